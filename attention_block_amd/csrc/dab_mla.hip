// Latent attention (MLA) decode over a latent cache: kernels, plan and C ABI
// (declared in include/dab.h).
//
// The ClusterFusion page (section 5.2) runs DeepSeek's latent attention by
// splitting the latent key/value cache across clusters and merging their
// partial results with a sparse reduction.  Here a chunk of one sequence's
// tokens is one workgroup, the partial softmax states go through memory and
// a second kernel merges them by log-sum-exp weights (the merge of the
// ClusterFusion page, section 3.2, written for a chunk count that varies per
// sequence).
//
// Every head of a sequence reads the same latent rows, so a chunk is a dense
// contraction: with nh = 128 heads, 2176 flops per 1152 bytes of cache.  The
// chunk kernel puts both products on the matrix cores
// (v_mfma_f32_16x16x32_bf16):
//   scores   S^T[t, h] = K[t, :] . Q[h, :]   A = 16 tokens x 32 dims of the
//            K rows [c_t | kr_t] from a token-major LDS tile, B = 16 heads'
//            query, held in registers for the whole chunk
//            (q * scale * log2 e, bf16);
//   values   O^T[r, h] += C^T[r, t] . P^T[t, h]   B = the weights, taken
//            straight from the score accumulators (a lane holds head l % 16,
//            tokens 4 (l / 16) + i of each 16-token tile: the k index of an
//            MFMA may be any fixed permutation, so these eight tokens are its
//            k slots), A = a transposed copy of the latent rows in LDS
//            ([dim][token], written from the load registers with 16-bit
//            stores), two 8-byte reads per fragment in that token order.
// A workgroup of four waves takes 64 heads (one wave: 16 heads where nh is
// not a multiple of 64); each wave owns a tile of 16 heads, its query
// fragments (72 registers) and its 16 x 512 output tile (128 accumulator
// registers).  Tokens go through LDS 32 at a time (rows of the token-major
// tile 1168 bytes apart, so that the 16 rows an operand read touches start
// 36 banks apart); with four waves the next 32 rows are requested into
// registers while a tile is computed, and the operand fragments of both
// products are read from LDS a few steps ahead of their MFMA.  The online
// softmax keeps a per-head reference that moves only when a score exceeds it
// by more than 2^8 (weights stay below 256, exact in fp32 and bf16), so the
// 512-wide output rows are rescaled almost never.
#include <hip/hip_runtime.h>
#include <math.h>

#include <atomic>

#include "dab.h"
#include "dab_mfma.h"

namespace dab {

dab_status record_hip_status(hipError_t e);    // the library's last-error record (dab_api.hip)

namespace mla {

using dev::as_bf16x8;
using dev::bf16x8;
using dev::f32x4;
using dev::u32x4;
using dev::lds_address;
using dev::lds_barrier;
using dev::lds_load16;
using dev::read_tr16;
using dev::wait_vm;

constexpr int kR = 512;                  // latent width
constexpr int kP = 64;                   // rotary key width
constexpr int kKD = kR + kP;             // score contraction: 576 = 18 steps of 32
constexpr int kSteps = kKD / 32;
constexpr int kDimTiles = kR / 16;       // output tiles of 16 latent dims
constexpr int kTB = 32;                  // tokens per LDS tile
constexpr int kCRow = kR + 8;            // bf16 per latent row of an LDS tile (1040 bytes: rows start 4 banks apart)
constexpr int kKrOff = kTB * kCRow;      // the tile's rotary keys follow its latent rows: 32 x 128 bytes, swizzled
constexpr int kTile = kKrOff + kTB * kP; // bf16 per LDS tile (37,376 bytes)
constexpr int kPieces = kKD / 8;         // 16-byte pieces per token row (64 latent + 8 rotary)
#ifndef DAB_MLA_DEPTH
#define DAB_MLA_DEPTH 4
#endif
constexpr int kDepth = DAB_MLA_DEPTH;    // operand fragments in flight (LDS reads ahead of their MFMA)
constexpr float kLazy = 8.f;             // the softmax reference moves when a score passes it by 2^8
constexpr int kMergeHeadThreads = 128;   // threads per head in the merge: four dims each
constexpr int kMaxHeads = 1024;
constexpr int kMaxChunk = 65536;

struct MlaArgs {
    const float* q_lat;       // [B, nh, R]
    const float* q_rope;      // [B, nh, P]
    const uint16_t* c_new;    // [B, R]
    const uint16_t* kr_new;   // [B, P]
    uint16_t* c_cache;        // [B, cap, R]
    uint16_t* kr_cache;       // [B, cap, P]
    const int32_t* pos;       // [B]
    float* out;               // [B, nh, R]
    float* part_ml;           // [B, splits, nh, 2]: (max, sum) per chunk and head, log2 units
    void* part_o;             // [B, splits, nh, R]: unnormalised weighted latent sums, fp32 or bf16 (below)
    int* err;                 // sticky device error flag
    int nh, cap, hblocks;     // heads, cache rows, workgroups of heads per chunk
    int splits;               // chunk slots per sequence (grid and partial layout)
    int fixed;                // > 0: every chunk has this many tokens
    int lmin;                 // automatic chunks: at least this many tokens
    float qscale;             // softmax_scale * log2(e)
};

// Tokens per chunk of a sequence of n attended tokens: a fixed length, or
// the shortest multiple of 32 that covers n in `splits` chunks, at least
// lmin.  Either way ceil(n / len) <= splits.
__host__ __device__ inline int chunk_len(int fixed, int splits, int lmin, int n) {
    if (fixed > 0) return fixed;
    int len = (n + splits - 1) / splits;
    len = len > lmin ? len : lmin;
    return (len + kTB - 1) / kTB * kTB;
}

__device__ inline bool seq_range(const MlaArgs& a, int b, int* p_out, int* len_out, int* nchunks_out) {
    const int p = a.pos[b];
    if (p < 0 || p >= a.cap) return false;
    const int n = p + 1;
    const int len = chunk_len(a.fixed, a.splits, a.lmin, n);
    *p_out = p;
    *len_out = len;
    *nchunks_out = (n + len - 1) / len;
    return true;
}

// Tiles of 32 token rows reach LDS by direct loads (global_load_lds_dwordx4:
// lane l's 16 bytes land at the LDS byte address in M0 + 16 l, no registers
// involved): one 64-lane load per 1 KB latent row, and one per eight tokens'
// 128-byte rotary keys, which sit together after the latent rows with their
// 16-byte pieces XOR-swizzled (piece q of token t at q ^ (t / 2 % 8)), so
// that the 16 rows an operand read touches hit distinct banks.  Each wave
// requests its share of the next tiles one load at a time between the MFMAs
// of a step: a direct load holds up its wave's issue for a while (~60 ns
// measured), long enough to stall the matrix cores if a tile's loads go out
// back to back.
// DEPTH tiles are in flight while one is computed, in DEPTH + 1 buffers.
// Each wave waits for its own loads with s_waitcnt vmcnt, then a bare
// s_barrier (inline asm, memory clobber: no fence, which would wait for every
// load in flight) makes the tile visible to all waves.  The direct loads are
// issued from inline asm: the compiler's builtin for them makes it wait for
// every one in flight (vmcnt(0)) before any LDS read it cannot prove
// disjoint, i.e. before every tile.  Rows past t1 read row t1 - 1 again;
// their weights are zero.
template <int NW>
struct TilePipe {
    static constexpr int DEPTH = NW >= 4 ? 3 : 1;
    static constexpr int NBUF = DEPTH + 1;
    static constexpr int TPW = kTB / NW;                   // latent rows each wave loads per tile
    static constexpr int KRW = kTB / 8 / NW > 0 ? kTB / 8 / NW : 1;   // rotary loads per wave (8 tokens each)
    static constexpr int PER_TILE = TPW + KRW;             // direct loads per wave and tile
    static_assert((DEPTH - 1) * PER_TILE <= 63, "vmcnt holds at most 63");
    static_assert(KRW * NW * 8 == kTB, "rotary loads must cover the tile");
};

// Chunk (sequence blockIdx.y; chunk s, head block hb from blockIdx.x).
// Workgroups are dispatched to the eight XCDs round-robin by linear index,
// so index x goes to XCD x % 8: slot x / 8 of an XCD takes head block
// slot % hblocks of chunk 8 (slot / hblocks) + x % 8, and the head blocks of
// one chunk run on one XCD one after the other, the later ones reading the
// chunk's rows from that XCD's L2.  gridDim.x is 8 hblocks ceil(splits / 8).
template <int NW, bool PB>
__global__ __launch_bounds__(64 * NW) void mla_chunk_kernel(MlaArgs a) {
    constexpr int NT = 64 * NW;
    constexpr int DEPTH = TilePipe<NW>::DEPTH, NBUF = TilePipe<NW>::NBUF, PT = TilePipe<NW>::PER_TILE;
    constexpr int TPW = TilePipe<NW>::TPW, KRW = TilePipe<NW>::KRW;
    __shared__ __attribute__((aligned(16))) uint16_t kt[NBUF][kTile];   // latent rows, then rotary keys

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int b = blockIdx.y, slot = blockIdx.x / 8;
    const int hb = slot % a.hblocks, s = slot / a.hblocks * 8 + blockIdx.x % 8;
    int p, len, nchunks;
    if (!seq_range(a, b, &p, &len, &nchunks)) {
        if (s == 0 && hb == 0 && t == 0) atomicOr(a.err, 1);
        return;
    }
    if (s >= nchunks) return;
    const int t0 = s * len, t1 = min(p + 1, t0 + len);
    const size_t row0 = (size_t)b * a.cap;
    const uint16_t* c_new = a.c_new + (size_t)b * kR;
    const uint16_t* kr_new = a.kr_new + (size_t)b * kP;

    // this wave's query fragments (head 16 (hb NW + wave) + m, dims 32 ks + 8 g .. + 8), requested first,
    // so that their latency runs under the issue of the first tiles' direct loads
    const int head = (hb * NW + wave) * 16 + m;
    f32x4 qraw[kSteps][2];
    {
        const size_t h = (size_t)b * a.nh + head;
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
            const int d = 32 * ks + 8 * g;
            const float* src = d < kR ? a.q_lat + h * kR + d : a.q_rope + h * kP + (d - kR);
            qraw[ks][0] = *reinterpret_cast<const f32x4*>(src);
            qraw[ks][1] = *reinterpret_cast<const f32x4*>(src + 4);
        }
    }

    // direct load i (0 <= i < PT) of this wave for tile j: latent row wave * TPW + i for i < TPW, else
    // the rotary keys of tokens 8 k .. 8 k + 7, k = wave * KRW + i - TPW (lane l: token 8 k + l / 8,
    // landing at piece l % 8, so it fetches piece (l % 8) ^ (token / 2 % 8))
    const uint32_t kt0 = lds_address(&kt[0][0]);
    auto issue = [&](int j, int i) {
        const uint32_t dst = kt0 + (uint32_t)(j % NBUF) * (kTile * 2);
        const int base = t0 + kTB * j;
        if (i < TPW) {
            const int r = wave * TPW + i;
            const int tok = min(base + r, t1 - 1);
            const uint16_t* cs = tok < p ? a.c_cache + (row0 + tok) * kR : c_new;
            lds_load16(cs + 8 * lane, dst + r * (kCRow * 2));
        } else {
            const int k = wave * KRW + (i - TPW), r = 8 * k + (lane >> 3);
            const int tok = min(base + r, t1 - 1);
            const uint16_t* ks = tok < p ? a.kr_cache + (row0 + tok) * kP : kr_new;
            lds_load16(ks + 8 * ((lane & 7) ^ ((r >> 1) & 7)), dst + kKrOff * 2 + 8 * k * (kP * 2));
        }
    };
    const int ntiles = (t1 - t0 + kTB - 1) / kTB;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (d < ntiles)
#pragma unroll
            for (int i = 0; i < PT; ++i) issue(d, i);

    bf16x8 qf[kSteps];
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
        const f32x4 x0 = qraw[ks][0], x1 = qraw[ks][1];
        const u32x4 v = {dev::pack_bf16x2(x0[0] * a.qscale, x0[1] * a.qscale),
                         dev::pack_bf16x2(x0[2] * a.qscale, x0[3] * a.qscale),
                         dev::pack_bf16x2(x1[0] * a.qscale, x1[1] * a.qscale),
                         dev::pack_bf16x2(x1[2] * a.qscale, x1[3] * a.qscale)};
        qf[ks] = as_bf16x8(v);
    }

    // the new token's rows are appended by the one workgroup whose chunk holds them (every chunk
    // reads the new token from c_new / kr_new, never from the cache row being written)
    if (hb == 0 && p >= t0 && p < t1) {
        for (int i = t; i < kPieces; i += NT) {
            if (i < kR / 8)
                *reinterpret_cast<u32x4*>(a.c_cache + (row0 + p) * kR + 8 * i) =
                    *reinterpret_cast<const u32x4*>(c_new + 8 * i);
            else
                *reinterpret_cast<u32x4*>(a.kr_cache + (row0 + p) * kP + 8 * (i - kR / 8)) =
                    *reinterpret_cast<const u32x4*>(kr_new + 8 * (i - kR / 8));
        }
    }

    f32x4 oacc[kDimTiles];
    float mref = -INFINITY, lsum = 0.f;
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int j = 0; j < ntiles; ++j) {
        // tile j has landed once at most min(DEPTH - 1, ntiles - 1 - j) later tiles' loads are in flight
        const int later = min(DEPTH - 1, ntiles - 1 - j);
        if constexpr (DEPTH >= 3) {
            if (later >= 2) wait_vm<2 * PT>();
            else if (later == 1) wait_vm<PT>();
            else wait_vm<0>();
        } else if constexpr (DEPTH == 2) {
            if (later >= 1) wait_vm<PT>();
            else wait_vm<0>();
        } else {
            wait_vm<0>();
        }
        lds_barrier();                     // every wave's loads of tile j are in; tile j - 1 is consumed
        const bool more = j + DEPTH < ntiles;    // tile j + DEPTH goes out during this tile's score steps
        const uint16_t* tile = kt[j % NBUF];

        // scores: S[token 16 tt + 4 g + i][head] = sum over e of sacc[e][tt][i] (the even and odd 32-dim
        // steps accumulate apart: four independent chains).  The K fragments of step ks + kDepth - 1
        // are requested while step ks is multiplied.
        f32x4 sacc[2][2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) sacc[e][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            bf16x8 fr[kDepth][2];
            auto read_k = [&](int ks, bf16x8 (&f)[2]) {
                if (ks < kR / 32) {
                    f[0] = as_bf16x8(*reinterpret_cast<const u32x4*>(tile + m * kCRow + 32 * ks + 8 * g));
                    f[1] = as_bf16x8(*reinterpret_cast<const u32x4*>(tile + (16 + m) * kCRow + 32 * ks + 8 * g));
                } else {
                    const int q = (4 * (ks - kR / 32) + g) ^ ((m >> 1) & 7);   // tokens m and 16 + m swizzle alike
                    f[0] = as_bf16x8(*reinterpret_cast<const u32x4*>(tile + kKrOff + m * kP + 8 * q));
                    f[1] = as_bf16x8(*reinterpret_cast<const u32x4*>(tile + kKrOff + (16 + m) * kP + 8 * q));
                }
            };
#pragma unroll
            for (int d = 0; d < kDepth - 1; ++d) read_k(d, fr[d]);
#pragma unroll
            for (int ks = 0; ks < kSteps; ++ks) {
                // this step's share of tile j + DEPTH's direct loads
#pragma unroll
                for (int i = ks * PT / kSteps; i < (ks + 1) * PT / kSteps; ++i)
                    if (more) issue(j + DEPTH, i);
                if (ks + kDepth - 1 < kSteps) read_k(ks + kDepth - 1, fr[(ks + kDepth - 1) % kDepth]);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    sacc[ks & 1][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[ks % kDepth][tt], qf[ks],
                                                                                sacc[ks & 1][tt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        sacc[0][0] += sacc[1][0];
        sacc[0][1] += sacc[1][1];

        // online softmax of this wave's heads; weights to bf16 in the k-slot order of the value product
        const int valid = t1 - t0 - kTB * j;           // tokens of this tile that are attended (>= 1)
        bf16x8 pf;
        {
            float mx = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * tt + 4 * g + i < valid) mx = fmaxf(mx, sacc[0][tt][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const bool move = mx > mref + kLazy;
            if (__ballot(move)) {
                const float mnew = move ? mx : mref;
                const float alpha = __builtin_amdgcn_exp2f(mref - mnew);   // 0 on the first tile
                lsum *= alpha;
#pragma unroll
                for (int dt = 0; dt < kDimTiles; ++dt) oacc[dt] *= alpha;
                mref = mnew;
            }
            uint32_t w[4];
            float rowsum = 0.f;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i2 = 0; i2 < 2; ++i2) {
                    float e[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int i = 2 * i2 + u;
                        e[u] = 16 * tt + 4 * g + i < valid ? __builtin_amdgcn_exp2f(sacc[0][tt][i] - mref) : 0.f;
                    }
                    w[2 * tt + i2] = dev::pack_bf16x2(e[0], e[1]);
                    // the sum takes the weights as rounded, so that they sum to the normaliser exactly
                    rowsum += __uint_as_float(w[2 * tt + i2] << 16) + __uint_as_float(w[2 * tt + i2] & 0xffff0000u);
                }
            lsum += rowsum;
            pf = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
        }

        // values: A = latent dim 16 dt + m of tokens 4 g + j, then 16 + 4 g + j (j = 0..3), two
        // transposing reads of the token-major tile: lane (m, g) addresses token 16 u + 4 g + m / 4,
        // dims 16 dt + 4 (m % 4) .. + 3.  The fragment of dim tile dt + kDepth - 1 is requested while
        // tile dt is multiplied.
        {
            bf16x8 fv[kDepth];
            auto read_c = [&](int dt) -> bf16x8 {
                // whole 64-bit results as two dwords each (per-element 16-bit extraction of the short4
                // result lost its upper dword in hipcc's code for gfx950)
                const uint16_t* at = tile + (4 * g + (m >> 2)) * kCRow + 16 * dt + 4 * (m & 3);
                const uint2 lo = __builtin_bit_cast(uint2, read_tr16(at));
                const uint2 hi = __builtin_bit_cast(uint2, read_tr16(at + 16 * kCRow));
                return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
            };
#pragma unroll
            for (int d = 0; d < kDepth - 1; ++d) fv[d] = read_c(d);
#pragma unroll
            for (int dt = 0; dt < kDimTiles; ++dt) {
                if (dt + kDepth - 1 < kDimTiles) fv[(dt + kDepth - 1) % kDepth] = read_c(dt + kDepth - 1);
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fv[dt % kDepth], pf, oacc[dt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // lane (m, g) holds dims 16 dt + 4 g + i of its head
    float l = lsum;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (nchunks == 1) {
        const float inv = 1.f / l;
        float* o = a.out + ((size_t)b * a.nh + head) * kR + 4 * g;
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) *reinterpret_cast<f32x4*>(o + 16 * dt) = oacc[dt] * inv;
    } else {
        const size_t sl = ((size_t)b * a.splits + s) * a.nh + head;
        if constexpr (PB) {
            uint16_t* o = static_cast<uint16_t*>(a.part_o) + sl * kR + 4 * g;
#pragma unroll
            for (int dt = 0; dt < kDimTiles; ++dt)
                *reinterpret_cast<uint2*>(o + 16 * dt) = uint2{dev::pack_bf16x2(oacc[dt][0], oacc[dt][1]),
                                                               dev::pack_bf16x2(oacc[dt][2], oacc[dt][3])};
        } else {
            float* o = static_cast<float*>(a.part_o) + sl * kR + 4 * g;
#pragma unroll
            for (int dt = 0; dt < kDimTiles; ++dt) *reinterpret_cast<f32x4*>(o + 16 * dt) = oacc[dt];
        }
        if (g == 0) {
            a.part_ml[2 * sl] = mref;
            a.part_ml[2 * sl + 1] = l;
        }
    }
}

// Merge of one sequence's chunks for one head (grid: nh x B), SUB sub-groups
// of 128 threads (four dims each): sub-group g takes chunks g, g + SUB, ...,
// PER of them per round, every statistic and partial row of a round requested
// together (and the first round with the position, for every chunk slot the
// workspace has: slots past the sequence's chunks are read and not used), so
// that the common case (up to SUB PER chunks) is one trip to memory.  Each
// sub-group keeps a running reference M_g (rescaling its sums when a round
// raises it), then the sub-groups' (M_g, sum, row) are combined in order
// through LDS.  (DeepSeek-V3 shape on MI355X, four sub-groups of 16: bs1 4K
// 6.9 -> 4.1 us, bs1 16K 19.8 -> 6.2 us against the former merge, maxima
// first and then the rows, 16 chunks at a time.)
template <int SUB, int PER, bool PB>
__global__ __launch_bounds__(SUB * kMergeHeadThreads) void mla_merge_kernel(MlaArgs a) {
    __shared__ float s_m[SUB], s_l[SUB];
    __shared__ f32x4 s_acc[SUB > 1 ? SUB - 1 : 1][kMergeHeadThreads];
    const int b = blockIdx.y, h = blockIdx.x;
    const int g = threadIdx.x / kMergeHeadThreads, i = threadIdx.x % kMergeHeadThreads, d = 4 * i;
    const size_t slot0 = (size_t)b * a.splits * a.nh + h, stride = a.nh;
    float mm[PER], ll[PER];
    f32x4 oo[PER];
    auto request = [&](int c0, int lim) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = c0 + g + SUB * u;
            if (c < lim) {                                  // past lim: never used
                const size_t slot = slot0 + (size_t)c * stride;
                mm[u] = a.part_ml[2 * slot];
                ll[u] = a.part_ml[2 * slot + 1];
                if constexpr (PB) {
                    const uint2 w2 = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.part_o) + slot * kR + d);
                    oo[u] = f32x4{__uint_as_float(w2.x << 16), __uint_as_float(w2.x & 0xffff0000u),
                                  __uint_as_float(w2.y << 16), __uint_as_float(w2.y & 0xffff0000u)};
                } else {
                    oo[u] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.part_o) + slot * kR + d);
                }
            }
        }
    };
    request(0, a.splits);
    int p, len, nchunks;
    if (!seq_range(a, b, &p, &len, &nchunks) || nchunks == 1) return;
    float M = -INFINITY, den = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nchunks; c0 += SUB * PER) {
        if (c0 > 0) request(c0, nchunks);
        float Mr = M;
#pragma unroll
        for (int u = 0; u < PER; ++u)
            if (c0 + g + SUB * u < nchunks) Mr = fmaxf(Mr, mm[u]);
        if (Mr > M) {                                      // the reference rises (always on the first round)
            const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mr);
            den *= r;
            acc *= r;
            M = Mr;
        }
#pragma unroll
        for (int u = 0; u < PER; ++u)
            if (c0 + g + SUB * u < nchunks) {
                const float w = __builtin_amdgcn_exp2f(mm[u] - M);
                den = fmaf(w, ll[u], den);
                acc += w * oo[u];
            }
    }
    if constexpr (SUB > 1) {
        // a sub-group without chunks (nchunks < SUB) keeps M = -inf and weighs 0 below; sub-group 0
        // always has chunk 0
        if (i == 0) {
            s_m[g] = M;
            s_l[g] = den;
        }
        if (g > 0) s_acc[g - 1][i] = acc;
        __syncthreads();
        if (g > 0) return;
        float Mt = M;
#pragma unroll
        for (int q = 1; q < SUB; ++q) Mt = fmaxf(Mt, s_m[q]);
        const float w0 = __builtin_amdgcn_exp2f(M - Mt);
        den *= w0;
        acc *= w0;
#pragma unroll
        for (int q = 1; q < SUB; ++q) {
            const float wq = s_m[q] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[q] - Mt);
            den = fmaf(wq, s_l[q], den);
            acc += wq * s_acc[q - 1][i];
        }
    }
    *reinterpret_cast<f32x4*>(a.out + ((size_t)b * a.nh + h) * kR + d) = acc * (1.f / den);
}

// ---------------------------------------------------------------------------
// host plan
// ---------------------------------------------------------------------------

struct MlaPlan {
    int B = 0, nh = 0, cap = 0, ht = 0, nw = 0, hblocks = 0, splits = 0, fixed = 0, lmin = 0;
    bool part_bf16 = false;   // partial rows stored in bf16
    float scale = 0.f;
    size_t off_ml = 0, off_o = 0, ws_bytes = 0;
};

// automatic chunks hold at least this many tokens (a chunk reads the query of all its heads, nh x 576
// values, once: as many bytes as ~250 cached tokens at nh = 128), and a sequence has at most
// kAutoMaxSplits of them (DeepSeek-V3 shape, batch 1, on MI355X with the sub-group merge: 4K in 128-token
// chunks 25.6 us against 30.7 in 256-token ones; 16K in 256-token chunks 35.5 us against 44.5 in 128)
constexpr int kAutoMinChunk = 128;
constexpr int kAutoMaxSplits = 64;

std::atomic<int> g_mla_cus[16];

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) {
        (void)hipGetLastError();
        return 0;
    }
    int cus = g_mla_cus[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
            (void)hipGetLastError();
            cus = -1;
        }
        g_mla_cus[dev].store(cus, std::memory_order_relaxed);
    }
    return cus > 0 ? cus : 0;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

dab_status make_plan(const dab_mla_config* cfg, MlaPlan* p) {
    if (!cfg) return DAB_ERR_INVALID_ARG;
    if (cfg->batch < 0 || cfg->n_heads <= 0 || cfg->cache_capacity <= 0 || !(cfg->softmax_scale > 0.f) ||
        !isfinite(cfg->softmax_scale) || cfg->kv_chunk < 0)
        return DAB_ERR_INVALID_ARG;
    if (cfg->kv_lora_rank != kR || cfg->rope_dim != kP || cfg->n_heads % 16 != 0 || cfg->n_heads > kMaxHeads)
        return DAB_ERR_UNSUPPORTED;
    if (cfg->kv_chunk != 0 && (cfg->kv_chunk % kTB != 0 || cfg->kv_chunk > kMaxChunk)) return DAB_ERR_UNSUPPORTED;
    if ((int64_t)cfg->batch * cfg->cache_capacity > (int64_t)1 << 31) return DAB_ERR_UNSUPPORTED;
    MlaPlan q;
    q.B = cfg->batch;
    q.nh = cfg->n_heads;
    q.cap = cfg->cache_capacity;
    q.scale = cfg->softmax_scale;
    // 64 heads per workgroup of four waves (two head tiles per wave spill at 512 registers), else
    // one wave of 16 heads
    q.ht = 1;
    // (A single sequence of at most 8192 tokens takes one-wave workgroups too: four times the
    // workgroups, each loading a quarter of the query, on more CUs; DeepSeek-V3 shape on MI355X, 4K:
    // 25.5 -> 22.0 us; at 16K the shared cache tiles pay more: 36.4 against 40.1 us.)
    q.nw = q.nh % 64 == 0 && !(q.B == 1 && q.cap <= 8192) ? 4 : 1;
    q.hblocks = q.nh / (16 * q.ht * q.nw);
    if (cfg->kv_chunk > 0) {
        q.fixed = cfg->kv_chunk;
        q.splits = (q.cap + q.fixed - 1) / q.fixed;
    } else {
        // one chunk workgroup per compute unit over the batch (the 128-head workgroup holds a
        // compute unit's registers), never more chunks than the capacity needs
        int cus = device_cus();
        if (cus <= 0) cus = 256;
        const int per_cu = q.nw == 1 ? 4 : 1;
        const int64_t wgs = (int64_t)q.B * q.hblocks;
        int sp = (int)(wgs > 0 ? ((int64_t)cus * per_cu + wgs - 1) / wgs : 1);
        const int most = min((q.cap + kAutoMinChunk - 1) / kAutoMinChunk, kAutoMaxSplits);
        sp = sp < 1 ? 1 : sp > most ? most : sp;
        q.splits = sp;
        q.lmin = kAutoMinChunk;
    }
    if ((int64_t)8 * q.hblocks * ((q.splits + 7) / 8) > (int64_t)1 << 30 || q.B > 65535) return DAB_ERR_UNSUPPORTED;
    q.off_ml = 256;
    const size_t slots = (size_t)q.B * q.splits * q.nh;
    q.off_o = align256(q.off_ml + slots * 2 * sizeof(float));
    // many heads (batch 16): the partial rows in bf16, half their traffic (DeepSeek-V3 shape, batch 16, on
    // MI355X: 56.5 -> 54.4 us); at batch 1 the merge of bf16 rows measured slower (16K: 4.6 -> 7.5 us)
    q.part_bf16 = (int64_t)q.B * q.nh >= 1024;
    q.ws_bytes = align256(q.off_o + slots * kR * (q.part_bf16 ? sizeof(uint16_t) : sizeof(float)));
    *p = q;
    return DAB_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

dab_status hip_status(hipError_t e) { return record_hip_status(e); }

template <typename K>
hipError_t launch(K kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t start, hipEvent_t stop, MlaArgs a) {
    void* args[] = {&a};
    const void* f = reinterpret_cast<const void*>(kernel);
    if (start || stop) return hipExtLaunchKernel(f, grid, block, args, 0, s, start, stop, 0);
    return hipLaunchKernel(f, grid, block, args, 0, s);
}

dab_status call(const dab_mla_config* cfg, const float* q_lat, const float* q_rope, const void* c_new,
                const void* kr_new, void* c_cache, void* kr_cache, const int32_t* pos, float* out, void* workspace,
                size_t workspace_bytes, void* stream, void* const* events, int n_events) {
    MlaPlan p;
    dab_status st = make_plan(cfg, &p);
    if (st != DAB_OK) return st;
    if (!workspace) return DAB_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DAB_ERR_INVALID_ARG;
    if (workspace_bytes < p.ws_bytes) return DAB_ERR_WORKSPACE;
    if (events) {
        if (n_events != 4) return DAB_ERR_INVALID_ARG;
        for (int i = 0; i < 4; ++i)
            if (!events[i]) return DAB_ERR_INVALID_ARG;
    }
    if (p.B == 0) return DAB_OK;
    const void* req[] = {q_lat, q_rope, c_new, kr_new, c_cache, kr_cache, out};
    for (const void* r : req)
        if (!r || !aligned(r, 16)) return DAB_ERR_INVALID_ARG;
    if (!pos || !aligned(pos, 4)) return DAB_ERR_INVALID_ARG;
    const size_t B = p.B, nh = p.nh, cap = p.cap;
    struct Span { const void* ptr; size_t n; bool written; };
    const Span spans[] = {
        {q_lat, B * nh * kR * 4, false}, {q_rope, B * nh * kP * 4, false}, {c_new, B * kR * 2, false},
        {kr_new, B * kP * 2, false},     {pos, B * 4, false},             {c_cache, B * cap * kR * 2, true},
        {kr_cache, B * cap * kP * 2, true}, {out, B * nh * kR * 4, true}, {workspace, p.ws_bytes, true},
    };
    const int ns = (int)(sizeof(spans) / sizeof(spans[0]));
    for (int i = 0; i < ns; ++i)
        for (int j = i + 1; j < ns; ++j)
            if ((spans[i].written || spans[j].written) && overlaps(spans[i].ptr, spans[i].n, spans[j].ptr, spans[j].n))
                return DAB_ERR_INVALID_ARG;

    MlaArgs a{};
    a.q_lat = q_lat;
    a.q_rope = q_rope;
    a.c_new = static_cast<const uint16_t*>(c_new);
    a.kr_new = static_cast<const uint16_t*>(kr_new);
    a.c_cache = static_cast<uint16_t*>(c_cache);
    a.kr_cache = static_cast<uint16_t*>(kr_cache);
    a.pos = pos;
    a.out = out;
    char* ws = static_cast<char*>(workspace);
    a.err = reinterpret_cast<int*>(ws);                 // the flags word at offset 0 of every workspace
    a.part_ml = reinterpret_cast<float*>(ws + p.off_ml);
    a.part_o = ws + p.off_o;
    a.nh = p.nh;
    a.cap = p.cap;
    a.hblocks = p.hblocks;
    a.splits = p.splits;
    a.fixed = p.fixed;
    a.lmin = p.lmin;
    a.qscale = p.scale * 1.4426950408889634f;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if (events)
        for (int i = 0; i < 4; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
    const dim3 grid((unsigned)(8 * p.hblocks * ((p.splits + 7) / 8)), (unsigned)p.B);
    hipError_t e;
    if (p.nw == 4 && p.part_bf16) e = launch(mla_chunk_kernel<4, true>, grid, dim3(256), s, ev[0], ev[1], a);
    else if (p.nw == 4) e = launch(mla_chunk_kernel<4, false>, grid, dim3(256), s, ev[0], ev[1], a);
    else if (p.part_bf16) e = launch(mla_chunk_kernel<1, true>, grid, dim3(64), s, ev[0], ev[1], a);
    else e = launch(mla_chunk_kernel<1, false>, grid, dim3(64), s, ev[0], ev[1], a);
    if (e == hipSuccess) e = hipGetLastError();
    if ((st = hip_status(e)) != DAB_OK) return st;
    // few heads (batch 1): four sub-groups of 16 chunks a round; many heads: one of 8
    if ((int64_t)p.B * p.nh < 1024)
        e = launch(mla_merge_kernel<4, 16, false>, dim3((unsigned)p.nh, (unsigned)p.B), dim3(4 * kMergeHeadThreads), s,
                   ev[2], ev[3], a);
    else
        e = launch(mla_merge_kernel<1, 8, true>, dim3((unsigned)p.nh, (unsigned)p.B), dim3(kMergeHeadThreads), s, ev[2],
                   ev[3], a);
    if (e == hipSuccess) e = hipGetLastError();
    return hip_status(e);
}

}  // namespace mla
}  // namespace dab

extern "C" {

size_t dab_mla_workspace_size(const dab_mla_config* cfg) {
    dab::mla::MlaPlan p;
    return dab::mla::make_plan(cfg, &p) == DAB_OK ? p.ws_bytes : 0;
}

dab_status dab_mla_decode_attn(const dab_mla_config* cfg, const float* q_lat, const float* q_rope, const void* c_new,
                               const void* kr_new, void* c_cache, void* kr_cache, const int32_t* pos, float* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return dab::mla::call(cfg, q_lat, q_rope, c_new, kr_new, c_cache, kr_cache, pos, out, workspace, workspace_bytes,
                          stream, nullptr, 0);
}

dab_status dab_mla_decode_attn_timed(const dab_mla_config* cfg, const float* q_lat, const float* q_rope,
                                     const void* c_new, const void* kr_new, void* c_cache, void* kr_cache,
                                     const int32_t* pos, float* out, void* workspace, size_t workspace_bytes,
                                     void* stream, void* const* events, int n_events) {
    if (!events) return DAB_ERR_INVALID_ARG;
    return dab::mla::call(cfg, q_lat, q_rope, c_new, kr_new, c_cache, kr_cache, pos, out, workspace, workspace_bytes,
                          stream, events, n_events);
}

}  // extern "C"

// Device code of the decode attention block (gfx950, wave64) shared by the
// kernels of the step.
//
// Work items:
//   QKV panel         (dab_gemv.h) four RoPE pairs of W_qkv rows for up to
//                     four sequences, all of K: RMSNorm folded in as a scale,
//                     RoPE, q and the new k/v written out, k/v appended to
//                     the caches.
//   attention chunk   (sequence b, kv head g, chunk c of 32..256 tokens):
//                     each K and V row is read once for the G query heads of
//                     the group; online softmax; the chunk's (max, sum,
//                     weighted values) are published and the last chunk of
//                     (b, g) merges them with log-sum-exp weights.
//   O panel           (dab_gemv.h) four W_o rows, all of K, plus the residual.
//
// The split of attention into chunks, and their hand-off through the
// memory-side cache, replace the thread-block clusters and the distributed
// shared memory reductions (ClusterReduce / ClusterGather) of the
// ClusterFusion page, sections 3.1-3.2: gfx950 has no distributed shared
// memory, so partials go through the Infinity Cache with device-coherent
// stores and loads, the cross-cluster route that page lists as future work
// (section 6).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dab_kernels.h"

namespace dab {
namespace dev {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
// Online softmax: how far (log2 units) a score may exceed the reference a
// chunk's weights are taken against before the reference moves.
constexpr float kRescaleSlack = 8.f;

// Profiling builds (-DDAB_TRACE) record a 100 MHz timestamp per workgroup at
// up to eight points: 0 start, 1 loads issued, 2 inputs staged, 3 end; in
// the workgroup that merges a group: 4 its start, 5 its loads issued, 6 its
// results published.
#ifdef DAB_TRACE
#define DAB_TRACE_POINT(args, slot) \
    do { if (threadIdx.x == 0 && (args).trace) \
        (args).trace[((args).trace_base + blockIdx.x) * 8 + (slot)] = __builtin_amdgcn_s_memrealtime(); } while (0)
#else
#define DAB_TRACE_POINT(args, slot) do { } while (0)
#endif

// ---------------------------------------------------------------------------
// element access: 8 consecutive elements per lane
// ---------------------------------------------------------------------------

template <typename T> struct Vec8;

template <> struct Vec8<uint16_t> {            // bf16: one 16-byte load
    u32x4 r;
    __device__ void load(const uint16_t* p) { r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
    __device__ void zero() { r = u32x4{0u, 0u, 0u, 0u}; }
    __device__ void unpack(float* f) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(r[i] << 16);
            f[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
        }
    }
    __device__ void pack(const float* f) {      // nearest-even, as stored
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)f[2 * i]);
            const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)f[2 * i + 1]);
            r[i] = lo | (hi << 16);
        }
    }
};

template <> struct Vec8<float> {               // fp32: two 16-byte loads
    f32x4 a, b;
    __device__ void load(const float* p) {
        a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
    }
    __device__ void zero() { a = f32x4{0.f, 0.f, 0.f, 0.f}; b = a; }
    __device__ void unpack(float* f) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
    }
    __device__ void pack(const float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { a[i] = f[i]; b[i] = f[4 + i]; }
    }
};

__device__ inline float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ inline float to_f32(float v) { return v; }

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 (nearest-even), lo in the low half.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// a.lo * b.lo + a.hi * b.hi + c over packed bf16 pairs (v_dot2c_f32_bf16).
__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c, false);
}

template <typename T> __device__ inline T from_f32(float f);
template <> __device__ inline float from_f32<float>(float f) { return f; }
template <> __device__ inline uint16_t from_f32<uint16_t>(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);   // v_cvt_pk_bf16_f32: nearest-even
}

// ---------------------------------------------------------------------------
// cross-lane reductions
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ inline float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR lanes (8 or 16); every lane of a group gets the sum.
template <int LPR>
__device__ inline float group_sum(float v) {
    v += dpp<0xB1>(v);                    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);                    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);                   // row_half_mirror: the two quads of a half row
    if (LPR == 16) v += dpp<0x140>(v);    // row_mirror: the two halves of a row
    return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// Weights of two online-softmax states (log2 units) relative to their max.
__device__ inline void lse_weights(float m1, float m2, float* w1, float* w2, float* mout) {
    const float M = fmaxf(m1, m2);
    const float Ms = M == kNegInf ? 0.f : M;
    *w1 = __builtin_amdgcn_exp2f(m1 - Ms);
    *w2 = __builtin_amdgcn_exp2f(m2 - Ms);
    *mout = M;
}

// ---------------------------------------------------------------------------
// hand-off between workgroups of one launch
// ---------------------------------------------------------------------------
//
// The eight XCD L2 caches are not coherent with one another.  An agent-scope
// fence would make every workgroup write back its L2 (buffer_wbl2, ~1 us,
// serialised per XCD).  Instead every value handed to another workgroup is
// stored and loaded with device-scope coherence (relaxed agent-scope atomic
// stores and loads: global_store / global_load ... sc1, which write through
// and read past the non-coherent L2).  A producer waits until its stores are
// acknowledged (s_waitcnt 0), meets its workgroup at a barrier, and one
// thread bumps a counter; consumers read the counter and then the data with
// sc1 loads.

__device__ inline void publish(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float fetch(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two consecutive published floats (8-byte aligned) in one device-coherent load.
__device__ inline void fetch2(const float* p, float* out) {
    const uint64_t w = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    out[0] = __uint_as_float((uint32_t)w);
    out[1] = __uint_as_float((uint32_t)(w >> 32));
}

// Two adjacent storage values (4- or 8-byte aligned) in one device-coherent store.
__device__ inline void publish_pair(uint16_t* p, uint16_t v0, uint16_t v1) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), (uint32_t)v0 | ((uint32_t)v1 << 16), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void publish_pair(float* p, float v0, float v1) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p),
                       (uint64_t)__float_as_uint(v0) | ((uint64_t)__float_as_uint(v1) << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes of published data in two device-coherent loads.
__device__ inline void fetch16(const void* p, uint32_t* w) {
    const uint64_t* q = static_cast<const uint64_t*>(p);
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w[0] = (uint32_t)lo;
    w[1] = (uint32_t)(lo >> 32);
    w[2] = (uint32_t)hi;
    w[3] = (uint32_t)(hi >> 32);
}

__device__ inline int load_counter(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline int bump(int* p) {
    return __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// +1 with no reply requested (the result is unused, so no return trip).
__device__ inline void add_counter(int* p) {
    (void)__hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void set_counter(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread's published stores are acknowledged, then the workgroup meets.
__device__ inline void drain_and_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // keeps the compiler from sinking stores
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// Thread-level bounded wait until *p >= target, SLEEP x 64 cycles between
// polls.  The bound (at least 0.2 s) cannot be reached in a correct run; if it is, bit 1 of the error flags is
// raised and the caller carries on, so every wave still exits.
constexpr int kSpinLimit = 1 << 21;
template <int SLEEP = 4>
__device__ inline void wait_at_least(const int* p, int target, int* flags) {
    for (int it = 0; it < kSpinLimit; ++it) {
        if (load_counter(p) >= target) return;
        __builtin_amdgcn_s_sleep(SLEEP);
    }
    __hip_atomic_fetch_or(flags, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival at a counter shared by `expected` workgroups; true in exactly one
// workgroup, the last to arrive, which also re-arms the counter for the next
// call.  Every thread's published stores are acknowledged first, so the last
// arriver sees all of them.
__device__ inline bool arrive_last(int* counter, int expected, int* s_flag) {
    drain_and_sync();
    if (threadIdx.x == 0) {
        const int prev = bump(counter);
        const bool last = prev == expected - 1;
        *s_flag = last;
        if (last) set_counter(counter, 0);
    }
    __syncthreads();
    return *s_flag != 0;
}

// Each sequence's split-KV chunk length and count, for the attention
// launches that follow (workgroup 0 of the QKV kernel): the rule's integer
// divisions are evaluated once per sequence instead of in front of every
// chunk's first loads.  Invalid positions get a count of 0; nothing reads it.
__device__ inline void publish_seq_chunks(const StepArgs& a) {
    if (!a.seq_chunk || blockIdx.x != 0) return;
    for (int b = threadIdx.x; b < a.B; b += blockDim.x) {
        const int p = a.pos[b];
        int len = 0, n = 0;
        if (p >= 0 && p < a.pos_end) {
            len = chunk_len(a.chunk, p);
            n = p > 0 ? (p + len - 1) / len : 1;
        }
        a.seq_chunk[2 * b] = len;
        a.seq_chunk[2 * b + 1] = n;
    }
}

// A sequence's chunk length and count: from the QKV kernel's table where
// there is one (request it before the position, so both loads overlap), else
// from the rule.
struct SeqChunk {
    int len, n;
};
__device__ inline SeqChunk seq_chunk_of(const StepArgs& a, int b, int p, const int2* pre) {
    if (pre) return SeqChunk{pre->x, pre->y};
    const int len = chunk_len(a.chunk, p);
    return SeqChunk{len, p > 0 ? (p + len - 1) / len : 1};
}

// A sequence's position is in the cache and within the max_position hint.
__device__ inline bool pos_valid(const StepArgs& a, int b, int* p_out) {
    const int p = a.pos[b];
    *p_out = p;
    return p >= 0 && p < a.pos_end;
}

// ---------------------------------------------------------------------------
// split-KV attention chunks
// ---------------------------------------------------------------------------
//
// LPR = D/8 lanes hold one token row (8 elements each); the workgroup's
// NSLOT = 256/LPR row slots each take U tokens of a buffer of HB = NSLOT * U
// tokens.  With grouped heads two half-batch buffers are in flight, the next
// requested before the current one is used, so a chunk of many half-batches
// streams without a round trip between them (see AttnGeom).  Scores are kept in log2 units (q is
// pre-scaled by log2(e)/sqrt(D)), so every exponential is an exp2.  The new
// token never comes from the cache: its k and v are taken from the fp32
// workspace copy the QKV kernel wrote, rounded to the storage type exactly
// as the appended row.

template <int D, int G>
struct AttnShared {
    float m[4][G], l[4][G];
    float o[4][G][D];
    float w[G][kMaxChunks];      // merge: chunk maxima, then their weights exp2(m - M)
    float cl[G][kMaxChunks];     // merge: chunk sums
    float red[4][G];
    float L[G];
    float acc[256 / D][G * D];   // merge: per-part weighted sums
};

template <int D, int G>
struct AttnGeom {
    static constexpr int LPR = D / 8;
    static constexpr int NSLOT = 256 / LPR;
    // One query head per kv head: one buffer of 8 tokens per slot, loaded,
    // used, then the next loaded (a 7B-sized step's chunks are one such
    // batch, and the single copy of the loop body measured faster there).
    // Grouped heads: two half-batch buffers of 4 tokens per slot (2 with
    // four or more heads, whose scores and accumulators take the
    // registers), the next requested before the current one is used.
    static constexpr bool PIPE = G > 1;
    static constexpr int U = G == 1 ? 8 : G >= 4 ? 2 : 4;
    static constexpr int HB = NSLOT * U;      // tokens per buffer (128 for D = 128, G = 1)
};

// 8 consecutive fp32 values of the workspace (32-byte aligned).  COHERENT:
// written in this launch by another workgroup, so read past the L2; else
// plain loads (the kernel boundary orders them after their writer).
template <bool COHERENT>
__device__ inline void load8(const float* p, float* f) {
    if constexpr (COHERENT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fetch2(p + 2 * i, f + 2 * i);
    } else {
        const f32x4 lo = reinterpret_cast<const f32x4*>(p)[0];
        const f32x4 hi = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[i] = lo[i]; f[4 + i] = hi[i]; }
    }
}

// Log-sum-exp merge of the chunk partials of (sequence b, kv group g) for its
// G query heads, by the chunk that arrived last: statistics first (one
// request per chunk and head), then the weighted outputs, every load of a
// round requested before any is used; deterministic (fixed order).
template <typename T, int D, int G, bool PUBLISH>
__device__ void merge_group(const StepArgs& a, int b, int g, int nchunk, AttnShared<D, G>& sm) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int nkv = a.nkv;
    DAB_TRACE_POINT(a, 4);
    const size_t pbase = ((size_t)b * a.nq + g * G) * a.maxc;   // head j, chunk cc: pbase + j * maxc + cc
    // thread (part, d) sums chunks part, part + PARTS, ... of every head, QB
    // chunks of each head per round (32 loads in flight); the first round is
    // requested together with the statistics
    constexpr int PARTS = 256 / D;
    constexpr int QB = merge_round(G);
    const int d = t % D, part = t / D;
    auto request = [&](int q0, float (&v)[G][QB]) {
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
            for (int q = 0; q < QB; ++q) {
                const int cc = part + (q0 + q) * PARTS;
                v[j][q] = cc < nchunk ? fetch(a.attn_o + (pbase + (size_t)j * a.maxc + cc) * D + d) : 0.f;
            }
    };
    float ml0[2] = {kNegInf, 0.f};
    if (t < G * nchunk) {
        const int j = t / nchunk, cc = t - j * nchunk;
        fetch2(a.attn_ml + (pbase + (size_t)j * a.maxc + cc) * 2, ml0);
    }
    float v0[G][QB];
    request(0, v0);
    if (t < G * nchunk) {
        const int j = t / nchunk, cc = t - j * nchunk;
        sm.w[j][cc] = ml0[0];
        sm.cl[j][cc] = ml0[1];
    }
    for (int idx = t + 256; idx < G * nchunk; idx += 256) {
        const int j = idx / nchunk, cc = idx - j * nchunk;
        float ml[2];
        fetch2(a.attn_ml + (pbase + (size_t)j * a.maxc + cc) * 2, ml);
        sm.w[j][cc] = ml[0];
        sm.cl[j][cc] = ml[1];
    }
    __syncthreads();
    DAB_TRACE_POINT(a, 5);
    // per head: M = max of the chunk maxima, weights exp2(m - M), L = sum w l
    float mx[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        float v = kNegInf;
        for (int cc = t; cc < nchunk; cc += 256) v = fmaxf(v, sm.w[j][cc]);
        mx[j] = wave_max(v);
        if (lane == 0) sm.red[wave][j] = mx[j];
    }
    __syncthreads();
    float lsum[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const float M = fmaxf(fmaxf(sm.red[0][j], sm.red[1][j]), fmaxf(sm.red[2][j], sm.red[3][j]));
        float v = 0.f;
        for (int cc = t; cc < nchunk; cc += 256) {
            const float w = __builtin_amdgcn_exp2f(sm.w[j][cc] - M);   // every chunk has a token: m finite
            v += w * sm.cl[j][cc];
            sm.w[j][cc] = w;
        }
        lsum[j] = wave_sum(v);
    }
    __syncthreads();                     // weights visible, sm.red read by everyone
#pragma unroll
    for (int j = 0; j < G; ++j)
        if (lane == 0) sm.red[wave][j] = lsum[j];
    // outputs, in fixed chunk order
    float acc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = 0.f;
    for (int q0 = 0; part + q0 * PARTS < nchunk; q0 += QB) {
        float v[G][QB];
        if (q0 == 0) {
#pragma unroll
            for (int j = 0; j < G; ++j)
#pragma unroll
                for (int q = 0; q < QB; ++q) v[j][q] = v0[j][q];
        } else {
            request(q0, v);
        }
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
            for (int q = 0; q < QB; ++q) {
                const int cc = part + (q0 + q) * PARTS;
                if (cc < nchunk) acc[j] += sm.w[j][cc] * v[j][q];
            }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) sm.acc[part][j * D + d] = acc[j];
    __syncthreads();
    for (int idx = t; idx < G * D; idx += 256) {
        const int j = idx / D;
        const float L = sm.red[0][j] + sm.red[1][j] + sm.red[2][j] + sm.red[3][j];
        float tot = 0.f;
#pragma unroll
        for (int q = 0; q < PARTS; ++q) tot += sm.acc[q][idx];
        const size_t ai = (size_t)b * a.n_q + (size_t)g * G * D + idx;   // head g*G + j, dim idx % D
        if constexpr (PUBLISH) {
            publish(a.a + ai, tot / L);
        } else {
            a.a[ai] = tot / L;
            if constexpr (sizeof(T) == 2) a.a16[ai] = from_f32<uint16_t>(tot / L);   // input of the MFMA projection
        }
    }
    if constexpr (PUBLISH) {
        // one more kv group of sequence b merged: once its output is stored
        // and acknowledged, every copy of the sequence's ready count goes up
        // by one (no reply awaited); the projection waits for nkv
        drain_and_sync();
        if (t < a.ready_copies) add_counter(&a.seq_ready[(b * kReadyCopies + t) * kReadyStride]);
    }
    DAB_TRACE_POINT(a, 6);
}

// PUBLISH: the output projection runs in the same launch, so the merged
// output is stored device-coherently and, once every head of the group is
// stored and acknowledged, the sequence's merge counter is bumped.
// WAITQ: the QKV projection runs in the same launch; after the first K/V
// loads are issued, wait until every panel of the group's q heads is done
// and read q device-coherently; the chunk that takes the new token waits for
// the panels of the group's k and v heads only before that token.
template <typename T, int D, int G, bool PUBLISH, bool WAITQ>
__device__ void attn_item(const StepArgs& a, int b, int g, int c, AttnShared<D, G>& sm, int* s_flag) {
    using Geo = AttnGeom<D, G>;
    constexpr int LPR = Geo::LPR, NSLOT = Geo::NSLOT, U = Geo::U, HB = Geo::HB;
    const int nkv = a.nkv;
    int2 pre;
    if (a.seq_chunk) pre = reinterpret_cast<const int2*>(a.seq_chunk)[b];
    int p;
    if (!pos_valid(a, b, &p)) return;
    // chunks cover the p cached tokens; the last one also takes the new token
    const SeqChunk sc = seq_chunk_of(a, b, p, a.seq_chunk ? &pre : nullptr);
    const int len = sc.len, nchunk = sc.n;             // this sequence's chunk length and count
    if (c >= nchunk) return;
    const int t0 = c * len;
    const int t1 = min(t0 + len, p);
    const bool has_new = c == nchunk - 1;
    const int nhb = (t1 - t0 + HB - 1) / HB;          // buffers of HB tokens (0 when there is no history)

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int slot = t / LPR, l = t % LPR;
    const size_t row = (size_t)nkv * D;
    const size_t base = ((size_t)b * a.cap * nkv + g) * D + l * 8;
    const T* Kp = static_cast<const T*>(a.k_cache) + base;
    const T* Vp = static_cast<const T*>(a.v_cache) + base;

    // 1. the first buffer(s) of history rows in flight
    Vec8<T> kA[U], vA[U], kB[U], vB[U];
    auto issue = [&](Vec8<T> (&kr)[U], Vec8<T> (&vr)[U], int hb0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tok = hb0 + slot + NSLOT * u;
            if (tok < t1) {
                kr[u].load(Kp + (size_t)tok * row);
                vr[u].load(Vp + (size_t)tok * row);
            } else {
                kr[u].zero();
                vr[u].zero();
            }
        }
    };
    issue(kA, vA, t0);
    if constexpr (Geo::PIPE) issue(kB, vB, t0 + HB);
    DAB_TRACE_POINT(a, 1);

    // 2. q of this group's heads, in log2 units
    // panel counts of this sequence's heads (panels per head: 4 RoPE pairs each)
    const int* hcnt = a.head_cnt + (a.head_cnt_per_seq ? b : b / a.qkv.nb) * (a.nq + 2 * nkv);
    if constexpr (WAITQ) {
        if (t == 0)
            for (int j = 0; j < G; ++j) wait_at_least<2>(hcnt + g * G + j, D / 8, a.flags);
        __syncthreads();
    }
    float qv[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        load8<WAITQ>(a.q + (size_t)b * a.n_q + (size_t)(g * G + j) * D + l * 8, qv[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[j][e] *= a.qscale;
    }
    // Grouped heads over a bf16 cache: scores and values by bf16 pair dot
    // products (v_dot2c_f32_bf16, fp32 accumulation), K and V used as they
    // are stored, q rounded to bf16 once per chunk, the weights p rounded to
    // bf16 for the values (each a relative 2^-9); the vector ALUs bound this
    // loop, and the unpacking and the separate multiplies were a third of it.
    constexpr bool DOT2 = sizeof(T) == 2 && G > 1;
    uint32_t qp[DOT2 ? G : 1][4];
    if constexpr (DOT2) {
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) qp[j][i] = pack_bf16x2(qv[j][2 * i], qv[j][2 * i + 1]);
    }
    // this lane's part of head j's score for a token row
    auto score = [&](const Vec8<T>& k, int j) {
        float d = 0.f;
        if constexpr (DOT2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) d = dot2_bf16(k.r[i], qp[j][i], d);
        } else {
            float kf[8];
            k.unpack(kf);
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf(qv[j][e], kf[e], d);
        }
        return d;
    };
    DAB_TRACE_POINT(a, 2);
    float m[G], ls[G], o[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = kNegInf;
        ls[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
    }

    // online-softmax update of this slot's state with its first nvalid
    // scores / value rows (nvalid >= 1)
    // Grouped heads: m[j] is the reference the weights are taken against, not
    // necessarily the running maximum: it moves (and l, o are rescaled) only
    // when a score exceeds it by more than kRescaleSlack, decided for the
    // whole wave at once, so most buffers skip the rescale (the 8B GQA layer
    // at batch 16: attention 56.3 -> 53.4 us on MI355X); every weight stays
    // below 2^kRescaleSlack.  One query head per kv head keeps the plain
    // update (m the running maximum): the 7B step measured 0.25 us slower
    // with the vote.
    auto absorb = [&](float (&s)[G][U], Vec8<T> (&vv)[U], int nvalid) {
        if constexpr (G == 1) {
            float mx = m[0];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (u < nvalid) mx = fmaxf(mx, s[0][u]);
            // at least one score is valid, so mx is finite here
            const float alpha = __builtin_amdgcn_exp2f(m[0] - mx);
            float pu[U], psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pu[u] = u < nvalid ? __builtin_amdgcn_exp2f(s[0][u] - mx) : 0.f;
                psum += pu[u];
            }
            ls[0] = ls[0] * alpha + psum;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[0][e] *= alpha;
            m[0] = mx;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u < nvalid) {
                    float vf[8];
                    vv[u].unpack(vf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[0][e] = fmaf(pu[u], vf[e], o[0][e]);
                }
            }
            return;
        }
        float mx[G];
        bool up = false;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            mx[j] = m[j];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (u < nvalid) mx[j] = fmaxf(mx[j], s[j][u]);
            up |= mx[j] > m[j] + kRescaleSlack;        // true for a first score (m = -inf)
        }
        if (__any(up)) {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                // at least one score is valid, so mx is finite here
                const float alpha = __builtin_amdgcn_exp2f(m[j] - mx[j]);
                ls[j] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[j][e] *= alpha;
                m[j] = mx[j];
            }
        }
        float pu[G][U];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pu[j][u] = u < nvalid ? __builtin_amdgcn_exp2f(s[j][u] - m[j]) : 0.f;
                psum += pu[j][u];
            }
            ls[j] += psum;
        }
        if constexpr (DOT2) {
            // token pairs (u, u + 1): their dims interleaved once for all heads
            // (rows past the valid ones are zeros with weight 0)
#pragma unroll
            for (int u = 0; u < U; u += 2) {
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t a0 = vv[u].r[i], a1 = vv[u + 1].r[i];
                    lo[i] = (a0 & 0xffffu) | (a1 << 16);            // dim 2i of both tokens
                    hi[i] = (a0 >> 16) | (a1 & 0xffff0000u);        // dim 2i + 1
                }
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    const uint32_t pp = pack_bf16x2(pu[j][u], pu[j][u + 1]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        o[j][2 * i] = dot2_bf16(pp, lo[i], o[j][2 * i]);
                        o[j][2 * i + 1] = dot2_bf16(pp, hi[i], o[j][2 * i + 1]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < G; ++j)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (u < nvalid) {
                        float vf[8];
                        vv[u].unpack(vf);
#pragma unroll
                        for (int e = 0; e < 8; ++e) o[j][e] = fmaf(pu[j][u], vf[e], o[j][e]);
                    }
                }
        }
    };

    // scores of one buffer starting at token hb0, then the update; every
    // lane of the workgroup runs it (the trip count is uniform), the lanes of
    // a slot agree on how many of its tokens are valid
    auto process = [&](Vec8<T> (&kr)[U], Vec8<T> (&vr)[U], int hb0) {
        float s[G][U];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < G; ++j) s[j][u] = group_sum<LPR>(score(kr[u], j));
        const int left = t1 - hb0 - slot;                  // this slot's tokens hb0 + slot + NSLOT*u < t1
        const int nvalid = left <= 0 ? 0 : min(U, (left + NSLOT - 1) / NSLOT);
        if (nvalid > 0) absorb(s, vr, nvalid);
    };

    if constexpr (Geo::PIPE) {
        for (int k = 0; k < nhb; k += 2) {
            process(kA, vA, t0 + k * HB);
            if (k + 2 < nhb) issue(kA, vA, t0 + (k + 2) * HB);
            if (k + 1 < nhb) {
                process(kB, vB, t0 + (k + 1) * HB);
                if (k + 3 < nhb) issue(kB, vB, t0 + (k + 3) * HB);
            }
        }
    } else {
        for (int k = 0; k < nhb; ++k) {
            if (k > 0) issue(kA, vA, t0 + k * HB);
            process(kA, vA, t0 + k * HB);
        }
    }

    // the new token, in slot 0 of the last chunk: its k and v come from the
    // workspace copy the QKV kernel wrote, rounded to the storage type
    // exactly as the appended cache row
    if constexpr (WAITQ) {
        if (has_new) {
            if (t == 0) {
                wait_at_least<2>(hcnt + a.nq + g, D / 8, a.flags);
                wait_at_least<2>(hcnt + a.nq + nkv + g, D / 8, a.flags);
            }
            __syncthreads();
        }
    }
    if (has_new && slot == 0) {
        const size_t kn = ((size_t)b * 2 * nkv + g) * D + l * 8;
        const size_t vn = kn + (size_t)nkv * D;
        float kf[8], vf[8];
        load8<WAITQ>(a.kv_new + kn, kf);
        load8<WAITQ>(a.kv_new + vn, vf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kf[e] = to_f32(from_f32<T>(kf[e]));
            vf[e] = to_f32(from_f32<T>(vf[e]));
        }
        float s[G][U];
        Vec8<T> vv[U];
        vv[0].pack(vf);
        if constexpr (DOT2) {
            Vec8<T> kk;
            kk.pack(kf);
#pragma unroll
            for (int u = 1; u < U; ++u) vv[u].zero();   // weight 0, and no garbage in a pair product
#pragma unroll
            for (int j = 0; j < G; ++j) {
                s[j][0] = group_sum<LPR>(score(kk, j));
#pragma unroll
                for (int u = 1; u < U; ++u) s[j][u] = 0.f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(qv[j][e], kf[e], d);
                s[j][0] = group_sum<LPR>(d);
#pragma unroll
                for (int u = 1; u < U; ++u) s[j][u] = 0.f;
            }
        }
        absorb(s, vv, 1);
    }

    // 3. merge the row slots of each wave (lanes LPR, 2 LPR, ... apart), then the waves
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float m2 = __shfl_xor(m[j], off);
            const float l2 = __shfl_xor(ls[j], off);
            float w1, w2, M;
            lse_weights(m[j], m2, &w1, &w2, &M);
            ls[j] = ls[j] * w1 + l2 * w2;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[j][e] = o[j][e] * w1 + __shfl_xor(o[j][e], off) * w2;
            m[j] = M;
        }
    }
    if (lane < LPR) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.o[wave][j][l * 8 + e] = o[j][e];
            if (lane == 0) {
                sm.m[wave][j] = m[j];
                sm.l[wave][j] = ls[j];
            }
        }
    }
    __syncthreads();
    for (int idx = t; idx < G * D; idx += 256) {
        const int j = idx / D, d = idx % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm.m[w][j]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float wt = sm.m[w][j] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sm.m[w][j] - M);
            L += sm.l[w][j] * wt;
            O += sm.o[w][j][d] * wt;
        }
        const size_t pi = ((size_t)b * a.nq + g * G + j) * a.maxc + c;
        publish(a.attn_o + pi * D + d, O);
        if (d == 0) {
            publish(a.attn_ml + pi * 2, M);
            publish(a.attn_ml + pi * 2 + 1, L);
        }
    }

    // 4. the last chunk of (b, g) to arrive merges all chunks of all G heads
    if (a.split_merge) return;           // merged by the merge kernel that follows
    if (!arrive_last(&a.attn_cnt[b * nkv + g], nchunk, s_flag)) return;
    merge_group<T, D, G, PUBLISH>(a, b, g, nchunk, sm);
}

}  // namespace dev
}  // namespace dab

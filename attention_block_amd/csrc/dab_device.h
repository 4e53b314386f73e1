// Device code of the decode attention block (gfx950, wave64), shared by the
// fused persistent kernel and the one-kernel-per-phase schedule.
//
// Work items:
//   gemv tile (QKV)   RMSNorm + a 256-column x KR-row tile of W_qkv for BG
//                     sequences; fp32 partials; the last tile of a slab sums
//                     them, scales by the RMS factor, applies RoPE, writes q
//                     and the new k/v (workspace, fp32) and appends k/v to the
//                     caches.
//   attention chunk   (sequence b, kv head g, chunk c of 128 or more tokens):
//                     each K and V row is read once for the G query heads of
//                     the group; online softmax; the chunk's (max, sum,
//                     weighted values) are published and the last chunk of
//                     (b, g) merges them with log-sum-exp weights.
//   gemv tile (O)     a 256-column x KR-row tile of W_o; the last tile of a
//                     slab adds the residual and rounds to the storage type.
//
// The split of the step into these items, and their hand-off through the
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

// Profiling builds (-DDAB_TRACE) record a 100 MHz timestamp per workgroup at
// up to eight points: 0 start, 1 loads issued, 2 dependencies met, 3 end;
// in the workgroup that finishes a slab or merges a group: 4 its start,
// 5 its inputs fetched, 6 its results published.
#ifdef DAB_TRACE
#define DAB_TRACE_POINT(args, slot) \
    do { if (threadIdx.x == 0 && (args).trace) \
        (args).trace[((args).trace_base + blockIdx.x) * 8 + (slot)] = __builtin_amdgcn_s_memrealtime(); } while (0)
#else
#define DAB_TRACE_POINT(args, slot) do { } while (0)
#endif
constexpr int kMaxRows = 128;      // largest KR (rows of W per GEMV tile)
constexpr int kSpinLimit = 1 << 21;

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

__device__ inline int load_counter(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline int bump(int* p) {
    return __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Thread 0 waits (bounded) until *p >= target.  The bound cannot be reached
// in a correct run; if it is, bit 1 of the error flags is raised and the
// caller carries on, so every wave still exits.
__device__ inline void wait_at_least(const int* p, int target, int* flags) {
    for (int it = 0; it < kSpinLimit; ++it) {
        if (load_counter(p) >= target) return;
        __builtin_amdgcn_s_sleep(4);
    }
    __hip_atomic_fetch_or(flags, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Published values.  The phased schedule publishes plain floats (each kernel
// boundary orders them); the fused schedule publishes 8-byte words
// {value, tag} with one 64-bit device-coherent store, the low-latency
// message format of RCCL's LL protocol.  A reader checks the tag against
// this call's tag and re-reads a word that has not landed yet, so a producer
// bumps its arrival counter without waiting for its stores to be
// acknowledged.  The tag is a signalling-NaN bit pattern derived from the
// call epoch, which no arithmetic result (and no float another call left in
// the workspace) can equal.  Buffers hold 8 bytes per element in both
// schedules; the phased one uses the low half as a float array.

__device__ inline uint32_t ll_tag(uint32_t epoch) { return 0x7F800001u + epoch % 0x3FFFFFu; }

template <bool LL>
__device__ inline void put(float* base, size_t i, float v, uint32_t tag) {
    if constexpr (LL) {
        const uint64_t w = ((uint64_t)tag << 32) | __float_as_uint(v);
        __hip_atomic_store(reinterpret_cast<uint64_t*>(base) + i, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        publish(base + i, v);
    }
}

__device__ inline uint64_t load_ll(const float* base, size_t i) {
    return __hip_atomic_load(reinterpret_cast<const uint64_t*>(base) + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Value of an LL word once it carries `tag` (re-read with a bounded wait).
__device__ inline float ll_value(uint64_t w, const float* base, size_t i, uint32_t tag, int* flags) {
    for (int it = 0; (uint32_t)(w >> 32) != tag; ++it) {
        if (it == kSpinLimit) {
            __hip_atomic_fetch_or(flags, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        w = load_ll(base, i);
    }
    return __uint_as_float((uint32_t)w);
}

template <bool LL>
__device__ inline float get(const float* base, size_t i, uint32_t tag, int* flags) {
    if constexpr (LL) return ll_value(load_ll(base, i), base, i, tag, flags);
    else return fetch(base + i);
}

// Published values base[i0 + j * stride] for the j < N whose bit is set in
// `valid` (the others are neither read nor waited for and come back 0), all
// requested before any is checked: a check may re-read, and later loads must
// not queue behind it.
template <bool LL, int N>
__device__ inline void get_n(const float* base, size_t i0, size_t stride, uint32_t valid, float* out, uint32_t tag,
                             int* flags) {
    if constexpr (LL) {
        uint64_t w[N];
#pragma unroll
        for (int j = 0; j < N; ++j) w[j] = (valid >> j) & 1u ? load_ll(base, i0 + j * stride) : 0;
#pragma unroll
        for (int j = 0; j < N; ++j) out[j] = (valid >> j) & 1u ? ll_value(w[j], base, i0 + j * stride, tag, flags) : 0.f;
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) out[j] = (valid >> j) & 1u ? fetch(base + i0 + j * stride) : 0.f;
    }
}

__device__ inline uint32_t low_bits(int n) { return n >= 32 ? 0xffffffffu : n <= 0 ? 0u : (1u << n) - 1u; }

// Sum of n published values base[i0], base[i0 + stride], ... in index order.
// Loads go out NB at a time so their round trips to the memory-side cache
// overlap; with n <= NB the whole sum costs one round trip.
template <int NB, bool LL>
__device__ inline float fetch_sum(const float* base, size_t i0, size_t stride, int n, uint32_t tag, int* flags) {
    float acc = 0.f;
    constexpr int NW = LL ? NB / 2 : NB;   // a tagged word takes two registers
    for (int k0 = 0; k0 < n; k0 += NW) {
        if constexpr (LL) {
            uint64_t w[NW];
#pragma unroll
            for (int j = 0; j < NW; ++j) w[j] = (k0 + j < n) ? load_ll(base, i0 + (size_t)(k0 + j) * stride) : 0;
#pragma unroll
            for (int j = 0; j < NW; ++j)
                if (k0 + j < n) acc += ll_value(w[j], base, i0 + (size_t)(k0 + j) * stride, tag, flags);
        } else {
            float v[NW];
#pragma unroll
            for (int j = 0; j < NW; ++j) v[j] = (k0 + j < n) ? fetch(base + i0 + (size_t)(k0 + j) * stride) : 0.f;
#pragma unroll
            for (int j = 0; j < NW; ++j) acc += v[j];
        }
    }
    return acc;
}

// Arrival at a counter shared by `expected` workgroups; true in exactly one
// workgroup, the last to arrive.  Phased: every thread's stores are
// acknowledged first.  Fused: readers check tags, so no wait.  With `rearm`
// the last arriver resets the counter (nobody waits on it); otherwise it
// stays at `expected` until the finaliser signals completion with one more
// bump.
template <bool LL>
__device__ inline bool arrive_last(int* counter, int expected, bool rearm, int* s_flag) {
    if constexpr (LL) __syncthreads();
    else drain_and_sync();
    if (threadIdx.x == 0) {
        const int prev = bump(counter);
        const bool last = prev == expected - 1;
        *s_flag = last;
        if (last && rearm) set_counter(counter, 0);
    }
    __syncthreads();
    return *s_flag != 0;
}

__device__ inline bool pos_valid(const StepArgs& a, int b, int* p_out) {
    const int p = a.pos[b];
    *p_out = p;
    return p >= 0 && p < a.cap;
}

// ---------------------------------------------------------------------------
// GEMV tiles
// ---------------------------------------------------------------------------
//
// Tile (slab, ks, batch group): columns [slab*256, +256) x rows [ks*KR, +KR)
// of W for BG batch rows.  Thread t: column group c8 = t % 32 (8 columns,
// one 16-byte bf16 load), row group rg = t / 32 (rows rg, rg+8, ...).  All
// KR/8 loads are issued first.  RMSNorm is applied as a scale after the sum:
// u = r * ((x .* w) @ W), r = (mean x^2 + eps)^(-1/2) a scalar per sequence,
// so the weight stream never waits for the norm; each tile also sums x^2
// over its rows and the slab's finaliser adds those sums up.

template <int BG>
struct GemvShared {
    float xs[BG][kMaxRows];
    f32x4 red[4][BG][64];        // per-wave column partials: 256 columns as 64 x float4
    float ssq[BG][4];
    float val[BG][256];
    float r[BG];
};

// Decode a GEMV work index over `tiles` tiles into (tile, batch group);
// false for padding.  Batch groups sharing a weight tile get work indices 8
// apart, so they run on one XCD and share its L2.
__device__ inline bool gemv_decode(int nbg, int tiles, int idx, int* tile, int* bgi) {
    if (nbg == 1) {
        *tile = idx;
        *bgi = 0;
        return idx < tiles;
    }
    const int lo = idx & 7, rest = idx >> 3;
    *bgi = rest % nbg;
    *tile = (rest / nbg) * 8 + lo;
    return *tile < tiles;
}

// Work indices a GEMV over `tiles` tiles takes (padding included).
__device__ __host__ inline int gemv_items(int nbg, int tiles) {
    return nbg == 1 ? tiles : (tiles + 7) / 8 * 8 * nbg;
}

template <typename T, int BG, bool QKV, bool FUSED>
__device__ void gemv_tile(const StepArgs& a, int slab, int ks, int bgi, uint32_t tag, GemvShared<BG>& sm,
                          int* s_flag) {
    const GemvPlanDev& g = QKV ? a.qkv : a.oproj;
    const int K = QKV ? a.H : a.n_q;
    const int N = QKV ? a.n_qkv : a.H;
    const int KR = g.rows;
    const int t = threadIdx.x, c8 = t & 31, rg = t >> 5, lane = t & 63, wave = t >> 6;
    const int n0 = slab * 256 + c8 * 8;
    const bool col_ok = n0 < N;
    const int kb = ks * KR;
    const int b0 = bgi * BG;
    const int B = a.B;

    // 1. weight stream: every load of the tile in flight before anything else
    const T* W = static_cast<const T*>(QKV ? a.w_qkv : a.w_o) + (size_t)(kb + rg) * N + n0;
    Vec8<T> wv[kMaxRows / 8];
#pragma unroll
    for (int u = 0; u < kMaxRows / 8; ++u) {
        if (col_ok && 8 * u < KR) wv[u].load(W + (size_t)(8 * u) * N);
        else wv[u].zero();
    }

    DAB_TRACE_POINT(a, 1);

    // 2. inputs of this tile's rows
    float sq[BG];
#pragma unroll
    for (int j = 0; j < BG; ++j) sq[j] = 0.f;
    if constexpr (QKV) {
        if (t < KR) {
#pragma unroll
            for (int j = 0; j < BG; ++j) {
                const int bb = b0 + j;
                float xv = 0.f;
                if (bb < B) {
                    const float x = to_f32(static_cast<const T*>(a.hidden)[(size_t)bb * K + kb + t]);
                    xv = x * to_f32(static_cast<const T*>(a.norm_w)[kb + t]);
                    sq[j] = x * x;
                }
                sm.xs[j][t] = xv;
            }
        }
#pragma unroll
        for (int j = 0; j < BG; ++j) {
            const float s = wave_sum(sq[j]);
            if (lane == 0) sm.ssq[j][wave] = s;
        }
    } else {
        // attention output rows [kb, kb+KR) = heads kb/D .. ; in the fused
        // schedule wait until every sequence of the group has them
        if (FUSED && t == 0) {
            for (int j = 0; j < BG; ++j) {
                const int bb = b0 + j;
                int p;
                if (bb >= B || !pos_valid(a, bb, &p)) continue;
                const int nchunk = p > 0 ? (p + a.T - 1) / a.T : 1;
                for (int h = kb / a.D; h <= (kb + KR - 1) / a.D; ++h)
                    wait_at_least(&a.attn_cnt[bb * a.nkv + h / a.G], nchunk + 1, a.flags);
            }
        }
        __syncthreads();
        if (t < KR) {
            // rows of sequences with a valid position only (the others have
            // no attention output and no output row)
            uint32_t valid = 0;
#pragma unroll
            for (int j = 0; j < BG; ++j) {
                int p;
                if (b0 + j < B && pos_valid(a, b0 + j, &p)) valid |= 1u << j;
            }
            float xv[BG];
            get_n<FUSED, BG>(a.a, (size_t)b0 * K + kb + t, K, valid, xv, tag, a.flags);
#pragma unroll
            for (int j = 0; j < BG; ++j) sm.xs[j][t] = b0 + j < B ? xv[j] : 0.f;
        }
    }
    __syncthreads();
    DAB_TRACE_POINT(a, 2);

    // 3. multiply-accumulate
    float acc[BG][8];
#pragma unroll
    for (int j = 0; j < BG; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
#pragma unroll
    for (int u = 0; u < kMaxRows / 8; ++u) {
        if (8 * u < KR) {
            float w8[8];
            wv[u].unpack(w8);
#pragma unroll
            for (int j = 0; j < BG; ++j) {
                const float xv = sm.xs[j][rg + 8 * u];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(xv, w8[e], acc[j][e]);
            }
        }
    }

    // 4. reduce the 8 row groups: lane pairs (l, l+32), then the 4 waves
#pragma unroll
    for (int j = 0; j < BG; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] += __shfl_xor(acc[j][e], 32);
    if (lane < 32) {
#pragma unroll
        for (int j = 0; j < BG; ++j) {
            sm.red[wave][j][2 * c8] = f32x4{acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
            sm.red[wave][j][2 * c8 + 1] = f32x4{acc[j][4], acc[j][5], acc[j][6], acc[j][7]};
        }
    }
    __syncthreads();
    const int n = slab * 256 + t;        // this thread's column from here on
    const float* redf = reinterpret_cast<const float*>(&sm.red[0][0][0]);
    float* part = QKV ? a.qkv_part : a.oproj_part;
#pragma unroll
    for (int j = 0; j < BG; ++j) {
        const int bb = b0 + j;
        if (bb < B && n < N) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) s += redf[(w * BG + j) * 256 + t];
            put<FUSED>(part, ((size_t)ks * B + bb) * N + n, s, tag);
        }
        if constexpr (QKV) {
            if (t == 0 && bb < B)
                put<FUSED>(a.ssq, ((size_t)slab * g.ksplit + ks) * B + bb,
                           sm.ssq[j][0] + sm.ssq[j][1] + sm.ssq[j][2] + sm.ssq[j][3], tag);
        }
    }

    // 5. the last tile of this slab finishes it
    int* cnt = (QKV ? a.qkv_cnt : a.oproj_cnt) + slab * g.nbg + bgi;
    if (!arrive_last<FUSED>(cnt, g.ksplit, !(QKV && FUSED), s_flag)) return;
    DAB_TRACE_POINT(a, 4);

    // every partial sum of this slab: one round trip per batch row (32 wide)
#pragma unroll
    for (int j = 0; j < BG; ++j) {
        const int bb = b0 + j;
        sm.val[j][t] = (bb < B && n < N)
                           ? fetch_sum<32, FUSED>(part, (size_t)bb * N + n, (size_t)B * N, g.ksplit, tag, a.flags)
                           : 0.f;
    }
    DAB_TRACE_POINT(a, 5);
    if constexpr (QKV) {
        if (t < BG) {
            const int bb = b0 + t;
            const float ss =
                bb < B ? fetch_sum<32, FUSED>(a.ssq, (size_t)slab * g.ksplit * B + bb, B, g.ksplit, tag, a.flags)
                       : 0.f;
            sm.r[t] = 1.0f / sqrtf(ss / (float)K + a.eps);
        }
        __syncthreads();
        const int D = a.D, half = D >> 1;
        const bool rot = n < a.n_q + a.nkv * D;         // q and k columns are rotated
        const int e = n % D;
        const int partner = e < half ? t + half : t - half;
#pragma unroll
        for (int j = 0; j < BG; ++j) {
            const int bb = b0 + j;
            if (bb >= B || n >= N) continue;
            int p;
            const bool ok = pos_valid(a, bb, &p);
            if (!ok && slab == 0 && t == 0)
                __hip_atomic_fetch_or(a.flags, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const float r = sm.r[j];
            float v = sm.val[j][t] * r;
            if (rot) {
                // angle pos * theta^(-2i/D), i = e mod D/2: formed and reduced
                // to [-pi, pi] in fp64 (fp32 would lose ~1e-3 rad at pos 16K),
                // then sin/cos in fp32
                const double ang = (double)p * exp2(-(2.0 * (e % half) / D) * a.log2_theta);
                const double two_pi = 6.283185307179586;
                float sn, cs;
                sincosf((float)(ang - two_pi * rint(ang / two_pi)), &sn, &cs);
                const float pv = sm.val[j][partner] * r;
                v = e < half ? v * cs - pv * sn : v * cs + pv * sn;
            }
            if (n < a.n_q) {
                put<FUSED>(a.q, (size_t)bb * a.n_q + n, v, tag);
            } else {
                const int kvn = n - a.n_q;
                const int is_v = kvn >= a.nkv * D;
                const int col = is_v ? kvn - a.nkv * D : kvn;
                put<FUSED>(a.kv_new, ((size_t)bb * 2 + is_v) * a.nkv * D + col, v, tag);
                if (ok) {
                    T* dst = static_cast<T*>(is_v ? a.v_cache : a.k_cache);
                    dst[((size_t)bb * a.cap + p) * a.nkv * D + col] = from_f32<T>(v);
                }
            }
        }
        if constexpr (FUSED) {
            __syncthreads();
            if (t == 0) bump(cnt);                       // slab ready: counter = ksplit + 1
        }
        DAB_TRACE_POINT(a, 6);
    } else {
#pragma unroll
        for (int j = 0; j < BG; ++j) {
            const int bb = b0 + j;
            int p;
            if (bb >= B || n >= N || !pos_valid(a, bb, &p)) continue;
            const float y = sm.val[j][t];
            const float x = to_f32(static_cast<const T*>(a.hidden)[(size_t)bb * N + n]);
            static_cast<T*>(a.out)[(size_t)bb * N + n] = from_f32<T>(x + y);
            if (a.dbg_y) a.dbg_y[(size_t)bb * N + n] = y;
        }
    }
}

// ---------------------------------------------------------------------------
// split-KV attention chunks
// ---------------------------------------------------------------------------
//
// LPR = D/8 lanes hold one token row (8 elements each); the workgroup's
// 256/LPR row slots take tokens slot, slot + NSLOT, ...; U tokens per slot
// are loaded per batch (16 loads of 16 bytes in flight per lane).  Scores
// are kept in log2 units (q is pre-scaled by log2(e)/sqrt(D)), so every
// exponential is an exp2.  The new token never comes from the cache: its
// k and v are taken from the workspace copy the QKV finaliser published,
// rounded to the storage type exactly as the appended row.

template <int D, int G>
struct AttnShared {
    float m[4][G], l[4][G];
    float o[4][G][D];
    float cm[kMaxChunks], cw[kMaxChunks];
    float red[8];
    float acc[256];
};

template <int D>
struct AttnGeom {
    static constexpr int LPR = D / 8;
    static constexpr int NSLOT = 256 / LPR;
    static constexpr int U = 8;
    static constexpr int BATCH = NSLOT * U;   // tokens per batch of loads (128 for D=128)
};

// Which QKV slab (of 256 columns) holds column `col`.
__device__ inline int slab_of(int col) { return col >> 8; }

template <typename T, int D, int G, bool FUSED>
__device__ void attn_item(const StepArgs& a, int b, int g, int c, uint32_t tag, AttnShared<D, G>& sm, int* s_flag) {
    using Geo = AttnGeom<D>;
    constexpr int LPR = Geo::LPR, NSLOT = Geo::NSLOT, U = Geo::U;
    const int nkv = a.nkv;
    int p;
    if (!pos_valid(a, b, &p)) return;
    // chunks cover the p cached tokens; the last one also takes the new token
    const int nchunk = p > 0 ? (p + a.T - 1) / a.T : 1;
    if (c >= nchunk) return;
    const int t0 = c * a.T;
    const int t1 = min(t0 + a.T, p);
    const bool has_new = c == nchunk - 1;

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int slot = t / LPR, l = t % LPR;
    const size_t row = (size_t)nkv * D;
    const size_t base = ((size_t)b * a.cap * nkv + g) * D + l * 8;
    const T* Kp = static_cast<const T*>(a.k_cache) + base;
    const T* Vp = static_cast<const T*>(a.v_cache) + base;

    // 1. first batch of history rows in flight
    Vec8<T> kr[U], vr[U];
    auto issue = [&](int tb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tok = tb + NSLOT * u;
            if (tok < t1) {
                kr[u].load(Kp + (size_t)tok * row);
                vr[u].load(Vp + (size_t)tok * row);
            } else {
                kr[u].zero();
                vr[u].zero();
            }
        }
    };
    issue(t0 + slot);
    DAB_TRACE_POINT(a, 1);

    // 2. wait for q of this group's heads (and the new k, v in the last chunk)
    if constexpr (FUSED) {
        if (t == 0) {
            const int bq = b / a.qkv_bg;
            const GemvPlanDev& q = a.qkv;
            const int ready = q.ksplit + 1;
            const int lo = slab_of(g * G * D), hi = slab_of((g + 1) * G * D - 1);
            for (int s = lo; s <= hi; ++s) wait_at_least(&a.qkv_cnt[s * q.nbg + bq], ready, a.flags);
            if (has_new) {
                wait_at_least(&a.qkv_cnt[slab_of(a.n_q + g * D) * q.nbg + bq], ready, a.flags);
                wait_at_least(&a.qkv_cnt[slab_of(a.n_q + (nkv + g) * D) * q.nbg + bq], ready, a.flags);
            }
        }
        __syncthreads();
    }
    DAB_TRACE_POINT(a, 2);

    float qv[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        get_n<FUSED, 8>(a.q, (size_t)b * a.n_q + (size_t)(g * G + j) * D + l * 8, 1, 0xffu, qv[j], tag, a.flags);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[j][e] *= a.qscale;
    }
    float m[G], ls[G], o[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = kNegInf;
        ls[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
    }

    // online-softmax update of this slot's state with n scores / value rows
    auto absorb = [&](float (&s)[G][U], Vec8<T> (&vv)[U], int nvalid) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float mx = m[j];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (u < nvalid) mx = fmaxf(mx, s[j][u]);
            // at least one score is valid, so mx is finite here
            const float alpha = __builtin_amdgcn_exp2f(m[j] - mx);
            float pu[U], psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pu[u] = u < nvalid ? __builtin_amdgcn_exp2f(s[j][u] - mx) : 0.f;
                psum += pu[u];
            }
            ls[j] = ls[j] * alpha + psum;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[j][e] *= alpha;
            m[j] = mx;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u < nvalid) {
                    float vf[8];
                    vv[u].unpack(vf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[j][e] = fmaf(pu[u], vf[e], o[j][e]);
                }
            }
        }
    };

    for (int tb = t0 + slot; tb < t1; tb += NSLOT * U) {
        if (tb != t0 + slot) issue(tb);
        float s[G][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[8];
            kr[u].unpack(kf);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(qv[j][e], kf[e], d);
                s[j][u] = group_sum<LPR>(d);
            }
        }
        // tokens tb + NSLOT*u < t1 are valid, u = 0 always
        const int nvalid = min(U, (t1 - tb + NSLOT - 1) / NSLOT);
        absorb(s, vr, nvalid);
    }

    // the new token, in slot 0 of the last chunk: its k and v come from the
    // workspace copy the QKV finaliser published, rounded to the storage type
    // exactly as the appended cache row
    if (has_new && slot == 0) {
        const size_t kn = ((size_t)b * 2 * nkv + g) * D + l * 8;
        const size_t vn = kn + (size_t)nkv * D;
        float kf[8], vf[8];
        get_n<FUSED, 8>(a.kv_new, kn, 1, 0xffu, kf, tag, a.flags);
        get_n<FUSED, 8>(a.kv_new, vn, 1, 0xffu, vf, tag, a.flags);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kf[e] = to_f32(from_f32<T>(kf[e]));
            vf[e] = to_f32(from_f32<T>(vf[e]));
        }
        float s[G][U];
        Vec8<T> vv[U];
        vv[0].pack(vf);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf(qv[j][e], kf[e], d);
            s[j][0] = group_sum<LPR>(d);
#pragma unroll
            for (int u = 1; u < U; ++u) s[j][u] = 0.f;
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
        put<FUSED>(a.attn_o, pi * D + d, O, tag);
        if (d == 0) {
            put<FUSED>(a.attn_ml, pi * 2, M, tag);
            put<FUSED>(a.attn_ml, pi * 2 + 1, L, tag);
        }
    }

    // 4. the last chunk of (b, g) merges all chunks.  Each head's chunk
    // statistics (m, l) and the first OB weighted outputs of every thread
    // are requested together, so short merges cost one round trip.
    int* cnt = &a.attn_cnt[b * nkv + g];
    if (!arrive_last<FUSED>(cnt, nchunk, !FUSED, s_flag)) return;
    DAB_TRACE_POINT(a, 4);
    constexpr int PARTS = 256 / D;       // threads per output element
    constexpr int OB = 8;                // chunks per thread in the first request
    const int d = t % D, part = t / D;
    for (int j = 0; j < G; ++j) {
        const int h = g * G + j;
        const size_t pbase = ((size_t)b * a.nq + h) * a.maxc;
        // this thread's chunks part, part + PARTS, ... below nchunk
        float ov[OB];
        {
            const int nv = part < nchunk ? (nchunk - part + PARTS - 1) / PARTS : 0;
            get_n<FUSED, OB>(a.attn_o, (pbase + part) * D + d, (size_t)PARTS * D, low_bits(nv), ov, tag, a.flags);
        }
        DAB_TRACE_POINT(a, 5);
        float mloc = kNegInf;
        for (int cc = t; cc < nchunk; cc += 256) {
            float ml[2];
            get_n<FUSED, 2>(a.attn_ml, (pbase + cc) * 2, 1, 0x3u, ml, tag, a.flags);
            sm.cm[cc] = ml[0];
            sm.cw[cc] = ml[1];            // l for now, weight below
            mloc = fmaxf(mloc, ml[0]);
        }
        mloc = wave_max(mloc);
        if (lane == 0) sm.red[wave] = mloc;
        __syncthreads();
        const float M = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
        float lloc = 0.f;
        for (int cc = t; cc < nchunk; cc += 256) {
            const float w = __builtin_amdgcn_exp2f(sm.cm[cc] - M);
            lloc += w * sm.cw[cc];
            sm.cw[cc] = w;
        }
        lloc = wave_sum(lloc);
        __syncthreads();                 // weights visible; sm.red[0..3] read by everyone
        if (lane == 0) sm.red[4 + wave] = lloc;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < OB; ++q) {
            const int cc = part + q * PARTS;
            if (cc < nchunk) acc += sm.cw[cc] * ov[q];
        }
        for (int c0 = part + OB * PARTS; c0 < nchunk; c0 += 8 * PARTS) {
            float v[8];
            get_n<FUSED, 8>(a.attn_o, (pbase + c0) * D + d, (size_t)PARTS * D,
                            low_bits((nchunk - c0 + PARTS - 1) / PARTS), v, tag, a.flags);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int cc = c0 + q * PARTS;
                if (cc < nchunk) acc += sm.cw[cc] * v[q];
            }
        }
        sm.acc[t] = acc;
        __syncthreads();
        const float L = sm.red[4] + sm.red[5] + sm.red[6] + sm.red[7];
        if (t < D) {
            float tot = 0.f;
#pragma unroll
            for (int q = 0; q < PARTS; ++q) tot += sm.acc[q * D + t];
            put<FUSED>(a.a, (size_t)b * a.n_q + (size_t)h * D + t, tot / L, tag);
        }
        __syncthreads();
    }
    if constexpr (FUSED) {
        __syncthreads();
        if (t == 0) bump(cnt);                          // group ready: counter = nchunk + 1
    }
    DAB_TRACE_POINT(a, 6);
}

}  // namespace dev
}  // namespace dab

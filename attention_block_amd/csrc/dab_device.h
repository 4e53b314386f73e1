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

__device__ inline bool pos_valid(const StepArgs& a, int b, int* p_out) {
    const int p = a.pos[b];
    *p_out = p;
    return p >= 0 && p < a.cap;
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
// k and v are taken from the fp32 workspace copy the QKV kernel wrote,
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

// PUBLISH: the output projection runs in the same launch, so the merged
// output is stored device-coherently and, once every head of the group is
// stored and acknowledged, the sequence's merge counter is bumped.
// WAITQ: the QKV projection runs in the same launch; after the K/V loads are
// issued, wait until every panel of the group's q heads and of its k and v
// heads is done, then read q and the new k, v device-coherently.
template <typename T, int D, int G, bool PUBLISH, bool WAITQ>
__device__ void attn_item(const StepArgs& a, int b, int g, int c, AttnShared<D, G>& sm, int* s_flag) {
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

    // 2. q of this group's heads, in log2 units
    if constexpr (WAITQ) {
        if (t == 0) {
            const int nheads = a.nq + 2 * nkv, panels = D / 8;      // panels per head: 4 RoPE pairs each
            const int* cnt = a.head_cnt + (b / a.qkv.nb) * nheads;
            for (int j = 0; j < G; ++j) wait_at_least<2>(cnt + g * G + j, panels, a.flags);
            wait_at_least<2>(cnt + a.nq + g, panels, a.flags);
            wait_at_least<2>(cnt + a.nq + nkv + g, panels, a.flags);
        }
        __syncthreads();
    }
    float qv[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        load8<WAITQ>(a.q + (size_t)b * a.n_q + (size_t)(g * G + j) * D + l * 8, qv[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[j][e] *= a.qscale;
    }
    DAB_TRACE_POINT(a, 2);
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
    // workspace copy the QKV kernel wrote, rounded to the storage type
    // exactly as the appended cache row
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
        publish(a.attn_o + pi * D + d, O);
        if (d == 0) {
            publish(a.attn_ml + pi * 2, M);
            publish(a.attn_ml + pi * 2 + 1, L);
        }
    }

    // 4. the last chunk of (b, g) merges all chunks.  Each head's chunk
    // statistics (m, l) and the first OB weighted outputs of every thread
    // are requested together, so short merges cost one round trip.
    int* cnt = &a.attn_cnt[b * nkv + g];
    if (!arrive_last(cnt, nchunk, s_flag)) return;
    DAB_TRACE_POINT(a, 4);
    constexpr int PARTS = 256 / D;       // threads per output element
    constexpr int OB = 16;               // chunks per thread in the first request (32 at D = 128)
    const int d = t % D, part = t / D;
    for (int j = 0; j < G; ++j) {
        const int h = g * G + j;
        const size_t pbase = ((size_t)b * a.nq + h) * a.maxc;
        float m0 = kNegInf, l0 = 0.f;
        if (t < nchunk) {
            m0 = fetch(a.attn_ml + (pbase + t) * 2);
            l0 = fetch(a.attn_ml + (pbase + t) * 2 + 1);
        }
        // this thread's chunks part, part + PARTS, ... below nchunk
        float ov[OB];
#pragma unroll
        for (int q = 0; q < OB; ++q) {
            const int cc = part + q * PARTS;
            ov[q] = cc < nchunk ? fetch(a.attn_o + (pbase + cc) * D + d) : 0.f;
        }
        DAB_TRACE_POINT(a, 5);
        float mloc = m0;
        if (t < nchunk) {
            sm.cm[t] = m0;
            sm.cw[t] = l0;               // l for now, weight below
        }
        for (int cc = t + 256; cc < nchunk; cc += 256) {
            const float mc = fetch(a.attn_ml + (pbase + cc) * 2);
            sm.cm[cc] = mc;
            sm.cw[cc] = fetch(a.attn_ml + (pbase + cc) * 2 + 1);
            mloc = fmaxf(mloc, mc);
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
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int cc = c0 + q * PARTS;
                v[q] = cc < nchunk ? fetch(a.attn_o + (pbase + cc) * D + d) : 0.f;
            }
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
            if constexpr (PUBLISH) publish(a.a + (size_t)b * a.n_q + (size_t)h * D + t, tot / L);
            else a.a[(size_t)b * a.n_q + (size_t)h * D + t] = tot / L;
        }
        __syncthreads();
    }
    if constexpr (PUBLISH) {
        // one more kv group of sequence b merged; the last one raises the
        // sequence's ready flags (every other group's output was stored and
        // acknowledged before its bump)
        drain_and_sync();
        if (t == 0) *s_flag = bump(&a.seq_cnt[b]) == nkv - 1;
        __syncthreads();
        if (*s_flag && t < kReadyCopies) set_counter(&a.seq_ready[(b * kReadyCopies + t) * kReadyStride], 1);
    }
    DAB_TRACE_POINT(a, 6);
}

}  // namespace dev
}  // namespace dab

// HIP kernels of the fused single-token decode attention block, gfx950.
//
// Three phases, each one kernel on the caller's stream:
//   1. gemv<QKV>  RMSNorm + QKV projection.  Workgroups take (column slab,
//                 row block) tiles of W_qkv, stream them once with 16-byte
//                 loads and write fp32 partial sums; the last workgroup to
//                 arrive at a slab sums the partials, applies the RMS scale,
//                 RoPE, and writes q (fp32) and the new k/v rows of the cache.
//   2. attn       split-KV attention.  Workgroups take (sequence, kv head,
//                 token chunk) items, read each K/V row once for all query
//                 heads of the group, keep an online softmax (max, sum,
//                 weighted values) and write one partial per head; the last
//                 workgroup to arrive at (sequence, kv head) merges the
//                 partials with log-sum-exp weights.
//   3. gemv<OPROJ> output projection; the last workgroup per slab adds the
//                 residual and rounds to the storage type.
//
// The hand-off between workgroups of one phase replaces the thread-block
// cluster reductions of the ClusterFusion page (section 3.1, ClusterReduce /
// ClusterGather): gfx950 has no distributed shared memory, so partials go
// through the memory-side Infinity Cache with device-coherent stores and
// loads (see `publish` / `arrive_last`), close to the route that page lists
// as future work (section 6, hierarchical clusters communicating via L2).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dab_kernels.h"

namespace dab {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// element access: 8 consecutive elements per lane
// ---------------------------------------------------------------------------

template <typename T> struct Vec8;

template <> struct Vec8<uint16_t> {           // bf16: one 16-byte load
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
};

template <> struct Vec8<float> {              // fp32: two 16-byte loads
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
};

__device__ inline float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ inline float to_f32(float v) { return v; }

template <typename T> __device__ inline T from_f32(float f);
template <> __device__ inline float from_f32<float>(float f) { return f; }
template <> __device__ inline uint16_t from_f32<uint16_t>(float f) {
    __bf16 h = (__bf16)f;                      // v_cvt_pk_bf16_f32: nearest-even
    return __builtin_bit_cast(uint16_t, h);
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
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror: combines the two quads of each half row
    if (LPR == 16) v += dpp<0x140>(v);   // row_mirror: combines the two halves of the row
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

// Merge of two online-softmax states in log2 units: (m, l) and weighted sums.
__device__ inline void lse_weights(float m1, float m2, float* w1, float* w2, float* mout) {
    const float M = fmaxf(m1, m2);
    const float Ms = M == kNegInf ? 0.f : M;
    *w1 = __builtin_amdgcn_exp2f(m1 - Ms);
    *w2 = __builtin_amdgcn_exp2f(m2 - Ms);
    *mout = M;
}

// Cross-workgroup hand-off without L2 write-back.
//
// The eight XCD L2 caches are not coherent with one another, and an
// agent-scope fence makes each workgroup write back its whole L2 (a
// buffer_wbl2 per workgroup, ~1 us each, serialised per XCD).  Instead,
// data handed to another workgroup of the same launch is stored and loaded
// with device-scope coherence bits (relaxed agent-scope atomic stores and
// loads compile to global_store/global_load ... sc1, which write through
// and read past the non-coherent L2).  A producer waits until its sc1
// stores are acknowledged (s_waitcnt 0), the workgroup meets at a barrier,
// and one thread bumps the arrival counter; the last arriver then reads the
// published data with sc1 loads.
__device__ inline void publish(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float fetch(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival at a counter shared by `expected` workgroups; returns true in
// exactly one workgroup, the last to arrive, which also re-arms the counter.
__device__ inline bool arrive_last(int* counter, int expected, int* s_flag) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // keeps the compiler from sinking the stores
    __builtin_amdgcn_s_waitcnt(0);                           // this wave's sc1 stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
        const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = (prev == expected - 1);
        if (prev == expected - 1) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return *s_flag != 0;
}

// Sum of n published floats p[0], p[stride], ... in index order.  Loads go
// out in batches of 16 so that their round trips to the memory-side cache
// overlap (a plain loop would wait for each one before the next).
__device__ inline float fetch_sum(const float* p, size_t stride, int n) {
    constexpr int NB = 16;
    float acc = 0.f;
    for (int k0 = 0; k0 < n; k0 += NB) {
        float v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) v[j] = (k0 + j < n) ? fetch(p + (size_t)(k0 + j) * stride) : 0.f;
#pragma unroll
        for (int j = 0; j < NB; ++j) acc += v[j];
    }
    return acc;
}

}  // namespace

// ---------------------------------------------------------------------------
// workspace fill (graph-safe replacement for a memset)
// ---------------------------------------------------------------------------

__global__ void fill_zero_kernel(uint32_t* p, size_t n_words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ---------------------------------------------------------------------------
// GEMV phases
// ---------------------------------------------------------------------------
//
// Tile (slab, ks, batch group): columns [slab*256, +256) x rows [ks*KR, +KR)
// of W for BG batch rows.  Thread t: column group c8 = t % 32 (8 columns,
// one 16-byte bf16 load), row group rg = t / 32 (rows rg, rg+8, ...).  The
// KR/8 loads of a thread are all issued before any arithmetic.
//
// RMSNorm is applied as a scale after the sum: u = r * ((x .* w) @ W) with
// r = (mean x^2 + eps)^(-1/2), a scalar per sequence, so the GEMV streams
// weights without waiting for the norm.  Each tile also sums x^2 over its
// rows; the slab's finaliser adds those sums up to get r.

template <typename T, int BG, int KR, bool QKV>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
    constexpr int NLD = KR / 8;
    __shared__ float xs[BG][KR];
    __shared__ f32x4 red[4][BG][64];     // per-wave column partials, 256 columns as 64 x float4
    __shared__ float s_ssq[BG][4];
    __shared__ float s_val[BG][256];
    __shared__ int s_last;

    int tile, bgi;
    if (a.nbg == 1) {
        tile = blockIdx.x;
        bgi = 0;
    } else {
        // groups that share a weight tile get workgroup ids 8 apart: same XCD
        const int lo = blockIdx.x & 7, rest = blockIdx.x >> 3;
        bgi = rest % a.nbg;
        tile = (rest / a.nbg) * 8 + lo;
        if (tile >= a.tiles) return;
    }
    const int slab = tile % a.slabs, ks = tile / a.slabs;
    const int t = threadIdx.x, c8 = t & 31, rg = t >> 5, lane = t & 63, wave = t >> 6;
    const int n0 = slab * 256 + c8 * 8;
    const bool col_ok = n0 < a.N;
    const int kb = ks * KR;
    const int b0 = bgi * BG;
    const int B = a.B;

    // 1. weight stream: all loads in flight before the staging below
    const T* W = static_cast<const T*>(a.W) + (size_t)(kb + rg) * a.N + n0;
    Vec8<T> wv[NLD];
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
        if (col_ok) wv[u].load(W + (size_t)(8 * u) * a.N);
        else wv[u].zero();
    }

    // 2. stage the input rows [kb, kb+KR) of each batch row
    float sq[BG];
#pragma unroll
    for (int j = 0; j < BG; ++j) sq[j] = 0.f;
    if (t < KR) {
#pragma unroll
        for (int j = 0; j < BG; ++j) {
            const int bb = b0 + j;
            float xv = 0.f;
            if (bb < B) {
                if constexpr (QKV) {
                    const float x = to_f32(static_cast<const T*>(a.hidden)[(size_t)bb * a.K + kb + t]);
                    xv = x * to_f32(static_cast<const T*>(a.norm_w)[kb + t]);
                    sq[j] = x * x;
                } else {
                    xv = a.xin[(size_t)bb * a.K + kb + t];
                }
            }
            xs[j][t] = xv;
        }
    }
    if constexpr (QKV) {
#pragma unroll
        for (int j = 0; j < BG; ++j) {
            const float s = wave_sum(sq[j]);
            if (lane == 0) s_ssq[j][wave] = s;
        }
    }
    __syncthreads();

    // 3. multiply-accumulate
    float acc[BG][8];
#pragma unroll
    for (int j = 0; j < BG; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
        float w8[8];
        wv[u].unpack(w8);
#pragma unroll
        for (int j = 0; j < BG; ++j) {
            const float xv = xs[j][rg + 8 * u];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(xv, w8[e], acc[j][e]);
        }
    }

    // 4. reduce the 8 row groups: lane pairs (l, l+32) then the 4 waves
#pragma unroll
    for (int j = 0; j < BG; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] += __shfl_xor(acc[j][e], 32);
    if (lane < 32) {
#pragma unroll
        for (int j = 0; j < BG; ++j) {
            red[wave][j][2 * c8] = f32x4{acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
            red[wave][j][2 * c8 + 1] = f32x4{acc[j][4], acc[j][5], acc[j][6], acc[j][7]};
        }
    }
    __syncthreads();
    const int n = slab * 256 + t;        // this thread's column from here on
    const float* redf = reinterpret_cast<const float*>(&red[0][0][0]);
#pragma unroll
    for (int j = 0; j < BG; ++j) {
        const int bb = b0 + j;
        if (bb < B && n < a.N) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) s += redf[(w * BG + j) * 256 + t];
            publish(&a.part[((size_t)ks * B + bb) * a.N + n], s);
        }
        if constexpr (QKV) {
            if (t == 0 && bb < B)
                publish(&a.ssq[((size_t)slab * a.ksplit + ks) * B + bb],
                        s_ssq[j][0] + s_ssq[j][1] + s_ssq[j][2] + s_ssq[j][3]);
        }
    }

    // 5. the last workgroup of this slab finishes it
    if (!arrive_last(&a.cnt[slab * a.nbg + bgi], a.ksplit, &s_last)) return;

#pragma unroll
    for (int j = 0; j < BG; ++j) {
        const int bb = b0 + j;
        float v = 0.f;
        if (bb < B && n < a.N) v = fetch_sum(a.part + (size_t)bb * a.N + n, (size_t)B * a.N, a.ksplit);
        s_val[j][t] = v;
    }
    if constexpr (QKV) {
        // RMS scale per batch row (same for every column)
        __shared__ float s_r[BG];
        if (t < BG) {
            const int bb = b0 + t;
            const float ss = bb < B ? fetch_sum(a.ssq + (size_t)slab * a.ksplit * B + bb, B, a.ksplit) : 0.f;
            s_r[t] = 1.0f / sqrtf(ss / (float)a.K + a.eps);
        }
        __syncthreads();
        const int half = a.D >> 1;
        const bool rot = n < a.n_q + a.nkv * a.D;       // q and k columns are rotated
        const int e = n % a.D;
        const int partner = e < half ? t + half : t - half;
        float cs = 1.f, sn = 0.f;
#pragma unroll
        for (int j = 0; j < BG; ++j) {
            const int bb = b0 + j;
            if (bb >= B || n >= a.N) continue;
            const int p = a.pos[bb];
            const bool pos_ok = p >= 0 && p < a.cap;
            if (!pos_ok && slab == 0 && t == 0) atomicOr(&a.flags[0], 1);
            const float r = s_r[j];
            float v = s_val[j][t] * r;
            if (rot) {
                // angle pos * theta^(-2i/D), i = e mod D/2, formed in fp64
                const int i = e % half;
                const double ang = (double)p * exp2(-(2.0 * i / a.D) * a.log2_theta);
                double sd, cd;
                sincos(ang, &sd, &cd);
                cs = (float)cd;
                sn = (float)sd;
                const float pv = s_val[j][partner] * r;
                v = e < half ? v * cs - pv * sn : v * cs + pv * sn;
            }
            if (n < a.n_q) {
                a.q[(size_t)bb * a.n_q + n] = v;
            } else if (pos_ok) {
                const int kvn = n - a.n_q;
                const bool is_k = kvn < a.nkv * a.D;
                const int gcol = is_k ? kvn : kvn - a.nkv * a.D;
                const size_t at = ((size_t)bb * a.cap + p) * a.nkv * a.D + gcol;
                T* dst = static_cast<T*>(is_k ? a.k_cache : a.v_cache);
                dst[at] = from_f32<T>(v);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < BG; ++j) {
            const int bb = b0 + j;
            if (bb >= B || n >= a.N) continue;
            const int p = a.pos[bb];
            if (p < 0 || p >= a.cap) continue;
            const float y = s_val[j][t];
            const float x = to_f32(static_cast<const T*>(a.hidden)[(size_t)bb * a.N + n]);
            static_cast<T*>(a.out)[(size_t)bb * a.N + n] = from_f32<T>(x + y);
            if (a.dbg_y) a.dbg_y[(size_t)bb * a.N + n] = y;
        }
    }
}

// ---------------------------------------------------------------------------
// split-KV attention
// ---------------------------------------------------------------------------
//
// Item (b, g, c): tokens [c*T, min((c+1)*T, pos_b+1)) of kv head g of
// sequence b, for the G query heads g*G .. g*G+G-1.  LPR = D/8 lanes hold
// one token row (8 elements each); the workgroup's 256/LPR row slots take
// tokens slot, slot + NSLOT, ...  Scores are kept in log2 units (q is
// pre-scaled by log2(e)/sqrt(D)) so every exponential is an exp2.

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
    constexpr int LPR = D / 8;
    constexpr int NSLOT = 256 / LPR;
    constexpr int U = 8;                 // tokens per slot per batch of loads
    __shared__ float s_m[4][G], s_l[4][G];
    __shared__ float s_o[4][G][D];
    __shared__ float s_cm[kMaxChunks], s_cw[kMaxChunks];
    __shared__ float s_red[8];
    __shared__ float s_acc[256];
    __shared__ int s_last;

    const int nkv = a.nkv;
    const int g = blockIdx.x % nkv;
    const int rest = blockIdx.x / nkv;
    const int c = rest % a.maxc;
    const int b = rest / a.maxc;
    const int p = a.pos[b];
    if (p < 0 || p >= a.cap) return;
    const int ntok = p + 1;
    const int nchunk = (ntok + a.T - 1) / a.T;
    if (c >= nchunk) return;
    const int t0 = c * a.T;
    const int t1 = min(t0 + a.T, ntok);

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int slot = t / LPR, l = t % LPR;

    float qv[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const float* qp = a.q + (size_t)b * a.nq * D + (size_t)(g * G + j) * D + l * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[j][e] = qp[e] * a.qscale;
    }
    float m[G], ls[G], o[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = kNegInf;
        ls[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
    }

    const size_t row = (size_t)nkv * D;
    const size_t base = ((size_t)b * a.cap * nkv + g) * D + l * 8;
    const T* Kp = static_cast<const T*>(a.k_cache) + base;
    const T* Vp = static_cast<const T*>(a.v_cache) + base;

    for (int tb = t0 + slot; tb < t1; tb += NSLOT * U) {
        Vec8<T> kr[U], vr[U];
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
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float mx = m[j];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (tb + NSLOT * u < t1) mx = fmaxf(mx, s[j][u]);
            // token tb is valid, so mx is finite here
            const float alpha = __builtin_amdgcn_exp2f(m[j] - mx);
            float pu[U], psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pu[u] = (tb + NSLOT * u < t1) ? __builtin_amdgcn_exp2f(s[j][u] - mx) : 0.f;
                psum += pu[u];
            }
            ls[j] = ls[j] * alpha + psum;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[j][e] *= alpha;
            m[j] = mx;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vf[8];
                vr[u].unpack(vf);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[j][e] = fmaf(pu[u], vf[e], o[j][e]);
            }
        }
    }

    // merge the row slots of each wave (lanes LPR, 2 LPR, ... apart)
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
            for (int e = 0; e < 8; ++e) s_o[wave][j][l * 8 + e] = o[j][e];
            if (lane == 0) {
                s_m[wave][j] = m[j];
                s_l[wave][j] = ls[j];
            }
        }
    }
    __syncthreads();
    // merge the 4 waves and write this chunk's partial for each head
    for (int idx = t; idx < G * D; idx += 256) {
        const int j = idx / D, d = idx % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][j]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float wt = s_m[w][j] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(s_m[w][j] - M);
            L += s_l[w][j] * wt;
            O += s_o[w][j][d] * wt;
        }
        const int h = g * G + j;
        const size_t pi = ((size_t)b * a.nq + h) * a.maxc + c;
        publish(&a.part_o[pi * D + d], O);
        if (d == 0) {
            publish(&a.part_ml[pi * 2], M);
            publish(&a.part_ml[pi * 2 + 1], L);
        }
    }

    if (!arrive_last(&a.cnt[b * nkv + g], nchunk, &s_last)) return;

    // last workgroup of (b, g): log-sum-exp merge of the chunk partials
    constexpr int PARTS = 256 / D;       // threads per output element
    for (int j = 0; j < G; ++j) {
        const int h = g * G + j;
        const size_t pbase = ((size_t)b * a.nq + h) * a.maxc;
        float mloc = kNegInf;
        for (int cc = t; cc < nchunk; cc += 256) {
            const float mc = fetch(&a.part_ml[(pbase + cc) * 2]);
            s_cm[cc] = mc;
            mloc = fmaxf(mloc, mc);
        }
        mloc = wave_max(mloc);
        if (lane == 0) s_red[wave] = mloc;
        __syncthreads();
        const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
        float lloc = 0.f;
        for (int cc = t; cc < nchunk; cc += 256) {
            const float w = __builtin_amdgcn_exp2f(s_cm[cc] - M);
            s_cw[cc] = w;
            lloc += w * fetch(&a.part_ml[(pbase + cc) * 2 + 1]);
        }
        lloc = wave_sum(lloc);
        __syncthreads();                     // s_red reads above are done
        if (lane == 0) s_red[4 + wave] = lloc;
        __syncthreads();
        const float L = s_red[4] + s_red[5] + s_red[6] + s_red[7];
        const int d = t % D, part = t / D;
        float acc = 0.f;
        for (int c0 = part; c0 < nchunk; c0 += 8 * PARTS) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int cc = c0 + j * PARTS;
                v[j] = cc < nchunk ? s_cw[cc] * fetch(&a.part_o[(pbase + cc) * D + d]) : 0.f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += v[j];
        }
        s_acc[t] = acc;
        __syncthreads();
        if (t < D) {
            float tot = 0.f;
#pragma unroll
            for (int q = 0; q < PARTS; ++q) tot += s_acc[q * D + t];
            a.a_out[(size_t)b * a.nq * D + (size_t)h * D + t] = tot / L;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

namespace {

template <typename T, int BG, bool QKV>
hipError_t launch_gemv_bg(const GemvArgs& a, int rows, int grid, hipStream_t s) {
    if (rows == 128) hipLaunchKernelGGL((gemv_kernel<T, BG, 128, QKV>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemv_kernel<T, BG, 64, QKV>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename T, bool QKV>
hipError_t launch_gemv_t(const GemvArgs& a, int bg, int rows, int grid, hipStream_t s) {
    switch (bg) {
        case 1: return launch_gemv_bg<T, 1, QKV>(a, rows, grid, s);
        case 2: return launch_gemv_bg<T, 2, QKV>(a, rows, grid, s);
        case 4: return launch_gemv_bg<T, 4, QKV>(a, rows, grid, s);
        default: return launch_gemv_bg<T, 8, QKV>(a, rows, grid, s);
    }
}

template <typename T, int D>
hipError_t launch_attn_d(const AttnArgs& a, int G, int grid, hipStream_t s) {
    switch (G) {
#define DAB_G(NG) case NG: hipLaunchKernelGGL((attn_kernel<T, D, NG>), dim3(grid), dim3(256), 0, s, a); break;
        DAB_G(1) DAB_G(2) DAB_G(3) DAB_G(4) DAB_G(5) DAB_G(6) DAB_G(7) DAB_G(8)
#undef DAB_G
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_attn_t(const AttnArgs& a, int D, int G, int grid, hipStream_t s) {
    return D == 128 ? launch_attn_d<T, 128>(a, G, grid, s) : launch_attn_d<T, 64>(a, G, grid, s);
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), words);
    return hipGetLastError();
}

hipError_t launch_gemv(const GemvArgs& a, bool bf16, bool qkv, int bg, int rows, int grid, hipStream_t s) {
    if (bf16) return qkv ? launch_gemv_t<uint16_t, true>(a, bg, rows, grid, s)
                         : launch_gemv_t<uint16_t, false>(a, bg, rows, grid, s);
    return qkv ? launch_gemv_t<float, true>(a, bg, rows, grid, s) : launch_gemv_t<float, false>(a, bg, rows, grid, s);
}

hipError_t launch_attn(const AttnArgs& a, bool bf16, int D, int G, int grid, hipStream_t s) {
    return bf16 ? launch_attn_t<uint16_t>(a, D, G, grid, s) : launch_attn_t<float>(a, D, G, grid, s);
}

}  // namespace dab

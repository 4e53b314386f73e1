// Kernel arguments and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dab_plan.h"

namespace dab {

// One GEMV phase: QKV (RMSNorm folded in, RoPE + cache append in the
// finaliser) or O-projection (residual in the finaliser).
struct GemvArgs {
    const void* W;          // [K, N] storage type, row-major
    const void* hidden;     // [B, H] storage type
    const void* norm_w;     // [H] storage type (QKV)
    const float* xin;       // [B, K] fp32 input rows (O-projection: attention output)
    float* part;            // [ksplit, B, N] fp32 partial sums
    float* ssq;             // [slabs, ksplit, B] partial sums of x^2 (QKV)
    int* cnt;               // [slabs * nbg] arrival counters, zero between calls
    int* flags;             // device error flags
    const int* pos;         // [B]
    float* q;               // [B, nq*D] rotated q, fp32 (QKV)
    void* k_cache;          // [B, cap, nkv, D] (QKV)
    void* v_cache;
    void* out;              // [B, H] (O-projection)
    float* dbg_y;           // [B, H] fp32 or null (O-projection)
    int B, K, N, slabs, ksplit, nbg, tiles;
    int cap, n_q, nkv, D;
    float eps;
    double log2_theta;
};

struct AttnArgs {
    const float* q;         // [B, nq*D] rotated q
    const void* k_cache;    // [B, cap, nkv, D]
    const void* v_cache;
    const int* pos;         // [B]
    float* part_o;          // [B, nq, maxc, D] unnormalised chunk outputs
    float* part_ml;         // [B, nq, maxc, 2] chunk (max, sum) in log2 units
    int* cnt;               // [B * nkv] arrival counters
    float* a_out;           // [B, nq*D] attention output
    int nq, nkv, cap, T, maxc;
    float qscale;           // log2(e) / sqrt(D)
};

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_gemv(const GemvArgs& a, bool bf16, bool qkv, int bg, int rows, int grid, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, bool bf16, int D, int G, int grid, hipStream_t s);

}  // namespace dab

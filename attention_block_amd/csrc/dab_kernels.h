// Kernel arguments and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dab_plan.h"

namespace dab {

// Finish counting in the fused schedule: sub-counters on separate 256-byte lines.
constexpr int kDoneShards = 16;
constexpr int kDoneStride = 64;

// Tiling of one GEMV phase as the kernels see it.
struct GemvPlanDev {
    int slabs;     // 256-column slabs
    int ksplit;    // row blocks (K / rows)
    int rows;      // KR: rows of W per tile (64 or 128)
    int nbg;       // batch groups
    int tiles;     // slabs * ksplit
    int items;     // work indices (tiles, padded per batch group)
};

// Everything one decode step needs, for every kernel of either schedule.
struct StepArgs {
    // caller tensors
    const void* hidden;     // [B, H]
    const void* norm_w;     // [H]
    const void* w_qkv;      // [H, n_qkv]
    const void* w_o;        // [n_q, H]
    void* k_cache;          // [B, cap, nkv, D]
    void* v_cache;
    const int* pos;         // [B]
    void* out;              // [B, H]
    float* dbg_y;           // [B, H] or null
    // workspace
    int* flags;             // error bits
    int* done;              // fused schedule: finished items, kDoneShards counters kDoneStride ints apart
    int* done_all;          // fused schedule: finished shards
    int* epoch;             // fused schedule: calls completed (message tags derive from it)
    int* qkv_cnt;           // [q slabs * nbg] tile arrivals (+1 when the slab is final)
    int* attn_cnt;          // [B * nkv] chunk arrivals (+1 when merged)
    int* oproj_cnt;         // [o slabs * nbg] tile arrivals
    // published buffers hold 8 bytes per element: {value, tag} words in the
    // fused schedule, a float array in the low half in the phased one
    float* qkv_part;        // [q ksplit, B, n_qkv]
    float* ssq;             // [q slabs, q ksplit, B]
    float* q;               // [B, n_q] rotated q
    float* kv_new;          // [B, 2, nkv, D] the new token's rotated k and v
    float* attn_o;          // [B, nq, maxc, D]
    float* attn_ml;         // [B, nq, maxc, 2]
    float* a;               // [B, n_q] attention output
    float* oproj_part;      // [o ksplit, B, H]
    // shapes and numerics
    int B, H, nq, nkv, D, G, cap, n_qkv, n_q;
    float eps, qscale;      // qscale = log2(e) / sqrt(D)
    double log2_theta;
    // plan
    GemvPlanDev qkv, oproj;
    int qkv_bg;             // batch rows per GEMV tile
    int T, maxc, attn_items;
    int total_items;        // fused schedule: work items of the whole step
    int item_lo;            // fused schedule: first work item of this launch (its workgroup 0)
    // fused schedule, unit order (one unit = all heads when not unitised)
    int units;              // number of units
    int unit_items;         // work items per unit
    int unit_slabs;         // QKV slabs per unit
    int unit_kv;            // kv heads per unit
    int unit_oks;           // output-projection row blocks per unit
#ifdef DAB_TRACE
    unsigned long long* trace;   // [items, 8] timestamps per workgroup (profiling builds only)
    int trace_base;              // item number of this launch's workgroup 0
#endif
};

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_fused(const StepArgs& a, bool bf16, hipStream_t s);
// two-stage schedule: QKV tiles alone, then attention and output tiles
hipError_t launch_two_stage(const StepArgs& a, bool bf16, int stage, hipStream_t s);
hipError_t launch_phase(const StepArgs& a, bool bf16, int phase, hipStream_t s);

// per-dtype instantiations of the fused kernel (separate translation units)
hipError_t launch_fused_bf16(const StepArgs& a, hipStream_t s);
hipError_t launch_fused_f32(const StepArgs& a, hipStream_t s);
hipError_t launch_stage_qkv_bf16(const StepArgs& a, hipStream_t s);
hipError_t launch_stage_qkv_f32(const StepArgs& a, hipStream_t s);

}  // namespace dab

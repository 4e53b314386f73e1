// Kernel arguments and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dab_plan.h"

namespace dab {

// One row-panel GEMV as the kernels see it.
struct PanelPlanDev {
    int panels;    // row panels: 4 waves x rows_per_wave rows of W
    int nb;        // batch rows per workgroup (1, 2 or 4)
    int nbg;       // batch groups: ceil(B / nb)
    int items;     // workgroups (panels, padded per batch group)
};

// Everything one decode step needs, for every kernel.
struct StepArgs {
    // caller tensors
    const void* hidden;     // [B, H]
    const void* norm_w;     // [H]
    const void* w_qkv;      // [n_qkv, H]: one output feature per row
    const void* w_o;        // [H, n_q]
    void* k_cache;          // [B, cap, nkv, D]
    void* v_cache;
    const int* pos;         // [B]
    void* out;              // [B, H]
    float* dbg_y;           // [B, H] or null
    // workspace
    int* flags;             // error bits
    int* attn_cnt;          // [B * nkv] chunk arrivals (re-armed by the merging workgroup)
    int* seq_ready;         // [B, kReadyCopies] x kReadyStride: kv groups of the sequence merged so far (one-launch attention + projection; re-armed by the QKV kernel)
    int* ready_done;        // [B, kReadyCopies] x kReadyStride: projection workgroups past their wait on each
                            // copy of seq_ready (whole step in one launch; the last one re-arms both)
    int* head_cnt;          // QKV panels done per (batch group, head) [qkv.nbg, nq + 2 nkv] (one-launch QKV +
                            // attention; re-armed by the output projection kernel) or per (sequence, head)
                            // [B, nq + 2 nkv] (whole step in one launch; re-armed by its projection panels)
    int head_cnt_per_seq;   // 1: head_cnt is per (sequence, head)
    int* hand;              // layer launch: the FFN workspace's hand-off of h (h_sub_at, h_flag_at), else null
    int ready_copies;       // copies of seq_ready in use: min(kReadyCopies, output projection panels)
    float* q;               // [B, n_q] rotated q
    float* kv_new;          // [B, 2, nkv, D] the new token's rotated k and v
    float* attn_o;          // [B, nq, maxc, D] chunk partial outputs
    float* attn_ml;         // [B, nq, maxc, 2] chunk (max, sum)
    float* a;               // [B, n_q] attention output
    uint16_t* a16;          // [B, n_q] the same rounded to bf16 (bf16 storage, phased schedule: MFMA input)
    // shapes and numerics
    int B, H, nq, nkv, D, G, cap, n_qkv, n_q;
    int pos_end;            // valid positions: [0, pos_end) (the max_position hint + 1, else cap)
    float eps, qscale;      // qscale = log2(e) / sqrt(D)
    double log2_theta;
    // plan
    PanelPlanDev qkv, oproj;
    ChunkRule chunk;        // split-KV chunk length of each sequence, from its position (chunk_len)
    int* seq_chunk;         // [B, 2] each sequence's chunk length and count, written by workgroup 0 of the
                            // QKV kernel for the attention launches after it (phased and attention +
                            // projection schedules), else null: the attention items evaluate the rule
    int maxc, attn_items;
    int split_merge;        // phased: chunk partials are merged by a kernel of their own
#ifdef DAB_TRACE
    unsigned long long* trace;   // [items, 8] timestamps per workgroup (profiling builds only)
    int trace_base;              // item number of this launch's workgroup 0
#endif
};

// Events a timed call records at a kernel's own start and end (null: untimed).
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};

// The FFN half of the layer, for both of its kernels.
struct FfnArgs {
    const void* hidden;     // [B, H] h
    const void* norm_w;     // [H]
    const void* w_gate;     // [F, H]
    const void* w_up;       // [F, H]
    const void* w_down;     // [H, F]
    void* out;              // [B, H]
    float* dbg_y;           // [B, H] or null
    float* m;               // [B, F] silu(g) * u (workspace; VALU panels)
    uint16_t* m16;          // [B, F] the same rounded to bf16 (workspace; MFMA panels)
    int B, H, F;
    float eps;
    int mfma;               // MFMA panels (bf16, batch >= 8): 16 sequences per workgroup
    int down_tiles;         // MFMA down panel: 1 or 2 tiles of 16 rows
    int gu_tiles;           // streamed gate/up panel: mixed tiles (8 features) per panel, 0: not streamed
    PanelPlanDev gu, down;
    int* hand;              // layer launch: hand-off of h from the projection panels (the down kernel
                            // re-arms its ready counts), else null
    int* flags;             // layer launch: the attention workspace's error bits, else null
    int h_panels;           // layer launch: the output projection's panels, which publish h
#ifdef DAB_TRACE
    unsigned long long* trace;
    int trace_base;
#endif
};

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// FFN kernel `phase` (0: RMSNorm + gate/up + silu, 1: down + residual).
hipError_t launch_ffn_phase(const FfnArgs& a, int dtype, int phase, hipStream_t s, const LaunchEvents& ev);
// Kernel `phase` of the plan's schedule (0 .. phase_count - 1).
hipError_t launch_phase(const StepArgs& a, const Plan& p, int phase, hipStream_t s, const LaunchEvents& ev);

// The layer in two launches after the QKV kernel: attention + output
// projection + FFN gate/up in one launch (the gate/up panels stream their
// weights before h is complete), then the FFN down kernel.  layer_overlap_ok:
// the plans this is built for.
bool layer_overlap_ok(const Plan& p, const FfnPlan& f);
hipError_t launch_layer_attn_ffn(const StepArgs& a, const FfnArgs& f, const Plan& p, const FfnPlan& fp, hipStream_t s,
                                 const LaunchEvents& ev);

// per-dtype instantiations (separate translation units)
hipError_t launch_phase_bf16(const StepArgs& a, const Plan& p, int phase, hipStream_t s, const LaunchEvents& ev);
hipError_t launch_phase_f32(const StepArgs& a, const Plan& p, int phase, hipStream_t s, const LaunchEvents& ev);
// Workgroups of the phased schedule's attention kernel one CU holds at once (0: unknown).
int attn_resident_bf16(int D, int G);
int attn_resident_f32(int D, int G);

}  // namespace dab

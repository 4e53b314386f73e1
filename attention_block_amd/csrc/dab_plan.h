// Host-side validation and launch planning of the decode attention block.
// Pure C++ (no HIP headers): the C ABI layer calls it before enqueueing
// anything, and the host sanitizer build exercises it on the CPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "dab.h"

namespace dab {

// Columns of one GEMV slab: 32 lanes x 8 columns (one 16-byte bf16 load each).
constexpr int kSlab = 256;
// Threads per workgroup of every kernel.
constexpr int kThreads = 256;
// Largest number of split-KV chunks per sequence the merge step stages.
constexpr int kMaxChunks = 1024;
// Largest query-head group per KV head the attention kernel keeps in registers.
constexpr int kMaxGroup = 8;
// Tokens per attention chunk in the fused schedule: one batch of loads,
// 256 / (D/8) row slots x 8 tokens.
inline int fused_chunk(int head_dim) { return 8 * 256 / (head_dim / 8); }

struct GemvPlan {
    int K = 0, N = 0;     // reduction length, output columns
    int slabs = 0;        // ceil(N / kSlab)
    int rows = 0;         // rows of W per workgroup (KR), 64 or 128
    int ksplit = 0;       // K / rows
    int bg = 0;           // batch rows per workgroup (1, 2, 4 or 8)
    int nbg = 0;          // ceil(B / bg)
    int tiles = 0;        // slabs * ksplit
    int grid = 0;         // work indices: tiles, padded per batch group
};

struct Plan {
    int B = 0, H = 0, nq = 0, nkv = 0, D = 0, cap = 0, dtype = 0, G = 0;
    int n_qkv = 0, n_q = 0;      // (nq + 2 nkv) D, nq D
    float theta = 0.f, eps = 0.f;
    int elem = 0;                // bytes per stored element

    int schedule = DAB_SCHEDULE_PHASED;   // resolved: FUSED, TWO_STAGE or PHASED
    bool fused = false;          // FUSED or TWO_STAGE: tagged hand-offs, fused device code
    GemvPlan qkv, oproj;
    int kv_chunk = 0, max_chunks = 0, attn_grid = 0;
    int total_items = 0;         // fused: qkv.grid + attn_grid + oproj.grid (+ unit padding)
    // fused unit order: units of unit_kv kv heads, each with unit_slabs QKV
    // slabs, its attention chunks and unit_oks output row blocks
    int units = 1, unit_items = 0, unit_slabs = 0, unit_kv = 0, unit_oks = 0;

    // workspace layout, byte offsets (each 256-byte aligned).  The flags
    // word is at offset 0, the finished-shard count at 4, the call epoch at
    // 8; the 16 finish sub-counters follow, one per 256 bytes.
    size_t off_flags = 0, off_done = 0, off_qkv_cnt = 0, off_attn_cnt = 0, off_oproj_cnt = 0;
    size_t off_qkv_part = 0, off_ssq = 0, off_q = 0, off_kv_new = 0;
    size_t off_attn_o = 0, off_attn_ml = 0, off_a = 0, off_oproj_part = 0;
    size_t ws_bytes = 0;

    // byte extents of the caller's tensors (for alias checks)
    size_t bytes_hidden = 0, bytes_norm = 0, bytes_wqkv = 0, bytes_wo = 0, bytes_cache = 0;
    size_t bytes_pos = 0, bytes_out = 0, bytes_dbg = 0;
};

// Validate `cfg` and fill `plan`.  Returns DAB_OK, DAB_ERR_INVALID_ARG or
// DAB_ERR_UNSUPPORTED.  Makes no HIP calls.
dab_status make_plan(const dab_config* cfg, Plan* plan);

// Validate the pointers of a call against a plan: non-null where required,
// 16-byte aligned, `out` disjoint from every other argument, workspace large
// enough.  Makes no HIP calls and dereferences nothing.
dab_status check_call(const Plan& p, const void* hidden, const void* norm_w, const void* w_qkv,
                      const void* w_o, const void* k_cache, const void* v_cache, const int32_t* pos,
                      const void* out, const float* dbg_y, const void* workspace, size_t ws_bytes);

}  // namespace dab

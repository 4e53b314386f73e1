// Host-side validation and launch planning of the decode attention block.
// Pure C++ (no HIP headers): the C ABI layer calls it before enqueueing
// anything, and the host sanitizer build exercises it on the CPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "dab.h"

namespace dab {

// Threads per workgroup of every kernel (four waves).
constexpr int kThreads = 256;
// Largest number of split-KV chunks per (sequence, kv head) the merge step
// stages (the chunk length grows with the context to stay below it).
constexpr int kMaxChunks = 256;
// Largest query-head group per KV head the attention kernel keeps in registers.
constexpr int kMaxGroup = 8;
// LDS a GEMV workgroup may give its fp32 input rows (nb x K floats).
constexpr int kPanelLds = 64 * 1024;
// Ready flags of a sequence's attention output (one-launch attention +
// projection): copies on separate 128-byte lines, so that the projection's
// workgroups, which poll them, spread over kReadyCopies addresses instead of
// queueing on one.
constexpr int kReadyCopies = 16;
constexpr int kReadyStride = 32;     // ints
// Hand-off of the attention block's output h to the FFN panels of the same
// launch (the overlapped layer), per sequence, each counter on a line of its
// own: the output-projection panels arrive at kHSub counters (panel p at
// p % kHSub), and the last arrival at each adds one, with no reply
// requested, to all kHCopies ready counts, which the FFN panels poll (2752
// of them for the 7B layer: about 43 per copy) until they reach the number
// of counters in use.  One counter for all 512 panels of the 7B layer
// measured 7.4 us of serialised arrivals; every panel adding to its counter
// in 8 sets, with the FFN panels polling all 16 counters of a set, measured
// 1.2 us slower than this.  In the FFN workspace, at off_hand; the last
// arrival at a counter re-arms it, the FFN down kernel the ready counts.
constexpr int kHSub = 16;
constexpr int kHCopies = 64;
constexpr int kHLines = kHSub + kHCopies;
constexpr int h_region(int B) { return B * kHLines * kReadyStride; }              // ints for B sequences
constexpr int h_sub_at(int b, int i) { return (b * kHLines + i) * kReadyStride; }
constexpr int h_flag_at(int b, int c) { return (b * kHLines + kHSub + c) * kReadyStride; }
// counters in use for a projection of `panels` panels
constexpr int h_subs(int panels) { return panels < kHSub ? panels : kHSub; }
// Chunks per thread and head that the attention kernel's in-launch merge
// requests at once (32 loads in flight per thread).
constexpr int merge_round(int G) { return G >= 8 ? 4 : 32 / G; }

#if defined(__HIPCC__)
#define DAB_HOST_DEVICE __host__ __device__
#else
#define DAB_HOST_DEVICE
#endif

// The split-KV chunk length rule.  The host evaluates it at the cache
// capacity (cap - 1 cached tokens) to size the grid (max_chunks chunk slots
// per (sequence, kv head)); every attention workgroup evaluates it at its own
// sequence's position, so that a sequence with far fewer tokens than the
// capacity still gets about `want` chunks instead of a few long ones.
struct ChunkRule {
    int fixed = 0;          // > 0: the caller's kv_chunk, the same for every sequence
    int want = 1;           // chunks per (sequence, kv head) aimed at
    int lo = 16, hi = 448;  // clamps of the length, in tokens
    int whole = 16;         // the length is rounded up to a multiple of this
    int want2 = 0;          // > 0: the two-per-CU rule: where pairs * chunks would exceed `resident`,
    int hi2 = 0;            //   chunks of ceil(p / want2) tokens where that is longer and at most hi2
    int pairs = 0;          //   (sequences x kv heads)
    int resident = 0;       //   (attention workgroups the device holds at once)
    int maxc = 1;           // chunk slots per (sequence, kv head) in the grid
};

// Chunk length for a sequence with `hist` cached tokens: never more than
// r.maxc chunks.
DAB_HOST_DEVICE inline int chunk_len(const ChunkRule& r, int hist) {
    if (r.fixed > 0) return r.fixed;
    const int h = hist > 0 ? hist : 1;
    int T = ((h + r.want - 1) / r.want + 15) / 16 * 16;
    if (T < r.lo) T = r.lo;
    if (T > r.hi) T = r.hi;
    T = (T + r.whole - 1) / r.whole * r.whole;
    if (r.want2 > 0 && (long long)r.pairs * ((h + T - 1) / T) > r.resident) {
        const int T1 = ((h + r.want2 - 1) / r.want2 + 15) / 16 * 16;
        if (T1 <= r.hi2 && T1 > T) T = T1;
    }
    const int floor = ((h + r.maxc - 1) / r.maxc + 15) / 16 * 16;
    return T > floor ? T : floor;
}

// Chunks of a sequence at position p (cached tokens): the last one also takes
// the new token; a sequence with no history has one chunk, for that token.
DAB_HOST_DEVICE inline int chunk_count(const ChunkRule& r, int p) {
    if (p <= 0) return 1;
    const int T = chunk_len(r, p);
    return (p + T - 1) / T;
}

// A row-panel GEMV y[b, n] = sum_k W[n, k] x[b, k] with W stored [N, K]
// (every output's K weights contiguous).  A workgroup owns `rows` = 4 waves
// x rows_per_wave outputs and all K for `nb` batch rows, so no partial sums
// cross workgroups.
struct PanelPlan {
    int K = 0, N = 0;
    bool mfma = false;      // MFMA panels: 16 or 32 rows x 16 or 32 sequences per workgroup (bf16, batch >= 8)
    int rows_per_wave = 0;  // 1 or 2 (the QKV panel: one RoPE pair per wave)
    int rows = 0;           // 4 * rows_per_wave
    int panels = 0;         // N / rows
    int nb = 0;             // batch rows per workgroup: 1, 2 or 4
    int nbg = 0;            // ceil(B / nb)
    int grid = 0;           // workgroups: panels, padded to a multiple of 8 per batch group
    size_t lds = 0;         // dynamic LDS bytes: nb * K floats
};

struct Plan {
    int B = 0, H = 0, nq = 0, nkv = 0, D = 0, cap = 0, dtype = 0, G = 0;
    int pos_end = 0;             // positions in [0, pos_end) are valid: max_position + 1, else cap
    int n_qkv = 0, n_q = 0;      // (nq + 2 nkv) D, nq D
    float theta = 0.f, eps = 0.f;
    int elem = 0;                // bytes per stored element

    int schedule = DAB_SCHEDULE_PHASED;   // resolved schedule (never AUTO)
    bool attn_oproj_ok = false;           // the one-launch attention + projection is built for this shape
    bool qkv_attn_ok = false;             // the one-launch QKV + attention is built for this shape
    bool fused_ok = false;                // the one-launch whole step is built for this shape
    PanelPlan qkv, oproj;
    int kv_chunk = 0, max_chunks = 0, attn_grid = 0;   // kv_chunk: the length at the capacity
    ChunkRule chunk;                                  // the length for each sequence's position
    bool split_merge = false;             // phased: the LSE merge runs as a kernel of its own

    // workspace layout, byte offsets (each 256-byte aligned); the flags
    // word is at offset 0
    size_t off_flags = 0, off_attn_cnt = 0, off_seq_ready = 0, off_ready_done = 0, off_head_cnt = 0;
    size_t off_q = 0, off_kv_new = 0;
    size_t off_attn_o = 0, off_attn_ml = 0, off_a = 0, off_a16 = 0, off_seq_chunk = 0;
    size_t ws_bytes = 0;

    // byte extents of the caller's tensors (for alias checks)
    size_t bytes_hidden = 0, bytes_norm = 0, bytes_wqkv = 0, bytes_wo = 0, bytes_cache = 0;
    size_t bytes_pos = 0, bytes_out = 0, bytes_dbg = 0;
};

// The FFN half of the layer: two row-panel GEMVs.  gu: W_gate and W_up
// (wave w of panel i takes row 4i + w of both, K = H, N = 2F counted as
// rows of the pair); down: W_down, two rows per wave, K = F.
struct FfnPlan {
    int B = 0, H = 0, F = 0, dtype = 0, elem = 0;
    float eps = 0.f;
    bool mfma = false;        // bf16, batch >= 8: MFMA panels for both GEMVs
    int gu_tiles = 0;         // gate/up on the streamed panel: mixed tiles (8 features, gate and up) per panel
    PanelPlan gu, down;
    size_t off_m = 0, off_m16 = 0, off_hand = 0, ws_bytes = 0;
    size_t bytes_hidden = 0, bytes_norm = 0, bytes_wgu = 0, bytes_wdown = 0, bytes_out = 0, bytes_dbg = 0;
};

dab_status make_ffn_plan(const dab_ffn_config* cfg, FfnPlan* plan);

dab_status check_ffn_call(const FfnPlan& p, const void* hidden, const void* norm_w, const void* w_gate,
                          const void* w_up, const void* w_down, const void* out, const float* dbg_y,
                          const void* workspace, size_t ws_bytes);

// Both halves' checks (h the attention block's out and the FFN's input),
// then every pair across the halves in which either side is written must
// not overlap.  Makes no HIP calls and dereferences nothing.
dab_status check_layer_call(const Plan& p, const FfnPlan& f, const void* hidden, const void* attn_norm_w,
                            const void* w_qkv, const void* w_o, const void* k_cache, const void* v_cache,
                            const int32_t* pos, const void* ffn_norm_w, const void* w_gate, const void* w_up,
                            const void* w_down, const void* h, const void* out, const void* workspace,
                            size_t ws_bytes, const void* ffn_workspace, size_t ffn_ws_bytes);

// Validate `cfg` and fill `plan`.  Returns DAB_OK, DAB_ERR_INVALID_ARG or
// DAB_ERR_UNSUPPORTED.  Makes no HIP calls.
// attn_cus, attn_per_cu: the device's compute units and how many workgroups
// of the phased schedule's attention kernel one of them holds at once for
// this shape, 0 if unknown; they only steer the split-KV chunk length.
dab_status make_plan(const dab_config* cfg, Plan* plan, int attn_cus = 0, int attn_per_cu = 0);

// Validate the pointers of a call against a plan: non-null where required,
// 16-byte aligned, `out` disjoint from every other argument, workspace large
// enough.  Makes no HIP calls and dereferences nothing.
dab_status check_call(const Plan& p, const void* hidden, const void* norm_w, const void* w_qkv,
                      const void* w_o, const void* k_cache, const void* v_cache, const int32_t* pos,
                      const void* out, const float* dbg_y, const void* workspace, size_t ws_bytes);

}  // namespace dab

/*
 * dab.h - C ABI of the fused single-token decode attention block for
 * AMD Instinct MI355X (gfx950).
 *
 * One call computes, for every sequence b of a batch, the decode step of a
 * pre-norm transformer attention block (the block composition listed in the
 * operator-fusion article, "LayerNorm + Attention" CUDA kernel page,
 * section 1; the fused dataflow of the ClusterFusion page, section 3.2):
 *
 *   r      = (mean_i x_i^2 + eps)^(-1/2),  xh = x * r * norm_w        RMSNorm
 *   u      = xh @ W_qkv^T        (packed outputs [Q | K | V])           QKV GEMV
 *   q, k   = RoPE(q, pos_b), RoPE(k, pos_b)   (rotate-half pairing)     RoPE
 *   cache  : K[b, pos_b] = k, V[b, pos_b] = v                           KV append
 *   a_h    = softmax(q_h . K[b, 0..pos_b, g(h)] / sqrt(D)) @ V[...]     attention
 *   out    = x + a @ W_o^T                                              O-proj + residual
 *
 * with g(h) = h / (n_q_heads / n_kv_heads) (grouped-query mapping of the
 * operator-fusion page, section 3).  RoPE angle for pair (j, j + D/2) is
 * pos_b * theta^(-2j/D).
 *
 * Weights are taken in the [out_features, in_features] layout (the layout of
 * a torch.nn.Linear weight): the transpose of the [in, out] matrices the
 * pages multiply by (the ClusterFusion page, section 1.1, multiplies the
 * hidden state by W_qkv and the attention output by W_out; the
 * operator-fusion page, section 3, indexes q_weight as [hidden_dim,
 * heads * head_dim]).  Each output's weights are then one contiguous row, so
 * at decode batch sizes one workgroup computes whole outputs and no partial
 * sums cross workgroups.  Weights are static: dab_pack_weight turns a matrix
 * in the pages' [in, out] layout into this one on the device, once, at load
 * time.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise,
 *     16-byte aligned, to memory of the device that is current when the
 *     call is made.  The caller owns every buffer; the library never
 *     allocates or frees device memory in these calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; no call below synchronises the
 *     device except dab_read_device_error.  The enqueue sequence contains
 *     only kernel launches, so it may be captured into a HIP graph.
 *   - Storage dtype DAB_BF16: hidden, norm_w, W_qkv, W_o, both caches and out
 *     hold bf16 and every sum accumulates in fp32.  Intermediates are fp32
 *     except where a matrix-core or pair-dot-product operand is rounded to
 *     bf16 (nearest-even, a relative 2^-9 each): with grouped heads
 *     (n_q_heads > n_kv_heads) attention rounds the pre-scaled q and the
 *     softmax weights to bf16 for v_dot2 products against the stored K and
 *     V; with a batch of 8 or more the phased schedule's matrix-core panels
 *     round x * norm_w and the attention output to bf16; the new token's k
 *     and v enter attention rounded to bf16, exactly as appended.
 *     DAB_F32: every tensor and every intermediate is fp32.
 *   - Errors a host can see (bad shapes, null or misaligned pointers,
 *     overlapping output, short workspace) return a status before anything
 *     is enqueued, and no buffer is touched.  A launch failure returns
 *     DAB_ERR_HIP.  An out-of-range pos[b] can only be seen on the device:
 *     that sequence is skipped (no cache write, its out row is left
 *     unwritten) and a sticky flag is raised in the workspace, readable with
 *     dab_read_device_error.
 */
#ifndef DAB_H
#define DAB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DAB_OK = 0,
    DAB_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size, aliasing */
    DAB_ERR_UNSUPPORTED = 2,  /* shape outside what the kernels implement     */
    DAB_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required   */
    DAB_ERR_HIP = 4           /* the HIP runtime reported an error            */
} dab_status;

typedef enum { DAB_F32 = 0, DAB_BF16 = 1 } dab_dtype;

/* Shape and numerics of one decode-block call. */
typedef struct {
    int32_t batch;           /* B >= 0 sequences (0: nothing to do)                     */
    int32_t hidden;          /* H, multiple of 64, at most 16384                        */
    int32_t n_q_heads;       /* nq >= 1                                                 */
    int32_t n_kv_heads;      /* nkv >= 1, divides nq, nq / nkv <= 8                     */
    int32_t head_dim;        /* D: 64 or 128; nq * D at most 16384                      */
    int32_t cache_capacity;  /* cap: token rows per sequence in each cache              */
    int32_t dtype;           /* dab_dtype                                               */
    float rope_theta;        /* RoPE base, > 0                                          */
    float eps;               /* RMSNorm epsilon, >= 0 (1e-6 in the pages' kernels)      */
    int32_t kv_chunk;        /* cached tokens per split-KV work item: 0 = automatic     */
                             /* (sized for the current device: see dab_workspace_size), */
                             /* else a multiple of 16 in [32, 4096]                     */
    int32_t schedule;        /* dab_schedule: how the step is laid out on the GPU        */
    int32_t max_position;    /* the largest position any sequence of the call holds      */
                             /* (0: not given, cap - 1), at most cap - 1.  It sizes the  */
                             /* split-KV grid and workspace from the tokens in use       */
                             /* rather than the capacity; a sequence beyond it is        */
                             /* rejected on the device as one past the capacity is (the  */
                             /* error flag, its row and cache left untouched)            */
} dab_config;

/*
 * DAB_SCHEDULE_PHASED runs one kernel per phase: QKV (RMSNorm, projection,
 * RoPE, append), split-KV attention (each (sequence, kv head) merged by its
 * last chunk), output projection with the residual.
 * DAB_SCHEDULE_ATTN_OPROJ runs the QKV kernel, then attention and the output
 * projection as one launch whose projection workgroups stream their weights
 * while the last attention chunks finish.  It needs n_q_heads / n_kv_heads
 * in {1, 2, 4, 8} and nq * D a multiple of 4096 (bf16) or 2048 (fp32).
 * DAB_SCHEDULE_QKV_ATTN runs QKV and attention as one launch whose attention
 * workgroups load their K/V rows while the QKV projection finishes, then
 * the output projection.  It needs n_q_heads / n_kv_heads in {1, 2, 4, 8}
 * and H a multiple of 4096 (bf16) or 2048 (fp32).
 * DAB_SCHEDULE_FUSED runs the whole step as one launch, its workgroups in
 * dependency order: the QKV projection's row panels (q, then k, then v
 * heads), the attention chunks, then the output projection's panels.  A
 * chunk waits only for the q panels of its kv group's query heads; the
 * chunk that also takes the new token waits for that group's k and v
 * panels before it; the output projection streams its weights as soon as
 * it has a slot and waits for its sequences' attention output.  It needs
 * n_q_heads / n_kv_heads in {1, 2, 4, 8}, nq * D a multiple of 4096 (bf16)
 * or 2048 (fp32), and batch <= 4.
 * AUTO picks the schedule measured fastest on MI355X: ATTN_OPROJ where it
 * applies with n_q_heads == n_kv_heads and batch <= 4, PHASED otherwise.
 * Every call is deterministic: every sum has a fixed order.  At one chunk
 * length (kv_chunk) the schedules give identical bits, except that the
 * phased schedule's matrix-core panels (bf16, batch of 8 or more) round
 * their operands to bf16 where the other schedules keep fp32.
 */
typedef enum {
    DAB_SCHEDULE_AUTO = 0,
    DAB_SCHEDULE_PHASED = 1,
    DAB_SCHEDULE_ATTN_OPROJ = 2,
    DAB_SCHEDULE_QKV_ATTN = 3,
    DAB_SCHEDULE_FUSED = 4
} dab_schedule;

/*
 * Bytes of device workspace one call with this configuration needs (0 when
 * the configuration is invalid).  The workspace holds q, the new k and v,
 * the split-KV partials, arrival counters and the device error flag.  It must
 * be initialised with dab_workspace_init before its first call; every call
 * re-arms the counters it uses, so later calls with the SAME configuration
 * (on one stream at a time) reuse it as is.  The layout depends on the
 * configuration: before a call with another configuration, initialise it
 * again.  With kv_chunk = 0 the chunk length, and so the size, also depends
 * on how many attention workgroups the current HIP device holds at once (read
 * from the runtime on first use, then cached per device): size and call on
 * the same device.  Without a device the size is the one of a device-free
 * plan.
 */
size_t dab_workspace_size(const dab_config* cfg);

/*
 * Zero `bytes` of workspace at `workspace` (device) with a fill kernel on
 * `stream`.  Returns DAB_ERR_INVALID_ARG for a null or misaligned pointer.
 */
dab_status dab_workspace_init(void* workspace, size_t bytes, void* stream);

/*
 * One decode step (all of the steps listed at the top of this header).
 *
 *   hidden   [B, H]              input hidden state x (read only)
 *   norm_w   [H]                 RMSNorm weight (read only)
 *   w_qkv    [(nq+2nkv)*D, H]    row-major, one output feature per row; row
 *                                blocks Q (nq*D), K (nkv*D), V (nkv*D), head-major
 *                                inside each block (row h*D + d: head h, dim d)
 *   w_o      [H, nq*D]           row-major, one output feature per row; column
 *                                h*D + d belongs to query head h
 *   k_cache, v_cache [B, cap, nkv, D]  token-major per sequence.  Rows
 *                                t < pos[b] are read; row pos[b] is written with
 *                                the new token's rotated k (resp. v), rounded to
 *                                the storage dtype; no other element changes.
 *   pos      int32 [B]           tokens already cached = index of the new token,
 *                                0 <= pos[b] < cap; attention covers pos[b] + 1
 *                                tokens (the history and the new one)
 *   out      [B, H]              x + a @ W_o, rounded to the storage dtype; must
 *                                not overlap any other argument
 *   dbg_y    [B, H] fp32 or NULL the pre-residual a @ W_o in fp32 (a test tap)
 *   workspace, workspace_bytes   device scratch of at least dab_workspace_size
 *                                bytes, initialised by dab_workspace_init for
 *                                this configuration (see dab_workspace_size)
 */
dab_status dab_decode_attn_block(const dab_config* cfg,
                                 const void* hidden, const void* norm_w,
                                 const void* w_qkv, const void* w_o,
                                 void* k_cache, void* v_cache,
                                 const int32_t* pos, void* out, float* dbg_y,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Same as dab_decode_attn_block, and also records `n_events` hipEvent_t
 * (passed as void*, created by the caller) for the kernels it enqueues on
 * `stream`: events[2i] at the start and events[2i + 1] at the end of kernel
 * i, taken by the kernel's own dispatch (hipExtLaunchKernel), so that
 * hipEventElapsedTime of the pair is the kernel's duration without the gaps
 * between kernels.  n_events must equal 2 * dab_phase_count(cfg).
 */
dab_status dab_decode_attn_block_timed(const dab_config* cfg,
                                       const void* hidden, const void* norm_w,
                                       const void* w_qkv, const void* w_o,
                                       void* k_cache, void* v_cache,
                                       const int32_t* pos, void* out, float* dbg_y,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream, void* const* events, int n_events);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as dab_decode_attn_block, with the same arguments, results and
 * errors, but no workspace argument.  Its workspace is a device array of
 * DAB_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held from
 * the library's load until the process ends; the call allocates nothing.
 * The first call on a device looks up that device's copy
 * (hipGetSymbolAddress), so make it outside a graph capture.  Every call
 * first clears the scratch's counter words with a fill kernel on `stream`
 * (so any configuration may follow any other), then enqueues the step's
 * kernels.  Calls on one GPU share its scratch: calls that overlap in time
 * on one GPU (on different streams, or the same graph launched twice
 * concurrently) race and give wrong results.  Returns DAB_ERR_WORKSPACE,
 * before anything is enqueued, when the configuration's workspace
 * (dab_workspace_size) exceeds DAB_NOALLOC_SCRATCH_BYTES.  The device error
 * flag of these calls is cleared by the next call and has no reader: a
 * sequence with an out-of-range pos is still skipped.
 */
#define DAB_NOALLOC_SCRATCH_BYTES (16u << 20)
dab_status dab_decode_attn_block_noalloc(const dab_config* cfg,
                                         const void* hidden, const void* norm_w,
                                         const void* w_qkv, const void* w_o,
                                         void* k_cache, void* v_cache,
                                         const int32_t* pos, void* out, float* dbg_y,
                                         void* stream);

/* Number of kernels one call enqueues for this configuration (0 if invalid). */
int dab_phase_count(const dab_config* cfg);

/* Name of kernel `i` (0-based) of a call, or NULL. */
const char* dab_phase_name(const dab_config* cfg, int i);

/*
 * Copy the workspace's sticky device error flag to *flag (host pointer) and
 * clear it.  Synchronises `stream`.  Bit 0: some pos[b] was outside [0, cap).
 * Bit 1: a workgroup of a one-launch schedule gave up waiting for its
 * inputs (a bounded wait that cannot expire in a correct run; results are
 * invalid).
 */
dab_status dab_read_device_error(void* workspace, void* stream, int32_t* flag);

/*
 * Test tap, not part of the step: copies the attention output a [B, nq*D]
 * (fp32, head-major: element b * nq*D + h*D + d is dim d of query head h)
 * that the last call with this configuration left in `workspace` to `dst`
 * (device, fp32, 16-byte aligned, must not overlap the workspace), with a
 * kernel on `stream` ordered after that call.  Every schedule keeps a in
 * the workspace.  Returns DAB_ERR_INVALID_ARG / DAB_ERR_UNSUPPORTED for a
 * bad configuration or pointer, DAB_ERR_WORKSPACE for a short workspace.
 */
dab_status dab_attention_output(const dab_config* cfg, const void* workspace, size_t workspace_bytes, float* dst,
                                void* stream);

/*
 * Weight layout conversion for callers that hold a matrix in the pages'
 * [in_features, out_features] layout (y = x @ W: the ClusterFusion page,
 * section 1.1, torch.mm(hidden_states, W_qkv) and torch.mm(attn_out,
 * W_out); the operator-fusion page, section 3, q_weight [hidden_dim,
 * num_heads * head_dim]).  Writes dst[o, i] = src[i, o], the
 * [out_features, in_features] layout every entry point here takes:
 *
 *   W_qkv [H, (nq+2nkv)*D]  -> [(nq+2nkv)*D, H]     (in = H)
 *   W_o   [nq*D, H]         -> [H, nq*D]            (in = nq*D)
 *   W_gate, W_up [H, F]     -> [F, H];  W_down [F, H] -> [H, F]
 *
 * src, dst: device, 16-byte aligned, in_features * out_features elements of
 * `dtype` each, caller-owned, not overlapping.  in_features at most
 * 65535 * 64, out_features at most 2^30.  One kernel on `stream`, no
 * allocation, no synchronisation; the bits are copied unchanged.  Returns
 * DAB_ERR_INVALID_ARG for a null, misaligned or overlapping pointer, a bad
 * size or dtype, DAB_ERR_HIP if the launch fails.
 */
dab_status dab_pack_weight(const void* src, void* dst, int64_t in_features, int64_t out_features, int32_t dtype,
                           void* stream);

/* Static, human-readable description of a status code. */
const char* dab_status_string(dab_status status);

/*
 * Name and description of the last HIP error that made a call on this
 * thread return DAB_ERR_HIP ("no error" if none).  The string is owned by
 * the library and valid until the next call on this thread.
 */
const char* dab_last_hip_error(void);

/* Library version string. */
const char* dab_version(void);

/*
 * Measurement aid, not part of the step: streams `bytes` of device memory at
 * `buffer` once with the 16-byte non-temporal loads the step's kernels use,
 * in 64 KB chunks as the row panels read their weights (DAB_READ_PROBE_BLOCKS
 * workgroups of 256 threads; workgroup w takes chunks w, w + blocks, ...;
 * thread t the vectors t, t + 256, ..., t + 15 * 256 of a chunk, sixteen
 * loads in flight, one wave-wide load covering 1 KB), and writes each
 * workgroup's XOR of the 32-bit words it read to out[workgroup] (device,
 * uint32), so that no load can be dropped.  Timed with events around it, it gives the HBM read bandwidth a
 * plain stream attains, the practical ceiling the step's kernels are set
 * against.  buffer: 16-byte aligned, bytes a multiple of 16; out: at least
 * DAB_READ_PROBE_BLOCKS * 4 bytes.  Asynchronous on `stream`; returns
 * DAB_ERR_INVALID_ARG on a null or misaligned pointer or a bad size.
 */
#define DAB_READ_PROBE_BLOCKS 2048
dab_status dab_read_probe(const void* buffer, size_t bytes, void* out, size_t out_bytes, void* stream);

/*
 * The feed-forward half of the decoder layer, the step after the attention
 * block: the operator-fusion article ("LayerNorm + Attention" CUDA kernel
 * page, section 1) lists a second RMS norm and the FFN after the O
 * projection and residual of each LLaMA-style block.  The pages do not
 * spell the FFN out; this is the LLaMA one (gated, SiLU):
 *
 *   r    = (mean_i h_i^2 + eps)^(-1/2),  hh = h * r * norm_w      RMSNorm
 *   g    = hh @ W_gate^T,  u = hh @ W_up^T                        [F] each
 *   m    = silu(g) * u,    silu(z) = z / (1 + exp(-z))
 *   out  = h + m @ W_down^T                                       down + residual
 *
 * Same conventions as the attention block (device pointers, 16-byte
 * alignment, [out_features, in_features] weights, bf16 or fp32 storage with
 * fp32 arithmetic, asynchronous on `stream`, kernel launches only).
 */
typedef struct {
    int32_t batch;         /* B >= 0 sequences (0: nothing to do)            */
    int32_t hidden;        /* H, multiple of 64, at most 16384               */
    int32_t intermediate;  /* F, multiple of 64, at most 16384               */
    int32_t dtype;         /* dab_dtype                                      */
    float eps;             /* RMSNorm epsilon, >= 0                          */
} dab_ffn_config;

/*
 * Bytes of device workspace one FFN call needs (0 when the configuration is
 * invalid): m [B, F] in fp32 and its bf16 copy, and the ready flags of
 * dab_decode_layer.  dab_decode_ffn_block writes what it reads, so for it the
 * workspace needs no initialisation; dab_decode_layer needs it zeroed once
 * (dab_workspace_init) before its first call, and leaves it ready for the
 * next.  Calls that share one workspace must not overlap.
 */
size_t dab_ffn_workspace_size(const dab_ffn_config* cfg);

/*
 * One FFN step for every sequence of the batch, two kernels: RMSNorm + gate
 * and up GEMVs + silu(g) * u, then the down GEMV + residual.
 *
 *   hidden   [B, H]     input h (read only)
 *   norm_w   [H]        RMSNorm weight (read only)
 *   w_gate   [F, H]     row-major, one output feature per row
 *   w_up     [F, H]     row-major, one output feature per row
 *   w_down   [H, F]     row-major, one output feature per row
 *   out      [B, H]     h + m @ W_down^T rounded to the storage dtype; must
 *                       not overlap any other argument
 *   dbg_y    [B, H] fp32 or NULL  the pre-residual m @ W_down^T (a test tap)
 *   workspace, workspace_bytes    at least dab_ffn_workspace_size bytes
 *
 * Returns DAB_ERR_INVALID_ARG / DAB_ERR_UNSUPPORTED / DAB_ERR_WORKSPACE
 * before anything is enqueued, DAB_ERR_HIP if a launch fails.
 */
dab_status dab_decode_ffn_block(const dab_ffn_config* cfg,
                                const void* hidden, const void* norm_w,
                                const void* w_gate, const void* w_up, const void* w_down,
                                void* out, float* dbg_y,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Same, recording events[0] / events[1] at the start / end of the first
 * kernel and events[2] / events[3] at those of the second (as in
 * dab_decode_attn_block_timed); n_events must be 4.
 */
dab_status dab_decode_ffn_block_timed(const dab_ffn_config* cfg,
                                      const void* hidden, const void* norm_w,
                                      const void* w_gate, const void* w_up, const void* w_down,
                                      void* out, float* dbg_y,
                                      void* workspace, size_t workspace_bytes, void* stream,
                                      void* const* events, int n_events);

/*
 * One decoder layer: the attention block, then the FFN on its output.  The
 * operator-fusion page, section 1, chains the two halves in this order
 * through the residual h.
 *
 * layer_schedule (dab_layer_schedule):
 *   DAB_LAYER_SEQUENTIAL  the attention block's kernels, then the FFN's, on
 *                         `stream` (what the two calls below enqueue).
 *   DAB_LAYER_OVERLAP     the FFN's weight stream started under the
 *                         attention block's tail, as the ClusterFusion page,
 *                         section 3.3, overlaps a stage's loads with the work
 *                         in front of it: after the QKV kernel one launch
 *                         holds the attention chunks, the output projection
 *                         and the FFN's gate/up panels, which load their rows
 *                         of W_gate and W_up as soon as they have a compute
 *                         unit and wait on device counters for h; the down
 *                         kernel follows (three kernels against four).
 *                         Built for the configurations dab_layer_overlapped
 *                         reports; DAB_ERR_UNSUPPORTED elsewhere.  On MI355X
 *                         it measured 0.8 to 1.5 us per layer slower than
 *                         SEQUENTIAL for the 7B layer at batch 1 (91.3
 *                         against 90.5 us at 4K tokens, 83.1 against 81.8 at
 *                         1K, 32 layers in a graph): the hand-off of h inside
 *                         the launch costs more than the kernel boundary it
 *                         removes.
 *   DAB_LAYER_AUTO        SEQUENTIAL (the faster on every configuration
 *                         measured).
 * Every schedule gives the same bits: those of h = dab_decode_attn_block(
 * hidden, ...) in `h` and out = dab_decode_ffn_block(h, ...) in `out`.
 *
 *   cfg, hidden .. pos        as dab_decode_attn_block (attn_norm_w its norm_w)
 *   ffn_cfg                   as dab_decode_ffn_block; batch, hidden and
 *                             dtype equal to cfg's
 *   ffn_norm_w .. w_down      as dab_decode_ffn_block
 *   h        [B, H]           the attention block's output (the FFN's input
 *                             and residual); must not overlap any other
 *                             argument
 *   out      [B, H]           the layer's output; must not overlap any other
 *                             argument
 *   workspace, ffn_workspace  as for the two calls; for DAB_LAYER_OVERLAP the
 *                             FFN workspace zeroed once before the first call
 *                             (see dab_ffn_workspace_size)
 *
 * Returns what the two calls return for their arguments (nothing enqueued on
 * an argument error); DAB_ERR_INVALID_ARG if the two configurations disagree
 * or layer_schedule is not a dab_layer_schedule.  Calls that share either
 * workspace must not overlap.
 */
typedef enum {
    DAB_LAYER_AUTO = 0,
    DAB_LAYER_SEQUENTIAL = 1,
    DAB_LAYER_OVERLAP = 2
} dab_layer_schedule;

dab_status dab_decode_layer(const dab_config* cfg, const dab_ffn_config* ffn_cfg,
                            const void* hidden, const void* attn_norm_w, const void* w_qkv, const void* w_o,
                            void* k_cache, void* v_cache, const int32_t* pos,
                            const void* ffn_norm_w, const void* w_gate, const void* w_up, const void* w_down,
                            void* h, void* out,
                            void* workspace, size_t workspace_bytes,
                            void* ffn_workspace, size_t ffn_workspace_bytes,
                            int32_t layer_schedule, void* stream);

/*
 * 1 if DAB_LAYER_OVERLAP is built for these configurations (one query head
 * per kv head on the one-launch attention + projection schedule, head dim 64
 * or 128, the FFN on its VALU panels (fp32, or bf16 below batch 8), H a whole
 * number of 4096 bf16 or 2048 fp32 values, the two projections' batch
 * grouping alike), 0 if not, -1 if a configuration is invalid or the two
 * disagree.
 */
int dab_layer_overlapped(const dab_config* cfg, const dab_ffn_config* ffn_cfg);

/*
 * Latent attention decode (DeepSeek's multi-head latent attention, MLA),
 * the second attention workload the ClusterFusion page runs through its
 * fused decode step (section 5.2: the latent key/value cache is split across
 * clusters and the partial results are merged with a sparse reduction; the
 * page measures it at 4K and 16K tokens).  The page gives no formulas; the
 * reading taken is the absorbed decode form of latent attention.  Every
 * cached token t of a sequence holds one latent row c_t (R = kv_lora_rank
 * values) and one rotary key kr_t (P = rope_dim values), both shared by all
 * heads; head h's query arrives already folded through the key
 * up-projection (q_lat_h, R values) with its rotary part q_rope_h (P values):
 *
 *   s_{h,t} = (q_lat_h . c_t + q_rope_h . kr_t) * softmax_scale
 *   o_h     = sum_t softmax_t(s_{h,.}) c_t        over t = 0 .. pos_b
 *
 * where token pos_b is the new token, whose rows are appended to the caches
 * at row pos_b and attended with the history.  o_h is a latent vector: the
 * value up-projection and the output projection follow outside this call.
 *
 * On MI355X the latent cache of one sequence is split into chunks of tokens,
 * each one workgroup that reads every cached row once for all of its heads
 * (scores and weighted sums on the matrix cores, bf16 operands, fp32
 * accumulation); the chunks' partial softmax states are merged by
 * log-sum-exp weights in a second kernel.
 */
typedef struct {
    int32_t batch;           /* B >= 0 sequences (0: nothing to do)                     */
    int32_t n_heads;         /* nh, a multiple of 16, at most 1024                      */
    int32_t kv_lora_rank;    /* R: 512                                                  */
    int32_t rope_dim;        /* P: 64                                                   */
    int32_t cache_capacity;  /* cap >= 1: token rows per sequence in each cache         */
    float softmax_scale;     /* > 0 (DeepSeek-V3: 1/sqrt(128 + 64))                     */
    int32_t kv_chunk;        /* tokens per chunk: 0 = automatic (sized per sequence from */
                             /* its position and the current device's compute units),  */
                             /* else a multiple of 32 in [32, 65536]                    */
} dab_mla_config;

/*
 * Bytes of device workspace one latent-attention call needs (0 when the
 * configuration is invalid): the device error flag, then the chunks'
 * partial softmax states (max, sum) and unnormalised latent outputs, fp32.
 * Every call writes each partial before it reads it, so the workspace needs
 * no initialisation beyond a zeroed flag word (dab_workspace_init once);
 * calls that share one workspace must not overlap.  With kv_chunk = 0 the
 * size depends on the current device's compute-unit count: size and call on
 * the same device.
 */
size_t dab_mla_workspace_size(const dab_mla_config* cfg);

/*
 * One latent-attention decode step for every sequence of the batch, two
 * kernels on `stream` (chunks, then the merge).
 *
 *   q_lat    fp32 [B, nh, R]     query folded through the key up-projection
 *   q_rope   fp32 [B, nh, P]     rotary part of the query (already rotated)
 *   c_new    bf16 [B, R]         the new token's latent row
 *   kr_new   bf16 [B, P]         the new token's rotary key (already rotated)
 *   c_cache  bf16 [B, cap, R]    token-major.  Rows t < pos[b] are read; row
 *   kr_cache bf16 [B, cap, P]    pos[b] is written with c_new[b] (resp.
 *                                kr_new[b]), bits unchanged; nothing else
 *                                is written
 *   pos      int32 [B]           tokens already cached = index of the new
 *                                token, 0 <= pos[b] < cap
 *   out      fp32 [B, nh, R]     o; must not overlap any other argument
 *   workspace, workspace_bytes   at least dab_mla_workspace_size bytes
 *
 * Numerics: q * softmax_scale * log2(e) and the softmax weights are rounded
 * to bf16 (nearest-even, relative 2^-9 each) as matrix-core operands; the
 * scores, the running max and sum and every weighted sum are fp32.  Every
 * sum has a fixed order: the call is deterministic.  Errors a host can see
 * return a status before anything is enqueued; an out-of-range pos[b]
 * leaves that sequence's rows untouched and sets bit 0 of the device flag
 * (dab_read_device_error).
 */
dab_status dab_mla_decode_attn(const dab_mla_config* cfg,
                               const float* q_lat, const float* q_rope,
                               const void* c_new, const void* kr_new,
                               void* c_cache, void* kr_cache, const int32_t* pos, float* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Same, recording events[0] / events[1] at the start / end of the chunk
 * kernel and events[2] / events[3] at those of the merge kernel (as in
 * dab_decode_attn_block_timed); n_events must be 4.
 */
dab_status dab_mla_decode_attn_timed(const dab_mla_config* cfg,
                                     const float* q_lat, const float* q_rope,
                                     const void* c_new, const void* kr_new,
                                     void* c_cache, void* kr_cache, const int32_t* pos, float* out,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* events, int n_events);

#ifdef __cplusplus
}
#endif

#endif /* DAB_H */

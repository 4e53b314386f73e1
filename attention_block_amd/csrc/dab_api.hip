// C ABI of the decode attention block (declared in include/dab.h).
// Validates on the host, then enqueues the three phase kernels on the
// caller's stream.  No allocation, no synchronisation
// (except in dab_read_device_error).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "dab.h"
#include "dab_kernels.h"
#include "dab_plan.h"

using dab::Plan;

namespace {

#ifdef DAB_TRACE
unsigned long long* g_trace = nullptr;
#endif

const char* const kPhasedNames[3] = {"qkv_rmsnorm_rope_append", "attention_split_kv", "oproj_residual"};
const char* const kPhasedSplitNames[4] = {"qkv_rmsnorm_rope_append", "attention_split_kv", "attention_merge",
                                          "oproj_residual"};
const char* const kAttnOprojNames[2] = {"qkv_rmsnorm_rope_append", "attention_oproj_residual"};
const char* const kQkvAttnNames[2] = {"qkv_attention_split_kv", "oproj_residual"};
const char* const kFusedNames[1] = {"decode_block_fused"};

thread_local char g_last_error[256] = "no error";

dab_status hip_status(hipError_t e) {
    if (e == hipSuccess) return DAB_OK;
    snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
    return DAB_ERR_HIP;
}

// The current device's compute units and how many workgroups of the phased
// attention kernel for cfg's shape one of them holds at once, cached per
// device, storage type, head dim and group; zeros without a device.  Every
// planning call goes through it, so the workspace size and the launch agree.
constexpr int kSlotDevices = 16;
std::atomic<int> g_cus[kSlotDevices];                               // 0: not yet asked; -1: unknown
std::atomic<int> g_per_cu[kSlotDevices][2][2][dab::kMaxGroup + 1];   // 0: not yet asked; -1: unknown

void attn_residency(const dab_config* cfg, int* cus_out, int* per_cu_out) {
    *cus_out = 0;
    *per_cu_out = 0;
    if (!cfg || cfg->n_kv_heads <= 0 || cfg->n_q_heads % cfg->n_kv_heads != 0) return;
    const int G = cfg->n_q_heads / cfg->n_kv_heads;
    const int di = cfg->head_dim == 128 ? 1 : cfg->head_dim == 64 ? 0 : -1;
    const int ti = cfg->dtype == DAB_BF16 ? 1 : cfg->dtype == DAB_F32 ? 0 : -1;
    if (G < 1 || G > dab::kMaxGroup || di < 0 || ti < 0) return;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kSlotDevices) {
        (void)hipGetLastError();
        return;
    }
    int cus = g_cus[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
            (void)hipGetLastError();
            cus = -1;
        }
        g_cus[dev].store(cus, std::memory_order_relaxed);
    }
    std::atomic<int>& slot = g_per_cu[dev][ti][di][G];
    int per_cu = slot.load(std::memory_order_relaxed);
    if (per_cu == 0) {
        per_cu = ti ? dab::attn_resident_bf16(cfg->head_dim, G) : dab::attn_resident_f32(cfg->head_dim, G);
        if (per_cu <= 0) per_cu = -1;
        slot.store(per_cu, std::memory_order_relaxed);
    }
    if (cus > 0 && per_cu > 0) {
        *cus_out = cus;
        *per_cu_out = per_cu;
    }
}

dab_status plan(const dab_config* cfg, Plan* p) {
    int cus, per_cu;
    attn_residency(cfg, &cus, &per_cu);
    return dab::make_plan(cfg, p, cus, per_cu);
}

int phase_count(const Plan& p) {
    return p.schedule == DAB_SCHEDULE_PHASED ? (p.split_merge ? 4 : 3) : p.schedule == DAB_SCHEDULE_FUSED ? 1 : 2;
}

dab::PanelPlanDev panel_dev(const dab::PanelPlan& g) {
    dab::PanelPlanDev d;
    d.panels = g.panels;
    d.nb = g.nb;
    d.nbg = g.nbg;
    d.items = g.grid;
    return d;
}

dab::StepArgs step_args(const Plan& p, const void* hidden, const void* norm_w, const void* w_qkv, const void* w_o,
                        void* k_cache, void* v_cache, const int32_t* pos, void* out, float* dbg_y, void* workspace) {
    char* ws = static_cast<char*>(workspace);
    auto f = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    auto n = [&](size_t off) { return reinterpret_cast<int*>(ws + off); };
    dab::StepArgs a{};
    a.hidden = hidden;
    a.norm_w = norm_w;
    a.w_qkv = w_qkv;
    a.w_o = w_o;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.pos = pos;
    a.out = out;
    a.dbg_y = dbg_y;
    a.flags = n(p.off_flags);
    a.attn_cnt = n(p.off_attn_cnt);
    a.seq_ready = n(p.off_seq_ready);
    a.ready_done = n(p.off_ready_done);
    a.head_cnt = n(p.off_head_cnt);
    a.head_cnt_per_seq = p.schedule == DAB_SCHEDULE_FUSED ? 1 : 0;
    a.ready_copies = p.oproj.panels < dab::kReadyCopies ? p.oproj.panels : dab::kReadyCopies;
    a.q = f(p.off_q);
    a.kv_new = f(p.off_kv_new);
    a.attn_o = f(p.off_attn_o);
    a.attn_ml = f(p.off_attn_ml);
    a.a = f(p.off_a);
    a.a16 = reinterpret_cast<uint16_t*>(ws + p.off_a16);
    a.seq_chunk = p.schedule == DAB_SCHEDULE_PHASED || p.schedule == DAB_SCHEDULE_ATTN_OPROJ
                      ? n(p.off_seq_chunk) : nullptr;
    a.B = p.B;
    a.H = p.H;
    a.nq = p.nq;
    a.nkv = p.nkv;
    a.D = p.D;
    a.G = p.G;
    a.cap = p.cap;
    a.pos_end = p.pos_end;
    a.n_qkv = p.n_qkv;
    a.n_q = p.n_q;
    a.eps = p.eps;
    a.qscale = (float)(1.4426950408889634 / sqrt((double)p.D));
    a.log2_theta = log2((double)p.theta);
    a.qkv = panel_dev(p.qkv);
    a.oproj = panel_dev(p.oproj);
    a.chunk = p.chunk;
    a.maxc = p.max_chunks;
    a.attn_items = p.attn_grid;
    a.split_merge = p.split_merge ? 1 : 0;
#ifdef DAB_TRACE
    a.trace = g_trace;
    a.trace_base = 0;
#endif
    return a;
}

dab_status enqueue(const Plan& p, const dab::StepArgs& a, hipStream_t s, void* const* events) {
    for (int phase = 0; phase < phase_count(p); ++phase) {
        dab::LaunchEvents ev;
        if (events) {
            ev.start = static_cast<hipEvent_t>(events[2 * phase]);
            ev.stop = static_cast<hipEvent_t>(events[2 * phase + 1]);
        }
        const dab_status st = hip_status(dab::launch_phase(a, p, phase, s, ev));
        if (st != DAB_OK) return st;
    }
    return DAB_OK;
}

dab_status call(const dab_config* cfg, const void* hidden, const void* norm_w, const void* w_qkv, const void* w_o,
                void* k_cache, void* v_cache, const int32_t* pos, void* out, float* dbg_y, void* workspace,
                size_t workspace_bytes, void* stream, void* const* events, int n_events) {
    Plan p;
    dab_status st = plan(cfg, &p);
    if (st != DAB_OK) return st;
    st = dab::check_call(p, hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, out, dbg_y, workspace,
                         workspace_bytes);
    if (st != DAB_OK) return st;
    if (events) {
        if (n_events != 2 * phase_count(p)) return DAB_ERR_INVALID_ARG;
        for (int i = 0; i < n_events; ++i)
            if (!events[i]) return DAB_ERR_INVALID_ARG;
    }
    if (p.B == 0) return DAB_OK;
    const dab::StepArgs a = step_args(p, hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, out, dbg_y, workspace);
    return enqueue(p, a, static_cast<hipStream_t>(stream), events);
}

// Scratch of the allocation-free entry point: the workspace of its calls, a
// file-scope device array of which every GPU holds its own copy at its own
// address.  In host code `scratch` only names the symbol; the address of a
// device's copy comes from hipGetSymbolAddress with that device current, once
// per device, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[DAB_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kSlotDevices];

dab_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kSlotDevices) return DAB_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p || ((uintptr_t)p % 256) != 0) return DAB_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DAB_OK;
}

dab_status call_noalloc(const dab_config* cfg, const void* hidden, const void* norm_w, const void* w_qkv,
                        const void* w_o, void* k_cache, void* v_cache, const int32_t* pos, void* out, float* dbg_y,
                        void* stream) {
    Plan p;
    dab_status st = plan(cfg, &p);
    if (st != DAB_OK) return st;
    if (p.ws_bytes > (size_t)DAB_NOALLOC_SCRATCH_BYTES) return DAB_ERR_WORKSPACE;
    // the pointer checks first, against a stand-in address (no device call yet)
    st = dab::check_call(p, hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, out, dbg_y,
                         reinterpret_cast<void*>((uintptr_t)256), DAB_NOALLOC_SCRATCH_BYTES);
    if (st != DAB_OK) return st;
    if (p.B == 0) return DAB_OK;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != DAB_OK) return st;
    st = dab::check_call(p, hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, out, dbg_y, ws,
                         DAB_NOALLOC_SCRATCH_BYTES);
    if (st != DAB_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the scratch keeps whatever the last call on this GPU left, of whatever
    // configuration: the words that must start at zero (error flags, arrival
    // and ready counts, panel counts: everything in front of q) are cleared
    // by a fill kernel, which a graph capture records like any other kernel
    st = hip_status(dab::launch_fill_zero(ws, p.off_q, s));
    if (st != DAB_OK) return st;
    const dab::StepArgs a = step_args(p, hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, out, dbg_y, ws);
    return enqueue(p, a, s, nullptr);
}

dab::FfnArgs ffn_args(const dab::FfnPlan& p, const void* hidden, const void* norm_w, const void* w_gate,
                      const void* w_up, const void* w_down, void* out, float* dbg_y, void* workspace);
dab_status ffn_enqueue(const dab::FfnPlan& p, dab::FfnArgs a, int first, hipStream_t s, void* const* events);

dab_status ffn_call(const dab_ffn_config* cfg, const void* hidden, const void* norm_w, const void* w_gate,
                    const void* w_up, const void* w_down, void* out, float* dbg_y, void* workspace,
                    size_t workspace_bytes, void* stream, void* const* events, int n_events) {
    dab::FfnPlan p;
    dab_status st = dab::make_ffn_plan(cfg, &p);
    if (st != DAB_OK) return st;
    st = dab::check_ffn_call(p, hidden, norm_w, w_gate, w_up, w_down, out, dbg_y, workspace, workspace_bytes);
    if (st != DAB_OK) return st;
    if (events) {
        if (n_events != 4) return DAB_ERR_INVALID_ARG;
        for (int i = 0; i < n_events; ++i)
            if (!events[i]) return DAB_ERR_INVALID_ARG;
    }
    if (p.B == 0) return DAB_OK;
    const dab::FfnArgs a = ffn_args(p, hidden, norm_w, w_gate, w_up, w_down, out, dbg_y, workspace);
    return ffn_enqueue(p, a, 0, static_cast<hipStream_t>(stream), events);
}

dab::FfnArgs ffn_args(const dab::FfnPlan& p, const void* hidden, const void* norm_w, const void* w_gate,
                      const void* w_up, const void* w_down, void* out, float* dbg_y, void* workspace) {
    dab::FfnArgs a{};
    a.hidden = hidden;
    a.norm_w = norm_w;
    a.w_gate = w_gate;
    a.w_up = w_up;
    a.w_down = w_down;
    a.out = out;
    a.dbg_y = dbg_y;
    a.m = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.off_m);
    a.m16 = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + p.off_m16);
    a.mfma = p.mfma ? 1 : 0;
    a.down_tiles = p.down.rows == 32 ? 2 : 1;
    a.gu_tiles = p.gu_tiles;
    a.B = p.B;
    a.H = p.H;
    a.F = p.F;
    a.eps = p.eps;
    a.gu = panel_dev(p.gu);
    a.down = panel_dev(p.down);
    return a;
}

// The FFN's kernels from `first` (0: gate/up, 1: down) on.
dab_status ffn_enqueue(const dab::FfnPlan& p, dab::FfnArgs a, int first, hipStream_t s, void* const* events) {
    for (int phase = first; phase < 2; ++phase) {
        dab::LaunchEvents ev;
        if (events) {
            ev.start = static_cast<hipEvent_t>(events[2 * phase]);
            ev.stop = static_cast<hipEvent_t>(events[2 * phase + 1]);
        }
#ifdef DAB_TRACE
        a.trace = g_trace;
        a.trace_base = phase == 0 ? 0 : p.gu.grid;
#endif
        const dab_status st = hip_status(dab::launch_ffn_phase(a, p.dtype, phase, s, ev));
        if (st != DAB_OK) return st;
    }
    return DAB_OK;
}

// Both plans of a layer call, checked against each other.
dab_status layer_plans(const dab_config* cfg, const dab_ffn_config* ffn_cfg, Plan* p, dab::FfnPlan* fp) {
    if (!cfg || !ffn_cfg) return DAB_ERR_INVALID_ARG;
    dab_status st = plan(cfg, p);
    if (st != DAB_OK) return st;
    st = dab::make_ffn_plan(ffn_cfg, fp);
    if (st != DAB_OK) return st;
    if (fp->B != p->B || fp->H != p->H || fp->dtype != p->dtype) return DAB_ERR_INVALID_ARG;
    return DAB_OK;
}

dab_status layer_call(const dab_config* cfg, const dab_ffn_config* ffn_cfg, const void* hidden,
                      const void* attn_norm_w, const void* w_qkv, const void* w_o, void* k_cache, void* v_cache,
                      const int32_t* pos, const void* ffn_norm_w, const void* w_gate, const void* w_up,
                      const void* w_down, void* h, void* out, void* workspace, size_t workspace_bytes,
                      void* ffn_workspace, size_t ffn_workspace_bytes, int32_t layer_schedule, void* stream) {
    if (layer_schedule != DAB_LAYER_AUTO && layer_schedule != DAB_LAYER_SEQUENTIAL &&
        layer_schedule != DAB_LAYER_OVERLAP)
        return DAB_ERR_INVALID_ARG;
    Plan p;
    dab::FfnPlan fp;
    dab_status st = layer_plans(cfg, ffn_cfg, &p, &fp);
    if (st != DAB_OK) return st;
    if (layer_schedule == DAB_LAYER_OVERLAP && !dab::layer_overlap_ok(p, fp)) return DAB_ERR_UNSUPPORTED;
    st = dab::check_layer_call(p, fp, hidden, attn_norm_w, w_qkv, w_o, k_cache, v_cache, pos, ffn_norm_w, w_gate,
                               w_up, w_down, h, out, workspace, workspace_bytes, ffn_workspace, ffn_workspace_bytes);
    if (st != DAB_OK) return st;
    if (p.B == 0) return DAB_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    dab::StepArgs a = step_args(p, hidden, attn_norm_w, w_qkv, w_o, k_cache, v_cache, pos, h, nullptr, workspace);
    dab::FfnArgs f = ffn_args(fp, h, ffn_norm_w, w_gate, w_up, w_down, out, nullptr, ffn_workspace);
    // AUTO: the sequential schedule, measured faster than the overlapped one
    // on MI355X wherever both are built (7B layer, batch 1: 92.2 against 93.1
    // us at 4K tokens, 83.6 against 85.1 at 1K)
    if (layer_schedule != DAB_LAYER_OVERLAP) {
        st = enqueue(p, a, s, nullptr);
        return st != DAB_OK ? st : ffn_enqueue(fp, f, 0, s, nullptr);
    }
    int* hand = reinterpret_cast<int*>(static_cast<char*>(ffn_workspace) + fp.off_hand);
    a.hand = hand;
    f.hand = hand;
    f.flags = a.flags;
    f.h_panels = p.oproj.panels;
    st = hip_status(dab::launch_phase(a, p, 0, s, dab::LaunchEvents{}));      // QKV
    if (st != DAB_OK) return st;
#ifdef DAB_TRACE
    a.trace_base = p.qkv.grid;
    f.trace = a.trace;
    f.trace_base = a.trace_base;
#endif
    st = hip_status(dab::launch_layer_attn_ffn(a, f, p, fp, s, dab::LaunchEvents{}));
    if (st != DAB_OK) return st;
#ifdef DAB_TRACE
    f.trace_base = a.trace_base + p.attn_grid + p.oproj.grid + fp.gu.grid;
#endif
    return hip_status(dab::launch_ffn_phase(f, fp.dtype, 1, s, dab::LaunchEvents{}));   // down (re-arms the flags)
}

}  // namespace

namespace dab {

// The status of a HIP result, recorded for dab_last_hip_error (other sources of the library report
// their launch failures through it).
dab_status record_hip_status(hipError_t e) { return hip_status(e); }

namespace {

__global__ void fill_zero_kernel(uint32_t* p, size_t n_words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// dst[o, i] = src[i, o]: a row-major [in, out] matrix rewritten as [out, in],
// through 64 x 64 tiles of LDS so that both the reads and the writes are
// whole rows of a tile.  Grid: (ceil(out / 64), ceil(in / 64)).
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E* src, E* dst, int64_t in_f, int64_t out_f) {
    __shared__ E tile[64][65];
    const int64_t o0 = (int64_t)blockIdx.x * 64, i0 = (int64_t)blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) {
        const int64_t i = i0 + r, o = o0 + tx;
        if (i < in_f && o < out_f) tile[r][tx] = src[i * out_f + o];
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int64_t o = o0 + r, i = i0 + tx;
        if (o < out_f && i < in_f) dst[o * in_f + i] = tile[tx][r];
    }
}

// n consecutive fp32 values from src to dst (device to device).
__global__ __launch_bounds__(256) void copy_f32_kernel(const float* src, float* dst, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));

// A plain stream over n16 16-byte vectors in chunks of 64 KB, as the
// row panels read their weights: workgroup w takes chunks w, w + G, ...
// (G workgroups); thread t reads vectors t, t + 256, ..., t + 15 * 256 of a
// chunk, all sixteen requested before any is used, so one wave-wide load
// covers 1 KB.  Each workgroup's XOR of its words goes to out.
__global__ __launch_bounds__(256) void read_probe_kernel(const probe_u32x4* p, size_t n16, uint32_t* out) {
    constexpr int V = 16;
    constexpr size_t kChunk = 256 * V;            // vectors per chunk
    __shared__ uint32_t red[4];
    uint32_t acc = 0u;
    for (size_t c = blockIdx.x; c * kChunk < n16; c += gridDim.x) {
        const size_t base = c * kChunk + threadIdx.x;
        probe_u32x4 v[V];
        if ((c + 1) * kChunk <= n16) {
#pragma unroll
            for (int k = 0; k < V; ++k) v[k] = __builtin_nontemporal_load(p + base + (size_t)k * 256);
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k)
                v[k] = base + (size_t)k * 256 < n16 ? __builtin_nontemporal_load(p + base + (size_t)k * 256)
                                                    : probe_u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < V; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
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

hipError_t launch_phase(const StepArgs& a, const Plan& p, int phase, hipStream_t s, const LaunchEvents& ev) {
#ifdef DAB_TRACE
    // phases trace at consecutive item numbers: QKV, attention, output
    // projection, then the merge kernel's workgroups (phased, split merge)
    StepArgs t = a;
    const bool merge = p.split_merge && phase == 2;
    const bool oproj_only = (phase == 2 && !p.split_merge) || phase == 3 ||
                            (phase == 1 && p.schedule == DAB_SCHEDULE_QKV_ATTN);
    t.trace_base = phase == 0 ? 0 : merge ? p.qkv.grid + p.attn_grid + p.oproj.grid
                 : oproj_only ? p.qkv.grid + p.attn_grid : p.qkv.grid;
    return p.dtype == DAB_BF16 ? launch_phase_bf16(t, p, phase, s, ev) : launch_phase_f32(t, p, phase, s, ev);
#else
    return p.dtype == DAB_BF16 ? launch_phase_bf16(a, p, phase, s, ev) : launch_phase_f32(a, p, phase, s, ev);
#endif
}

}  // namespace dab

extern "C" {

#ifdef DAB_TRACE
// Profiling builds only: device buffer of [grid, 4] timestamps for later calls (null: off).
void dab_trace_set_buffer(void* p) { g_trace = static_cast<unsigned long long*>(p); }
// Profiling builds only: workgroups of the QKV, attention, output projection and merge kernels.
dab_status dab_trace_layout(const dab_config* cfg, int32_t* grids) {
    Plan p;
    const dab_status st = plan(cfg, &p);
    if (st != DAB_OK) return st;
    grids[0] = p.qkv.grid;
    grids[1] = p.attn_grid;
    grids[2] = p.oproj.grid;
    grids[3] = p.split_merge ? p.B * p.nq : 0;
    return DAB_OK;
}
#endif

size_t dab_workspace_size(const dab_config* cfg) {
    Plan p;
    if (plan(cfg, &p) != DAB_OK) return 0;
    return p.ws_bytes;
}

dab_status dab_read_probe(const void* buffer, size_t bytes, void* out, size_t out_bytes, void* stream) {
    if (!buffer || !out || ((uintptr_t)buffer % 16) != 0 || ((uintptr_t)out % 4) != 0 || bytes % 16 != 0 ||
        out_bytes < (size_t)DAB_READ_PROBE_BLOCKS * 4)
        return DAB_ERR_INVALID_ARG;
    hipLaunchKernelGGL(dab::read_probe_kernel, dim3(DAB_READ_PROBE_BLOCKS), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const dab::probe_u32x4*>(buffer), bytes / 16,
                       static_cast<uint32_t*>(out));
    return hip_status(hipGetLastError());
}

dab_status dab_pack_weight(const void* src, void* dst, int64_t in_features, int64_t out_features, int32_t dtype,
                           void* stream) {
    if (!src || !dst || ((uintptr_t)src % 16) != 0 || ((uintptr_t)dst % 16) != 0) return DAB_ERR_INVALID_ARG;
    if (dtype != DAB_F32 && dtype != DAB_BF16) return DAB_ERR_INVALID_ARG;
    if (in_features <= 0 || out_features <= 0 || in_features > 65535LL * 64 || out_features > (1LL << 30))
        return DAB_ERR_INVALID_ARG;
    const size_t bytes = (size_t)in_features * (size_t)out_features * (dtype == DAB_BF16 ? 2 : 4);
    const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
    if (s < d + bytes && d < s + bytes) return DAB_ERR_INVALID_ARG;
    const dim3 grid((unsigned)((out_features + 63) / 64), (unsigned)((in_features + 63) / 64));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == DAB_BF16)
        hipLaunchKernelGGL(dab::transpose_kernel<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(src),
                           static_cast<uint16_t*>(dst), in_features, out_features);
    else
        hipLaunchKernelGGL(dab::transpose_kernel<uint32_t>, grid, dim3(256), 0, st, static_cast<const uint32_t*>(src),
                           static_cast<uint32_t*>(dst), in_features, out_features);
    return hip_status(hipGetLastError());
}

dab_status dab_attention_output(const dab_config* cfg, const void* workspace, size_t workspace_bytes, float* dst,
                                void* stream) {
    Plan p;
    dab_status st = plan(cfg, &p);
    if (st != DAB_OK) return st;
    if (!workspace || ((uintptr_t)workspace % 256) != 0 || !dst || ((uintptr_t)dst % 16) != 0)
        return DAB_ERR_INVALID_ARG;
    if (workspace_bytes < p.ws_bytes) return DAB_ERR_WORKSPACE;
    const size_t n = (size_t)p.B * p.n_q;
    if (n == 0) return DAB_OK;
    const float* a = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + p.off_a);
    if ((uintptr_t)dst < (uintptr_t)(static_cast<const char*>(workspace) + p.ws_bytes) &&
        (uintptr_t)workspace < (uintptr_t)(dst + n))
        return DAB_ERR_INVALID_ARG;
    size_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(dab::copy_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), a,
                       dst, n);
    return hip_status(hipGetLastError());
}

dab_status dab_workspace_init(void* workspace, size_t bytes, void* stream) {
    if (!workspace || ((uintptr_t)workspace % 256) != 0) return DAB_ERR_INVALID_ARG;
    return hip_status(dab::launch_fill_zero(workspace, bytes, static_cast<hipStream_t>(stream)));
}

dab_status dab_decode_attn_block(const dab_config* cfg, const void* hidden, const void* norm_w, const void* w_qkv,
                                 const void* w_o, void* k_cache, void* v_cache, const int32_t* pos, void* out,
                                 float* dbg_y, void* workspace, size_t workspace_bytes, void* stream) {
    return call(cfg, hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, out, dbg_y, workspace, workspace_bytes,
                stream, nullptr, 0);
}

dab_status dab_decode_attn_block_timed(const dab_config* cfg, const void* hidden, const void* norm_w,
                                       const void* w_qkv, const void* w_o, void* k_cache, void* v_cache,
                                       const int32_t* pos, void* out, float* dbg_y, void* workspace,
                                       size_t workspace_bytes, void* stream, void* const* events, int n_events) {
    if (!events) return DAB_ERR_INVALID_ARG;
    return call(cfg, hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, out, dbg_y, workspace, workspace_bytes,
                stream, events, n_events);
}

dab_status dab_decode_attn_block_noalloc(const dab_config* cfg, const void* hidden, const void* norm_w,
                                         const void* w_qkv, const void* w_o, void* k_cache, void* v_cache,
                                         const int32_t* pos, void* out, float* dbg_y, void* stream) {
    return call_noalloc(cfg, hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, out, dbg_y, stream);
}

int dab_phase_count(const dab_config* cfg) {
    Plan p;
    return plan(cfg, &p) == DAB_OK ? phase_count(p) : 0;
}

const char* dab_phase_name(const dab_config* cfg, int i) {
    Plan p;
    if (plan(cfg, &p) != DAB_OK || i < 0 || i >= phase_count(p)) return nullptr;
    return p.schedule == DAB_SCHEDULE_ATTN_OPROJ ? kAttnOprojNames[i]
         : p.schedule == DAB_SCHEDULE_QKV_ATTN ? kQkvAttnNames[i]
         : p.schedule == DAB_SCHEDULE_FUSED ? kFusedNames[i]
         : p.split_merge ? kPhasedSplitNames[i] : kPhasedNames[i];
}

dab_status dab_read_device_error(void* workspace, void* stream, int32_t* flag) {
    if (!workspace || !flag || ((uintptr_t)workspace % 256) != 0) return DAB_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t host = 0;
    // the flags word sits at offset 0 of every workspace layout
    dab_status st = hip_status(hipMemcpyAsync(&host, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    if (st == DAB_OK) st = hip_status(hipStreamSynchronize(s));
    if (st != DAB_OK) return st;
    *flag = host;
    return hip_status(dab::launch_fill_zero(workspace, sizeof(int32_t), s));
}

const char* dab_status_string(dab_status status) {
    switch (status) {
        case DAB_OK: return "ok";
        case DAB_ERR_INVALID_ARG: return "invalid argument (null, misaligned or overlapping pointer, bad size)";
        case DAB_ERR_UNSUPPORTED: return "unsupported shape (head_dim not 64/128, hidden or intermediate not a "
                                         "multiple of 64, hidden, intermediate or n_q_heads * head_dim above "
                                         "16384, group > 8, or too many KV chunks)";
        case DAB_ERR_WORKSPACE: return "workspace missing or too small";
        case DAB_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* dab_last_hip_error(void) { return g_last_error; }

size_t dab_ffn_workspace_size(const dab_ffn_config* cfg) {
    dab::FfnPlan p;
    if (dab::make_ffn_plan(cfg, &p) != DAB_OK) return 0;
    return p.ws_bytes;
}

dab_status dab_decode_ffn_block(const dab_ffn_config* cfg, const void* hidden, const void* norm_w, const void* w_gate,
                                const void* w_up, const void* w_down, void* out, float* dbg_y, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return ffn_call(cfg, hidden, norm_w, w_gate, w_up, w_down, out, dbg_y, workspace, workspace_bytes, stream,
                    nullptr, 0);
}

dab_status dab_decode_ffn_block_timed(const dab_ffn_config* cfg, const void* hidden, const void* norm_w,
                                      const void* w_gate, const void* w_up, const void* w_down, void* out,
                                      float* dbg_y, void* workspace, size_t workspace_bytes, void* stream,
                                      void* const* events, int n_events) {
    if (!events) return DAB_ERR_INVALID_ARG;
    return ffn_call(cfg, hidden, norm_w, w_gate, w_up, w_down, out, dbg_y, workspace, workspace_bytes, stream,
                    events, n_events);
}

dab_status dab_decode_layer(const dab_config* cfg, const dab_ffn_config* ffn_cfg, const void* hidden,
                            const void* attn_norm_w, const void* w_qkv, const void* w_o, void* k_cache,
                            void* v_cache, const int32_t* pos, const void* ffn_norm_w, const void* w_gate,
                            const void* w_up, const void* w_down, void* h, void* out, void* workspace,
                            size_t workspace_bytes, void* ffn_workspace, size_t ffn_workspace_bytes,
                            int32_t layer_schedule, void* stream) {
    return layer_call(cfg, ffn_cfg, hidden, attn_norm_w, w_qkv, w_o, k_cache, v_cache, pos, ffn_norm_w, w_gate, w_up,
                      w_down, h, out, workspace, workspace_bytes, ffn_workspace, ffn_workspace_bytes, layer_schedule,
                      stream);
}

int dab_layer_overlapped(const dab_config* cfg, const dab_ffn_config* ffn_cfg) {
    Plan p;
    dab::FfnPlan fp;
    if (layer_plans(cfg, ffn_cfg, &p, &fp) != DAB_OK) return -1;
    return dab::layer_overlap_ok(p, fp) ? 1 : 0;
}

const char* dab_version(void) { return "dab 0.1.0 (gfx950)"; }

}  // extern "C"

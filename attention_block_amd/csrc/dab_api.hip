// C ABI of the decode attention block (declared in include/dab.h).
// Validates on the host, then enqueues the three phase kernels on the
// caller's stream.  No allocation, no synchronisation (except in
// dab_read_device_error).
#include <hip/hip_runtime.h>
#include <math.h>

#include "dab.h"
#include "dab_kernels.h"
#include "dab_plan.h"

using dab::Plan;

namespace {

constexpr int kPhases = 3;
const char* const kPhaseNames[kPhases] = {"qkv_rmsnorm_rope_append", "attention_split_kv", "oproj_residual"};

dab_status hip_status(hipError_t e) { return e == hipSuccess ? DAB_OK : DAB_ERR_HIP; }

dab_status record(void* const* events, int i, hipStream_t s) {
    if (!events) return DAB_OK;
    return hip_status(hipEventRecord(static_cast<hipEvent_t>(events[i]), s));
}

dab_status enqueue(const Plan& p, const void* hidden, const void* norm_w, const void* w_qkv, const void* w_o,
                   void* k_cache, void* v_cache, const int32_t* pos, void* out, float* dbg_y, void* workspace,
                   hipStream_t s, void* const* events) {
    char* ws = static_cast<char*>(workspace);
    const bool bf16 = p.dtype == DAB_BF16;
    int* flags = reinterpret_cast<int*>(ws + p.off_flags);
    float* q = reinterpret_cast<float*>(ws + p.off_q);
    float* a = reinterpret_cast<float*>(ws + p.off_a);
    dab_status st;

    dab::GemvArgs g{};
    g.W = w_qkv;
    g.hidden = hidden;
    g.norm_w = norm_w;
    g.part = reinterpret_cast<float*>(ws + p.off_qkv_part);
    g.ssq = reinterpret_cast<float*>(ws + p.off_ssq);
    g.cnt = reinterpret_cast<int*>(ws + p.off_qkv_cnt);
    g.flags = flags;
    g.pos = pos;
    g.q = q;
    g.k_cache = k_cache;
    g.v_cache = v_cache;
    g.B = p.B;
    g.K = p.H;
    g.N = p.n_qkv;
    g.slabs = p.qkv.slabs;
    g.ksplit = p.qkv.ksplit;
    g.nbg = p.qkv.nbg;
    g.tiles = p.qkv.tiles;
    g.cap = p.cap;
    g.n_q = p.n_q;
    g.nkv = p.nkv;
    g.D = p.D;
    g.eps = p.eps;
    g.log2_theta = log2((double)p.theta);

    if ((st = record(events, 0, s)) != DAB_OK) return st;
    if ((st = hip_status(dab::launch_gemv(g, bf16, true, p.qkv.bg, p.qkv.rows, p.qkv.grid, s))) != DAB_OK) return st;
    if ((st = record(events, 1, s)) != DAB_OK) return st;

    dab::AttnArgs at{};
    at.q = q;
    at.k_cache = k_cache;
    at.v_cache = v_cache;
    at.pos = pos;
    at.part_o = reinterpret_cast<float*>(ws + p.off_attn_o);
    at.part_ml = reinterpret_cast<float*>(ws + p.off_attn_ml);
    at.cnt = reinterpret_cast<int*>(ws + p.off_attn_cnt);
    at.a_out = a;
    at.nq = p.nq;
    at.nkv = p.nkv;
    at.cap = p.cap;
    at.T = p.kv_chunk;
    at.maxc = p.max_chunks;
    at.qscale = (float)(1.4426950408889634 / sqrt((double)p.D));
    if ((st = hip_status(dab::launch_attn(at, bf16, p.D, p.G, p.attn_grid, s))) != DAB_OK) return st;
    if ((st = record(events, 2, s)) != DAB_OK) return st;

    dab::GemvArgs o{};
    o.W = w_o;
    o.hidden = hidden;
    o.xin = a;
    o.part = reinterpret_cast<float*>(ws + p.off_oproj_part);
    o.cnt = reinterpret_cast<int*>(ws + p.off_oproj_cnt);
    o.flags = flags;
    o.pos = pos;
    o.out = out;
    o.dbg_y = dbg_y;
    o.B = p.B;
    o.K = p.n_q;
    o.N = p.H;
    o.slabs = p.oproj.slabs;
    o.ksplit = p.oproj.ksplit;
    o.nbg = p.oproj.nbg;
    o.tiles = p.oproj.tiles;
    o.cap = p.cap;
    o.n_q = p.n_q;
    o.nkv = p.nkv;
    o.D = p.D;
    if ((st = hip_status(dab::launch_gemv(o, bf16, false, p.oproj.bg, p.oproj.rows, p.oproj.grid, s))) != DAB_OK)
        return st;
    return record(events, 3, s);
}

dab_status call(const dab_config* cfg, const void* hidden, const void* norm_w, const void* w_qkv, const void* w_o,
                void* k_cache, void* v_cache, const int32_t* pos, void* out, float* dbg_y, void* workspace,
                size_t workspace_bytes, void* stream, void* const* events, int n_events) {
    Plan p;
    dab_status st = dab::make_plan(cfg, &p);
    if (st != DAB_OK) return st;
    st = dab::check_call(p, hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, out, dbg_y, workspace,
                         workspace_bytes);
    if (st != DAB_OK) return st;
    if (events) {
        if (n_events != kPhases + 1) return DAB_ERR_INVALID_ARG;
        for (int i = 0; i < n_events; ++i)
            if (!events[i]) return DAB_ERR_INVALID_ARG;
    }
    if (p.B == 0) return DAB_OK;
    return enqueue(p, hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, out, dbg_y, workspace,
                   static_cast<hipStream_t>(stream), events);
}

}  // namespace

extern "C" {

size_t dab_workspace_size(const dab_config* cfg) {
    Plan p;
    if (dab::make_plan(cfg, &p) != DAB_OK) return 0;
    return p.ws_bytes;
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

int dab_phase_count(const dab_config* cfg) {
    Plan p;
    return dab::make_plan(cfg, &p) == DAB_OK ? kPhases : 0;
}

const char* dab_phase_name(const dab_config* cfg, int i) {
    if (dab_phase_count(cfg) == 0 || i < 0 || i >= kPhases) return nullptr;
    return kPhaseNames[i];
}

dab_status dab_read_device_error(void* workspace, void* stream, int32_t* flag) {
    if (!workspace || !flag || ((uintptr_t)workspace % 256) != 0) return DAB_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t host = 0;
    // the flags word sits at offset 0 of every workspace layout
    if (hipMemcpyAsync(&host, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return DAB_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return DAB_ERR_HIP;
    *flag = host;
    if (dab::launch_fill_zero(workspace, sizeof(int32_t), s) != hipSuccess) return DAB_ERR_HIP;
    return DAB_OK;
}

const char* dab_status_string(dab_status status) {
    switch (status) {
        case DAB_OK: return "ok";
        case DAB_ERR_INVALID_ARG: return "invalid argument (null, misaligned or overlapping pointer, bad size)";
        case DAB_ERR_UNSUPPORTED: return "unsupported shape (head_dim not 64/128, hidden not a multiple of 64, "
                                         "group > 8, or too many KV chunks)";
        case DAB_ERR_WORKSPACE: return "workspace missing or too small";
        case DAB_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* dab_version(void) { return "dab 0.1.0 (gfx950)"; }

}  // extern "C"

// The fused decode step: one launch for the whole step.
//
// Workgroup i runs work item i.  Items are numbered in dependency order, unit
// by unit: a unit is a group of kv heads (one 256-column slab of keys), and
// its items are the QKV tiles of its query, key and value slabs, then its
// attention chunks, then the output-projection row blocks of its query
// heads.  Later units stream from HBM while earlier ones hand over.
// An item issues its HBM loads (weight tile or K/V rows) before it waits on
// the counters of the items it depends on, so the three streams overlap.
// An item only ever waits on lower-numbered items.  Each XCD dispatches its
// share of the grid in workgroup-id order, so when a workgroup runs, every
// lower-numbered workgroup of its XCD has been dispatched, and the lowest
// unfinished item can always proceed: the schedule cannot deadlock.  Each
// wait is bounded besides (see wait_at_least), so a broken assumption shows
// up as an error flag, never as a hang.  The workgroup that finishes last
// re-arms every counter for the next call; the finish count is spread over
// 16 sub-counters on separate cache lines, since same-address atomics from
// thousands of workgroups serialise.
//
// A launch may start at item a.item_lo (the two-stage schedule runs the QKV
// tiles in a kernel of their own first, then items from the first attention
// chunk on); the launch that ends at the last item re-arms the counters.
//
// This replaces the one-kernel-per-cluster launch of the ClusterFusion page
// (section 3.2) and its CUDA-graph / overlap tuning (section 3.3): without
// thread-block clusters, one grid-wide item order gives the overlap.
#pragma once

#include "dab_device.h"

namespace dab {
namespace dev {

// Attention work index -> (sequence, kv head, chunk) over `nkv` kv heads;
// kv head fastest, so concurrent items read neighbouring rows of one token
// range.
__device__ inline void attn_decode(const StepArgs& a, int nkv, int i, int* b, int* g, int* c) {
    *g = i % nkv;
    const int rest = i / nkv;
    *c = rest % a.maxc;
    *b = rest / a.maxc;
}

// Global QKV slab of slab `sl` of unit `u`: the unit's G query slabs, then
// its key slab, then its value slab (one slab of 256 columns holds 256/D
// heads).  With a single unit the slabs are taken in order.
__device__ inline int unit_qkv_slab(const StepArgs& a, int u, int sl) {
    if (a.units == 1) return sl;
    if (sl < a.G) return u * a.G + sl;
    const int kv_base = (sl == a.G) ? a.n_q : a.n_q + a.nkv * a.D;
    return kv_base / 256 + u;
}

template <typename T, int BG, int D, int G>
__global__ __launch_bounds__(256) void fused_step_kernel(StepArgs a) {
    __shared__ union {
        GemvShared<BG> gemv;
        AttnShared<D, G> attn;
    } sm;
    __shared__ int s_flag;

    const int tk = a.item_lo + blockIdx.x;
    DAB_TRACE_POINT(a, 0);
    // this call's message tag; the epoch only changes at the end of a launch
    const uint32_t tag = ll_tag((uint32_t)load_counter(a.epoch) + 1u);
    // unit u = a group of kv heads: its QKV tiles, its attention chunks, its
    // output-projection row blocks, in that order; units follow one another
    const int u = tk / a.unit_items;
    const int r = tk % a.unit_items;
    const int q_tiles = a.unit_slabs * a.qkv.ksplit;
    const int q_items = gemv_items(a.qkv.nbg, q_tiles);
    const int a_items = a.B * a.unit_kv * a.maxc;
    if (r < q_items) {
        int tile, bgi;
        if (gemv_decode(a.qkv.nbg, q_tiles, r, &tile, &bgi))
            gemv_tile<T, BG, true, true>(a, unit_qkv_slab(a, u, tile % a.unit_slabs), tile / a.unit_slabs, bgi, tag,
                                         sm.gemv, &s_flag);
    } else if (r < q_items + a_items) {
        int b, g, c;
        attn_decode(a, a.unit_kv, r - q_items, &b, &g, &c);
        attn_item<T, D, G, true>(a, b, u * a.unit_kv + g, c, tag, sm.attn, &s_flag);
    } else {
        const int o_tiles = a.unit_oks * a.oproj.slabs;
        int tile, bgi;
        if (gemv_decode(a.oproj.nbg, o_tiles, r - q_items - a_items, &tile, &bgi))
            gemv_tile<T, BG, false, true>(a, tile % a.oproj.slabs, u * a.unit_oks + tile / a.oproj.slabs, bgi, tag,
                                          sm.gemv, &s_flag);
    }

    // the last workgroup to finish re-arms the counters for the next call.
    // Wave 0 first waits for its own counter updates to land, so none of
    // them can arrive after the re-arm.
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_s_waitcnt(0);
        const int n = a.total_items - a.item_lo;              // workgroups of this launch
        const int sub = blockIdx.x % kDoneShards;
        const int n_sub = (n - sub + kDoneShards - 1) / kDoneShards;   // of this shard
        bool last = bump(&a.done[sub * kDoneStride]) == n_sub - 1;
        if (last) last = bump(a.done_all) == min(kDoneShards, n) - 1;   // non-empty shards
        s_flag = last;
    }
    __syncthreads();
    DAB_TRACE_POINT(a, 3);
    if (s_flag) {
        const int nq = a.qkv.slabs * a.qkv.nbg, na = a.B * a.nkv;
        for (int i = threadIdx.x; i < nq; i += 256) set_counter(&a.qkv_cnt[i], 0);
        for (int i = threadIdx.x; i < na; i += 256) set_counter(&a.attn_cnt[i], 0);
        if (threadIdx.x < kDoneShards) set_counter(&a.done[threadIdx.x * kDoneStride], 0);
        if (threadIdx.x == 0) {
            set_counter(a.done_all, 0);
            set_counter(a.epoch, load_counter(a.epoch) + 1);   // next call's tag
        }
    }
}

// First stage of the two-stage schedule: the QKV tiles alone (tagged
// partials, finalisers publish tagged q and new k/v).  A kernel of its own
// so that its register budget, and so its occupancy, is the GEMV's.
template <typename T, int BG>
__global__ __launch_bounds__(256) void stage_qkv_kernel(StepArgs a) {
    __shared__ GemvShared<BG> sm;
    __shared__ int s_flag;
    const uint32_t tag = ll_tag((uint32_t)load_counter(a.epoch) + 1u);
    const int q_tiles = a.unit_slabs * a.qkv.ksplit;
    int tile, bgi;
    DAB_TRACE_POINT(a, 0);
    if (gemv_decode(a.qkv.nbg, q_tiles, blockIdx.x, &tile, &bgi))
        gemv_tile<T, BG, true, true>(a, unit_qkv_slab(a, 0, tile % a.unit_slabs), tile / a.unit_slabs, bgi, tag, sm,
                                     &s_flag);
    DAB_TRACE_POINT(a, 3);
}

template <typename T>
hipError_t launch_stage_qkv_t(const StepArgs& a, hipStream_t s) {
    const dim3 grid(a.qkv.items), block(256);
    switch (a.qkv_bg) {
        case 1: hipLaunchKernelGGL((stage_qkv_kernel<T, 1>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((stage_qkv_kernel<T, 2>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((stage_qkv_kernel<T, 4>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((stage_qkv_kernel<T, 8>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

template <typename T, int BG, int D>
hipError_t launch_fused_g(const StepArgs& a, hipStream_t s) {
    const dim3 grid(a.total_items - a.item_lo), block(256);
    switch (a.G) {
        case 1: hipLaunchKernelGGL((fused_step_kernel<T, BG, D, 1>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((fused_step_kernel<T, BG, D, 2>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((fused_step_kernel<T, BG, D, 4>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((fused_step_kernel<T, BG, D, 8>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int BG>
hipError_t launch_fused_bg(const StepArgs& a, hipStream_t s) {
    return a.D == 128 ? launch_fused_g<T, BG, 128>(a, s) : launch_fused_g<T, BG, 64>(a, s);
}

template <typename T>
hipError_t launch_fused_t(const StepArgs& a, hipStream_t s) {
    switch (a.qkv_bg) {
        case 1: return launch_fused_bg<T, 1>(a, s);
        case 2: return launch_fused_bg<T, 2>(a, s);
        case 4: return launch_fused_bg<T, 4>(a, s);
        default: return launch_fused_bg<T, 8>(a, s);
    }
}

}  // namespace dev
}  // namespace dab

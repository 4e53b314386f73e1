// The fused decode step: one launch for the whole step.
//
// Workgroup i runs work item i.  Items are numbered in dependency order: all
// QKV tiles, then every attention chunk, then every output-projection tile.
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
// This replaces the one-kernel-per-cluster launch of the ClusterFusion page
// (section 3.2) and its CUDA-graph / overlap tuning (section 3.3): without
// thread-block clusters, one grid-wide item order gives the overlap.
#pragma once

#include "dab_device.h"

namespace dab {
namespace dev {

// Attention work index -> (sequence, kv head, chunk); kv head fastest, so
// concurrent items read whole token rows (all heads) of one token range.
__device__ inline void attn_decode(const StepArgs& a, int i, int* b, int* g, int* c) {
    *g = i % a.nkv;
    const int rest = i / a.nkv;
    *c = rest % a.maxc;
    *b = rest / a.maxc;
}

template <typename T, int BG, int D, int G>
__global__ __launch_bounds__(256) void fused_step_kernel(StepArgs a) {
    __shared__ union {
        GemvShared<BG> gemv;
        AttnShared<D, G> attn;
    } sm;
    __shared__ int s_flag;

    const int tk = blockIdx.x;
    DAB_TRACE_POINT(a, 0);
    if (tk < a.qkv.items) {
        int tile, bgi;
        if (gemv_decode(a.qkv, tk, &tile, &bgi)) gemv_tile<T, BG, true>(a, tile, bgi, true, sm.gemv, &s_flag);
    } else if (tk < a.qkv.items + a.attn_items) {
        int b, g, c;
        attn_decode(a, tk - a.qkv.items, &b, &g, &c);
        attn_item<T, D, G>(a, b, g, c, true, sm.attn, &s_flag);
    } else {
        int tile, bgi;
        if (gemv_decode(a.oproj, tk - a.qkv.items - a.attn_items, &tile, &bgi))
            gemv_tile<T, BG, false>(a, tile, bgi, true, sm.gemv, &s_flag);
    }

    // the last workgroup to finish re-arms the counters for the next call
    drain_and_sync();
    if (threadIdx.x == 0) {
        const int sub = tk % kDoneShards;
        const int n_sub = (a.total_items - sub + kDoneShards - 1) / kDoneShards;   // items of this shard
        bool last = bump(&a.done[sub * kDoneStride]) == n_sub - 1;
        if (last) last = bump(a.done_all) == min(kDoneShards, a.total_items) - 1;   // non-empty shards
        s_flag = last;
    }
    __syncthreads();
    DAB_TRACE_POINT(a, 3);
    if (s_flag) {
        const int nq = a.qkv.slabs * a.qkv.nbg, na = a.B * a.nkv;
        for (int i = threadIdx.x; i < nq; i += 256) set_counter(&a.qkv_cnt[i], 0);
        for (int i = threadIdx.x; i < na; i += 256) set_counter(&a.attn_cnt[i], 0);
        if (threadIdx.x < kDoneShards) set_counter(&a.done[threadIdx.x * kDoneStride], 0);
        if (threadIdx.x == 0) set_counter(a.done_all, 0);
    }
}

template <typename T, int BG, int D>
hipError_t launch_fused_g(const StepArgs& a, hipStream_t s) {
    const dim3 grid(a.total_items), block(256);
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

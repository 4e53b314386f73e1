// Host driver of the launch planner (dab_plan.cpp is plain C++): prints the
// split-KV chunk choice of a configuration for a given number of compute
// units and resident attention workgroups per unit.  Built with g++ by tests/test_plan_host.py.
//   plan_host B H nq nkv D cap dtype schedule cus per_cu [pos_probe]
// It also walks every position below the capacity: the largest chunk count,
// the positions whose chunks would not fit the grid or cover the tokens, and
// the chunk length at pos_probe.
//   plan_host ffn B H F dtype
// prints the FFN plan's panels and workspace layout, and the status of the
// layer call's pointer check (the attention block of H / 128 heads of 128,
// this FFN) on disjoint synthetic addresses, then with pairs of arguments
// made to overlap: h and w_gate, out and the attention workspace, the two
// workspaces, and two read-only inputs shared by both halves.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dab_plan.h"

namespace {

int ffn_main(int argc, char** argv) {
    if (argc != 6) {
        fprintf(stderr, "usage: plan_host ffn B H F dtype\n");
        return 2;
    }
    dab_ffn_config f{};
    f.batch = atoi(argv[2]);
    f.hidden = atoi(argv[3]);
    f.intermediate = atoi(argv[4]);
    f.dtype = atoi(argv[5]);
    f.eps = 1e-6f;
    dab::FfnPlan fp;
    const dab_status st = dab::make_ffn_plan(&f, &fp);
    if (st != DAB_OK) {
        printf("%d\n", (int)st);
        return 0;
    }
    // the hand-off region of the overlapped layer lies inside the workspace, after m and its bf16 copy
    const size_t hand_end = fp.off_hand + sizeof(int32_t) * (size_t)dab::h_region(fp.B);
    const int layout_ok = fp.off_m16 >= sizeof(float) * (size_t)fp.B * fp.F &&
                          fp.off_hand >= fp.off_m16 + sizeof(uint16_t) * (size_t)fp.B * fp.F &&
                          hand_end <= fp.ws_bytes && fp.off_hand % 256 == 0;
    // the layer call's check: an attention block of H / 128 heads of 128 over a cache of 64 tokens
    dab_config c{};
    c.batch = f.batch;
    c.hidden = f.hidden;
    c.n_q_heads = c.n_kv_heads = f.hidden / 128;
    c.head_dim = 128;
    c.cache_capacity = 64;
    c.dtype = f.dtype;
    c.rope_theta = 1e4f;
    c.eps = 1e-6f;
    dab::Plan p;
    if (dab::make_plan(&c, &p) != DAB_OK) {
        printf("%d %d bad-attention-plan\n", (int)st, layout_ok);
        return 0;
    }
    enum { HIDDEN, ANORM, WQKV, WO, KC, VC, POS, FNORM, WG, WU, WD, H, OUT, WS, FWS, N };
    uintptr_t ptr[N];
    for (int i = 0; i < N; ++i) ptr[i] = ((uintptr_t)1 << 40) + ((uintptr_t)i << 32);   // 4 GiB apart
    auto check = [&](const uintptr_t* q) {
        auto v = [&](int i) { return reinterpret_cast<const void*>(q[i]); };
        return (int)dab::check_layer_call(p, fp, v(HIDDEN), v(ANORM), v(WQKV), v(WO), v(KC), v(VC),
                                          reinterpret_cast<const int32_t*>(q[POS]), v(FNORM), v(WG), v(WU), v(WD),
                                          v(H), v(OUT), v(WS), p.ws_bytes, v(FWS), fp.ws_bytes);
    };
    auto overlapped = [&](int a, int b) {
        uintptr_t q[N];
        memcpy(q, ptr, sizeof(q));
        q[b] = q[a] + 256;
        return check(q);
    };
    printf("%d %d %d %d %d %d %d %d %zu %d %d %d %d %d\n", (int)st, fp.mfma ? 1 : 0, fp.gu_tiles, fp.gu.panels,
           fp.gu.nb, fp.down.panels, layout_ok, (int)(fp.off_hand / 256), fp.ws_bytes, check(ptr),
           overlapped(H, WG), overlapped(OUT, WS), overlapped(WS, FWS), overlapped(WG, HIDDEN));
    return 0;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc > 1 && strcmp(argv[1], "ffn") == 0) return ffn_main(argc, argv);
    if (argc != 11 && argc != 12) {
        fprintf(stderr, "usage: plan_host B H nq nkv D cap dtype schedule cus per_cu [pos_probe]\n");
        return 2;
    }
    dab_config c{};
    c.batch = atoi(argv[1]);
    c.hidden = atoi(argv[2]);
    c.n_q_heads = atoi(argv[3]);
    c.n_kv_heads = atoi(argv[4]);
    c.head_dim = atoi(argv[5]);
    c.cache_capacity = atoi(argv[6]);
    c.dtype = atoi(argv[7]);
    c.rope_theta = 1e4f;
    c.eps = 1e-6f;
    c.kv_chunk = 0;
    c.schedule = atoi(argv[8]);
    dab::Plan p;
    const dab_status st = dab::make_plan(&c, &p, atoi(argv[9]), atoi(argv[10]));
    // every position the capacity allows: the per-sequence chunk length fits the grid's slots and the
    // chunks cover the cached tokens; the largest count, and the length at position pos_probe
    int worst = 0, bad = 0;
    for (int pos = 0; st == DAB_OK && pos < c.cache_capacity; ++pos) {
        const int n = dab::chunk_count(p.chunk, pos);
        const int len = dab::chunk_len(p.chunk, pos);
        if (n > worst) worst = n;
        if (n > p.max_chunks || len % 16 != 0 || (pos > 0 && (n * len < pos || (n - 1) * len >= pos))) ++bad;
    }
    const int probe = argc > 11 ? atoi(argv[11]) : 0;
    printf("%d %d %d %d %d %d %d %d %d\n", (int)st, p.schedule, p.kv_chunk, p.max_chunks, p.attn_grid,
           p.split_merge ? 1 : 0, worst, bad, dab::chunk_len(p.chunk, probe));
    return 0;
}

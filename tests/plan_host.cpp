// Host driver of the launch planner (dab_plan.cpp is plain C++): prints the
// split-KV chunk choice of a configuration for a given number of compute
// units and resident attention workgroups per unit.  Built with g++ by tests/test_plan_host.py.
//   plan_host B H nq nkv D cap dtype schedule cus per_cu [pos_probe]
// It also walks every position below the capacity: the largest chunk count,
// the positions whose chunks would not fit the grid or cover the tokens, and
// the chunk length at pos_probe.
#include <stdio.h>
#include <stdlib.h>

#include "dab_plan.h"

int main(int argc, char** argv) {
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

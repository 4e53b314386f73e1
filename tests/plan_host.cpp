// Host driver of the launch planner (dab_plan.cpp is plain C++): prints the
// split-KV chunk choice of a configuration for a given number of compute
// units and resident attention workgroups per unit.  Built with g++ by tests/test_plan_host.py.
//   plan_host B H nq nkv D cap dtype schedule cus per_cu
#include <stdio.h>
#include <stdlib.h>

#include "dab_plan.h"

int main(int argc, char** argv) {
    if (argc != 11) {
        fprintf(stderr, "usage: plan_host B H nq nkv D cap dtype schedule cus per_cu\n");
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
    printf("%d %d %d %d %d %d\n", (int)st, p.schedule, p.kv_chunk, p.max_chunks, p.attn_grid, p.split_merge ? 1 : 0);
    return 0;
}

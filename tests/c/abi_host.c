/* A plain C11 caller of the host half of include/wave.h: builds a plan,
 * reads its view, packs its descriptor and exercises the error path.  No
 * GPU call is made.  Prints the facts the CPU test checks. */
#include <stdio.h>
#include <stdlib.h>

#include "wave.h"

int main(int argc, char** argv) {
  wave_plan_params p = {0};
  p.B = argc > 1 ? atoi(argv[1]) : 7;
  p.K = argc > 2 ? atoi(argv[2]) : 4;
  p.policy = WAVE_PROGRESSIVE;
  p.sched = WAVE_SCHED_WAVE;
  p.history_cap = -1;
  p.chunk_len = 4680;
  wave_plan_t* plan = NULL;
  if (wave_plan(&p, &plan) != WAVE_OK) {
    fprintf(stderr, "wave_plan: %s\n", wave_last_error());
    return 1;
  }
  wave_plan_view v;
  if (wave_plan_view_get(plan, &v) != WAVE_OK) return 2;
  size_t bytes = 0;
  if (wave_plan_desc_size(plan, &bytes) != WAVE_OK || bytes == 0) return 3;
  int32_t* desc = (int32_t*)malloc(bytes);
  if (!desc || wave_plan_desc_pack(plan, desc, bytes) != WAVE_OK) return 4;
  if (wave_plan_desc_pack(plan, desc, bytes - 4) != WAVE_ERR_INVALID_ARG) return 5;

  printf("rounds %d nodes %d phys %d desc_bytes %zu\n", v.num_rounds, v.num_nodes, v.num_phys_slots, bytes);
  const int t = v.num_rounds > 6 ? 6 : v.num_rounds - 1;
  for (int32_t i = v.round_node_begin[t]; i < v.round_node_begin[t + 1]; ++i) {
    const wave_node* n = &v.nodes[i];
    printf("round %d node %d %d ctx", t, n->chunk, n->level);
    for (int32_t e = n->ctx_begin; e < n->ctx_begin + n->ctx_count; ++e)
      printf(" %d:%d", v.ctx[e].chunk, v.ctx[e].level);
    printf("\n");
  }
  wave_plan_t* bad = NULL;
  wave_plan_params q = p;
  q.K = 0;
  const int32_t rc = wave_plan(&q, &bad);
  printf("bad K: rc %d plan %s message %s\n", rc, bad ? "set" : "null", wave_last_error()[0] ? "set" : "empty");
  free(desc);
  wave_plan_destroy(plan);
  return 0;
}

/* Host-only use of the C ABI from plain C (no GPU needed): the header compiles as C11,
 * the library links, and calls return the documented statuses before touching a GPU. */
#include <stdalign.h>
#include <stdio.h>
#include <string.h>

#include "graph_attn.h"

static alignas(256) unsigned char buf[4096]; /* stands in for device pointers */

#define CHECK(cond, code)                                 \
  do {                                                    \
    if (!(cond)) {                                        \
      fprintf(stderr, "check failed: %s\n", #cond);       \
      return code;                                        \
    }                                                     \
  } while (0)

int main(void) {
  const int32_t indptr[] = {0, 2, 3, 3, 5};
  const int32_t indices[] = {1, 2, 0, 0, 3};
  const int32_t bad_indices[] = {1, 2, 0, 0, 9};
  ga_plan_opts o;
  ga_plan* p = NULL;
  ga_plan_info info;
  size_t bytes = 0;
  void* d = buf;

  CHECK(strncmp(graph_attn_version(), "graph_attn", 10) == 0, 1);
  CHECK(graph_attn_plan_opts_default(&o) == GA_OK, 2);
  CHECK(graph_attn_plan_create(indptr, bad_indices, 4, 5, &o, &p) == GA_ERR_BAD_GRAPH, 3);
  CHECK(graph_attn_plan_create(indptr, indices, 4, 5, &o, &p) == GA_OK && p != NULL, 4);
  CHECK(graph_attn_plan_get_info(p, &info) == GA_OK, 5);
  CHECK(info.n_nodes == 4 && info.n_edges == 5 && info.has_csc == 1, 6);
  CHECK(info.max_in_degree == 2 && info.rows_sorted == 1 && info.uploaded == 0, 7);
  CHECK(graph_attn_plan_device_bytes(p, &bytes) == GA_OK && bytes > 0, 8);
  CHECK(graph_attn_fwd_workspace_bytes(p, 8, 32, &bytes) == GA_OK, 9);
  /* valid arguments, plan not uploaded: refused before any HIP call */
  CHECK(graph_attn_fwd(p, GA_SCORE_DOT, GA_BF16, 8, 32, 0.17f, 0.2f, d, d, d, d, (float*)d, d,
                       1 << 20, NULL) == GA_ERR_NOT_READY, 10);
  CHECK(graph_attn_fwd(p, GA_SCORE_DOT, GA_BF16, 8, 12, 0.17f, 0.2f, d, d, d, d, (float*)d, d,
                       1 << 20, NULL) == GA_ERR_UNSUPPORTED, 11);
  CHECK(graph_attn_reduce_fwd(p, GA_REDUCE_MAX, GA_F32, 64, d, d, (int32_t*)d, d, d, 1 << 20,
                              NULL) == GA_ERR_NOT_READY, 12);
  CHECK(graph_attn_reduce_bwd(p, GA_F32, 64, NULL, NULL, d, d, d, 1 << 20, NULL) ==
            GA_ERR_INVALID_ARG, 13);
  CHECK(strncmp(graph_attn_status_string(GA_ERR_WORKSPACE), "GA_ERR_WORKSPACE", 16) == 0, 14);
  graph_attn_plan_destroy(p);
  graph_attn_plan_destroy(NULL);
  puts("abi_smoke ok");
  return 0;
}

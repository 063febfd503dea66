/*
 * A plain C client of libmsa, built by tests/test_c_client.py with gcc
 * against include/msa.h alone.
 *
 *   msa_c_client cpu   validation and workspace queries, no device needed:
 *                      prints one line per query.
 *   msa_c_client gpu   a small fp32 forward on the default stream of device 0
 *                      with inputs from a fixed 32-bit LCG; prints the block
 *                      ids and the bit patterns of out and lse as hex words.
 *
 * The GPU mode uses the HIP runtime's C API for memory (the library itself
 * allocates nothing).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "msa.h"

static msa_problem_t make_problem(int32_t n_q, int32_t n_k, int32_t h_q, int32_t h_kv, int32_t d, int32_t d_idx,
                                  int32_t topk, int32_t dtype) {
  msa_problem_t p;
  memset(&p, 0, sizeof p);
  p.batch = 1;
  p.n_q = n_q;
  p.n_k = n_k;
  p.h_q = h_q;
  p.h_kv = h_kv;
  p.d = d;
  p.d_idx = d_idx;
  p.block_size = 128;
  p.topk = topk;
  p.dtype = dtype;
  p.q_offset = n_k - n_q;
  p.softmax_scale = 0.f;
  p.sched = MSA_SCHED_AUTO;
  p.idx_format = MSA_IDX_PLAIN;
  p.kv_format = MSA_IDX_PLAIN;
  return p;
}

static int cpu_mode(void) {
  msa_problem_t ok = make_problem(32768, 32768, 64, 8, 128, 128, 16, MSA_BF16);
  msa_problem_t bad_g = make_problem(4096, 4096, 12, 4, 64, 32, 4, MSA_F32);   /* Hq / Hkv = 3 */
  msa_problem_t bad_pos = make_problem(4096, 2048, 8, 2, 64, 32, 4, MSA_F32);  /* q_offset < 0 */
  msa_problem_t bad_d = make_problem(4096, 4096, 8, 2, 96, 32, 4, MSA_F32);    /* d = 96 */
  printf("validate ok %d\n", (int)msa_validate(&ok));
  printf("validate group3 %d\n", (int)msa_validate(&bad_g));
  printf("validate offset %d\n", (int)msa_validate(&bad_pos));
  printf("validate d96 %d\n", (int)msa_validate(&bad_d));
  printf("validate null %d\n", (int)msa_validate(NULL));
  for (int op = MSA_OP_INDEX_TOPK; op <= MSA_OP_INDEXER_KL; ++op) {
    size_t full = 0, least = 0;
    const msa_status_t st = msa_workspace_size(&ok, op, &full, &least);
    printf("workspace %d %d %zu %zu\n", op, (int)st, full, least);
  }
  printf("status %s\n", msa_status_string(MSA_ERR_UNSUPPORTED));
  return 0;
}

/* The HIP runtime's C API, declared here so that the client needs no HIP
 * header: hipMalloc, hipMemcpy (kinds 1 = host to device, 2 = device to host),
 * hipDeviceSynchronize and hipFree, each returning hipError_t (0 = success). */
extern int hipMalloc(void** ptr, size_t size);
extern int hipMemcpy(void* dst, const void* src, size_t size, int kind);
extern int hipDeviceSynchronize(void);
extern int hipFree(void* ptr);

static uint32_t lcg_state = 12345u;
static float lcg_uniform(void) { /* in [-0.5, 0.5): 24 random bits */
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)(lcg_state >> 8) * (1.0f / 16777216.0f) - 0.5f;
}

static void* upload(size_t n) {
  float* h = (float*)malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) h[i] = lcg_uniform();
  void* d = NULL;
  if (hipMalloc(&d, n * sizeof(float)) != 0 || hipMemcpy(d, h, n * sizeof(float), 1) != 0) {
    fprintf(stderr, "upload failed\n");
    exit(2);
  }
  free(h);
  return d;
}

static int gpu_mode(void) {
  const msa_problem_t p = make_problem(512, 1024, 8, 2, 64, 32, 4, MSA_F32);
  const size_t nq = (size_t)p.batch * p.n_q, nk = (size_t)p.batch * p.n_k;
  /* inputs in this order: q, k, v, idx_q, idx_k */
  void* q = upload(nq * p.h_q * p.d);
  void* k = upload(nk * p.h_kv * p.d);
  void* v = upload(nk * p.h_kv * p.d);
  void* iq = upload(nq * p.h_kv * p.d_idx);
  void* ik = upload(nk * p.h_kv * p.d_idx);
  const size_t n_ids = nq * p.h_kv * p.topk, n_out = nq * p.h_q * p.d, n_lse = nq * p.h_q;
  void *ids = NULL, *out = NULL, *lse = NULL, *ws = NULL;
  size_t full = 0, least = 0;
  if (msa_workspace_size(&p, MSA_OP_FORWARD, &full, &least) != MSA_OK) return 3;
  if (hipMalloc(&ids, n_ids * 4) || hipMalloc(&out, n_out * 4) || hipMalloc(&lse, n_lse * 4) ||
      hipMalloc(&ws, full)) {
    fprintf(stderr, "allocation failed\n");
    return 2;
  }
  const msa_status_t st = msa_forward(&p, q, k, v, iq, ik, (int32_t*)ids, out, (float*)lse, ws, full, NULL);
  if (st != MSA_OK) {
    fprintf(stderr, "msa_forward: %s (hip %d)\n", msa_status_string(st), msa_last_hip_error());
    return 4;
  }
  if (hipDeviceSynchronize() != 0) return 5;
  int32_t* h_ids = (int32_t*)malloc(n_ids * 4);
  uint32_t* h_out = (uint32_t*)malloc(n_out * 4);
  uint32_t* h_lse = (uint32_t*)malloc(n_lse * 4);
  if (hipMemcpy(h_ids, ids, n_ids * 4, 2) || hipMemcpy(h_out, out, n_out * 4, 2) ||
      hipMemcpy(h_lse, lse, n_lse * 4, 2))
    return 6;
  printf("ids");
  for (size_t i = 0; i < n_ids; ++i) printf(" %d", h_ids[i]);
  printf("\nout");
  for (size_t i = 0; i < n_out; ++i) printf(" %08x", h_out[i]);
  printf("\nlse");
  for (size_t i = 0; i < n_lse; ++i) printf(" %08x", h_lse[i]);
  printf("\n");
  void* bufs[] = {q, k, v, iq, ik, ids, out, lse, ws};
  for (int i = 0; i < 9; ++i) hipFree(bufs[i]);
  free(h_ids);
  free(h_out);
  free(h_lse);
  return 0;
}

int main(int argc, char** argv) {
  if (argc > 1 && strcmp(argv[1], "gpu") == 0) return gpu_mode();
  return cpu_mode();
}

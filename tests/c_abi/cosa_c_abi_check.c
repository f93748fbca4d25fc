/* A plain C caller of libcosa: the boundary used without Python or torch.
 *
 *   cosa_c_abi_check --host-only   argument validation, sizing helpers, status strings
 *                                  (no device call: every argument is checked on the
 *                                  host before the library touches the GPU)
 *   cosa_c_abi_check               the above, then the proxy, the ordered walk and the
 *                                  dense kernel on a small ragged GQA problem: at full
 *                                  budgets with the skip test off every list is a
 *                                  permutation of the candidate blocks and the walk is
 *                                  the dense softmax attention, so the sparse output and
 *                                  log-sum-exp must equal the dense ones (up to rounding
 *                                  order).
 * Exit status 0 on success; the first failed check is printed. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cosa.h"

#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      fprintf(stderr, "c abi check failed: ");    \
      fprintf(stderr, __VA_ARGS__);               \
      fprintf(stderr, "\n");                      \
      exit(1);                                    \
    }                                             \
  } while (0)

#define HIP(call)                                                           \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    CHECK(e_ == hipSuccess, "%s: %s", #call, hipGetErrorString(e_));        \
  } while (0)

enum { B = 1, HQ = 4, HKV = 2, N = 1000, D = 128, BLK = 128 };

static uint16_t to_bf16(float f) {   /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static float uniform_pm1(void) {   /* 64-bit LCG, top 24 bits */
  rng = rng * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((rng >> 40) & 0xffffff) / 8388608.0f - 1.0f;
}

static cosa_shape make_shape(void) {
  cosa_shape s;
  memset(&s, 0, sizeof s);
  s.batch = B;
  s.q_heads = HQ;
  s.kv_heads = HKV;
  s.seq_len = N;
  s.head_dim = D;
  s.block = BLK;
  s.causal = 1;
  s.scale = 0.0f;
  s.dtype = COSA_BF16;
  s.seq_lens = NULL;
  return s;
}

static cosa_kap_params full_kap(void) {
  cosa_kap_params p;
  memset(&p, 0, sizeof p);
  p.budget = 1.0;
  p.mass = 1.0;
  return p;
}

static void host_checks(void) {
  const cosa_shape s = make_shape();
  const cosa_kap_params kp = full_kap();
  const int nb = (N + BLK - 1) / BLK;
  CHECK(cosa_version() > 0, "version %d", cosa_version());
  CHECK(cosa_list_capacity(&s, 1.0) == nb, "capacity at full budget %d", cosa_list_capacity(&s, 1.0));
  CHECK(cosa_list_capacity(&s, 0.1) == 1, "capacity at budget 0.1 %d", cosa_list_capacity(&s, 0.1));
  CHECK(cosa_kap_workspace_bytes(&s, &kp) > 0, "workspace size");
  CHECK(strlen(cosa_status_string(COSA_ERR_INVALID_ARG)) > 0, "status string");

  /* invalid calls are rejected before any device work (all pointers are bogus here) */
  void* bogus = (void*)(uintptr_t)0x1000;
  int32_t* ib = (int32_t*)bogus;
  int r = cosa_proxy_select(&s, &kp, NULL, bogus, bogus, 1 << 30, ib, ib, ib, NULL, nb, NULL);
  CHECK(r == COSA_ERR_INVALID_ARG, "null q accepted (%d)", r);
  cosa_kap_params bad = kp;
  bad.budget = 0.0;
  r = cosa_proxy_select(&s, &bad, bogus, bogus, bogus, 1 << 30, ib, ib, ib, NULL, nb, NULL);
  CHECK(r == COSA_ERR_INVALID_ARG, "budget 0 accepted (%d)", r);
  r = cosa_proxy_select(&s, &kp, bogus, bogus, bogus, 16, ib, ib, ib, NULL, nb, NULL);
  CHECK(r == COSA_ERR_INVALID_ARG, "short workspace accepted (%d)", r);
  cosa_shape odd = s;
  odd.head_dim = 96;
  r = cosa_dense_attn(&odd, bogus, bogus, bogus, bogus, NULL, NULL);
  CHECK(r == COSA_ERR_UNSUPPORTED, "head_dim 96 accepted (%d)", r);
  cosa_osk_params op;
  memset(&op, 0, sizeof op);
  op.tight_budget = 1.5;
  r = cosa_ordered_sparse_attn(&s, &op, bogus, bogus, bogus, ib, ib, nb, NULL, bogus, NULL, NULL,
                               NULL, NULL);
  CHECK(r == COSA_ERR_INVALID_ARG, "tight budget 1.5 accepted (%d)", r);
  printf("c abi host checks ok (libcosa %d)\n", cosa_version());
}

static void device_checks(void) {
  const cosa_shape s = make_shape();
  const cosa_kap_params kp = full_kap();
  const int nb = (N + BLK - 1) / BLK;
  const int kmax = cosa_list_capacity(&s, kp.budget);
  const size_t nq = (size_t)B * HQ * N * D, nkv = (size_t)B * HKV * N * D;
  uint16_t* hq = malloc(nq * 2);
  uint16_t* hk = malloc(nkv * 2);
  uint16_t* hv = malloc(nkv * 2);
  CHECK(hq && hk && hv, "host allocation");
  for (size_t t = 0; t < nq; ++t) hq[t] = to_bf16(2.0f * uniform_pm1());
  for (size_t t = 0; t < nkv; ++t) hk[t] = to_bf16(2.0f * uniform_pm1());
  for (size_t t = 0; t < nkv; ++t) hv[t] = to_bf16(uniform_pm1());

  void *q, *k, *v, *os, *od, *ws;
  float *ls, *ld;
  int32_t *idx, *cnt, *hrm;
  const size_t wsb = cosa_kap_workspace_bytes(&s, &kp);
  HIP(hipMalloc(&q, nq * 2));
  HIP(hipMalloc(&k, nkv * 2));
  HIP(hipMalloc(&v, nkv * 2));
  HIP(hipMalloc(&os, nq * 2));
  HIP(hipMalloc(&od, nq * 2));
  HIP(hipMalloc((void**)&ls, (size_t)B * HQ * N * 4));
  HIP(hipMalloc((void**)&ld, (size_t)B * HQ * N * 4));
  HIP(hipMalloc(&ws, wsb));
  HIP(hipMalloc((void**)&idx, (size_t)B * HQ * nb * kmax * 4));
  HIP(hipMalloc((void**)&cnt, (size_t)B * HQ * nb * 4));
  HIP(hipMalloc((void**)&hrm, (size_t)B * HQ * nb * 4));
  HIP(hipMemcpy(q, hq, nq * 2, hipMemcpyHostToDevice));
  HIP(hipMemcpy(k, hk, nkv * 2, hipMemcpyHostToDevice));
  HIP(hipMemcpy(v, hv, nkv * 2, hipMemcpyHostToDevice));

  int r = cosa_proxy_select(&s, &kp, q, k, ws, wsb, idx, cnt, hrm, NULL, kmax, NULL);
  CHECK(r == COSA_OK, "cosa_proxy_select: %s", cosa_status_string(r));
  cosa_osk_params op;
  memset(&op, 0, sizeof op);
  op.tight_budget = 1.0;
  op.cap_mode = COSA_CAP_COMPUTED;
  op.skip_mode = COSA_SKIP_OFF;
  r = cosa_ordered_sparse_attn(&s, &op, q, k, v, idx, cnt, kmax, NULL, os, ls, NULL, NULL, NULL);
  CHECK(r == COSA_OK, "cosa_ordered_sparse_attn: %s", cosa_status_string(r));
  r = cosa_dense_attn(&s, q, k, v, od, ld, NULL);
  CHECK(r == COSA_OK, "cosa_dense_attn: %s", cosa_status_string(r));
  HIP(hipDeviceSynchronize());

  int32_t* hidx = malloc((size_t)B * HQ * nb * kmax * 4);
  int32_t* hcnt = malloc((size_t)B * HQ * nb * 4);
  uint16_t* hos = malloc(nq * 2);
  uint16_t* hod = malloc(nq * 2);
  float* hls = malloc((size_t)B * HQ * N * 4);
  float* hld = malloc((size_t)B * HQ * N * 4);
  CHECK(hidx && hcnt && hos && hod && hls && hld, "host allocation");
  HIP(hipMemcpy(hidx, idx, (size_t)B * HQ * nb * kmax * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(hcnt, cnt, (size_t)B * HQ * nb * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(hos, os, nq * 2, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(hod, od, nq * 2, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(hls, ls, (size_t)B * HQ * N * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(hld, ld, (size_t)B * HQ * N * 4, hipMemcpyDeviceToHost));

  /* every list of query block i is a permutation of the blocks 0..i */
  for (int h = 0; h < HQ; ++h)
    for (int i = 0; i < nb; ++i) {
      const int c = hcnt[h * nb + i];
      CHECK(c == i + 1, "head %d block %d: %d listed blocks", h, i, c);
      int seen[64] = {0};
      for (int p = 0; p < c; ++p) {
        const int j = hidx[((size_t)h * nb + i) * kmax + p];
        CHECK(j >= 0 && j <= i && !seen[j], "head %d block %d: entry %d = %d", h, i, p, j);
        seen[j] = 1;
      }
    }
  /* the full-budget walk is the dense attention */
  double worst = 0.0, worst_lse = 0.0;
  for (int h = 0; h < HQ; ++h)
    for (int t = 0; t < N; ++t) {
      for (int d = 0; d < D; ++d) {
        const size_t e = ((size_t)h * N + t) * D + d;
        const double diff = fabs((double)from_bf16(hos[e]) - (double)from_bf16(hod[e]));
        if (diff > worst) worst = diff;
      }
      const double dl = fabs((double)hls[h * N + t] - (double)hld[h * N + t]);
      if (dl > worst_lse) worst_lse = dl;
    }
  CHECK(worst <= 1e-2, "sparse vs dense output differ by %g", worst);
  CHECK(worst_lse <= 1e-3, "sparse vs dense lse differ by %g", worst_lse);
  printf("c abi device checks ok: %d heads x %d blocks, |O_sparse - O_dense| <= %.3g, |lse| <= %.3g\n",
         HQ, nb, worst, worst_lse);

  /* both stages pipelined over the two KV heads on two streams: bitwise the serial calls */
  {
    void* op2;
    float* lp;
    int32_t *idx2, *cnt2, *hrm2;
    HIP(hipMalloc(&op2, nq * 2));
    HIP(hipMalloc((void**)&lp, (size_t)B * HQ * N * 4));
    HIP(hipMalloc((void**)&idx2, (size_t)B * HQ * nb * kmax * 4));
    HIP(hipMalloc((void**)&cnt2, (size_t)B * HQ * nb * 4));
    HIP(hipMalloc((void**)&hrm2, (size_t)B * HQ * nb * 4));
    hipStream_t sp, sw;
    hipEvent_t ev;
    HIP(hipStreamCreate(&sp));
    HIP(hipStreamCreate(&sw));
    HIP(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    r = cosa_prefill(&s, &kp, &op, q, k, v, ws, wsb, idx2, cnt2, hrm2, kmax, op2, lp, HKV,
                     (void*)sp, (void*)sw, (void*)ev);
    CHECK(r == COSA_OK, "cosa_prefill: %s", cosa_status_string(r));
    HIP(hipStreamSynchronize(sw));
    int32_t* hidx2 = malloc((size_t)B * HQ * nb * kmax * 4);
    uint16_t* hop2 = malloc(nq * 2);
    float* hlp = malloc((size_t)B * HQ * N * 4);
    CHECK(hidx2 && hop2 && hlp, "host allocation");
    HIP(hipMemcpy(hidx2, idx2, (size_t)B * HQ * nb * kmax * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(hop2, op2, nq * 2, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(hlp, lp, (size_t)B * HQ * N * 4, hipMemcpyDeviceToHost));
    CHECK(memcmp(hidx, hidx2, (size_t)B * HQ * nb * kmax * 4) == 0, "pipelined lists differ");
    CHECK(memcmp(hos, hop2, nq * 2) == 0, "pipelined output differs");
    CHECK(memcmp(hls, hlp, (size_t)B * HQ * N * 4) == 0, "pipelined lse differs");
    /* a grouping that does not divide the KV heads is rejected */
    r = cosa_prefill(&s, &kp, &op, q, k, v, ws, wsb, idx2, cnt2, hrm2, kmax, op2, lp, 3,
                     (void*)sp, (void*)sw, (void*)ev);
    CHECK(r == COSA_ERR_INVALID_ARG, "3 groups of 2 KV heads accepted (%d)", r);
    printf("c abi pipelined prefill ok: %d groups, bitwise the serial calls\n", HKV);
    HIP(hipEventDestroy(ev));
    HIP(hipStreamDestroy(sp));
    HIP(hipStreamDestroy(sw));
    hipFree(op2); hipFree(lp); hipFree(idx2); hipFree(cnt2); hipFree(hrm2);
    free(hidx2); free(hop2); free(hlp);
  }

  hipFree(q); hipFree(k); hipFree(v); hipFree(os); hipFree(od); hipFree(ls); hipFree(ld);
  hipFree(ws); hipFree(idx); hipFree(cnt); hipFree(hrm);
  free(hq); free(hk); free(hv); free(hidx); free(hcnt); free(hos); free(hod); free(hls); free(hld);
}

int main(int argc, char** argv) {
  host_checks();
  if (argc > 1 && strcmp(argv[1], "--host-only") == 0) return 0;
  device_checks();
  return 0;
}

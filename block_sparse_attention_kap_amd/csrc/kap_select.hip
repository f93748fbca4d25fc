// KAP steps 3-5: MaxNorm, HRM flags, flag-group ordering and budgeted selection.
//
// CoSA technical summary (gist.science, pt), section 2.2 "Kernel-Aware Proxy":
// MaxNorm turns the block-max scores of each pooled row into relative ranking
// contributions; blocks holding some row's maximum are flagged HRM ("Have
// RowMax"); the computation-order mask lists the HRM blocks first and then the
// others by estimated score.  The authors' abstract: the proxy keeps blocks under a
// moderate budget, and the order of the mask is the order in which the kernel's
// inner loop visits KV pages.
//
// Readings fixed here: MaxNorm is c[r][j] = exp(P[r][j] - max_j' P[r][j']); the
// block score is S[j] = sum (or max) over the R_b pooled rows of the query block,
// added in ascending row order in fp32; a row's HRM block is the lowest j attaining
// its maximum; the order is (HRM desc, S desc, j asc); query block i keeps
// k_i = min(n_i, max(1, ceil(rho * n_i))) blocks.
//
// One workgroup per (batch*head, query block), heaviest (largest i) first.  The
// candidates are packed into 64-bit keys (HRM bit | fp32 bits of S >= 0 | ~j) whose
// unsigned order is exactly the visiting order, and bitonic-sorted in LDS.
#include "cosa_common.hpp"
#include "cosa_launch.hpp"

namespace cosa {

constexpr int SEL_NT = 256;
constexpr int SEL_MAX_M = 8192;  // largest power of two >= nb supported
constexpr int SEL_MAX_RB = 128;

__global__ __launch_bounds__(SEL_NT) void kap_select_kernel(SelectLaunch a) {
  extern __shared__ unsigned long long keys[];
  __shared__ float rmax[SEL_MAX_RB];
  __shared__ int rarg[SEL_MAX_RB];
  __shared__ int hcount[SEL_NT / 64];

  const int i = a.nb - 1 - (int)blockIdx.x;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = a.causal ? i + 1 : a.nb;
  int M = 1;
  while (M < n) M <<= 1;
  const float* P0 = a.P + ((long)bh * a.Np + (long)i * a.Rb) * a.nb;

  // Row maxima and the lowest block attaining each: one wave per row.
  for (int s = wave; s < a.Rb; s += SEL_NT / 64) {
    const float* row = P0 + (long)s * a.nb;
    float best = -__builtin_inff();
    int bj = 0x7fffffff;
    for (int j = lane; j < n; j += 64) {
      const float v = row[j];
      if (v > best) {  // ascending j per lane: strict > keeps the lowest index
        best = v;
        bj = j;
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const float ob = __shfl_xor(best, off, 64);
      const int oj = __shfl_xor(bj, off, 64);
      if (ob > best || (ob == best && oj < bj)) {
        best = ob;
        bj = oj;
      }
    }
    if (lane == 0) {
      rmax[s] = best;
      rarg[s] = bj;
    }
  }
  __syncthreads();

  // Block scores, HRM flags and sort keys.
  int myh = 0;
  for (int j = tid; j < M; j += SEL_NT) {
    unsigned long long key = 0ull;
    if (j < n) {
      float S = 0.0f;
      bool hrm = (a.force_sink && j == 0) || (a.force_diag && j == (i < n ? i : n - 1));
      for (int s = 0; s < a.Rb; ++s) {
        const float c = expf(P0[(long)s * a.nb + j] - rmax[s]);
        S = a.agg_mode == 0 ? S + c : fmaxf(S, c);
        hrm |= (rarg[s] == j);
      }
      myh += hrm ? 1 : 0;
      key = ((unsigned long long)(hrm ? 1u : 0u) << 63) |
            ((unsigned long long)(__float_as_uint(S) & 0x7fffffffu) << 32) |
            (unsigned long long)(0xffffffffu - (unsigned)j);
    }
    keys[j] = key;
  }
  for (int off = 32; off > 0; off >>= 1) myh += __shfl_xor(myh, off, 64);
  if (lane == 0) hcount[wave] = myh;
  __syncthreads();

  // Bitonic sort, descending.
  for (int kk = 2; kk <= M; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int t = tid; t < (M >> 1); t += SEL_NT) {
        const int i1 = 2 * jj * (t / jj) + (t % jj);
        const int i2 = i1 + jj;
        const unsigned long long x = keys[i1];
        const unsigned long long y = keys[i2];
        const bool desc = (i1 & kk) == 0;
        if (desc ? (x < y) : (x > y)) {
          keys[i1] = y;
          keys[i2] = x;
        }
      }
      __syncthreads();
    }
  }

  const long unit = (long)bh * a.nb + i;
  const int kcnt = (int)fmin((double)n, fmax(1.0, ceil(a.budget * (double)n)));
  for (int p = tid; p < a.kmax; p += SEL_NT) {
    int idx = -1;
    float sc = 0.0f;
    if (p < kcnt) {
      const unsigned long long key = keys[p];
      idx = (int)(0xffffffffu - (unsigned)(key & 0xffffffffull));
      sc = __uint_as_float((unsigned)((key >> 32) & 0x7fffffffull));
    }
    a.visit_idx[unit * a.kmax + p] = idx;
    if (a.visit_score) a.visit_score[unit * a.kmax + p] = sc;
  }
  if (tid == 0) {
    int hc = 0;
    for (int w = 0; w < SEL_NT / 64; ++w) hc += hcount[w];
    a.visit_cnt[unit] = kcnt;
    a.hrm_cnt[unit] = hc;
  }
}

hipError_t launch_select(const SelectLaunch& a, hipStream_t s) {
  int M = 1;
  while (M < a.nb) M <<= 1;
  if (M > SEL_MAX_M || a.Rb > SEL_MAX_RB) return hipErrorInvalidValue;
  const size_t lds = (size_t)M * sizeof(unsigned long long);
  hipLaunchKernelGGL(kap_select_kernel, dim3(a.nb, a.bh), dim3(SEL_NT), lds, s, a);
  return hipGetLastError();
}

}  // namespace cosa

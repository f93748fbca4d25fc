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
// One workgroup per (batch*head, query block), heaviest (largest i) first.  Each
// candidate becomes a 64-bit key (HRM bit | fp32 bits of S >= 0 | ~j) whose unsigned
// order is exactly the visiting order, so the list is the k largest keys in
// descending order.  The k-th largest key is found by an MSB-first radix select
// (8-bit digits, LDS histograms), the keys at or above it are compacted, and each is
// placed by its rank among them.  All counts are integers, so the result does not
// depend on the order of the LDS atomics.  The radix rounds read each key through an
// order-preserving map of its S field (shifted down by the unit's smallest S and up as
// far as its largest allows), so that the first digit already spreads the candidates:
// the raw bits of block scores in (0, R_b] share their exponent bits, so their first
// digit alone would fall into a few crowded bins.
//
// With share (one list per KV head, for GQA) the workgroup of (batch, KV head, i)
// takes the pooled rows of the group's query heads, heads ascending, as the rows of
// the query block: S sums over all of them in that order and HRM is their union.
//
// With order_mode SCORE the HRM bit is left out of the key (plain top-k by S, the
// ranking of a single-criterion proxy); the HRM count is still reported.
//
// Cumulative-mass selection (optional): the list is cut to the shortest prefix of the
// visiting order whose score sum reaches mass * (sum of S over all candidates), but
// never beyond k_i.  Sums are fp32 in a fixed order: the total as per-thread partial
// sums over j = tid, tid + 256, ... reduced in lane and wave order; the prefix sums
// sequentially along the list.
#include "cosa_common.hpp"
#include "cosa_launch.hpp"

namespace cosa {

constexpr int SEL_NT = 256;
constexpr int SEL_NW = SEL_NT / 64;
constexpr int SEL_MAX_NB = 4096;
constexpr int SEL_MAX_ROWS = 1024;  // pooled rows of a unit (heads x rows per block)

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), by data-parallel
// moves between lanes: shifts by 1, 2, 4, 8 inside each row of 16 lanes (lanes shifted in
// from outside the row add 0), then the last lane of row 0 is added to row 1, of row 2 to
// row 3, and the last lane of row 1 (by then the sum of rows 0 and 1) to rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// (max, lowest index attaining it) over the 64 lanes of a wave, left in lane 63: the same
// lane pattern as wave_inclusive_sum with the pair combine; lanes with no source take
// (-inf, INT_MAX), which changes nothing.
__device__ __forceinline__ void argmax_step(float& best, int& bj, float ob, int oj) {
  if (ob > best || (ob == best && oj < bj)) {
    best = ob;
    bj = oj;
  }
}
#define COSA_ARGMAX_DPP(CTRL, ROWM)                                                             \
  argmax_step(best, bj,                                                                         \
              __int_as_float(__builtin_amdgcn_update_dpp((int)0xff800000, __float_as_int(best), \
                                                         CTRL, ROWM, 0xf, false)),              \
              __builtin_amdgcn_update_dpp(0x7fffffff, bj, CTRL, ROWM, 0xf, false))
__device__ __forceinline__ void wave_argmax(float& best, int& bj) {
  COSA_ARGMAX_DPP(0x111, 0xf);
  COSA_ARGMAX_DPP(0x112, 0xf);
  COSA_ARGMAX_DPP(0x114, 0xf);
  COSA_ARGMAX_DPP(0x118, 0xf);
  COSA_ARGMAX_DPP(0x142, 0xa);
  COSA_ARGMAX_DPP(0x143, 0xc);
}
#undef COSA_ARGMAX_DPP

__global__ __launch_bounds__(SEL_NT) void kap_select_kernel(SelectLaunch a) {
  extern __shared__ unsigned long long keys[];  // n candidate keys, then the top k
  __shared__ float rmax[SEL_MAX_ROWS];
  __shared__ int rarg[SEL_MAX_ROWS];
  __shared__ int hist[2][256];                  // one per radix round, alternating
  __shared__ int hcount[SEL_NW];
  __shared__ int sel_digit, sel_rem, sel_cnt, nsel, kfinal;
  __shared__ float wsum[SEL_NW];
  __shared__ unsigned wsmin[SEL_NW], wsmax[SEL_NW];

  const int i = a.nb - 1 - (int)blockIdx.x;
  const int by = blockIdx.y;                          // batch * heads of the lists
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int G = a.share ? a.group : 1;                // query heads whose rows form the unit
  const int b = a.share ? by / a.Hkv : by / a.Hq;
  const int bh0 = a.share ? b * a.Hq + (by - b * a.Hkv) * a.group : by;   // first query head
  const int Lb = a.sl.of(b, a.N);                     // tokens of this batch entry
  const int nbv = (Lb + a.block - 1) / a.block;       // its blocks
  const long unit = (long)by * a.nb + i;
  if (i >= nbv) {                                     // past the end: an empty list
    for (int p = tid; p < a.kmax; p += SEL_NT) {
      a.visit_idx[unit * a.kmax + p] = -1;
      if (a.visit_score) a.visit_score[unit * a.kmax + p] = 0.0f;
    }
    if (tid == 0) {
      a.visit_cnt[unit] = 0;
      a.hrm_cnt[unit] = 0;
    }
    return;
  }
  const int n = a.causal ? i + 1 : nbv;
  const long ldp = p_pitch(a.nb);                     // row pitch of P
  const float* P0 = a.P + ((long)bh0 * a.Np + (long)i * a.Rb) * ldp;
  const long hstride = (long)a.Np * ldp;              // next query head's P
  // pooled rows of this block per head (fewer in a partial last block)
  const int Rb = min(a.Rb, (Lb + a.g - 1) / a.g - i * a.Rb);
  const float NEG = -__builtin_inff();

  // ---- row maxima and the lowest block attaining each: one wave per pooled row
  for (int s = wave; s < G * Rb; s += SEL_NW) {
    const int hs = s / Rb;
    const float* row = P0 + hs * hstride + (long)(s - hs * Rb) * ldp;
    float best = NEG;
    int bj = 0x7fffffff;
    for (int j0 = lane; j0 < n; j0 += 64 * 16) {   // 16 loads in flight per lane
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = (j0 + 64 * u < n) ? row[j0 + 64 * u] : NEG;
#pragma unroll
      for (int u = 0; u < 16; ++u)  // ascending j per lane: strict > keeps the lowest index
        if (v[u] > best) {
          best = v[u];
          bj = j0 + 64 * u;
        }
    }
    wave_argmax(best, bj);
    if (lane == 63) {
      rmax[s] = best;
      rarg[s] = bj;
    }
  }
  __syncthreads();

  // ---- block scores, HRM flags, sort keys (two blocks per thread and pass, so that
  // their loads are in flight together; each block's sum keeps its own ascending row order;
  // four would keep more loads in flight but cost occupancy: 92 registers instead of 58)
  constexpr int NBT = 2;
  int myh = 0;
  float mysum = 0.0f;
  unsigned sminb = 0x7fffffffu, smaxb = 0u;   // range of the bits of S over the candidates
  for (int j = tid; j < n; j += NBT * SEL_NT) {
    int je[NBT];
    float S[NBT];
    bool hrm[NBT];
#pragma unroll
    for (int e = 0; e < NBT; ++e) {
      je[e] = j + e * SEL_NT < n ? j + e * SEL_NT : j;   // past the end: block j again (unused)
      S[e] = 0.0f;
      hrm[e] = (a.force_sink && je[e] == 0) || (a.force_diag && je[e] == (i < n ? i : n - 1));
    }
    for (int hs = 0; hs < G; ++hs) {
      const float* Ph = P0 + hs * hstride;
      const float* rm = rmax + hs * Rb;
      const int* ra = rarg + hs * Rb;
      int s = 0;
      for (; s + 4 <= Rb; s += 4) {
        float pv[NBT][4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < NBT; ++e) pv[e][u] = Ph[(s + u) * ldp + je[e]];
#pragma unroll
        for (int e = 0; e < NBT; ++e)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float c = expf(pv[e][u] - rm[s + u]);
            S[e] = a.agg_mode == 0 ? S[e] + c : fmaxf(S[e], c);
            hrm[e] |= (ra[s + u] == je[e]);
          }
      }
      for (; s < Rb; ++s) {
#pragma unroll
        for (int e = 0; e < NBT; ++e) {
          const float c = expf(Ph[s * ldp + je[e]] - rm[s]);
          S[e] = a.agg_mode == 0 ? S[e] + c : fmaxf(S[e], c);
          hrm[e] |= (ra[s] == je[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < NBT; ++e) {
      if (j + e * SEL_NT >= n) break;
      myh += hrm[e] ? 1 : 0;
      mysum += S[e];
      const unsigned sb = __float_as_uint(S[e]) & 0x7fffffffu;
      sminb = sminb < sb ? sminb : sb;
      smaxb = smaxb > sb ? smaxb : sb;
      keys[je[e]] = ((unsigned long long)((hrm[e] && a.order_mode == 0) ? 1u : 0u) << 63) |
                    ((unsigned long long)(__float_as_uint(S[e]) & 0x7fffffffu) << 32) |
                    (unsigned long long)(0xffffffffu - (unsigned)je[e]);
    }
  }
  myh = __builtin_amdgcn_readlane(wave_inclusive_sum(myh), 63);
  for (int off = 32; off > 0; off >>= 1) mysum += __shfl_xor(mysum, off, 64);
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned a0 = (unsigned)__shfl_xor((int)sminb, off, 64), a1 = (unsigned)__shfl_xor((int)smaxb, off, 64);
    sminb = sminb < a0 ? sminb : a0;
    smaxb = smaxb > a1 ? smaxb : a1;
  }
  if (lane == 0) {
    hcount[wave] = myh;
    wsum[wave] = mysum;
    wsmin[wave] = sminb;
    wsmax[wave] = smaxb;
  }
  hist[0][tid] = 0;
  __syncthreads();
  // The radix select runs on keys whose S field is shifted down by the smallest S of the unit and
  // up as far as the largest allows: an order-preserving map onto the whole 31-bit field, so that
  // the first 8-bit digit already spreads the candidates (the raw bits of S share their top bits).
  unsigned smin = wsmin[0], smax = wsmax[0];
#pragma unroll
  for (int w = 1; w < SEL_NW; ++w) {
    smin = smin < wsmin[w] ? smin : wsmin[w];
    smax = smax > wsmax[w] ? smax : wsmax[w];
  }
  const unsigned srange = smax - smin;
  const int ssh = srange ? __clz(srange) - 1 : 0;
  auto tkey = [&](unsigned long long key) -> unsigned long long {
    const unsigned hi = (unsigned)(key >> 32);
    const unsigned thi = (hi & 0x80000000u) | (((hi & 0x7fffffffu) - smin) << ssh);
    return ((unsigned long long)thi << 32) | (key & 0xffffffffull);
  };

  // ---- radix select: the smallest key T such that exactly k keys are >= T
  int kcnt = (int)fmin((double)n, fmax(1.0, ceil(a.budget * (double)n)));
  kcnt = kcnt < a.kmax ? kcnt : a.kmax;  // the host guarantees kmax >= every k_i
  unsigned long long T = 0ull;
  if (kcnt < n) {
    unsigned long long prefix = 0ull, mask = 0ull;
    int rem = kcnt;
    for (int shift = 56, rnd = 0; shift >= 0; shift -= 8, ++rnd) {
      int* H = hist[rnd & 1];
      hist[(rnd + 1) & 1][tid] = 0;  // the next round's (its last reader, the scan of the round
                                     // before this one, finished before the previous barrier)
      for (int e = tid; e < n; e += SEL_NT) {
        const unsigned long long key = tkey(keys[e]);
        if ((key & mask) == prefix) atomicAdd(&H[(int)((key >> shift) & 255ull)], 1);
      }
      __syncthreads();
      if (wave == 0) {
        // lane L owns digits 255-4L .. 252-4L (descending); counts above each digit
        int c[4], loc = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c[q] = H[255 - 4 * lane - q];
          loc += c[q];
        }
        const int incl = wave_inclusive_sum(loc);
        int above = incl - loc;
        if (above < rem && rem <= incl) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (above < rem && rem <= above + c[q]) {
              sel_digit = 255 - 4 * lane - q;
              sel_rem = rem - above;
              sel_cnt = c[q];
            }
            above += c[q];
          }
        }
      }
      __syncthreads();
      const int d = sel_digit;
      rem = sel_rem;
      prefix |= (unsigned long long)d << shift;
      mask |= 255ull << shift;
      if (sel_cnt == rem) break;  // every key with this prefix is taken
    }
    T = prefix;
  }

  // ---- compact the top k (arbitrary order), then place each by its rank
  unsigned long long* top = keys + n;
  if (tid == 0) nsel = 0;
  __syncthreads();
  for (int e = tid; e < n; e += SEL_NT) {
    const unsigned long long key = keys[e];
    if (tkey(key) >= T) {
      const int slot = atomicAdd(&nsel, 1);  // exactly kcnt keys pass; the cap only guards the buffer
      if (slot < a.kmax) top[slot] = key;
    }
  }
  __syncthreads();

  // rank placement into keys[0 .. kcnt) (free again after the compaction)
  for (int t = tid; t < kcnt; t += SEL_NT) {
    const unsigned long long key = top[t];
    int r = 0;
#pragma unroll 8
    for (int u = 0; u < kcnt; ++u) r += top[u] > key ? 1 : 0;
    keys[r] = key;
  }
  if (tid == 0) kfinal = kcnt;
  __syncthreads();
  if (a.sel_mode == 1 && tid == 0) {
    float total = 0.0f;
    for (int w = 0; w < SEL_NW; ++w) total += wsum[w];
    const float goal = a.mass * total;
    float cum = 0.0f;
    int kf = kcnt;
    for (int r = 0; r < kcnt; ++r) {
      cum += __uint_as_float((unsigned)((keys[r] >> 32) & 0x7fffffffull));
      if (cum >= goal) {
        kf = r + 1;
        break;
      }
    }
    kfinal = kf;
  }
  __syncthreads();
  const int kout = kfinal;
  for (int p = tid; p < a.kmax; p += SEL_NT) {
    int idx = -1;
    float sc = 0.0f;
    if (p < kout) {
      const unsigned long long key = keys[p];
      idx = (int)(0xffffffffu - (unsigned)(key & 0xffffffffull));
      sc = __uint_as_float((unsigned)((key >> 32) & 0x7fffffffull));
    }
    a.visit_idx[unit * a.kmax + p] = idx;
    if (a.visit_score) a.visit_score[unit * a.kmax + p] = sc;
  }
  if (tid == 0) {
    int hc = 0;
    for (int w = 0; w < SEL_NW; ++w) hc += hcount[w];
    a.visit_cnt[unit] = kout;
    a.hrm_cnt[unit] = hc;
  }
}

hipError_t launch_select(const SelectLaunch& a, hipStream_t s) {
  const int G = a.share ? a.group : 1;
  if (a.nb > SEL_MAX_NB || G * a.Rb > SEL_MAX_ROWS || a.kmax > a.nb) return hipErrorInvalidValue;
  const size_t lds = (size_t)(a.nb + a.kmax) * sizeof(unsigned long long);
  if (lds > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute((const void*)kap_select_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int units = a.share ? a.bh / a.group : a.bh;   // batch * (KV or query) heads
  hipLaunchKernelGGL(kap_select_kernel, dim3(a.nb, units), dim3(SEL_NT), lds, s, a);
  return hipGetLastError();
}

}  // namespace cosa

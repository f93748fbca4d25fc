// KAP step 2: approximate scores of pooled queries against pooled keys, max-pooled
// over the keys of each block.
//
// CoSA technical summary (gist.science, pt), section 2.2 "Kernel-Aware Proxy",
// block ranking: approximate scores from the downsampled Q and K, then MaxPool over
// the keys (which keeps each row's maximum inside its block).
//
// P[bh][r][j] = max over pooled keys t of block j with t <= r (causal) of
// scale * q~_r . k~_t.  One wave owns 32 pooled query rows and walks the pooled key
// tiles (32 keys each) up to its causal limit.  The dot products are a dense
// contraction: v_mfma_f32_32x32x16_bf16 (fp32 inputs: v_mfma_f32_32x32x2_f32) with
// fp32 accumulation; the block max is a lane reduction over the 32 key columns.
#include "cosa_common.hpp"
#include "cosa_launch.hpp"

namespace cosa {

template <typename T, int D>
__global__ __launch_bounds__(64) void kap_score_kernel(const T* __restrict__ qp,
                                                       const T* __restrict__ kp,
                                                       float* __restrict__ P, int Hq, int group,
                                                       int Hkv, int Np, int nb, int Rb, int causal,
                                                       float scale) {
  typedef Mfma<T> M;
  constexpr int NS = D / M::KSTEP;
  const int r0 = blockIdx.x * 32;
  const int bh = blockIdx.y;
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int bkv = b * Hkv + h / group;
  const int lane = threadIdx.x;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const T* qb = qp + (long)bh * Np * D;
  const T* kb = kp + (long)bkv * Np * D;
  float* Pb = P + (long)bh * Np * nb;

  // A operand: pooled query row r0+n (clamped for loads; rows >= Np are never stored).
  typename M::frag qa[NS];
  {
    const int r = min(r0 + n, Np - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) qa[s] = load_frag(qb + (long)r * D + s * M::KSTEP + hh * M::KPL);
  }
  const int t_end = causal ? min(Np, r0 + 32) : Np;  // exclusive
  const int ntile = (t_end + 31) / 32;
  const float NEG = -__builtin_inff();
  float run[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) run[x] = NEG;

  for (int kt = 0; kt < ntile; ++kt) {
    const int t0 = kt * 32;
    const int t = t0 + n;  // this lane's key column
    const int tl = min(t, Np - 1);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      typename M::frag kf = load_frag(kb + (long)tl * D + s * M::KSTEP + hh * M::KPL);
      acc = M::mma(qa[s], kf, acc);  // C[row][key]
    }
    float v[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int r = r0 + 8 * (x >> 2) + 4 * hh + (x & 3);
      float s_ = acc[x] * scale;
      if (t >= Np || (causal && t > r)) s_ = NEG;
      v[x] = s_;
    }
    // max over the key columns of each block inside this tile
    const int span = Rb < 32 ? Rb : 32;
    for (int off = 1; off < span; off <<= 1) {
#pragma unroll
      for (int x = 0; x < 16; ++x) v[x] = fmaxf(v[x], __shfl_xor(v[x], off, 64));
    }
#pragma unroll
    for (int x = 0; x < 16; ++x) run[x] = fmaxf(run[x], v[x]);
    const bool block_done = Rb <= 32 || ((t0 + 32) % Rb == 0) || kt == ntile - 1;
    if (block_done) {
      if ((n % span) == 0) {
        const int j = t / Rb;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int r = r0 + 8 * (x >> 2) + 4 * hh + (x & 3);
          const bool ok = r < Np && j < nb && (!causal || j <= r / Rb);
          if (ok) Pb[(long)r * nb + j] = run[x];
        }
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) run[x] = NEG;
    }
  }
}

template <typename T>
static hipError_t launch_score_t(const ScoreLaunch& a, hipStream_t s) {
  dim3 grid((a.Np + 31) / 32, a.bh);
  if (a.D == 128)
    hipLaunchKernelGGL((kap_score_kernel<T, 128>), grid, dim3(64), 0, s, (const T*)a.qp,
                       (const T*)a.kp, a.P, a.Hq, a.group, a.Hkv, a.Np, a.nb, a.Rb, a.causal,
                       a.scale);
  else
    hipLaunchKernelGGL((kap_score_kernel<T, 64>), grid, dim3(64), 0, s, (const T*)a.qp,
                       (const T*)a.kp, a.P, a.Hq, a.group, a.Hkv, a.Np, a.nb, a.Rb, a.causal,
                       a.scale);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreLaunch& a, hipStream_t s) {
  return a.bf16 ? launch_score_t<bf16_t>(a, s) : launch_score_t<float>(a, s);
}

}  // namespace cosa

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

// bf16 variant.  A block max needs only the key tile that holds the block, so the work
// splits freely over (row tile, chunk of SC_KC key tiles): one wave each, many waves
// per SIMD to cover memory latency, and the next key tile's fragments are loaded while
// the current one is multiplied.  The contraction index is permuted identically on
// both operands (lane half h, step s, element e <-> d = h*D/2 + 8s + e) so that every
// lane reads one contiguous half row.  Block maxima are collected in LDS and written
// out as whole row segments (partial-line scattered stores are slow on HBM).
constexpr int SC_KC = 8;

template <int D>
__global__ __launch_bounds__(64) void kap_score_bf16_kernel(const bf16_t* __restrict__ qp,
                                                            const bf16_t* __restrict__ kp,
                                                            float* __restrict__ P, int Hq,
                                                            int group, int Hkv, int Np, int nb,
                                                            int Rb, int causal, float scale) {
  constexpr int NS = D / 16;
  const int lane = threadIdx.x;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int r0 = blockIdx.y * 32;
  const int bh = blockIdx.z;
  const int t_end = causal ? min(Np, r0 + 32) : Np;
  const int ntile = (t_end + 31) / 32;
  const int kt0 = blockIdx.x * SC_KC;
  if (kt0 >= ntile) return;
  const int kt1 = min(kt0 + SC_KC, ntile);
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int bkv = b * Hkv + h / group;
  const bf16_t* qb = qp + (long)bh * Np * D;
  const bf16_t* kb = kp + (long)bkv * Np * D;
  float* Pb = P + (long)bh * Np * nb;
  extern __shared__ float Ps[];            // [32 rows][bpc blocks] of this chunk
  const int bpc = (SC_KC * 32 + Rb - 1) / Rb;
  const int jlo = (kt0 * 32) / Rb;

  bf16x8 qa[NS], kf[NS], kn[NS];
  {
    const bf16_t* q = qb + (long)min(r0 + n, Np - 1) * D + hh * (D / 2);
#pragma unroll
    for (int s = 0; s < NS; ++s) qa[s] = load_frag(q + 8 * s);
    const bf16_t* k = kb + (long)min(kt0 * 32 + n, Np - 1) * D + hh * (D / 2);
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[s] = load_frag(k + 8 * s);
  }
  const float NEG = -__builtin_inff();
  float run[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) run[x] = NEG;
  for (int kt = kt0; kt < kt1; ++kt) {
    if (kt + 1 < kt1) {
      const bf16_t* k = kb + (long)min((kt + 1) * 32 + n, Np - 1) * D + hh * (D / 2);
#pragma unroll
      for (int s = 0; s < NS; ++s) kn[s] = load_frag(k + 8 * s);
    }
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < NS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kf[s], acc, 0, 0, 0);
    const int t0 = kt * 32;
    const int t = t0 + n;
    float v[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int r = r0 + 8 * (x >> 2) + 4 * hh + (x & 3);
      float s_ = acc[x] * scale;
      if (t >= Np || (causal && t > r)) s_ = NEG;
      v[x] = s_;
    }
    const int span = Rb < 32 ? Rb : 32;
    for (int off = 1; off < span; off <<= 1) {
#pragma unroll
      for (int x = 0; x < 16; ++x) v[x] = fmaxf(v[x], __shfl_xor(v[x], off, 64));
    }
#pragma unroll
    for (int x = 0; x < 16; ++x) run[x] = fmaxf(run[x], v[x]);
    // a block spanning several key tiles ends on a multiple of Rb (chunks are aligned
    // to it: SC_KC * 32 is a multiple of every Rb <= 128) or at the causal limit
    const bool block_done = Rb <= 32 || ((t0 + 32) % Rb == 0) || kt == ntile - 1;
    if (block_done) {
      if ((n % span) == 0) {
        const int jc = t / Rb - jlo;
#pragma unroll
        for (int x = 0; x < 16; ++x) Ps[(8 * (x >> 2) + 4 * hh + (x & 3)) * bpc + jc] = run[x];
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) run[x] = NEG;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[s] = kn[s];
  }
  // the wave's 32 rows x nbc blocks, written row by row with consecutive lanes
  __syncthreads();
  const int nbc = (min(kt1 * 32, t_end) + Rb - 1) / Rb - jlo;
  for (int idx = lane; idx < 32 * nbc; idx += 64) {
    const int rl = idx / nbc;
    const int c = idx - rl * nbc;
    const int r = r0 + rl;
    const int j = jlo + c;
    if (r < Np && j < nb && (!causal || j <= r / Rb)) Pb[(long)r * nb + j] = Ps[rl * bpc + c];
  }
}

template <typename T>
static hipError_t launch_score_t(const ScoreLaunch& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    dim3 g2(((a.Np + 31) / 32 + SC_KC - 1) / SC_KC, (a.Np + 31) / 32, a.bh);
    const size_t lds = (size_t)32 * ((SC_KC * 32 + a.Rb - 1) / a.Rb) * sizeof(float);
    if (a.D == 128)
      hipLaunchKernelGGL((kap_score_bf16_kernel<128>), g2, dim3(64), lds, s, (const bf16_t*)a.qp,
                         (const bf16_t*)a.kp, a.P, a.Hq, a.group, a.Hkv, a.Np, a.nb, a.Rb,
                         a.causal, a.scale);
    else
      hipLaunchKernelGGL((kap_score_bf16_kernel<64>), g2, dim3(64), lds, s, (const bf16_t*)a.qp,
                         (const bf16_t*)a.kp, a.P, a.Hq, a.group, a.Hkv, a.Np, a.nb, a.Rb,
                         a.causal, a.scale);
    return hipGetLastError();
  }
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

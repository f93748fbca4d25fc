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

// bf16 variant: a workgroup of four waves covers 128 pooled query rows and shares
// each tile of 32 pooled keys through LDS.  Tiles are copied HBM -> LDS with
// global_load_lds into two alternating buffers (16-byte chunks of a key row are
// XOR-swizzled by the row so that the MFMA operand reads hit distinct banks), one
// barrier per tile.
typedef __attribute__((address_space(3))) void* lds_void_t;

template <int D>
__global__ __launch_bounds__(256) void kap_score_bf16_kernel(const bf16_t* __restrict__ qp,
                                                             const bf16_t* __restrict__ kp,
                                                             float* __restrict__ P, int Hq,
                                                             int group, int Hkv, int Np, int nb,
                                                             int Rb, int causal, float scale) {
  constexpr int NS = D / 16;
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int CHUNKS = 32 * CPR;           // per tile
  constexpr int CPT = CHUNKS / 256;          // copies per thread per tile
  __shared__ __attribute__((aligned(1024))) bf16_t Kt[2][32 * D];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int bh = blockIdx.y;
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int bkv = b * Hkv + h / group;
  const int rw0 = blockIdx.x * 128 + wave * 32;   // this wave's first pooled row
  const bf16_t* qb = qp + (long)bh * Np * D;
  const bf16_t* kb = kp + (long)bkv * Np * D;
  float* Pb = P + (long)bh * Np * nb;

  bf16x8 qa[NS];
  {
    const int r = min(rw0 + n, Np - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) qa[s] = load_frag(qb + (long)r * D + s * 16 + hh * 8);
  }
  const int wg_last = min(Np, blockIdx.x * 128 + 128);
  const int ntile = causal ? (wg_last + 31) / 32 : (Np + 31) / 32;          // workgroup
  const int ntile_w = causal ? (min(Np, rw0 + 32) + 31) / 32 : ntile;       // this wave
  auto issue = [&](int kt) {
    const int t0 = kt * 32;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = c * 256 + tid;
      const int row = chunk / CPR;
      const int pos = chunk % CPR;
      const int src_row = min(t0 + row, Np - 1);
      const int col = pos ^ (row & (CPR - 1));
      bf16_t* dst = &Kt[kt & 1][(c * 256 + (tid & ~63)) * 8];
      __builtin_amdgcn_global_load_lds((const void*)(kb + (long)src_row * D + col * 8),
                                       (lds_void_t)dst, 16, 0, 0);
    }
  };
  const float NEG = -__builtin_inff();
  float run[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) run[x] = NEG;
  issue(0);
  for (int kt = 0; kt < ntile; ++kt) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this thread's copies of tile kt landed
    __syncthreads();                     // everyone's; buffer (kt+1)&1 is free again
    if (kt + 1 < ntile) issue(kt + 1);
    if (kt >= ntile_w) continue;
    const bf16_t* kr = &Kt[kt & 1][n * D];
    const int sw = n & (CPR - 1);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 kf = load_frag(kr + (((2 * s + hh) ^ sw) * 8));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kf, acc, 0, 0, 0);  // C[row][key]
    }
    const int t0 = kt * 32;
    const int t = t0 + n;
    float v[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int r = rw0 + 8 * (x >> 2) + 4 * hh + (x & 3);
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
    const bool block_done = Rb <= 32 || ((t0 + 32) % Rb == 0) || kt == ntile_w - 1;
    if (block_done) {
      if ((n % span) == 0) {
        const int j = t / Rb;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int r = rw0 + 8 * (x >> 2) + 4 * hh + (x & 3);
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
  if constexpr (sizeof(T) == 2) {
    dim3 g2((a.Np + 127) / 128, a.bh);
    if (a.D == 128)
      hipLaunchKernelGGL((kap_score_bf16_kernel<128>), g2, dim3(256), 0, s, (const bf16_t*)a.qp,
                         (const bf16_t*)a.kp, a.P, a.Hq, a.group, a.Hkv, a.Np, a.nb, a.Rb,
                         a.causal, a.scale);
    else
      hipLaunchKernelGGL((kap_score_bf16_kernel<64>), g2, dim3(256), 0, s, (const bf16_t*)a.qp,
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

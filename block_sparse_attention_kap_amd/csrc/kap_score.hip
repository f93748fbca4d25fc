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
                                                       float scale, int N, int g, SeqLens sl) {
  typedef Mfma<T> M;
  constexpr int NS = D / M::KSTEP;
  const int r0 = blockIdx.x * 32;
  const int bh = blockIdx.y;
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int Npv = (sl.of(b, N) + g - 1) / g;   // pooled rows of this batch entry
  if (r0 >= Npv) return;
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
    const int r = min(r0 + n, Npv - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) qa[s] = load_frag(qb + (long)r * D + s * M::KSTEP + hh * M::KPL);
  }
  const int t_end = causal ? min(Npv, r0 + 32) : Npv;  // exclusive
  const int ntile = (t_end + 31) / 32;
  const float NEG = -__builtin_inff();
  float run[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) run[x] = NEG;

  for (int kt = 0; kt < ntile; ++kt) {
    const int t0 = kt * 32;
    const int t = t0 + n;  // this lane's key column
    const int tl = min(t, Npv - 1);
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
      if (t >= Npv || (causal && t > r)) s_ = NEG;
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
          const bool ok = r < Npv && j < nb && (!causal || j <= r / Rb);
          if (ok) Pb[(long)r * nb + j] = run[x];
        }
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) run[x] = NEG;
    }
  }
}

// bf16 variant.  A block max needs only the key tile that holds the block, so the work
// splits freely over key ranges.  A workgroup of four waves (32 pooled query rows each)
// owns 128 rows and a range of up to SC_CPW chunks of SC_CK pooled keys.  Its query
// rows and each key chunk, all contiguous in HBM, are copied into LDS with
// global_load_lds (every copy instruction reads one contiguous 1 KB run); key chunks
// alternate between two buffers so that the next one lands while the current one is
// multiplied.  16-byte chunks of each LDS row are XOR-swizzled by the row so that the
// MFMA operand reads hit distinct banks.  Block maxima are collected in LDS and
// written out as whole row segments.
constexpr int SC_CK = 64;                        // pooled keys per chunk (two 32-key tiles)
constexpr int SC_CPW = 16;                       // chunks per workgroup at most
typedef __attribute__((address_space(3))) void* lds_void_t;

template <int D>
__device__ __forceinline__ void stage_rows(const bf16_t* g, int rows_avail, bf16_t* lds, int nrows,
                                           int tid, int wave_base) {
  // nrows x D bf16 rows; source rows past rows_avail are clamped (their results are unused)
  constexpr int CPR = D / 8;
  for (int c0 = 0; c0 < nrows * CPR; c0 += 256) {
    const int chunk = c0 + tid;
    const int row = chunk / CPR;
    const int pos = chunk % CPR;
    const int col = pos ^ (row & (CPR - 1));
    const int src = min(row, rows_avail - 1);
    __builtin_amdgcn_global_load_lds((const void*)(g + (long)src * D + col * 8),
                                     (lds_void_t)(lds + (c0 + wave_base) * 8), 16, 0, 0);
  }
}

template <int D>
__global__ __launch_bounds__(256) void kap_score_bf16_kernel(const bf16_t* __restrict__ qp,
                                                             const bf16_t* __restrict__ kp,
                                                             float* __restrict__ P, int Hq,
                                                             int group, int Hkv, int Np, int nb,
                                                             int Rb, int causal, float scale,
                                                             int N, int g, SeqLens sl) {
  constexpr int NS = D / 16;
  constexpr int CPR = D / 8;
  const int lrb = __builtin_ctz(Rb);             // Rb is a power of two: divisions are shifts
  __shared__ __attribute__((aligned(1024))) bf16_t Qs[128 * D];
  __shared__ __attribute__((aligned(1024))) bf16_t Ks[2][SC_CK * D];
  extern __shared__ float Ps[];                  // [4 waves][32 rows][bpc blocks]
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int wave_base = __builtin_amdgcn_readfirstlane(tid & ~63);
  const int R0 = blockIdx.y * 128;               // first pooled query row of the workgroup
  const int C0 = blockIdx.x * SC_CPW;            // first chunk of the key range
  const int bh = blockIdx.z;
  const int b = bh / Hq;
  const int Npv = (sl.of(b, N) + g - 1) / g;                 // pooled rows of this batch entry
  if (R0 >= Npv) return;
  const int wg_end = causal ? min(Npv, R0 + 128) : Npv;      // keys the workgroup needs
  const int nchunk = min(SC_CPW, (wg_end - C0 * SC_CK + SC_CK - 1) / SC_CK);
  if (nchunk <= 0) return;
  const int h = bh - b * Hq;
  const int bkv = b * Hkv + h / group;
  const bf16_t* qb = qp + (long)bh * Np * D;
  const bf16_t* kb = kp + (long)bkv * Np * D;
  float* Pb = P + (long)bh * Np * nb;
  const int bpc = Rb <= SC_CK ? (SC_CK >> lrb) : 1;   // blocks per chunk (a power of two)
  const int lbpc = __builtin_ctz(bpc);
  float* Pw = Ps + wave * 32 * bpc;

  const int r0 = R0 + wave * 32;                 // this wave's rows
  const int t_end = causal ? min(Npv, r0 + 32) : Npv;
  const float NEG = -__builtin_inff();
  const int span = Rb < 32 ? Rb : 32;

  stage_rows<D>(qb + (long)R0 * D, Npv - R0, Qs, 128, tid, wave_base);
  stage_rows<D>(kb + (long)C0 * SC_CK * D, Npv - C0 * SC_CK, Ks[0], SC_CK, tid, wave_base);
  bf16x8 qa[NS];
  float run[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) run[x] = NEG;
  for (int c = 0; c < nchunk; ++c) {
    const int K0 = (C0 + c) * SC_CK;
    __builtin_amdgcn_s_waitcnt(0x0F70);          // this thread's copies of chunk c landed
    __syncthreads();                             // everyone's; buffer (c+1)&1 is free again
    if (c + 1 < nchunk)
      stage_rows<D>(kb + (long)(K0 + SC_CK) * D, Npv - K0 - SC_CK, Ks[(c + 1) & 1], SC_CK, tid, wave_base);
    if (c == 0) {
      const int row = wave * 32 + n;
      const bf16_t* qr = Qs + row * D;
#pragma unroll
      for (int s = 0; s < NS; ++s) qa[s] = load_frag(qr + (((2 * s + hh) ^ (row & (CPR - 1))) * 8));
    }
    const int kt_end = min(SC_CK / 32, (t_end - K0 + 31) / 32);   // key tiles this wave needs
    const bf16_t* kbuf = Ks[c & 1];
    for (int kt = 0; kt < kt_end; ++kt) {
      const int krow = kt * 32 + n;
      const bf16_t* kr = kbuf + krow * D;
      f32x16 acc0 = {}, acc1 = {};
#pragma unroll
      for (int s = 0; s < NS; s += 2) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], load_frag(kr + (((2 * s + hh) ^ (krow & (CPR - 1))) * 8)), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s + 1], load_frag(kr + (((2 * s + 2 + hh) ^ (krow & (CPR - 1))) * 8)), acc1, 0, 0, 0);
      }
      const int t0 = K0 + kt * 32;
      const int t = t0 + n;
      float v[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) v[x] = (acc0[x] + acc1[x]) * scale;   // C[row][key]
      if (t0 + 31 >= Npv || (causal && t0 + 31 > r0)) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int r = r0 + 8 * (x >> 2) + 4 * hh + (x & 3);
          if (t >= Npv || (causal && t > r)) v[x] = NEG;
        }
      }
      if (span >= 2) {
#pragma unroll
        for (int x = 0; x < 16; ++x)  // xor 1 inside each quad
          v[x] = fmaxf(v[x], __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[x]), 0xB1, 0xF, 0xF, true)));
      }
      if (span >= 4) {
#pragma unroll
        for (int x = 0; x < 16; ++x)  // xor 2 inside each quad
          v[x] = fmaxf(v[x], __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[x]), 0x4E, 0xF, 0xF, true)));
      }
      for (int off = 4; off < span; off <<= 1) {
#pragma unroll
        for (int x = 0; x < 16; ++x) v[x] = fmaxf(v[x], __shfl_xor(v[x], off, 64));
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) run[x] = fmaxf(run[x], v[x]);
      // a block spanning several key tiles ends on a multiple of Rb or at this wave's
      // causal limit; ranges start on multiples of SC_CPW * SC_CK, a multiple of Rb
      const bool block_done = Rb <= 32 || ((t0 + 32) & (Rb - 1)) == 0 || t0 + 32 >= t_end;
      if (block_done) {
        if ((n & (span - 1)) == 0) {
          const int jc = (t >> lrb) - (K0 >> lrb);
#pragma unroll
          for (int x = 0; x < 16; ++x) Pw[(8 * (x >> 2) + 4 * hh + (x & 3)) * bpc + jc] = run[x];
        }
#pragma unroll
        for (int x = 0; x < 16; ++x) run[x] = NEG;
      }
    }
    // flush this chunk's complete blocks: the wave's 32 rows x nbc blocks, row by row
    if (kt_end > 0 && (Rb <= SC_CK || ((K0 + SC_CK) & (Rb - 1)) == 0 || K0 + kt_end * 32 >= t_end)) {
      const int jlo = K0 >> lrb;
      const int jhi = Rb <= SC_CK ? ((min(K0 + kt_end * 32, t_end) + Rb - 1) >> lrb) : jlo + 1;
      __builtin_amdgcn_wave_barrier();
      for (int idx = lane; idx < 32 * bpc; idx += 64) {
        const int rl = idx >> lbpc;
        const int j = jlo + (idx & (bpc - 1));
        const int r = r0 + rl;
        if (j < jhi && r < Npv && j < nb && (!causal || j <= (r >> lrb))) Pb[(long)r * nb + j] = Pw[idx];
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

template <typename T>
static hipError_t launch_score_t(const ScoreLaunch& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    const int nchunks = (a.Np + SC_CK - 1) / SC_CK;
    dim3 g2((nchunks + SC_CPW - 1) / SC_CPW, (a.Np + 127) / 128, a.bh);
    const size_t lds = (size_t)4 * 32 * ((SC_CK + a.Rb - 1) / a.Rb) * sizeof(float);
    if (a.D == 128)
      hipLaunchKernelGGL((kap_score_bf16_kernel<128>), g2, dim3(256), lds, s, (const bf16_t*)a.qp,
                         (const bf16_t*)a.kp, a.P, a.Hq, a.group, a.Hkv, a.Np, a.nb, a.Rb,
                         a.causal, a.scale, a.N, a.g, a.sl);
    else
      hipLaunchKernelGGL((kap_score_bf16_kernel<64>), g2, dim3(256), lds, s, (const bf16_t*)a.qp,
                         (const bf16_t*)a.kp, a.P, a.Hq, a.group, a.Hkv, a.Np, a.nb, a.Rb,
                         a.causal, a.scale, a.N, a.g, a.sl);
    return hipGetLastError();
  }
  dim3 grid((a.Np + 31) / 32, a.bh);
  if (a.D == 128)
    hipLaunchKernelGGL((kap_score_kernel<T, 128>), grid, dim3(64), 0, s, (const T*)a.qp,
                       (const T*)a.kp, a.P, a.Hq, a.group, a.Hkv, a.Np, a.nb, a.Rb, a.causal,
                       a.scale, a.N, a.g, a.sl);
  else
    hipLaunchKernelGGL((kap_score_kernel<T, 64>), grid, dim3(64), 0, s, (const T*)a.qp,
                       (const T*)a.kp, a.P, a.Hq, a.group, a.Hkv, a.Np, a.nb, a.Rb, a.causal,
                       a.scale, a.N, a.g, a.sl);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreLaunch& a, hipStream_t s) {
  return a.bf16 ? launch_score_t<bf16_t>(a, s) : launch_score_t<float>(a, s);
}

}  // namespace cosa

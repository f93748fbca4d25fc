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
  const long ldp = p_pitch(nb);
  float* Pb = P + (long)bh * Np * ldp;

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
          if (ok) Pb[r * ldp + j] = run[x];
        }
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) run[x] = NEG;
    }
  }
}

// bf16 variant.  A block max needs only the key tile that holds the block, so the work
// splits freely over key ranges.  A workgroup of four waves (32 pooled query rows each)
// owns 128 rows and a range of up to SC_CPW chunks of SC_CK pooled keys.  Each wave reads
// its query rows into registers once; the key chunks, contiguous in HBM, are copied into
// LDS with global_load_lds (every copy instruction reads one contiguous 1 KB run) and
// alternate between two buffers so that the next one lands while the current one is
// multiplied.  16-byte chunks of each LDS row are XOR-swizzled by the row so that the
// MFMA operand reads hit distinct banks.
//
// The product is formed as C[key][row] = K~ Q~^T: lane (n, h) holds query row n and the
// keys 8i + 4h + j (i, j = 0..3) of each 32-key tile, so the maximum over RB <= 4
// consecutive keys is taken inside the lane, RB = 8 adds one exchange with lane n+32,
// larger blocks reduce further inside the lane and run across tiles.  The scale is
// applied to the block maxima: rounding a product with a positive scale preserves order,
// so max(scale * x) == scale * max(x) exactly.  Block maxima are collected in LDS (one
// buffer per wave, columns XOR-swizzled by the row, 40 KB per workgroup in all at D = 128
// and RB = 4: four workgroups per CU) and written out one chunk later as 16-byte pieces of
// row segments (all of a wave's LDS reads first, then its stores), so that the wait for
// the next chunk's copy finds the stores long issued.
constexpr int SC_CK = 64;                        // pooled keys per chunk (two 32-key tiles)
constexpr int SC_CPW = 16;                       // chunks per workgroup at most
typedef __attribute__((address_space(3))) bf16_t lds_bf16_t;

// One copy instruction: 16 bytes per lane from global memory to LDS at lds_base + 16 * lane.
// Written as inline assembly so that the compiler does not see it write LDS: its own
// tracking cannot tell the two key buffers apart and would wait for the next chunk's copy
// before every read of the current one.  The kernel waits for its copies itself
// (vmcnt(0) before the barrier that publishes a chunk).  M0 (the LDS destination) is a
// reserved register the compiler does not track through inline assembly; nothing else in
// these kernels uses it, and every copy sets it first.
__device__ __forceinline__ void copy16_to_lds(const bf16_t* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory");
}


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
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_bf16_t*)(lds + (c0 + wave_base) * 8));
    copy16_to_lds(g + (long)src * D + col * 8, la);
  }
}

constexpr int sc_bpc(int rb) { return rb <= SC_CK ? SC_CK / rb : 1; }   // blocks per chunk

template <int V>
struct IntC {
  static constexpr int value = V;
};

template <int D, int RB>
__global__ __launch_bounds__(256) void kap_score_bf16_kernel(const bf16_t* __restrict__ qp,
                                                             const bf16_t* __restrict__ kp,
                                                             float* __restrict__ P, int Hq,
                                                             int group, int Hkv, int Np, int nb,
                                                             int causal, float scale,
                                                             int N, int g, SeqLens sl) {
  constexpr int NS = D / 16;
  constexpr int CPR = D / 8;
  constexpr int LRB = __builtin_ctz(RB);
  constexpr int BPC = sc_bpc(RB);
  constexpr int SWM = (BPC < 16 ? BPC : 16) - 1;  // column swizzle of the staged maxima
  constexpr int LBPC = __builtin_ctz(BPC);
  constexpr int RSTEP = 64 / BPC;                // rows one store instruction covers in a flush
  __shared__ __attribute__((aligned(1024))) bf16_t Ks[2][SC_CK * D];
  __shared__ float Ps[4 * 32 * BPC];             // [4 waves][32 rows][BPC], swizzled
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
  const long ldp = p_pitch(nb);
  float* Pb = P + (long)bh * Np * ldp;

  const int r0 = R0 + wave * 32;                 // this wave's rows
  const int r = r0 + n;                          // this lane's row
  const int t_end = causal ? min(Npv, r0 + 32) : Npv;
  const float NEG = -__builtin_inff();

  stage_rows<D>(kb + (long)C0 * SC_CK * D, Npv - C0 * SC_CK, Ks[0], SC_CK, tid, wave_base);
  bf16x8 qa[NS];                                 // B operand: pooled query row r (clamped)
  {
    const bf16_t* qr = qb + (long)min(r, Npv - 1) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) qa[s] = load_frag(qr + (2 * s + hh) * 8);
  }
  // A operand offsets inside a chunk buffer: key row n of each 32-key tile, 16-byte chunk
  // 2s + h, swizzled by the row (the same for every tile since 32 is a multiple of CPR)
  int koff[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) koff[s] = n * D + (((2 * s + hh) ^ (n & (CPR - 1))) * 8);
  // flush geometry: lane covers block jlo + fj of rows fr, fr + RSTEP, ... of the wave
  const int fj = lane & (BPC - 1);
  const int fr = lane >> LBPC;
  // staged maxima of a wave: row r, block c at r * BPC + (c ^ ((r >> 1) & SWM)); at BPC = 16 the
  // 64 lanes of one write (rows n = 0..31, blocks c and c + 1) then fall on distinct banks
  // (the odd rows sit 16 banks over the even ones), without padding
  auto pidx = [](int row, int col) { return row * BPC + (col ^ ((row >> 1) & SWM)); };

  bool pend = false;                             // the previous chunk's block maxima to write
  int pjlo = 0, pjhi = 0;
  auto flush = [&](const float* Pw, int jlo, int jhi) {
    __builtin_amdgcn_wave_barrier();
    if constexpr (BPC >= 4) {
      // 16-byte pieces of four consecutive blocks of one row, every LDS read issued before
      // the first store.  A piece that starts below jhi is stored whole: its blocks at or
      // past jhi (and those above a row's diagonal block) are never read, and the padded
      // pitch keeps them inside the row.
      constexpr int PPR = BPC / 4;               // pieces per row
      constexpr int NPL = (32 * PPR + 63) / 64;  // pieces per lane
      float4 pv[NPL];
#pragma unroll
      for (int it = 0; it < NPL; ++it) {
        const int pc = lane + 64 * it;
        const int row = (pc / PPR) & 31, c0 = 4 * (pc % PPR);
        pv[it] = make_float4(Pw[pidx(row, c0)], Pw[pidx(row, c0 + 1)], Pw[pidx(row, c0 + 2)],
                             Pw[pidx(row, c0 + 3)]);
      }
#pragma unroll
      for (int it = 0; it < NPL; ++it) {
        const int pc = lane + 64 * it;
        const int rr = r0 + pc / PPR;
        const int j = jlo + 4 * (pc % PPR);
        if (pc < 32 * PPR && rr < Npv && j < jhi) *(float4*)(Pb + rr * ldp + j) = pv[it];
      }
    } else {
      const int j = jlo + fj;
      if (j < jhi && j < nb) {
        for (int rl = fr; rl < 32; rl += RSTEP) {
          const int rr = r0 + rl;
          if (rr < Npv && (!causal || j <= (rr >> LRB))) Pb[rr * ldp + j] = Pw[pidx(rl, fj)];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  float run = NEG;                               // blocks spanning several tiles (RB > 32)
  // one chunk; the buffer index is a template constant so that every LDS address is an
  // immediate offset from the lane's base
  auto chunk = [&](int c, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int K0 = (C0 + c) * SC_CK;
    __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): this thread's copies of chunk c landed
    __syncthreads();                             // everyone's; the other buffer is free again
    if (c + 1 < nchunk)
      stage_rows<D>(kb + (long)(K0 + SC_CK) * D, Npv - K0 - SC_CK, Ks[BUF ^ 1], SC_CK, tid, wave_base);
    // the previous chunk's maxima are read (in program order, so before this chunk's
    // writes to the same LDS rows: one wave's LDS operations execute in order)
    if (pend) flush(Ps + wave * 32 * BPC, pjlo, pjhi);
    float* Pw = Ps + wave * 32 * BPC;
    const int kt_end = min(SC_CK / 32, (t_end - K0 + 31) / 32);   // key tiles this wave needs
#pragma unroll
    for (int kt = 0; kt < SC_CK / 32; ++kt) {
      if (kt >= kt_end) break;
      const bf16_t* kbuf = Ks[BUF] + kt * 32 * D;
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_frag(kbuf + koff[s]), qa[s], acc, 0, 0, 0);
      const int t0 = K0 + kt * 32;
      // keys past the end or above the diagonal (tiles that reach them only): a loop of 0
      // or 1 trips with an opaque limit keeps the compares off the other tiles
      for (int once = (t0 + 31 >= Npv || (causal && t0 + 31 > r0)) ? 1 : 0; once > 0; --once) {
        int lim = min(Npv - 1, causal ? r : Npv - 1) - t0 - 4 * hh;   // last key offset kept
        asm volatile("" : "+v"(lim));
#pragma unroll
        for (int x = 0; x < 16; ++x)
          if (8 * (x >> 2) + (x & 3) > lim) acc[x] = NEG;
      }
      const int jc0 = (t0 - K0) >> LRB;          // first block of this tile in the chunk
      if constexpr (RB == 1) {
#pragma unroll
        for (int x = 0; x < 16; ++x) Pw[pidx(n, jc0 + 8 * (x >> 2) + 4 * hh + (x & 3))] = acc[x] * scale;
      } else if constexpr (RB == 2) {
#pragma unroll
        for (int y = 0; y < 8; ++y)
          Pw[pidx(n, jc0 + 4 * (y >> 1) + 2 * hh + (y & 1))] = fmaxf(acc[2 * y], acc[2 * y + 1]) * scale;
      } else {
        float q[4];                              // maxima over each group of 4 keys
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = fmaxf(fmaxf(acc[4 * i], acc[4 * i + 1]), fmaxf(acc[4 * i + 2], acc[4 * i + 3]));
        if constexpr (RB == 4) {
#pragma unroll
          for (int i = 0; i < 4; ++i) Pw[pidx(n, jc0 + 2 * i + hh)] = q[i] * scale;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) q[i] = fmaxf(q[i], __shfl_xor(q[i], 32, 64));   // keys 8i .. 8i+7
          if constexpr (RB == 8) {
            if (hh == 0) {
#pragma unroll
              for (int i = 0; i < 4; ++i) Pw[pidx(n, jc0 + i)] = q[i] * scale;
            }
          } else if constexpr (RB == 16) {
            if (hh == 0) {
              Pw[pidx(n, jc0)] = fmaxf(q[0], q[1]) * scale;
              Pw[pidx(n, jc0 + 1)] = fmaxf(q[2], q[3]) * scale;
            }
          } else {
            run = fmaxf(run, fmaxf(fmaxf(q[0], q[1]), fmaxf(q[2], q[3])));
            // a block spanning several key tiles ends on a multiple of RB or at this wave's
            // causal limit; ranges start on multiples of SC_CPW * SC_CK, a multiple of RB
            const bool block_done = RB <= 32 || ((t0 + 32) & (RB - 1)) == 0 || t0 + 32 >= t_end;
            if (block_done) {
              if (hh == 0) Pw[pidx(n, jc0)] = run * scale;
              run = NEG;
            }
          }
        }
      }
    }
    // this chunk's complete blocks, written at the next chunk (or after the last)
    pend = kt_end > 0 && (RB <= SC_CK || ((K0 + SC_CK) & (RB - 1)) == 0 || K0 + kt_end * 32 >= t_end);
    if (pend) {
      pjlo = K0 >> LRB;
      pjhi = RB <= SC_CK ? ((min(K0 + kt_end * 32, t_end) + RB - 1) >> LRB) : pjlo + 1;
    }
  };
  for (int c = 0; c < nchunk; c += 2) {
    chunk(c, IntC<0>{});
    if (c + 1 < nchunk) chunk(c + 1, IntC<1>{});
  }
  if (pend) flush(Ps + wave * 32 * BPC, pjlo, pjhi);
}

template <int D>
static hipError_t launch_score_bf16(const ScoreLaunch& a, hipStream_t s) {
  const int nchunks = (a.Np + SC_CK - 1) / SC_CK;
  dim3 g2((nchunks + SC_CPW - 1) / SC_CPW, (a.Np + 127) / 128, a.bh);
  const bf16_t* qp = (const bf16_t*)a.qp;
  const bf16_t* kp = (const bf16_t*)a.kp;
#define COSA_SCORE_CASE(RBV)                                                                     \
  case RBV:                                                                                      \
    hipLaunchKernelGGL((kap_score_bf16_kernel<D, RBV>), g2, dim3(256), 0, s, qp, kp, a.P, a.Hq,    \
                       a.group, a.Hkv, a.Np, a.nb, a.causal, a.scale, a.N, a.g, a.sl);            \
    break;
  switch (a.Rb) {
    COSA_SCORE_CASE(1)
    COSA_SCORE_CASE(2)
    COSA_SCORE_CASE(4)
    COSA_SCORE_CASE(8)
    COSA_SCORE_CASE(16)
    COSA_SCORE_CASE(32)
    COSA_SCORE_CASE(64)
    COSA_SCORE_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef COSA_SCORE_CASE
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_score_t(const ScoreLaunch& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    return a.D == 128 ? launch_score_bf16<128>(a, s) : launch_score_bf16<64>(a, s);
  } else {
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
}

hipError_t launch_score(const ScoreLaunch& a, hipStream_t s) {
  return a.bf16 ? launch_score_t<bf16_t>(a, s) : launch_score_t<float>(a, s);
}

}  // namespace cosa

// OSK: ordered block-sparse flash attention with in-kernel skipping, and the dense
// causal baseline built from the same tile machinery.
//
// CoSA technical summary (gist.science, pt), section 2.3 "Ordered-Skipping Kernel":
// blocks the proxy did not select are never touched (the visit list is the
// remapped page table); a listed block whose local maximum is negligible against
// the running online-softmax statistics is skipped inside the kernel; the others
// are computed.  Section 2.1: online-softmax accumulation does not depend on the
// order in which key blocks are visited, so the list order is free.  The authors'
// abstract: the kernel skips more blocks under a tightened budget.
//
// Readings fixed here: the skip test (MAXDIFF or MASS, every row of the query block
// must pass, first computed block never tested), skipped blocks leave m, l and the
// accumulator unchanged, and the tightened budget caps the computed (or visited)
// blocks at k'_i = min(k_i, max(1, ceil(rho' * n_i))).
//
// Work decomposition: one workgroup per (batch, query head, query block i) with
// BLK/32 waves; wave w owns query rows 32w .. 32w+31.  Per visited block the K tile
// (row-major) and the V tile (transposed) are staged in LDS; each wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so that lane (n, h) holds 16 keys of
// query row n per 32-key subtile.  Row statistics then need one lane exchange
// (lane ^ 32), the probabilities feed O^T += V^T P^T as the B operand straight from
// registers (the contraction index is permuted identically on both operands), and
// each lane's O^T accumulator belongs to a single query row.
//
// Ragged sequences (block does not divide the length L of a batch entry, which is N
// or its own length in a varlen batch): the last block holds L - (nb_L-1)*BLK rows.  Keys past the end are masked like causally hidden ones; query rows past the
// end are computed as copies of the last real row (same logits, same mask, hence the
// same skip vote, so the block's decision is that of its real rows) and not stored.
// Loads past the end read zeros (buffer range) or the last real row (clamped index).
// Query blocks past the end of their entry do no work.
//
// Launch order: query blocks heaviest first (i descending); the G query heads that
// share a KV head at the same i run back to back on one XCD (workgroups are dealt
// round-robin over the 8 XCDs), so their overlapping K/V pages hit that XCD's L2.
#include "attn_tiles.hpp"
#include "cosa_common.hpp"
#include "cosa_launch.hpp"

namespace cosa {

template <typename T, int BLK, int D>
struct AttnTile {
  static constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16 bytes
  static constexpr int KP = D + EPC;                // K row pitch (16-byte pad)
  static constexpr int VP = BLK + 4;                // V^T row pitch
  static constexpr int NW = BLK / 32;
  static constexpr int NT = NW * 64;
};

template <typename T, int BLK, int D>  // fp32 tiles
__device__ __forceinline__ void stage_tile(const T* __restrict__ Kg, const T* __restrict__ Vg,
                                           T* Ks, T* Vt, int tid, int valid) {
  // rows past `valid` (the end of a ragged sequence) repeat the last real row; their
  // logits are masked
  typedef AttnTile<T, BLK, D> TT;
  constexpr int EPC = TT::EPC;
  constexpr int CPR = D / EPC;  // 16-byte chunks per row
#pragma unroll
  for (int c = tid; c < BLK * CPR; c += TT::NT) {
    const int row = c / CPR;
    const int ch = c - row * CPR;
    *reinterpret_cast<u32x4*>(Ks + row * TT::KP + ch * EPC) =
        *reinterpret_cast<const u32x4*>(Kg + (long)min(row, valid - 1) * D + ch * EPC);
  }
  // V: each item is 4 consecutive keys x one 16-byte chunk, written transposed.
#pragma unroll
  for (int c = tid; c < (BLK / 4) * CPR; c += TT::NT) {
    const int qd = c / CPR;
    const int ch = c - qd * CPR;
    u32x4 r[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      r[rr] = *reinterpret_cast<const u32x4*>(Vg + (long)min(4 * qd + rr, valid - 1) * D + ch * EPC);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32x4 o;
      o[0] = r[0][e];
      o[1] = r[1][e];
      o[2] = r[2][e];
      o[3] = r[3][e];
      *reinterpret_cast<u32x4*>(Vt + (ch * 4 + e) * TT::VP + 4 * qd) = o;
    }
  }
}

// fp32 inputs: register-staged tiles (V written transposed) and v_mfma_f32_32x32x2_f32.
template <typename T, int BLK, int D, bool SPARSE>
__global__ __launch_bounds__(BLK * 2) void attn_kernel(AttnLaunch a) {
  static_assert(sizeof(T) == 4, "the fp32 tile loop");
  typedef AttnTile<T, BLK, D> TT;
  typedef Mfma<T> M;
  constexpr int NS = D / M::KSTEP;   // k-steps of Q.K^T
  constexpr int NKT = BLK / 32;      // 32-key subtiles per block
  constexpr int NDT = D / 32;        // 32-dim subtiles of the output
  __shared__ __attribute__((aligned(16))) T Ks[BLK * TT::KP];
  __shared__ __attribute__((aligned(16))) T Vt[D * TT::VP];
  __shared__ int vote[TT::NW];

  // ---- unit of work (XCD-aware, heaviest first)
  const int G = a.group;
  const int wg = blockIdx.x;
  const int xcd = wg & 7;
  const int slot = wg >> 3;
  const int ag = slot / G;
  const int gm = slot - ag * G;
  const long grp = (long)ag * 8 + xcd;
  const long bhk = (long)a.Bt * a.Hkv;
  if (grp >= bhk * a.nb) return;
  const int i = a.nb - 1 - (int)(grp / bhk);
  const int rem = (int)(grp % bhk);
  const int b = rem / a.Hkv;
  const int kvh = rem - b * a.Hkv;
  const int h = kvh * G + gm;
  const long bh = (long)b * a.Hq + h;
  const long bkv = (long)b * a.Hkv + kvh;
  const long unit = bh * a.nb + i;

  const int tid = threadIdx.x;
  const int Lb = a.sl.of(b, a.N);                    // tokens of this batch entry
  const int nbv = (Lb + BLK - 1) / BLK;              // its blocks
  if (i >= nbv) {                                    // past the end of the entry: no work
    if (SPARSE && a.visit_status)
      for (int pp = tid; pp < a.kmax; pp += TT::NT) a.visit_status[unit * a.kmax + pp] = 0;
    if (SPARSE && a.tile_counts && tid == 0) a.tile_counts[unit * 2] = a.tile_counts[unit * 2 + 1] = 0;
    return;
  }
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int rloc = wave * 32 + n;  // query row inside the block
  const int rows_valid = min(BLK, Lb - i * BLK);
  const int rq = min(rloc, rows_valid - 1);          // rows past the end copy the last one
  const int nvk = Lb - (nbv - 1) * BLK;              // keys in the last block
  const T* Qg = (const T*)a.q + (bh * a.N + (long)i * BLK + rq) * D;
  const T* Kb = (const T*)a.k + bkv * a.N * D;
  const T* Vb = (const T*)a.v + bkv * a.N * D;

  typename M::frag qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qf[s] = load_frag(Qg + s * M::KSTEP + hh * M::KPL);

  const float NEG = -__builtin_inff();
  float m = NEG;    // running max, log2 units
  float l = 0.0f;   // running denominator
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};

  const int ncand = a.causal ? i + 1 : nbv;
  const long lunit = (a.shared_lists ? bkv : bh) * a.nb + i;   // the list this head walks
  int kl = ncand, kprime = ncand;
  if constexpr (SPARSE) {
    kl = a.visit_cnt[lunit];
    kl = kl < 0 ? 0 : (kl > a.kmax ? a.kmax : kl);
    const int kb = (int)fmin((double)ncand, fmax(1.0, ceil(a.tight_budget * (double)ncand)));
    kprime = kl < kb ? kl : kb;
  }
  const int32_t* lst = SPARSE ? a.visit_idx + lunit * a.kmax : nullptr;
  uint8_t* st = (SPARSE && a.visit_status) ? a.visit_status + unit * a.kmax : nullptr;
  int ncomp = 0, nvis = 0;
  int p = 0;
  for (; p < kl; ++p) {
    if constexpr (SPARSE) {
      if (a.cap_mode == 0 ? (ncomp == kprime) : (p == kprime)) break;
    }
    int j = p, phys = p;
    if constexpr (SPARSE) {
      j = lst[p];
      if (j < 0 || j >= ncand) break;
      phys = a.page_table ? a.page_table[(long)b * a.nb + j] : j;
      if (phys < 0 || phys >= a.nb) break;
    }
    const bool tail = j == nbv - 1 && nvk < BLK;    // partial last block (never paged)
    stage_tile<T, BLK, D>(Kb + (long)phys * BLK * D, Vb + (long)phys * BLK * D, Ks, Vt, tid,
                          tail ? nvk : BLK);
    __syncthreads();

    // ---- S^T = K Q^T for this wave's 32 rows
    f32x16 sacc[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      sacc[kt] = f32x16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        typename M::frag kf = load_frag(Ks + (32 * kt + n) * TT::KP + s * M::KSTEP + hh * M::KPL);
        sacc[kt] = M::mma(kf, qf[s], sacc[kt]);
      }
    }
    const bool diag = a.causal && j == i;
    const int lim = min(diag ? rq : BLK - 1, tail ? nvk - 1 : BLK - 1);   // last visible key
    float mloc = NEG;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        float v = sacc[kt][x] * a.scale_log2;
        const int key = 32 * kt + 8 * (x >> 2) + 4 * hh + (x & 3);
        if (key > lim) v = NEG;
        sacc[kt][x] = v;
        mloc = fmaxf(mloc, v);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    ++nvis;

    bool skip = false;
    if constexpr (SPARSE) {
      if (a.skip_mode != 0 && ncomp > 0) {
        float stat = mloc - m;
        if (a.skip_mode == 2) {
          stat += __log2f((float)(lim + 1)) - __log2f(l);
        }
        const bool pass = stat <= a.skip_thr_log2;
        const unsigned long long bal = __ballot(pass);
        if (lane == 0) vote[wave] = (bal == ~0ull) ? 1 : 0;
        __syncthreads();
        int all = 1;
#pragma unroll
        for (int w = 0; w < TT::NW; ++w) all &= vote[w];
        skip = all != 0;
      }
    }
    if (skip) {
      if (st && tid == 0) st[p] = 2;
      __syncthreads();
      continue;
    }

    // ---- online softmax update
    const float mnew = fmaxf(m, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    float rs = 0.0f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const float pv = __builtin_amdgcn_exp2f(sacc[kt][x] - mnew);
        sacc[kt][x] = pv;
        rs += pv;
      }
    }
    rs += __shfl_xor(rs, 32, 64);
    l = alpha * l + rs;
    m = mnew;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;

    // ---- O^T += V^T P^T (fp32 MFMA 32x32x2: one key per step)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const T* vrow = Vt + (32 * dt + n) * TT::VP + 4 * hh;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int key = 32 * kt + 8 * (x >> 2) + (x & 3);
          oacc[dt] = M::mma(load_frag(vrow + key), sacc[kt][x], oacc[dt]);
        }
      }
    }
    ++ncomp;
    if (st && tid == 0) st[p] = 1;
    __syncthreads();
  }

  // ---- epilogue
  if (st) {
    for (int pp = p + tid; pp < a.kmax; pp += TT::NT) st[pp] = 0;
  }
  if (SPARSE && a.tile_counts && tid == 0) {
    a.tile_counts[unit * 2] = nvis;
    a.tile_counts[unit * 2 + 1] = ncomp;
  }
  const float linv = ncomp > 0 ? 1.0f / l : 0.0f;
  T* Og = (T*)a.out + (bh * a.N + (long)i * BLK + rloc) * D;
  if (rloc >= rows_valid) return;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d0 = 32 * dt + 8 * ii + 4 * hh;
      f32x4 o;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) o[jj] = oacc[dt][4 * ii + jj] * linv;
      *reinterpret_cast<f32x4*>(Og + d0) = o;
    }
  }
  if (a.lse && hh == 0) {
    a.lse[bh * a.N + (long)i * BLK + rloc] = ncomp > 0 ? (m + __log2f(l)) * LN2 : NEG;
  }
}

// ---------------------------------------------------------------------------
// bf16 tile loop for gfx950 (tile copies, swizzles and the transposed V read are in
// attn_tiles.hpp).  One K buffer and one V buffer: the next K tile is fetched while
// the current one is turned into probabilities and multiplied with V, and the next
// V tile while the next Q.K^T runs, so the copies overlap the math with two barriers
// per tile.
//
// MODE 0: dense; 1: sparse walk, block vote; 2: sparse walk, one vote per 32-row group;
// 3: sparse walk of a list shared by the query heads of a KV head, HP of those heads per
// workgroup (eight waves), so that each K/V tile copied into LDS serves HP query blocks
// (launched for block 64: four heads per workgroup).
// Every head keeps its own softmax state, block vote and computed-tile cap: a head that
// reached its cap idles while the walk goes on for the others.
template <int BLK, int D, int MODE>
__global__ __launch_bounds__(MODE == 3 ? 512 : BLK * 2, MODE == 3 ? 1 : 2) void attn2_kernel(AttnLaunch a) {
  constexpr bool SPARSE = MODE > 0;
  constexpr bool GROUPV = MODE == 2;
  constexpr bool MULTI = MODE == 3;
  constexpr bool DEFERV = MODE == 1;          // V copies deferred after a skipped tile
  constexpr int NWH = BLK / 32;               // waves per query block (32 rows each)
  constexpr int HP = MULTI ? 8 / NWH : 1;     // query heads per workgroup
  constexpr int NWT = NWH * HP;               // waves per workgroup
  typedef Tile2<BLK, D, NWT * 64> TT;
  constexpr int NS = D / 16;
  constexpr int NKT = BLK / 32;
  constexpr int NDT = D / 32;
  __shared__ __attribute__((aligned(1024))) bf16_t Ks[BLK * D];
  __shared__ __attribute__((aligned(1024))) bf16_t Vs[BLK * D];
  __shared__ int vote[NWT];
  // Sparse walks stage their list in LDS, translated to physical pages, so that the
  // loop touches no global memory but the tiles.
  __shared__ uint16_t pages[SPARSE ? COSA_MAX_NB : 1];

  const int G = a.group;
  const int GP = MULTI ? (G + HP - 1) / HP : G;   // workgroups per (KV head, query block)
  const int wg = blockIdx.x;
  const int xcd = wg & 7;
  const int slot = wg >> 3;
  const int ag = slot / GP;
  const int gm = slot - ag * GP;
  const long grp = (long)ag * 8 + xcd;
  const long bhk = (long)a.Bt * a.Hkv;
  if (grp >= bhk * a.nb) return;
  const int i = a.nb - 1 - (int)(grp / bhk);
  const int rem = (int)(grp % bhk);
  const int b = rem / a.Hkv;
  const int kvh = rem - b * a.Hkv;

  const int tid = threadIdx.x;
  // (several heads: the wave's index and all that follows from it held in scalar registers)
  const int wave = MULTI ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int hp = MULTI ? wave / NWH : 0;          // head of this wave inside the workgroup
  const int rwave = wave - hp * NWH;              // its 32-row group inside the query block
  const int htid = tid - hp * NWH * 64;           // thread index inside the head's waves
  const int hg = MULTI ? gm * HP + hp : gm;       // head inside the KV group
  const bool head_ok = !MULTI || hg < G;          // (the last workgroup of an odd group)
  const int h = kvh * G + (head_ok ? hg : G - 1);
  const long bh = (long)b * a.Hq + h;
  const long bkv = (long)b * a.Hkv + kvh;
  const long unit = bh * a.nb + i;
  const int rloc = rwave * 32 + n;
  const int Lb = a.sl.of(b, a.N);                    // tokens of this batch entry
  const int nbv = (Lb + BLK - 1) / BLK;              // its blocks
  if (i >= nbv) {                                    // past the end of the entry: no work
    if (!head_ok) return;
    if (SPARSE && a.visit_status)
      for (int pp = htid; pp < a.kmax; pp += NWH * 64) a.visit_status[unit * a.kmax + pp] = 0;
    if (SPARSE && a.tile_counts && htid == 0) a.tile_counts[unit * 2] = a.tile_counts[unit * 2 + 1] = 0;
    return;
  }
  const int rows_valid = min(BLK, Lb - i * BLK);     // real query rows of this block
  const int rq = min(rloc, rows_valid - 1);          // rows past the end copy the last one
  const int nvk = Lb - (nbv - 1) * BLK;              // keys in the last block
  const int tail_bit = nvk < BLK ? TAIL_BIT : 0;
  const int wave_base = __builtin_amdgcn_readfirstlane(tid & ~63);  // scalar: copy slab of this wave
  // one descriptor per KV head (a head is at most 4096 blocks x 32 KB < 2^32 bytes); its
  // range ends with the entry's tokens, so rows past them read as zeros.  With a page table
  // the pages may sit anywhere in the head's N rows (always whole blocks), so it covers them.
  const uint32_t kv_bytes = (uint32_t)((a.page_table ? a.N : Lb) * D * 2);
  const i32x4 krs = make_rsrc((const bf16_t*)a.k + bkv * a.N * D, kv_bytes);
  const i32x4 vrs = make_rsrc((const bf16_t*)a.v + bkv * a.N * D, kv_bytes);
  constexpr int TILE_BYTES = BLK * D * 2;

  const int ncand = a.causal ? i + 1 : nbv;
  int kl = ncand, kprime = ncand;
  int ph = -1;  // encoded position being processed
  if constexpr (SPARSE) {
    const long lunit = (a.shared_lists ? bkv : bh) * a.nb + i;   // the list this head walks
    kl = a.visit_cnt[lunit];
    kl = kl < 0 ? 0 : (kl > a.kmax ? a.kmax : kl);
    const int kb = (int)fmin((double)ncand, fmax(1.0, ceil(a.tight_budget * (double)ncand)));
    kprime = kl < kb ? kl : kb;
    const int32_t* lst = a.visit_idx + lunit * a.kmax;
    const int32_t* pt = a.page_table ? a.page_table + (long)b * a.nb : nullptr;
    auto encode = [&](int jq) -> int {
      const int pq = (jq >= 0 && jq < ncand) ? (pt ? pt[jq] : jq) : -1;
      return (pq >= 0 && pq < a.nb)
                 ? (pq | (jq == i ? DIAG_BIT : 0) | (jq == nbv - 1 ? tail_bit : 0))
                 : STOP;
    };
    for (int q = tid; q < kl; q += TT::NT) pages[q] = (uint16_t)encode(lst[q]);
    if (kl > 0 && kprime > 0) {
      const int e0 = encode(lst[0]);
      ph = e0 == STOP ? -1 : e0;
    }
  } else {
    ph = kl > 0 ? ((i == 0 ? DIAG_BIT : 0) | (nbv == 1 ? tail_bit : 0)) : -1;
  }

  const float NEG = -__builtin_inff();
  float m = NEG, l = 0.0f;
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
  int ncomp = 0, nvis = 0, p = 0;
  bf16x8 qf[NS];
  {
    const bf16_t* Qg = (const bf16_t*)a.q + (bh * a.N + (long)i * BLK + rq) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = load_frag(Qg + s * 16 + hh * 8);
  }
  if (ph >= 0) {
    issue_tile<BLK, D, false, TT::NT>(krs, (ph & PAGE_MASK) * TILE_BYTES, Ks, tid, wave_base);
    issue_tile<BLK, D, true, TT::NT>(vrs, (ph & PAGE_MASK) * TILE_BYTES, Vs, tid, wave_base);
  }
  wait_copies();
  __syncthreads();

  bool hdone = !head_ok;   // this wave's head takes no part in the rest of the walk
  int p_end = -1;          // the position where its computed-tile cap ended its walk
  // Block vote: after a skipped tile the next tile's V is not copied ahead (skips come in runs,
  // and a skipped tile needs no V); it is copied once the vote says the tile is computed.
  bool vdefer = false;
  while (ph >= 0) {
    // ---- S^T = K Q^T.  Fragment reads run PFK MFMAs ahead of their use; scheduling
    // barriers keep that order (left alone, the scheduler pulls each read down to just
    // before its MFMA and exposes the LDS latency every other MFMA).
    f32x16 sacc[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) sacc[kt] = f32x16{};
    {   // (a head past its cap still forms S here; skipping it costs more registers)
      const bf16_t* kbase = Ks + n * D;
      const int sw = swz_k<D>(n);  // the same for row n of every 32-key subtile
      auto kfrag = [&](int idx) {
        const int kt = idx / NS, s = idx % NS;
        return load_frag(kbase + kt * 32 * D + (((2 * s + hh) ^ sw) * 8));
      };
      // the four subtile accumulators take turns, so consecutive MFMAs are independent
      auto kfrag_i = [&](int idx) { return kfrag((idx % NKT) * NS + idx / NKT); };
      constexpr int PFK = 3;
      bf16x8 kf[PFK];
#pragma unroll
      for (int u = 0; u < PFK; ++u) kf[u] = kfrag_i(u);
#pragma unroll
      for (int idx = 0; idx < NKT * NS; ++idx) {
        const bf16x8 kcur = kf[idx % PFK];
        if (idx + PFK < NKT * NS) kf[idx % PFK] = kfrag_i(idx + PFK);
        __builtin_amdgcn_sched_barrier(0);
        sacc[idx % NKT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur, qf[idx / NKT], sacc[idx % NKT], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const bool diag = a.causal && (ph & DIAG_BIT);
    const bool tail = (ph & TAIL_BIT) != 0;
    const int last_key = min(diag ? rq : BLK - 1, tail ? nvk - 1 : BLK - 1);  // last visible key
    // a loop of 0 or 1 trips keeps the mask off the other tiles (no if-conversion);
    // the lane's limit is made opaque so that the 64 compares are not hoisted out of
    // the tile loop into 64 live scalar masks
    for (int once = (diag || tail) ? 1 : 0; once > 0; --once) {
      int lim = last_key - 4 * hh;  // slot key offset 32kt + 8(x/4) + (x%4) must not exceed it
      asm volatile("" : "+v"(lim));
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int x = 0; x < 16; ++x)
          if (32 * kt + 8 * (x >> 2) + (x & 3) > lim) sacc[kt][x] = NEG;
    }
    float mq[4] = {NEG, NEG, NEG, NEG};   // four independent chains instead of one
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int x = 0; x < 16; ++x) mq[x & 3] = fmaxf(mq[x & 3], sacc[kt][x]);
    const float mraw = halves_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3])));
    const float mloc = mraw * a.scale_log2;
    nvis += hdone ? 0 : 1;

    // decision code of this wave for this tile: 1 compute, 2 skip, 0 idle (with the
    // per-group vote, a group that reached its cap leaves later tiles to the others)
    int code = 1;
    bool pass = false;   // every row of this wave passes the skip test
    if constexpr (SPARSE) {
      // a row group wholly past the end of the sequence takes no part
      const bool live = !GROUPV || wave * 32 < rows_valid;
      const bool active = live && !(GROUPV && a.cap_mode == 0 && ncomp == kprime);
      if (a.skip_mode != 0 && ncomp > 0 && !hdone) {
        float stat = mloc - m;
        if (a.skip_mode == 2) {
          stat += __log2f((float)(last_key + 1)) - __log2f(l);   // log of the visible keys
        }
        pass = __ballot(stat <= a.skip_thr_log2) == ~0ull;
      }
      if (MULTI) {
        if (lane == 0)
          vote[wave] = (pass ? 1 : 0) | (hdone ? 2 : 0) | (a.skip_mode != 0 && ncomp > 0 ? 4 : 0) | (ncomp << 3);
      } else if (GROUPV) {
        code = !active ? 0 : (pass ? 2 : 1);
        if (lane == 0) vote[wave] = code | ((live ? ncomp + (code == 1 ? 1 : 0) : kprime) << 2);
      } else if (a.skip_mode != 0 && ncomp > 0) {
        if (lane == 0) vote[wave] = pass ? 1 : 0;
      }
    }
    // the staged list entry of the next position, read before the barrier so that its LDS
    // latency hides behind it (the list does not change during the walk)
    const int pn = p + 1;
    int e_next = STOP;
    if constexpr (SPARSE) {
      if (pn < kl) e_next = pages[pn];
    }
    wait_copies();      // V of this tile has landed
    __syncthreads();    // B1: votes visible, K buffer free, V tile visible
    int st_byte = 1;    // status of this position (per-group vote: 2 bits per group)
    bool all_capped = false;
    // Block vote: the block skips only if every wave's rows pass, so a wave with a failing
    // row knows the tile is computed without reading the others' votes; only a wave whose
    // rows all pass waits for the LDS round trip after B1 (and then a skip is likely, so
    // nothing is formed ahead of the decision).
    const bool voted = SPARSE && !GROUPV && a.skip_mode != 0 && ncomp > 0 && pass;
    int vw[NWH];   // the votes of this wave's head
    if constexpr (SPARSE) {
      if (GROUPV) {
        st_byte = 0;
        bool done = true;
#pragma unroll
        for (int w = 0; w < TT::NW; ++w) {
          const int v = vote[w];
          st_byte |= (v & 3) << (2 * w);
          done &= (v >> 2) == kprime;
        }
        all_capped = done;
      } else if (voted) {
        int z = 0;   // a lane-varying zero: uniform loads would be moved to scalar registers,
        asm volatile("" : "+v"(z));   // and waited for, at once
#pragma unroll
        for (int w = 0; w < NWH; ++w) vw[w] = vote[hp * NWH + w + z];
      }
    }
    // the next position, and its K tile fetched behind this tile's P.V
    int ph_next = -1;
    auto next_position = [&]() {
      const int ncomp_next = ncomp + (code == 1 ? 1 : 0);
      if constexpr (MULTI) {
        // the walk ends when every head has reached its cap (none can before position k')
        bool capped = pn == kprime;
        if (a.cap_mode == 0 && pn >= kprime) {   // every head's votes decide
          int z = 0;
          asm volatile("" : "+v"(z));
          int all_done = 1;
#pragma unroll
          for (int hq = 0; hq < HP; ++hq) {
            bool allp = true;
#pragma unroll
            for (int w = 0; w < NWH; ++w) allp &= (vote[hq * NWH + w + z] & 1) != 0;
            const int v0 = vote[hq * NWH + z];
            const bool dn = (v0 & 2) != 0;
            const int cd = dn ? 0 : ((v0 & 4) && allp ? 2 : 1);
            all_done &= (dn || (v0 >> 3) + (cd == 1 ? 1 : 0) == kprime) ? 1 : 0;
          }
          capped = __builtin_amdgcn_readfirstlane(all_done) != 0;
        }
        if (!capped && pn < kl) ph_next = e_next == STOP ? -1 : e_next;
      } else if constexpr (SPARSE) {
        const bool capped = a.cap_mode == 0 ? (GROUPV ? all_capped : ncomp_next == kprime)
                                            : (pn == kprime);
        if (!capped && pn < kl) ph_next = e_next == STOP ? -1 : e_next;
      } else {
        if (pn < kl) ph_next = pn | (pn == i ? DIAG_BIT : 0) | (pn == nbv - 1 ? tail_bit : 0);
      }
      if (ph_next >= 0) issue_tile<BLK, D, false, TT::NT>(krs, (ph_next & PAGE_MASK) * TILE_BYTES, Ks, tid, wave_base);
    };
    // an undecided block vote can change the next position only at the computed-tile cap
    // (there the position is taken after the decision; elsewhere code = 1 gives the same)
    const bool early = MULTI || !voted || a.cap_mode != 0 || ncomp + 1 < kprime;
    if (early) next_position();

    uint32_t pk[NKT * 8];   // P as bf16 pairs: word w holds slots 2(w%8), 2(w%8)+1 of chunk w/8
    float mnew = m, alpha = 1.0f, rs = 0.0f;
    auto probabilities = [&]() {
      mnew = fmaxf(m, mloc);
      alpha = __builtin_amdgcn_exp2f(m - mnew);
      const float c = a.scale_log2;
      // four partial row sums keep the adds off one dependent chain; P is packed as soon as
      // a pair is formed, so that the P.V MFMAs read finished registers
      float rq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][x], c, -mnew));
          sacc[kt][x] = pv;
          if (x & 1) pk[kt * 8 + x / 2] = cvt_pk_bf16(sacc[kt][x - 1], pv);
          rq[x & 3] += pv;
        }
      rs = halves_sum((rq[0] + rq[1]) + (rq[2] + rq[3]));
    };
    if (voted) {
      int all = 1;
#pragma unroll
      for (int w = 0; w < NWH; ++w) all &= vw[w] & 1;
      code = __builtin_amdgcn_readfirstlane(all) ? 2 : 1;
    }
    if (MULTI && hdone) code = 0;
    // a computed tile whose V was not copied ahead: copy it now, behind the probabilities
    const bool vlate = DEFERV && vdefer && code == 1;
    if (vlate) issue_tile<BLK, D, true, TT::NT>(vrs, (ph & PAGE_MASK) * TILE_BYTES, Vs, tid, wave_base);
    if (code == 1) probabilities();
    if constexpr (SPARSE && !GROUPV) st_byte = code;
    if (!early) next_position();
    if (vlate) {
      wait_copies();      // this tile's V (and the next K, if issued) has landed
      __syncthreads();    // everyone's
    }

    if (code == 1) {
      l = alpha * l + rs;
      m = mnew;
      if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
      }
      // ---- O^T += V^T P^T (V fragment reads run PFV MFMAs ahead, order pinned as above)
      const int G4 = lane >> 4;
      const int i16 = lane & 15;
      const int rr = i16 >> 2;
      const int c4 = i16 & 3;
      const int keyb = 4 * hh + rr;          // key offset inside each 16-key step
      const int swv = swz_v<D>(keyb);        // the same for rows keyb + 8 and keyb + 16t
      const int sub = 4 * (c4 & 1);
      const bf16_t* vbase = Vs + keyb * D + sub;
      auto vfrag = [&](int idx) {
        const int t = idx / NDT, dt = idx % NDT;
        const int cd = 4 * dt + 2 * (G4 & 1) + (c4 >> 1);
        const bf16_t* p0 = vbase + (16 * t) * D + ((cd ^ swv) * 8);
        const bf16x4 lo = read_tr(p0);
        const bf16x4 hi = read_tr(p0 + 8 * D);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      constexpr int PFV = 3;
      bf16x8 vf[PFV];
#pragma unroll
      for (int u = 0; u < PFV; ++u) vf[u] = vfrag(u);
      bf16x8 pf;
#pragma unroll
      for (int idx = 0; idx < (BLK / 16) * NDT; ++idx) {
        const int t = idx / NDT;
        if (idx % NDT == 0) {
          const u32x4 w4 = {pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]};
          pf = __builtin_bit_cast(bf16x8, w4);
        }
        const bf16x8 vcur = vf[idx % PFV];
        if (idx + PFV < (BLK / 16) * NDT) vf[idx % PFV] = vfrag(idx + PFV);
        __builtin_amdgcn_sched_barrier(0);
        oacc[idx % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur, pf, oacc[idx % NDT], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (SPARSE) {
      if (a.visit_status && htid == 0 && !hdone) a.visit_status[unit * a.kmax + p] = (uint8_t)st_byte;
    }
    ncomp += code == 1 ? 1 : 0;
    if (MULTI && !hdone && a.cap_mode == 0 && ncomp == kprime) {
      hdone = true;
      p_end = pn;
    }
    wait_copies();      // next K tile has landed
    __syncthreads();    // B2: V buffer free, next K visible
    if constexpr (DEFERV) vdefer = code == 2;   // uniform: the block's decision
    if (ph_next >= 0 && !vdefer)
      issue_tile<BLK, D, true, TT::NT>(vrs, (ph_next & PAGE_MASK) * TILE_BYTES, Vs, tid, wave_base);
    ph = ph_next;
    p = pn;
  }

  // ---- epilogue
  if (!head_ok) return;
  if constexpr (SPARSE) {
    const int p0 = p_end >= 0 ? p_end : p;   // first position this head did not reach
    if (a.visit_status)
      for (int pp = p0 + htid; pp < a.kmax; pp += NWH * 64) a.visit_status[unit * a.kmax + pp] = 0;
    if (a.tile_counts) {
      int total = ncomp;
      if (GROUPV) {  // computed tiles summed over the row groups
        if (lane == 0) vote[wave] = ncomp;
        __syncthreads();
        total = 0;
#pragma unroll
        for (int w = 0; w < TT::NW; ++w) total += vote[w];
      }
      if (htid == 0) {
        a.tile_counts[unit * 2] = nvis;
        a.tile_counts[unit * 2 + 1] = total;
      }
    }
  }
  const float linv = ncomp > 0 ? 1.0f / l : 0.0f;
  bf16_t* Og = (bf16_t*)a.out + (bh * a.N + (long)i * BLK + rloc) * D;
  if (rloc >= rows_valid) return;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d0 = 32 * dt + 8 * ii + 4 * hh;
      u32x2 o;
      o[0] = cvt_pk_bf16(oacc[dt][4 * ii] * linv, oacc[dt][4 * ii + 1] * linv);
      o[1] = cvt_pk_bf16(oacc[dt][4 * ii + 2] * linv, oacc[dt][4 * ii + 3] * linv);
      *reinterpret_cast<u32x2*>(Og + d0) = o;
    }
  }
  if (a.lse && hh == 0) {
    a.lse[bh * a.N + (long)i * BLK + rloc] = ncomp > 0 ? (m + __log2f(l)) * LN2 : NEG;
  }
}

template <typename T, int BLK, int D>
static hipError_t launch_attn_t(const AttnLaunch& a, hipStream_t s) {
  const long groups = (long)a.Bt * a.Hkv * a.nb;
  const long grid = ((groups + 7) / 8) * 8 * a.group;
  if constexpr (sizeof(T) == 2) {
    // Block 64 with lists shared by a KV head's query heads: four of those heads share each
    // K/V tile in one workgroup.  (At block 128 two heads per workgroup run slower than one
    // workgroup per head: the two waves of each SIMD then move through the tile in lockstep
    // and contend for the matrix core and the VALU at the same moments, which outweighs the
    // halved copies.)
    if (BLK == 64 && a.sparse && a.shared_lists && !a.vote_group && a.group > 1) {
      if constexpr (BLK == 64) {
        constexpr int HP = 8 / (BLK / 32);
        const long grid3 = ((groups + 7) / 8) * 8 * ((a.group + HP - 1) / HP);
        hipLaunchKernelGGL((attn2_kernel<BLK, D, 3>), dim3((unsigned)grid3), dim3(512), 0, s, a);
      }
    } else if (a.sparse && a.vote_group)
      hipLaunchKernelGGL((attn2_kernel<BLK, D, 2>), dim3((unsigned)grid), dim3(BLK * 2), 0, s, a);
    else if (a.sparse)
      hipLaunchKernelGGL((attn2_kernel<BLK, D, 1>), dim3((unsigned)grid), dim3(BLK * 2), 0, s, a);
    else
      hipLaunchKernelGGL((attn2_kernel<BLK, D, 0>), dim3((unsigned)grid), dim3(BLK * 2), 0, s, a);
  } else {
    if (a.sparse)
      hipLaunchKernelGGL((attn_kernel<T, BLK, D, true>), dim3((unsigned)grid), dim3(BLK * 2), 0, s, a);
    else
      hipLaunchKernelGGL((attn_kernel<T, BLK, D, false>), dim3((unsigned)grid), dim3(BLK * 2), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_attn_dt(const AttnLaunch& a, hipStream_t s) {
  if (a.block == 128)
    return a.D == 128 ? launch_attn_t<T, 128, 128>(a, s) : launch_attn_t<T, 128, 64>(a, s);
  return a.D == 128 ? launch_attn_t<T, 64, 128>(a, s) : launch_attn_t<T, 64, 64>(a, s);
}

hipError_t launch_attn(const AttnLaunch& a, hipStream_t s) {
  return a.bf16 ? launch_attn_dt<bf16_t>(a, s) : launch_attn_dt<float>(a, s);
}

}  // namespace cosa

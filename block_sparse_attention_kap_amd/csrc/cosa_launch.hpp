// Internal launch descriptors shared by the host API and the kernel files.
// Arguments here are already validated by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cosa.h"

namespace cosa {

// Tokens of every batch entry (a varlen batch), passed by value to the kernels.
struct SeqLens {
  int varlen;                       // 0: every entry holds N tokens
  int len[COSA_MAX_VARLEN_BATCH];
  __host__ __device__ int of(int b, int N) const { return varlen ? len[b] : N; }
};

// Row pitch (floats) of the proxy scores P[bh][r][*]: the block count rounded up to a
// multiple of 4, so that every row starts 16-byte aligned and 16-byte stores of four
// consecutive blocks never cross into the next row.
__host__ __device__ inline int p_pitch(int nb) { return (nb + 3) & ~3; }

struct PoolLaunch {
  const void* x0;  // Q  [rows0 * g, D]
  void* y0;        // Q~ [rows0, D]
  long chunks0;    // rows0 * cpr
  const void* x1;  // K
  void* y1;        // K~
  long chunks1;
  int cpr;  // 16-byte chunks per row
  int g;
  int N, Np;  // rows and pooled rows per head (N % g != 0: the last group is partial)
  int H0, H1; // heads of x0 and x1 (to find the batch entry of a row)
  int stride_mode;
  int bf16;
  SeqLens sl;
};

struct ScoreLaunch {
  const void* qp;  // [Bt*Hq, Np, D]
  const void* kp;  // [Bt*Hkv, Np, D]
  float* P;        // [Bt*Hq, Np, p_pitch(nb)]
  int bh;          // Bt*Hq
  int Hq, group, Hkv;
  int Np, nb, Rb, D;
  int causal;
  float scale;
  int bf16;
  int g;      // pooling size (valid pooled rows of entry b: ceil(len_b / g))
  int N;
  SeqLens sl;
};

struct SelectLaunch {
  const float* P;
  int bh, Hq, Np, nb, Rb, causal;
  int share, group, Hkv;  // share: one list per KV head over the rows of its `group` heads
  double budget;
  int agg_mode, force_sink, force_diag;
  int sel_mode;   // 0 top-k, 1 cumulative mass
  int order_mode; // 0 HRM first, 1 score only
  float mass;
  int32_t* visit_idx;
  int32_t* visit_cnt;
  int32_t* hrm_cnt;
  float* visit_score;
  int kmax;
  int N, g, block;
  SeqLens sl;
};

struct AttnLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* visit_idx;
  const int32_t* visit_cnt;
  const int32_t* page_table;
  uint8_t* visit_status;
  int32_t* tile_counts;
  int Bt, Hq, Hkv, group, N, nb, kmax, causal;  // nb = ceil(N / block)
  float scale_log2;     // softmax scale * log2(e)
  int cap_mode, skip_mode;
  float skip_thr_log2;  // MAXDIFF: tau*log2(e); MASS: log2(eps)
  double tight_budget;
  int vote_group;       // 1: each 32-row group votes, counts and stops on its own
  int D, block, bf16;
  int sparse;
  int shared_lists;  // lists indexed by KV head
  SeqLens sl;
};

hipError_t launch_pool(const PoolLaunch& a, hipStream_t s);
hipError_t launch_score(const ScoreLaunch& a, hipStream_t s);
hipError_t launch_select(const SelectLaunch& a, hipStream_t s);
hipError_t launch_attn(const AttnLaunch& a, hipStream_t s);

}  // namespace cosa

// Host side of libcosa: argument validation, workspace layout and kernel launches.
// Every check runs before the first HIP call, so an invalid call has no effect.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "../../include/cosa.h"
#include "cosa_launch.hpp"

namespace {

constexpr int MAX_NB = 4096;

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int elem_bytes(int dtype) { return dtype == COSA_BF16 ? 2 : 4; }

// Blocks per sequence; the last one is partial when block does not divide seq_len.
int num_blocks(const cosa_shape* s) { return (s->seq_len + s->block - 1) / s->block; }

// Shape checks shared by every entry point.
int check_shape(const cosa_shape* s) {
  if (!s) return COSA_ERR_INVALID_ARG;
  if (s->batch < 1 || s->q_heads < 1 || s->kv_heads < 1 || s->seq_len < 1 || s->block < 1 ||
      s->head_dim < 1)
    return COSA_ERR_INVALID_ARG;
  if (s->q_heads % s->kv_heads) return COSA_ERR_INVALID_ARG;
  if (s->causal != 0 && s->causal != 1) return COSA_ERR_INVALID_ARG;
  if (!(s->scale >= 0.0f) || !isfinite(s->scale)) return COSA_ERR_INVALID_ARG;
  if (s->dtype != COSA_F32 && s->dtype != COSA_BF16) return COSA_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return COSA_ERR_UNSUPPORTED;
  if (s->block != 64 && s->block != 128) return COSA_ERR_UNSUPPORTED;
  if (num_blocks(s) > MAX_NB) return COSA_ERR_UNSUPPORTED;
  // the proxy launches one grid row per (batch entry, head): a grid dimension holds 65535
  if ((long)s->batch * s->q_heads > 65535) return COSA_ERR_UNSUPPORTED;
  // every tensor offset fits comfortably in 64 bits; keep element counts below 2^62
  const double elems = (double)s->batch * s->q_heads * s->seq_len * s->head_dim;
  if (elems > 4.0e18) return COSA_ERR_INVALID_ARG;
  if (s->seq_lens) {
    if (s->batch > COSA_MAX_VARLEN_BATCH) return COSA_ERR_UNSUPPORTED;
    for (int b = 0; b < s->batch; ++b)
      if (s->seq_lens[b] < 1 || s->seq_lens[b] > s->seq_len) return COSA_ERR_INVALID_ARG;
  }
  return COSA_OK;
}

// Does some batch entry end inside a block?
bool has_partial_block(const cosa_shape* s) {
  if (s->seq_len % s->block) return true;
  if (s->seq_lens)
    for (int b = 0; b < s->batch; ++b)
      if (s->seq_lens[b] % s->block) return true;
  return false;
}

cosa::SeqLens seq_lens_of(const cosa_shape* s) {
  cosa::SeqLens v;
  v.varlen = s->seq_lens != nullptr;
  for (int b = 0; b < COSA_MAX_VARLEN_BATCH; ++b)
    v.len[b] = (v.varlen && b < s->batch) ? s->seq_lens[b] : s->seq_len;
  return v;
}

bool budget_ok(double r) { return r > 0.0 && r <= 1.0 && isfinite(r); }

int budget_count(double rho, int n) {
  double k = ceil(rho * (double)n);
  if (k < 1.0) k = 1.0;
  if (k > (double)n) k = (double)n;
  return (int)k;
}

int resolve_pool(const cosa_shape* s, const cosa_kap_params* kp) {
  return kp->pool > 0 ? kp->pool : s->block / 4;
}

int check_kap(const cosa_shape* s, const cosa_kap_params* kp) {
  if (!kp) return COSA_ERR_INVALID_ARG;
  if (!budget_ok(kp->budget)) return COSA_ERR_INVALID_ARG;
  if (kp->pool < 0) return COSA_ERR_INVALID_ARG;
  const int g = resolve_pool(s, kp);
  if (!pow2(g) || s->block % g) return COSA_ERR_INVALID_ARG;
  if (kp->pool_mode != COSA_POOL_MEAN && kp->pool_mode != COSA_POOL_STRIDE)
    return COSA_ERR_INVALID_ARG;
  if (kp->agg_mode != COSA_AGG_SUM && kp->agg_mode != COSA_AGG_MAX) return COSA_ERR_INVALID_ARG;
  if (kp->sel_mode != COSA_SEL_TOPK && kp->sel_mode != COSA_SEL_CUMMASS) return COSA_ERR_INVALID_ARG;
  if (kp->sel_mode == COSA_SEL_CUMMASS && !(kp->mass > 0.0 && kp->mass <= 1.0)) return COSA_ERR_INVALID_ARG;
  if ((kp->force_sink != 0 && kp->force_sink != 1) || (kp->force_diag != 0 && kp->force_diag != 1))
    return COSA_ERR_INVALID_ARG;
  if (kp->order_mode != COSA_ORDER_HRM_FIRST && kp->order_mode != COSA_ORDER_SCORE)
    return COSA_ERR_INVALID_ARG;
  if (kp->share_kv != 0 && kp->share_kv != 1) return COSA_ERR_INVALID_ARG;
  if (kp->share_kv && (s->q_heads / s->kv_heads) * (s->block / g) > 1024) return COSA_ERR_UNSUPPORTED;
  return COSA_OK;
}

int capacity(const cosa_shape* s, double budget) {
  const int nb = num_blocks(s);
  // k(n) is non-decreasing in n; the largest candidate count is nb either way
  return budget_count(budget, nb);
}

struct WsLayout {
  size_t qp, kp, P, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const cosa_shape* s, const cosa_kap_params* kp) {
  const int g = resolve_pool(s, kp);
  const size_t Np = (size_t)(s->seq_len + g - 1) / g;
  const size_t nb = (size_t)num_blocks(s);
  const size_t eb = elem_bytes(s->dtype);
  WsLayout w;
  w.qp = 0;
  w.kp = align256((size_t)s->batch * s->q_heads * Np * s->head_dim * eb);
  w.P = w.kp + align256((size_t)s->batch * s->kv_heads * Np * s->head_dim * eb);
  w.total = w.P + align256((size_t)s->batch * s->q_heads * Np * cosa::p_pitch((int)nb) * sizeof(float));
  return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? COSA_OK : COSA_ERR_HIP; }

float resolved_scale(const cosa_shape* s) {
  return s->scale > 0.0f ? s->scale : (float)(1.0 / sqrt((double)s->head_dim));
}

}  // namespace

extern "C" {

int cosa_version(void) { return 10000; }

const char* cosa_status_string(int status) {
  switch (status) {
    case COSA_OK:
      return "ok";
    case COSA_ERR_INVALID_ARG:
      return "invalid argument";
    case COSA_ERR_UNSUPPORTED:
      return "unsupported configuration";
    case COSA_ERR_HIP:
      return "HIP runtime error";
    case COSA_ERR_SCRATCH:
      return "problem too large for the static scratch of cosa_proxy_select_noalloc";
    default:
      return "unknown status";
  }
}

int cosa_list_capacity(const cosa_shape* shape, double budget) {
  const int rc = check_shape(shape);
  if (rc) return rc;
  if (!budget_ok(budget)) return COSA_ERR_INVALID_ARG;
  return capacity(shape, budget);
}

size_t cosa_kap_workspace_bytes(const cosa_shape* shape, const cosa_kap_params* kap) {
  if (check_shape(shape) || check_kap(shape, kap)) return 0;
  return ws_layout(shape, kap).total;
}

}  // extern "C"

namespace {

// The three proxy kernels on validated arguments, the workspace laid out by ws_layout(s, kp).
int proxy_run(const cosa_shape* s, const cosa_kap_params* kp, const void* q, const void* k,
              void* workspace, int32_t* visit_idx, int32_t* visit_cnt, int32_t* hrm_cnt,
              float* visit_score, int kmax, hipStream_t st) {
  const WsLayout w = ws_layout(s, kp);
  const int nb = num_blocks(s);
  int rc;
  const int g = resolve_pool(s, kp);
  const int Np = (s->seq_len + g - 1) / g;  // pooled rows per head (last group may be partial)
  const int bf16 = s->dtype == COSA_BF16;
  char* ws = (char*)workspace;
  const int cpr = s->head_dim * elem_bytes(s->dtype) / 16;

  cosa::PoolLaunch pl;
  pl.x0 = q;
  pl.y0 = ws + w.qp;
  pl.chunks0 = (long)s->batch * s->q_heads * Np * cpr;
  pl.x1 = k;
  pl.y1 = ws + w.kp;
  pl.chunks1 = (long)s->batch * s->kv_heads * Np * cpr;
  pl.cpr = cpr;
  pl.g = g;
  pl.N = s->seq_len;
  pl.Np = Np;
  pl.H0 = s->q_heads;
  pl.H1 = s->kv_heads;
  pl.sl = seq_lens_of(s);
  pl.stride_mode = kp->pool_mode == COSA_POOL_STRIDE;
  pl.bf16 = bf16;
  rc = hip_status(cosa::launch_pool(pl, st));
  if (rc) return rc;

  cosa::ScoreLaunch sl;
  sl.qp = ws + w.qp;
  sl.kp = ws + w.kp;
  sl.P = (float*)(ws + w.P);
  sl.bh = s->batch * s->q_heads;
  sl.Hq = s->q_heads;
  sl.Hkv = s->kv_heads;
  sl.group = s->q_heads / s->kv_heads;
  sl.Np = Np;
  sl.nb = nb;
  sl.Rb = s->block / g;
  sl.D = s->head_dim;
  sl.causal = s->causal;
  sl.scale = resolved_scale(s);
  sl.bf16 = bf16;
  sl.g = g;
  sl.N = s->seq_len;
  sl.sl = pl.sl;
  rc = hip_status(cosa::launch_score(sl, st));
  if (rc) return rc;

  cosa::SelectLaunch se;
  se.P = sl.P;
  se.bh = sl.bh;
  se.Hq = s->q_heads;
  se.share = kp->share_kv;
  se.group = s->q_heads / s->kv_heads;
  se.Hkv = s->kv_heads;
  se.Np = Np;
  se.nb = nb;
  se.Rb = sl.Rb;
  se.causal = s->causal;
  se.budget = kp->budget;
  se.agg_mode = kp->agg_mode;
  se.force_sink = kp->force_sink;
  se.force_diag = kp->force_diag;
  se.sel_mode = kp->sel_mode;
  se.order_mode = kp->order_mode;
  se.mass = (float)kp->mass;
  se.visit_idx = visit_idx;
  se.visit_cnt = visit_cnt;
  se.hrm_cnt = hrm_cnt;
  se.visit_score = visit_score;
  se.kmax = kmax;
  se.N = s->seq_len;
  se.g = g;
  se.block = s->block;
  se.sl = pl.sl;
  return hip_status(cosa::launch_select(se, st));
}

// Proxy workspace for callers that cannot allocate: one static array per GPU (each device
// holds its own copy from the load of this code until the process ends).  Host code reaches
// it only through the device address hipGetSymbolAddress gives, looked up once per device.
constexpr size_t SCRATCH_BYTES = (size_t)COSA_NOALLOC_SCRATCH_MIB << 20;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
std::atomic<void*> scratch_ptr[MAX_DEVICES];

// The device address of this GPU's scratch array (the current device), or nullptr.
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    // two threads may both look it up on a first call: they store the same address
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

int cosa_proxy_select(const cosa_shape* s, const cosa_kap_params* kp, const void* q,
                      const void* k, void* workspace, size_t workspace_bytes, int32_t* visit_idx,
                      int32_t* visit_cnt, int32_t* hrm_cnt, float* visit_score, int kmax,
                      void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  rc = check_kap(s, kp);
  if (rc) return rc;
  if (!q || !k || !workspace || !visit_idx || !visit_cnt || !hrm_cnt) return COSA_ERR_INVALID_ARG;
  if ((uintptr_t)workspace & 255) return COSA_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k) & 15) return COSA_ERR_INVALID_ARG;
  if (workspace_bytes < ws_layout(s, kp).total) return COSA_ERR_INVALID_ARG;
  if (kmax < capacity(s, kp->budget) || kmax > num_blocks(s)) return COSA_ERR_INVALID_ARG;
  return proxy_run(s, kp, q, k, workspace, visit_idx, visit_cnt, hrm_cnt, visit_score, kmax,
                   (hipStream_t)stream);
}

int cosa_proxy_select_noalloc(const cosa_shape* s, const cosa_kap_params* kp, const void* q,
                              const void* k, int32_t* visit_idx, int32_t* visit_cnt,
                              int32_t* hrm_cnt, float* visit_score, int kmax, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  rc = check_kap(s, kp);
  if (rc) return rc;
  if (!q || !k || !visit_idx || !visit_cnt || !hrm_cnt) return COSA_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k) & 15) return COSA_ERR_INVALID_ARG;
  const int nb = num_blocks(s);
  if (kmax < capacity(s, kp->budget) || kmax > nb) return COSA_ERR_INVALID_ARG;
  // The layer is cut into slices whose workspace fits the array: one batch entry and a group
  // of hk KV heads with all their query heads, else (lists per query head) gq query heads of
  // one KV head.  Every (batch, head, query block) unit is computed exactly as in one call.
  const int G = s->q_heads / s->kv_heads;
  cosa_shape sub = *s;
  sub.batch = 1;
  sub.seq_lens = nullptr;
  int hk = 0, gq = G;
  for (int d = s->kv_heads; d >= 1 && !hk; --d) {
    if (s->kv_heads % d) continue;
    sub.q_heads = d * G;
    sub.kv_heads = d;
    if (ws_layout(&sub, kp).total <= SCRATCH_BYTES) hk = d;
  }
  if (!hk) {
    if (kp->share_kv) return COSA_ERR_SCRATCH;   // a shared list needs every query head at once
    hk = 1;
    gq = 0;
    for (int d = G - 1; d >= 1 && !gq; --d) {
      if (G % d) continue;
      sub.q_heads = d;
      sub.kv_heads = 1;
      if (ws_layout(&sub, kp).total <= SCRATCH_BYTES) gq = d;
    }
    if (!gq) return COSA_ERR_SCRATCH;
  }
  void* ws = scratch_of_current_device();
  if (!ws) return COSA_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  const size_t eb = (size_t)elem_bytes(s->dtype);
  const size_t row = (size_t)s->seq_len * s->head_dim * eb;  // bytes of one head of q or k
  const int HL = kp->share_kv ? s->kv_heads : s->q_heads;   // heads the lists are indexed by
  sub.q_heads = hk * (gq == G ? G : gq);
  sub.kv_heads = hk;
  for (int b = 0; b < s->batch; ++b) {
    sub.seq_lens = s->seq_lens ? s->seq_lens + b : nullptr;
    for (int kv0 = 0; kv0 < s->kv_heads; kv0 += hk) {
      for (int g0 = 0; g0 < G; g0 += gq) {
        const long hq0 = (long)b * s->q_heads + (long)kv0 * G + g0;   // first query head
        const long hv0 = (long)b * s->kv_heads + kv0;                  // first KV head
        const long l0 = (long)b * HL + (kp->share_kv ? kv0 : (long)kv0 * G + g0);  // first list
        rc = proxy_run(&sub, kp, (const char*)q + hq0 * row, (const char*)k + hv0 * row, ws,
                       visit_idx + l0 * nb * kmax, visit_cnt + l0 * nb, hrm_cnt + l0 * nb,
                       visit_score ? visit_score + l0 * nb * kmax : nullptr, kmax, st);
        if (rc) return rc;
      }
    }
  }
  return COSA_OK;
}

static int check_osk(const cosa_osk_params* op) {
  if (!op) return COSA_ERR_INVALID_ARG;
  if (!budget_ok(op->tight_budget)) return COSA_ERR_INVALID_ARG;
  if (op->cap_mode != COSA_CAP_COMPUTED && op->cap_mode != COSA_CAP_VISITED)
    return COSA_ERR_INVALID_ARG;
  if (op->skip_mode < COSA_SKIP_OFF || op->skip_mode > COSA_SKIP_MASS) return COSA_ERR_INVALID_ARG;
  if (op->skip_mode == COSA_SKIP_MASS && !(op->skip_param > 0.0f && isfinite(op->skip_param)))
    return COSA_ERR_INVALID_ARG;
  if (op->skip_mode == COSA_SKIP_MAXDIFF && !isfinite(op->skip_param)) return COSA_ERR_INVALID_ARG;
  if (op->vote_rows != 0 && op->vote_rows != 32) return COSA_ERR_INVALID_ARG;
  if (op->shared_lists != 0 && op->shared_lists != 1) return COSA_ERR_INVALID_ARG;
  return COSA_OK;
}

static int attn_common(const cosa_shape* s, const cosa_osk_params* op, const void* q,
                       const void* k, const void* v, const int32_t* visit_idx,
                       const int32_t* visit_cnt, int kmax, const int32_t* page_table, void* out,
                       float* lse, uint8_t* visit_status, int32_t* tile_counts, void* stream,
                       int sparse) {
  cosa::AttnLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.visit_idx = visit_idx;
  a.visit_cnt = visit_cnt;
  a.page_table = page_table;
  a.visit_status = visit_status;
  a.tile_counts = tile_counts;
  a.Bt = s->batch;
  a.Hq = s->q_heads;
  a.Hkv = s->kv_heads;
  a.group = s->q_heads / s->kv_heads;
  a.N = s->seq_len;
  a.nb = num_blocks(s);
  a.kmax = kmax;
  a.causal = s->causal;
  a.scale_log2 = (float)((double)resolved_scale(s) * 1.4426950408889634);
  a.cap_mode = sparse ? op->cap_mode : 0;
  a.skip_mode = sparse ? op->skip_mode : 0;
  a.skip_thr_log2 = 0.0f;
  if (sparse && op->skip_mode == COSA_SKIP_MASS) a.skip_thr_log2 = (float)log2((double)op->skip_param);
  if (sparse && op->skip_mode == COSA_SKIP_MAXDIFF)
    a.skip_thr_log2 = (float)((double)op->skip_param * 1.4426950408889634);
  a.tight_budget = sparse ? op->tight_budget : 1.0;
  a.vote_group = (sparse && op->vote_rows == 32 && s->dtype == COSA_BF16) ? 1 : 0;
  a.D = s->head_dim;
  a.block = s->block;
  a.bf16 = s->dtype == COSA_BF16;
  a.sparse = sparse;
  a.shared_lists = sparse ? op->shared_lists : 0;
  a.sl = seq_lens_of(s);
  return hip_status(cosa::launch_attn(a, (hipStream_t)stream));
}

int cosa_ordered_sparse_attn(const cosa_shape* s, const cosa_osk_params* op, const void* q,
                             const void* k, const void* v, const int32_t* visit_idx,
                             const int32_t* visit_cnt, int kmax, const int32_t* page_table,
                             void* out, float* lse, uint8_t* visit_status, int32_t* tile_counts,
                             void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  rc = check_osk(op);
  if (rc) return rc;
  if (op->vote_rows == 32 && s->dtype != COSA_BF16) return COSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !visit_idx || !visit_cnt || !out) return COSA_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return COSA_ERR_INVALID_ARG;
  const int nb = num_blocks(s);
  if (kmax < 1 || kmax > nb) return COSA_ERR_INVALID_ARG;
  // a ragged sequence keeps its partial block last; pages are whole blocks
  if (page_table && has_partial_block(s)) return COSA_ERR_UNSUPPORTED;
  return attn_common(s, op, q, k, v, visit_idx, visit_cnt, kmax, page_table, out, lse,
                     visit_status, tile_counts, stream, 1);
}

int cosa_prefill(const cosa_shape* s, const cosa_kap_params* kp, const cosa_osk_params* op,
                 const void* q, const void* k, const void* v, void* workspace,
                 size_t workspace_bytes, int32_t* visit_idx, int32_t* visit_cnt, int32_t* hrm_cnt,
                 int kmax, void* out, float* lse, int head_chunks,
                 void* stream_proxy, void* stream_walk, void* event) {
  // everything the two per-group calls check, once, for the whole layer
  int rc = check_shape(s);
  if (rc) return rc;
  rc = check_kap(s, kp);
  if (rc) return rc;
  rc = check_osk(op);
  if (rc) return rc;
  if (op->vote_rows == 32 && s->dtype != COSA_BF16) return COSA_ERR_UNSUPPORTED;
  if (op->shared_lists != kp->share_kv) return COSA_ERR_INVALID_ARG;
  if (!q || !k || !v || !out || !workspace || !visit_idx || !visit_cnt || !hrm_cnt || !event)
    return COSA_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return COSA_ERR_INVALID_ARG;
  if ((uintptr_t)workspace & 255) return COSA_ERR_INVALID_ARG;
  if (workspace_bytes < ws_layout(s, kp).total) return COSA_ERR_INVALID_ARG;
  const int nb = num_blocks(s);
  if (kmax < capacity(s, kp->budget) || kmax > nb) return COSA_ERR_INVALID_ARG;
  if (head_chunks < 1 || s->kv_heads % head_chunks != 0) return COSA_ERR_INVALID_ARG;

  hipStream_t sp = (hipStream_t)stream_proxy, sw = (hipStream_t)stream_walk;
  hipEvent_t ev = (hipEvent_t)event;
  // the lists and the workspace may still be in use by walks queued earlier on stream_walk
  rc = hip_status(hipEventRecord(ev, sw));
  if (rc) return rc;
  rc = hip_status(hipStreamWaitEvent(sp, ev, 0));
  if (rc) return rc;

  const int G = s->q_heads / s->kv_heads;
  const int hk = s->kv_heads / head_chunks;       // KV heads per group
  const int HL = kp->share_kv ? s->kv_heads : s->q_heads;   // heads the lists are indexed by
  const int hl = kp->share_kv ? hk : hk * G;
  const size_t es = (size_t)elem_bytes(s->dtype);
  const size_t row = (size_t)s->seq_len * s->head_dim * es;  // bytes of one head of q, k, v
  for (int b = 0; b < s->batch; ++b) {
    for (int c = 0; c < head_chunks; ++c) {
      // one batch entry and one group of KV heads: a contiguous slice of every tensor
      cosa_shape sub = *s;
      sub.batch = 1;
      sub.q_heads = hk * G;
      sub.kv_heads = hk;
      sub.seq_lens = s->seq_lens ? s->seq_lens + b : nullptr;
      const long hq0 = (long)b * s->q_heads + (long)c * hk * G;   // first query head
      const long hv0 = (long)b * s->kv_heads + (long)c * hk;      // first KV head
      const long l0 = (long)b * HL + (long)c * hl;                // first list head
      const char* qs = (const char*)q + hq0 * row;
      const char* ks = (const char*)k + hv0 * row;
      const char* vs = (const char*)v + hv0 * row;
      int32_t* idx = visit_idx + l0 * nb * kmax;
      int32_t* cnt = visit_cnt + l0 * nb;
      int32_t* hrm = hrm_cnt + l0 * nb;
      rc = cosa_proxy_select(&sub, kp, qs, ks, workspace, workspace_bytes, idx, cnt, hrm, nullptr,
                             kmax, sp);
      if (rc) return rc;
      rc = hip_status(hipEventRecord(ev, sp));
      if (rc) return rc;
      rc = hip_status(hipStreamWaitEvent(sw, ev, 0));
      if (rc) return rc;
      rc = cosa_ordered_sparse_attn(&sub, op, qs, ks, vs, idx, cnt, kmax, nullptr,
                                    (char*)out + hq0 * row, lse ? lse + hq0 * s->seq_len : nullptr,
                                    nullptr, nullptr, sw);
      if (rc) return rc;
    }
  }
  return COSA_OK;
}

int cosa_dense_attn(const cosa_shape* s, const void* q, const void* k, const void* v, void* out,
                    float* lse, void* stream) {
  const int rc = check_shape(s);
  if (rc) return rc;
  if (!q || !k || !v || !out) return COSA_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return COSA_ERR_INVALID_ARG;
  return attn_common(s, nullptr, q, k, v, nullptr, nullptr, 1, nullptr, out, lse, nullptr, nullptr,
                     stream, 0);
}

}  // extern "C"

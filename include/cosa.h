/*
 * cosa.h -- C ABI of libcosa: CoSA block-sparse prefill attention on gfx950.
 *
 * The operations follow the paper "CoSA: Accelerating Long-Context Inference
 * via Proxy-Kernel Co-Designed Sparse Attention" (arXiv 2607.25291) as
 * described on its public pages:
 *   - the authors' abstract: a proxy (KAP) selects blocks under a moderate
 *     budget and emits an ordered mask giving the order in which the kernel's
 *     inner loop visits KV pages; the kernel (OSK) applies it and skips more
 *     blocks under a tightened budget from online-softmax statistics;
 *   - the gist.science technical summary (pt), section 2.2 (KAP: downsampled
 *     queries and keys, approximate scores, MaxPool over keys, MaxNorm, HRM
 *     flags, HRM-first ordering) and section 2.3 (OSK: mask-skipped blocks
 *     via KV-page remapping, in-kernel skipped blocks from the running max,
 *     computed blocks).
 * The pages print no formula, constant or API.  Every open rule is a
 * parameter below; its default is the plainest reading of the pages.
 *
 * Conventions (all entry points):
 *   - Tensors are device pointers owned by the caller, contiguous, layout
 *     [batch, heads, seq, dim] (BHSD).  Query head h reads KV head
 *     h / (q_heads / kv_heads).
 *   - The library allocates and frees no device memory; scratch memory is
 *     passed in as a workspace (cosa_proxy_select_noalloc instead uses a
 *     static device array of its own, one per GPU).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  The return value reports argument validation and launch
 *     status only.  All validation happens on the host before any HIP call;
 *     on an error nothing is launched and no output is written.
 *   - Calls keep no state from one to the next and are thread-safe, except
 *     cosa_proxy_select_noalloc, whose calls on one GPU share its static
 *     scratch array and must not overlap.  Results are bitwise
 *     deterministic from run to run (no atomics in any reduction).
 *   - Supported: head_dim in {64, 128}, block in {64, 128},
 *     ceil(seq_len / block) <= 4096, q_heads % kv_heads == 0,
 *     batch * q_heads <= 65535, dtype in {COSA_F32, COSA_BF16}; any
 *     seq_len >= 1 (see cosa_shape).  Outside these: COSA_ERR_UNSUPPORTED.
 */
#ifndef COSA_H
#define COSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  COSA_OK = 0,
  COSA_ERR_INVALID_ARG = -1,  /* a null required pointer, a bad size or value */
  COSA_ERR_UNSUPPORTED = -2,  /* valid in principle, not built (dtype, dims)  */
  COSA_ERR_HIP = -3,          /* the HIP runtime refused a launch            */
  COSA_ERR_SCRATCH = -4       /* needs more than the static scratch of
                                 cosa_proxy_select_noalloc holds             */
} cosa_status;

typedef enum { COSA_F32 = 0, COSA_BF16 = 1 } cosa_dtype;

#define COSA_MAX_VARLEN_BATCH 128

/* Problem shape.  scale = 0 selects 1/sqrt(head_dim).
 *   seq_len   rows of the seq axis of every tensor.  nb = ceil(seq_len / block)
 *             blocks; when block does not divide seq_len the last block is
 *             partial (its missing keys are masked, its missing rows not
 *             computed) and the last pooled group of the proxy averages the rows
 *             that exist (still times 2^-log2(g)).
 *   seq_lens  nullable HOST array [batch] (a varlen batch): entry b is a sequence
 *             of seq_lens[b] tokens, 1 <= seq_lens[b] <= seq_len, held in the first
 *             seq_lens[b] rows of its seq axis; the rows after them are padding that
 *             is never read (except K and V pages a page table names, see
 *             cosa_ordered_sparse_attn).  Query blocks of entry b at or past
 *             ceil(seq_lens[b] / block) get empty lists (visit_cnt 0) and no work,
 *             and rows at or past seq_lens[b] of out and lse are not written.  At
 *             most COSA_MAX_VARLEN_BATCH entries; read during the call only.
 *             NULL: every entry holds seq_len tokens. */
typedef struct {
  int batch, q_heads, kv_heads, seq_len, head_dim, block;
  int causal;   /* 1: token-causal attention, 0: full attention */
  float scale;  /* softmax scale applied to q.k                  */
  int dtype;    /* cosa_dtype of Q, K, V and O                   */
  const int32_t* seq_lens;
} cosa_shape;

enum { COSA_POOL_MEAN = 0, COSA_POOL_STRIDE = 1 };
enum { COSA_AGG_SUM = 0, COSA_AGG_MAX = 1 };
enum { COSA_SEL_TOPK = 0, COSA_SEL_CUMMASS = 1 };
enum { COSA_ORDER_HRM_FIRST = 0, COSA_ORDER_SCORE = 1 };
enum { COSA_CAP_COMPUTED = 0, COSA_CAP_VISITED = 1 };
enum { COSA_SKIP_OFF = 0, COSA_SKIP_MAXDIFF = 1, COSA_SKIP_MASS = 2 };
enum { COSA_STATUS_NOT_REACHED = 0, COSA_STATUS_COMPUTED = 1, COSA_STATUS_SKIPPED = 2 };

/* Proxy (KAP) parameters.
 *   budget     rho in (0, 1]: query block i keeps k_i = min(n_i, max(1, ceil(rho*n_i)))
 *              of its n_i candidate blocks (n_i = i+1 causal, nb otherwise);
 *              the product is formed in IEEE double.
 *   pool       g, a power of two dividing block; 0 selects block/4.
 *   pool_mode  MEAN: fp32 sum of g consecutive rows in ascending order, times
 *              2^-log2(g), rounded to the dtype (RNE); STRIDE: first row of each group.
 *   agg_mode   how the per-row MaxNorm contributions exp(P - rowmax) of the
 *              pooled rows of a query block combine into its block score.
 *   sel_mode   TOPK keeps k_i blocks.  CUMMASS keeps the shortest prefix of the ordered
 *              list whose score sum reaches mass * (sum of S over all candidates),
 *              at least 1 and at most k_i blocks; mass in (0, 1].
 *   force_sink, force_diag: treat block 0 / the diagonal block as HRM.
 *   order_mode HRM_FIRST (default): HRM blocks first, then by S; SCORE: by S alone,
 *              the single-criterion ranking of a plain top-k proxy (for ablations).
 *   share_kv   0 (default): one list per query head.  1: one list per KV head, shared
 *              by its q_heads/kv_heads query heads (GQA): the pooled rows of all of
 *              them (heads ascending) are the rows of the query block, so S sums their
 *              MaxNorm contributions and the HRM flags are the union of theirs; the
 *              lists are then [batch, kv_heads, nb, kmax].  Needs
 *              (q_heads/kv_heads) * block / g <= 1024. */
typedef struct {
  double budget;
  int pool;
  int pool_mode;
  int agg_mode;
  int sel_mode;
  double mass;
  int force_sink;
  int force_diag;
  int order_mode;
  int share_kv;
} cosa_kap_params;

/* Kernel (OSK) parameters.
 *   tight_budget rho' in (0, 1]: the walk of query block i stops once the
 *              cap k'_i = min(k_i, max(1, ceil(rho'*n_i))) is reached, counted
 *              in visited blocks (CAP_VISITED: the walk covers the first k'_i listed
 *              blocks and the skip test drops some of them, so skipping raises the
 *              sparsity; the reading the Python binding and the benchmark use) or
 *              computed blocks (CAP_COMPUTED: a skipped block extends the walk).
 *   skip_mode  after the first computed block, a listed block is skipped (no
 *              exp, no P.V, statistics unchanged) iff every row r of the query
 *              block satisfies
 *                MAXDIFF: m_loc[r] - m[r] <= skip_param (tau), or
 *                MASS:    m_loc[r] - m[r] + ln nv[r] - ln l[r] <= ln(skip_param) (eps),
 *              where m_loc is the block's row max of the scaled logits, m and
 *              l the running max and denominator, nv the visible keys of the
 *              row in the block.
 *   vote_rows  0: the whole query block votes (default).  32: every group of 32 rows
 *              decides, counts its cap and stops on its own (a finer granularity of
 *              the skip test; bf16 only).  Then visit_status packs 2 bits per group
 *              (group g in bits 2g..2g+1) and tile_counts[...][1] sums the computed
 *              tiles over the groups.
 *   shared_lists 0: visit_idx/visit_cnt hold one list per query head.  1: one list per
 *              KV head ([batch, kv_heads, nb, ...], from share_kv), walked by each of
 *              its query heads; visit_status and tile_counts stay per query head. */
typedef struct {
  double tight_budget;
  int cap_mode;
  int skip_mode;
  float skip_param;
  int vote_rows;
  int shared_lists;
} cosa_osk_params;

/* Capacity kmax of a visit list: the largest k_i over the query blocks.
 * Returns kmax >= 1, or a negative cosa_status. */
int cosa_list_capacity(const cosa_shape* shape, double budget);

/* Bytes of device workspace cosa_proxy_select needs (pooled Q and K plus the
 * block-level proxy scores), or 0 if the arguments are invalid. */
size_t cosa_kap_workspace_bytes(const cosa_shape* shape, const cosa_kap_params* kap);

/* Stage 1, the Kernel-Aware Proxy (gist.science technical summary, section 2.2; the
 * authors' abstract, first stage): for every (batch, query head, query block i)
 * pool Q and K, score pooled rows against pooled keys (pool-level causal:
 * key pool t visible from query pool r iff t <= r), max-pool the scores over
 * the keys of each block (P), MaxNorm each pooled row (exp(P - rowmax)),
 * aggregate over the rows of the block (S), flag HRM blocks (the lowest block
 * holding a row's maximum), sort the candidates by (HRM desc, S desc, j asc)
 * and keep the first k_i.
 *   q          [batch, q_heads, seq_len, head_dim]  dtype
 *   k          [batch, kv_heads, seq_len, head_dim] dtype
 *   workspace  device scratch of at least cosa_kap_workspace_bytes(); 256-byte aligned
 *   visit_idx  out [batch, q_heads, nb, kmax] int32: the ordered list, -1 padded
 *              (kv_heads in place of q_heads here and below with share_kv)
 *   visit_cnt  out [batch, q_heads, nb] int32: k_i (CUMMASS: the cut length)
 *   hrm_cnt    out [batch, q_heads, nb] int32: number of HRM candidates of block i
 *              (HRM blocks are the first min(hrm_cnt, k_i) entries of the list)
 *   visit_score out, nullable [batch, q_heads, nb, kmax] float: S in list order, 0 padded
 *   kmax       list capacity, >= cosa_list_capacity(shape, kap->budget) */
int cosa_proxy_select(const cosa_shape* shape, const cosa_kap_params* kap,
                      const void* q, const void* k,
                      void* workspace, size_t workspace_bytes,
                      int32_t* visit_idx, int32_t* visit_cnt, int32_t* hrm_cnt,
                      float* visit_score, int kmax, void* stream);

/* Size of the static device array cosa_proxy_select_noalloc uses as its workspace (MiB). */
#define COSA_NOALLOC_SCRATCH_MIB 128

/* cosa_proxy_select for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same lists, bitwise,
 * with no workspace argument.  The workspace is a static device array of
 * COSA_NOALLOC_SCRATCH_MIB MiB that every GPU the library runs on holds from the first use
 * until the process ends; its address is looked up once per device (on the first call with
 * that device current).  The call allocates and frees nothing.  When the layer's workspace
 * (cosa_kap_workspace_bytes) exceeds the array, the layer is proxied in slices on `stream`,
 * one after another: one batch entry and a group of KV heads with their query heads, or
 * (lists per query head only) a group of the query heads of one KV head.  If even one query
 * head (share_kv: one KV head with all its query heads) needs more than the array holds, the
 * call returns COSA_ERR_SCRATCH and launches nothing.
 * Every call on a GPU uses that GPU's one array: calls that overlap in time on one GPU (on
 * different streams, or from several threads) race on it and give undefined lists.
 * The array needs no clearing: every byte of it a call reads was written by that call.
 * Arguments, outputs and the other errors are those of cosa_proxy_select. */
int cosa_proxy_select_noalloc(const cosa_shape* shape, const cosa_kap_params* kap,
                              const void* q, const void* k,
                              int32_t* visit_idx, int32_t* visit_cnt, int32_t* hrm_cnt,
                              float* visit_score, int kmax, void* stream);

/* Stage 2, the Ordered-Skipping Kernel (gist.science technical summary, section 2.3,
 * and section 2.1 for the order-free accumulation; the authors' abstract, second stage):
 * for every (batch, query head, query block i) walk visit_idx[..i..][0 .. visit_cnt-1]
 * in order with online softmax, apply the skip test and the tightened-budget cap, and
 * write O = acc / l over the computed blocks.  Blocks not in the list are never read.
 *   q, k, v      BHSD device tensors of the dtype (k and v: kv_heads)
 *   visit_idx    [batch, q_heads, nb, kmax] int32 (e.g. from cosa_proxy_select;
 *                kv_heads in place of q_heads with shared_lists)
 *   visit_cnt    [batch, q_heads, nb] int32, entries in [1, kmax] (idem)
 *   page_table   nullable [batch, nb] int32: logical block j of entry b lives in
 *                physical page page_table[b*nb + j] of k and v, i.e. rows
 *                page*block .. page*block + block-1 of that entry's KV head; NULL =
 *                identity.  Any page in [0, nb) may be named, also one at or past
 *                the end of a varlen entry's own tokens.  Pages are whole blocks:
 *                with a partial last block (seq_len, or some seq_lens[b], not a
 *                multiple of block) a page table is COSA_ERR_UNSUPPORTED
 *   out          [batch, q_heads, seq_len, head_dim] dtype
 *   lse          nullable [batch, q_heads, seq_len] float: m + ln l (natural log)
 *   visit_status nullable [batch, q_heads, nb, kmax] uint8: COSA_STATUS_* per position
 *   tile_counts  nullable [batch, q_heads, nb, 2] int32: visited, computed
 * A malformed list entry (not a valid candidate of block i, or a page index
 * outside [0, nb)) ends that walk at that position; the entry and the ones
 * after it are reported NOT_REACHED.  A walk that computed no block writes
 * zeros to out and -inf to lse. */
int cosa_ordered_sparse_attn(const cosa_shape* shape, const cosa_osk_params* osk,
                             const void* q, const void* k, const void* v,
                             const int32_t* visit_idx, const int32_t* visit_cnt, int kmax,
                             const int32_t* page_table,
                             void* out, float* lse, uint8_t* visit_status,
                             int32_t* tile_counts, void* stream);

/* Both stages over one layer (the proxy, then the kernel on its ordered lists, as the authors'
 * abstract chains them), pipelined across two streams: the KV heads of every batch
 * entry are split into head_chunks groups of kv_heads / head_chunks heads (each with its
 * query heads); the proxy of a group runs on stream_proxy while the walk of the group before
 * it runs on stream_walk, so that the proxy's memory-bound passes overlap the walk's matrix
 * work.  The outputs are bitwise those of cosa_proxy_select followed by
 * cosa_ordered_sparse_attn over the whole layer (without visit_score, visit_status and
 * tile_counts).
 *   shape, kap, osk, q, k, v, workspace, visit_idx, visit_cnt, hrm_cnt, kmax, out, lse:
 *                as in those two calls (workspace sized for the whole layer by
 *                cosa_kap_workspace_bytes); osk->shared_lists must equal kap->share_kv.  Both
 *                stages read the one k, in logical block order (no page table: a paged KV
 *                cache calls the two stages itself, the proxy on the logical K)
 *   head_chunks  >= 1 and a divisor of kv_heads
 *   event        a hipEvent_t created by the caller; recorded and waited on during the call
 *   stream_proxy, stream_walk: hipStream_t; the same stream for both gives the serial order
 * Ordering: the call first makes stream_proxy wait for the work already queued on stream_walk
 * (so the lists and the workspace of an earlier call are free again); the caller makes both
 * streams wait for the producers of q, k and v, and the consumers of out, lse and the lists
 * wait for stream_walk, which ends with the last walk.  All arguments are validated before the
 * first HIP call; a HIP error part-way returns COSA_ERR_HIP with earlier groups queued. */
int cosa_prefill(const cosa_shape* shape, const cosa_kap_params* kap,
                 const cosa_osk_params* osk, const void* q, const void* k, const void* v,
                 void* workspace, size_t workspace_bytes,
                 int32_t* visit_idx, int32_t* visit_cnt, int32_t* hrm_cnt, int kmax,
                 void* out, float* lse,
                 int head_chunks, void* stream_proxy, void* stream_walk, void* event);

/* Dense softmax attention (causal if shape->causal) in natural block order: the
 * baseline the sparse path is measured against (the authors' abstract and section 4 of
 * the gist.science technical summary report CoSA's attention speedup over dense
 * attention at 128K context).  Arguments as in cosa_ordered_sparse_attn: q, k, v BHSD
 * device tensors of the dtype, out [batch, q_heads, seq_len, head_dim] dtype, lse
 * nullable [batch, q_heads, seq_len] float (natural log).  Validation as for every
 * entry point: nothing is launched on an invalid argument. */
int cosa_dense_attn(const cosa_shape* shape, const void* q, const void* k, const void* v,
                    void* out, float* lse, void* stream);

/* Static description of a status code. */
const char* cosa_status_string(int status);

/* Library version (major*10000 + minor*100 + patch). */
int cosa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* COSA_H */

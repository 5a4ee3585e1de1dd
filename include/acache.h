/*
 * acache.h -- C ABI of the ACache slot-mapped bidirectional attention engine
 * for AMD Instinct MI355X (gfx950).
 *
 * Method: "Affix Cache for Diffusion Large Language Models" (ACache),
 * arXiv 2608.26140.  A shared affix F = {l, ..., l+L-1} has its KV cache
 * computed once and stored in a shared region.  Each request runs a one-shot
 * probe (Section 3.2, Eqs. 4-5), keeps the K affix tokens of largest
 * masked-to-affix attention mass as Anchor Tokens (Eq. 6), recomputes only
 * the anchors and its own positions into private slots (Section 3.3,
 * Section 4.1 write-side map), and attends through a per-request read-slot
 * map that names, for every logical position, the physical slot to read
 * (Section 4.1, Section 4.3, Appendix C.1).
 *
 * Conventions for every call below
 *  - Pointers are device pointers unless marked (host).  The caller owns all
 *    memory; the library never allocates, frees or keeps a pointer after a
 *    call returns.  Scratch memory comes from a caller workspace whose size
 *    the matching *_workspace_bytes query reports.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and return after enqueueing.  They hold no mutable global state
 *    (acache_mapped_attention_shared_noalloc aside: it keeps one fixed scratch
 *    array per GPU); calls on different streams may run concurrently when
 *    their outputs do not overlap.
 *  - Return value: ACACHE_OK (0) or a negative status.  Scalar, shape,
 *    alignment and pointer checks run on the host before anything is
 *    enqueued, so an error return means nothing was launched.  Table
 *    *contents* (slot ids, offsets) are trusted by the compute calls; the
 *    checked mode checks them first: acache_check_slots (a device pre-pass,
 *    synchronous) and acache_scatter_private_checked (that pre-pass, then
 *    the scatter only when it passes), or acache_validate_slots on host
 *    copies.  A kernel launch failure returns ACACHE_EDEVICE.
 *  - Element types: Q, the pool, scatter sources and attention outputs share
 *    the pool's dtype (ACACHE_F32 or ACACHE_BF16); scores and LSE are fp32;
 *    indices and offsets are int32.  Vector pointers must be 16-byte aligned.
 *  - head_dim is 16, 32, 64 or 128; page_size is a power of two <= 256;
 *    n_q_heads is a multiple of n_kv_heads and query head h reads KV head
 *    h / (n_q_heads / n_kv_heads).
 *  - Size limits of the bf16 head_dim-128 kernels (ESHAPE, before anything
 *    is enqueued): one layer of the pool below 4 GiB, and one page of one
 *    layer (n_kv_heads * page_size rows of 256 bytes) below 16 MiB, since
 *    row offsets are 32-bit byte offsets formed with 24-bit products.
 */
#ifndef ACACHE_H
#define ACACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden default visibility; the declarations of
 * this header are its only exported symbols. */
#if defined(__GNUC__)
#pragma GCC visibility push(default)
#endif

typedef void* acache_stream_t; /* hipStream_t */

enum acache_status {
  ACACHE_OK = 0,
  ACACHE_EINVAL = -1,     /* null pointer, bad scalar (rate, K, scale, layer range) */
  ACACHE_EDTYPE = -2,     /* unknown dtype */
  ACACHE_ESHAPE = -3,     /* unsupported head_dim / page_size / head grouping / size limit */
  ACACHE_ERANGE = -4,     /* slot or index out of range (checked mode, acache_validate_slots) */
  ACACHE_EREGION = -5,    /* slot outside the region its request may read or write (checked mode) */
  ACACHE_EDUP = -6,       /* duplicate scatter destination (checked mode) */
  ACACHE_EWORKSPACE = -7, /* workspace missing or too small */
  ACACHE_EDEVICE = -8,    /* HIP launch error */
  ACACHE_EALIGN = -9      /* pointer not 16-byte aligned */
};

enum acache_dtype { ACACHE_F32 = 0, ACACHE_BF16 = 1 };

/*
 * Paged KV pool (Section 4.1: KV lives in paged physical slots; the shared
 * region and each request's private region are sets of pages).
 * k, v: [n_layers][n_pages][n_kv_heads][page_size][head_dim], dtype `dtype`.
 * Physical slot s is page s / page_size, row s % page_size.
 */
typedef struct acache_kv_pool {
  void* k;
  void* v;
  int32_t dtype;
  int32_t n_layers;
  int32_t n_pages;
  int32_t page_size;
  int32_t n_kv_heads;
  int32_t head_dim;
} acache_kv_pool;

/* Library version (major*10000 + minor*100 + patch). */
int acache_version(void);

/* Static text for a status code. */
const char* acache_status_string(int status);

/*
 * Anchor count for an affix of L tokens at anchor ratio `rate` (Section 5,
 * Default Settings: ratios 0 to 1; ratio 0 is direct reuse, 1 is full
 * recomputation, Section 5.1).  K = ceil(rate * L - 1e-9), clamped to [0, L].
 * K_out (host).  EINVAL if rate is NaN or outside [0, 1], L < 0 or K_out NULL.
 */
int acache_anchor_count(int32_t L, double rate, int32_t* K_out);

/*
 * One-shot anchor probe, Section 3.2, Eq. (4)-(5).
 *
 * Every non-affix row of the batch attends over the L affix keys held in the
 * shared region (the affix KV is fixed past state; affix rows are not
 * forwarded):  O_aff = softmax(q K_aff^T * scale) V_aff,
 *               LSE_aff = logsumexp(q K_aff^T * scale)   (natural log).
 * For the initially masked rows k of request b the Eq. (4) weights
 * a_jk = exp(q_k . k_j * scale - LSE_aff,k) are summed over query heads,
 * masked rows and layers into scores[b][j]  (Eq. 5; the softmax normalises
 * over the affix keys, exactly as Eq. (4) writes it).
 *
 *  pool            pool; layers layer_begin .. layer_begin+n_layers-1 are read
 *  q               [n_layers][n_rows][n_q_heads][head_dim]: probe queries of
 *                  all non-affix rows of all requests (local layer index)
 *  n_rows          rows in q (any order; all rows share the affix)
 *  masked_rows     [n_masked] row indices into q of the initially masked rows,
 *                  request b's at masked_offsets[b] .. masked_offsets[b+1]-1
 *  masked_offsets  [B+1]
 *  n_masked        masked_offsets[B] (host copy, sizes the launch); at most n_rows
 *  max_masked      max over b of masked_offsets[b+1]-masked_offsets[b] (host;
 *                  a smaller value gives wrong scores for the longer requests)
 *  shared_slots    [L] physical slot of affix offset j
 *  scale           softmax scale, normally 1/sqrt(head_dim) (Eq. 4)
 *  scores          [B][L] fp32, ACCUMULATED (+=), so per-layer-group calls sum
 *                  to Eq. (5); the caller zeroes it once per request batch
 *  o_aff           nullable [n_layers][n_rows][n_q_heads][head_dim]
 *  lse_aff         nullable [n_layers][n_rows][n_q_heads] fp32
 *  workspace       >= acache_probe_workspace_bytes(...) bytes, 256-B aligned
 * Deterministic: the same inputs give the same bits (no atomics).
 */
int acache_probe_workspace_bytes(int32_t n_rows, int32_t B, int32_t L, int32_t n_q_heads,
                                 int32_t n_layers, int32_t lse_given, size_t* bytes /*host*/);

int acache_probe_scores(const acache_kv_pool* pool, const void* q, int32_t n_rows,
                        const int32_t* masked_rows, const int32_t* masked_offsets,
                        int32_t n_masked, int32_t max_masked, const int32_t* shared_slots,
                        int32_t L, int32_t B, int32_t n_q_heads, int32_t layer_begin,
                        int32_t n_layers, float scale, float* scores, void* o_aff,
                        float* lse_aff, void* workspace, size_t workspace_bytes,
                        acache_stream_t stream);

/*
 * The two halves of acache_probe_scores, for callers that schedule them
 * separately (same semantics, same arguments).
 *
 * acache_probe_attention: O_aff and LSE_aff of every probe row over the affix
 * (the O(N H P L) probe forward of Section 3.2).  lse_aff is required (the
 * column mass reads it); o_aff is nullable.  No workspace.
 *
 * acache_probe_column_mass: the Eq. (4) weights of the masked rows,
 * a_jk = exp(q_k . k_j * scale - LSE_aff,k), summed over query heads, masked
 * rows and layers and ADDED to scores[b][j] (Eq. 5), in a fixed order.  Reads
 * the lse_aff written by acache_probe_attention for the same q.  Workspace of
 * acache_probe_column_mass_workspace_bytes(...) bytes, 256-B aligned.
 */
int acache_probe_attention(const acache_kv_pool* pool, const void* q, int32_t n_rows,
                           const int32_t* shared_slots, int32_t L, int32_t n_q_heads,
                           int32_t layer_begin, int32_t n_layers, float scale, void* o_aff,
                           float* lse_aff, acache_stream_t stream);

int acache_probe_column_mass_workspace_bytes(int32_t n_rows, int32_t B, int32_t L, int32_t n_q_heads,
                                             int32_t n_layers, size_t* bytes /*host*/);

int acache_probe_column_mass(const acache_kv_pool* pool, const void* q, int32_t n_rows,
                             const int32_t* masked_rows, const int32_t* masked_offsets,
                             int32_t n_masked, int32_t max_masked, const int32_t* shared_slots,
                             int32_t L, int32_t B, int32_t n_q_heads, int32_t layer_begin,
                             int32_t n_layers, float scale, const float* lse_aff, float* scores,
                             void* workspace, size_t workspace_bytes, acache_stream_t stream);

/*
 * Arguments of the per-request maps (Section 4.1 dual mapping, Section 4.2
 * admission-time preparation).  All requests share the affix span
 * F = {affix_l .. affix_l+L-1} and its shared slots.
 *
 * For request b with logical length T_b = seq_len[b] and anchors A_b, the
 * recompute set R_b = A_b u ([0, T_b) \ F) is taken in ascending logical
 * order; its i-th member receives private slot
 *     private_pages[private_page_offsets[b] + i / page_size] * page_size + i % page_size.
 * Outputs:
 *   read_slot[kv_offsets[b] + p]  = shared_slots[p - affix_l] for p in F \ A_b,
 *                                   else the private slot of p;
 *   recompute_pos[rc_offsets[b] + i]  = i-th member of R_b (logical position);
 *   recompute_slot[rc_offsets[b] + i] = its private slot (the write-side map).
 * kv_offsets[b+1]-kv_offsets[b] must equal T_b and rc_offsets[b+1]-rc_offsets[b]
 * must equal K + T_b - L; request b needs ceil((K + T_b - L)/page_size) pages.
 * recompute_slot with rc_offsets is also the DropNA read table (Section 5.3,
 * Figure 5: the same anchors with the non-anchor affix cache discarded):
 * acache_mapped_attention over (recompute_slot, rc_offsets) is the DropNA
 * attention.
 */
typedef struct acache_map_args {
  int32_t B;
  int32_t affix_l;
  int32_t L;
  int32_t K;
  int32_t page_size;
  int32_t max_seq_len;               /* host: max T_b, sizes the launch */
  const int32_t* seq_len;            /* [B] */
  const int32_t* shared_slots;       /* [L] */
  const int32_t* private_pages;      /* flat page list */
  const int32_t* private_page_offsets; /* [B+1] */
  const int32_t* kv_offsets;         /* [B+1] */
  const int32_t* rc_offsets;         /* [B+1] */
  int32_t* read_slot;                /* out [kv_offsets[B]] */
  int32_t* recompute_pos;            /* out [rc_offsets[B]], nullable */
  int32_t* recompute_slot;           /* out [rc_offsets[B]], nullable */
} acache_map_args;

/*
 * Anchor set, Section 3.2, Eq. (6): A_b = TopK({scores[b][j]}, K), S = F \ A_b.
 * Exact radix select on the fp32 bit patterns: larger score first, equal
 * scores go to the lower offset j, NaN ranks below every number, -0 equals +0.
 * anchors [B][K] receives affix_l + j in ascending order.
 * L <= 32768.  If `maps` is not NULL the maps are then built from these
 * anchors on the same stream (maps->K, L, affix_l, B must agree).
 */
int acache_topk_anchors(const float* scores, int32_t B, int32_t L, int32_t K,
                        int32_t affix_l, int32_t* anchors, const acache_map_args* maps,
                        acache_stream_t stream);

/* Build the two maps from given anchors ([B][K], ascending, inside F). */
int acache_build_maps(const int32_t* anchors, const acache_map_args* maps,
                      acache_stream_t stream);

/*
 * Write-side scatter of recomputed K/V, Section 4.3 and Appendix C.1 (store
 * before attend).  For every local layer n, row i and KV head g:
 *   pool.k[layer_begin+n][slot dst_slots[i]][g][:] = k_src[n][i][g][:]  (same for v)
 * k_src, v_src: [n_layers][n_rows][n_kv_heads][head_dim], pool dtype.  A
 * bit-exact copy.  Destinations must be distinct private slots (checked on the
 * host by acache_validate_slots; duplicates would race).  n_rows = 0 is a no-op.
 */
int acache_scatter_private(const acache_kv_pool* pool, const void* k_src, const void* v_src,
                           const int32_t* dst_slots, int32_t n_rows, int32_t layer_begin,
                           int32_t n_layers, acache_stream_t stream);

/*
 * Destination slots of a decode block (Section 4.3, block decoding: the
 * block's KV goes to the private slots its positions read from):
 *   dst_slots[b*block_len + i] = read_slot[kv_offsets[b] + block_start[b] + i].
 */
int acache_block_slots(const int32_t* read_slot, const int32_t* kv_offsets,
                       const int32_t* block_start, int32_t B, int32_t block_len,
                       int32_t* dst_slots, acache_stream_t stream);

/*
 * Read-slot attention, Section 4.3 and Appendix C.1.  For request b, each of
 * its query rows r in q_offsets[b] .. q_offsets[b+1]-1 and query head h:
 *   O[r][h] = sum_{p < T_b} softmax_p(q[r][h] . K[s_p] * scale) V[s_p],
 *   s_p = read_slot[kv_offsets[b] + p], K/V of KV head h / (n_q_heads/n_kv_heads).
 * Bidirectional (no mask), ragged queries and keys, every logical position
 * read exactly once in logical order.
 *  q    [n_layers][n_q][n_q_heads][head_dim]; out the same shape (pool dtype);
 *  lse  nullable [n_layers][n_q][n_q_heads] fp32 (natural log).
 *  max_q_per_req, max_kv_per_req: host maxima that size the launch.
 * A request with T_b = 0 gets O = 0 and LSE = -inf.
 */
int acache_mapped_attention_workspace_bytes(int32_t B, int32_t n_q, int32_t n_q_heads,
                                            int32_t n_layers, size_t* bytes /*host*/);

int acache_mapped_attention(const acache_kv_pool* pool, const void* q, const int32_t* q_offsets,
                            int32_t n_q, int32_t max_q_per_req, const int32_t* read_slot,
                            const int32_t* kv_offsets, int32_t max_kv_per_req, int32_t B,
                            int32_t n_q_heads, int32_t layer_begin, int32_t n_layers, float scale,
                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                            acache_stream_t stream);

/*
 * Read-slot attention of a batch that shares one affix, Section 4.3 and
 * Appendix C.1 (the shared region is stored once and read by every request,
 * Section 4.1).  The result is defined exactly as for acache_mapped_attention
 * with the same q, read_slot and kv_offsets; the extra arguments only say
 * which slots the requests share, so that the shared region is read once per
 * group of requests instead of once per request:
 *   shared_slots [L]  slot of affix key j; position affix_l + j of request b
 *                     is read from the shared pass when
 *                     read_slot[kv_offsets[b] + affix_l + j] == shared_slots[j],
 *                     every other position from its own read slot.
 * Any read table gives the same result as acache_mapped_attention (up to fp32
 * summation order); the gain needs most affix positions routed to
 * shared_slots, as the maps of acache_build_maps / acache_topk_anchors do.
 * Decode blocks (max_q_per_req <= 32) of bf16 pools with head_dim 128 and
 * batches of B >= 2 requests take the two-pass path, unless each KV head
 * serves G > 1 query heads with G * max_q_per_req >= 128 (then the work is
 * bound by the matrix units, not by HBM reads); every other case runs
 * acache_mapped_attention itself, with no workspace needed (the size query
 * returns 0).
 * Requests must satisfy T_b <= max_kv_per_req (positions past it are not
 * read).  The workspace (size from the query below, given the same pool,
 * B, n_q, max_q_per_req, n_q_heads, n_layers, max_kv_per_req and L) holds
 * each request's list of non-shared read slots and its affix exclusion bits
 * (B * (4 * max_kv_per_req + L / 8) bytes, about); it is rewritten by every
 * call, so calls that share a workspace must not overlap.
 */
int acache_mapped_attention_shared_workspace_bytes(const acache_kv_pool* pool, int32_t B, int32_t n_q,
                                                   int32_t max_q_per_req, int32_t n_q_heads, int32_t n_layers,
                                                   int32_t max_kv_per_req, int32_t L, size_t* bytes /*host*/);

int acache_mapped_attention_shared(const acache_kv_pool* pool, const void* q, const int32_t* q_offsets,
                                   int32_t n_q, int32_t max_q_per_req, const int32_t* read_slot,
                                   const int32_t* kv_offsets, int32_t max_kv_per_req,
                                   const int32_t* shared_slots, int32_t affix_l, int32_t L, int32_t B,
                                   int32_t n_q_heads, int32_t layer_begin, int32_t n_layers, float scale,
                                   void* out, float* lse, void* workspace, size_t workspace_bytes,
                                   acache_stream_t stream);

/*
 * acache_mapped_attention_shared for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and result, without the workspace: the plan lives in a fixed
 * device array of the library, 8 MiB on each GPU it runs on (held until the
 * process ends), taken on the current device (hipGetDevice; the stream must
 * belong to it).  The call allocates nothing.  A call whose plan needs more
 * than 8 MiB (the size acache_mapped_attention_shared_workspace_bytes reports
 * for the same arguments) returns EWORKSPACE with nothing enqueued.  Every
 * call on one GPU shares the array: calls that overlap on one GPU (other
 * streams, or other host threads) race and must not be issued.
 */
int acache_mapped_attention_shared_noalloc(const acache_kv_pool* pool, const void* q,
                                           const int32_t* q_offsets, int32_t n_q, int32_t max_q_per_req,
                                           const int32_t* read_slot, const int32_t* kv_offsets,
                                           int32_t max_kv_per_req, const int32_t* shared_slots,
                                           int32_t affix_l, int32_t L, int32_t B, int32_t n_q_heads,
                                           int32_t layer_begin, int32_t n_layers, float scale, void* out,
                                           float* lse, acache_stream_t stream);

/*
 * Store-then-attend of the recompute phase, Section 4.3 and Appendix C.1:
 * the recomputed K/V rows are written to their private slots through the
 * write-side map and the attention reads the full context through the
 * read-slot map.  The result is defined as
 *   acache_scatter_private(pool, k_src, v_src, src_slot, n_src, ...);
 *   acache_mapped_attention(pool, q, q_offsets, ..., read_slot, kv_offsets, ...);
 * on the same stream: pool slots src_slot[i] hold the source rows afterwards,
 * and out / lse are those of the attention.
 *  k_src, v_src [n_layers][n_src][n_kv_heads][head_dim] (pool dtype, 16-byte
 *               aligned); request b's rows are src_offsets[b] .. src_offsets[b+1]
 *               (src_offsets [B+1], always given) and row i holds logical
 *               position src_pos[i] of its request, to be stored at src_slot[i].
 *  q, q_offsets, n_q, max_q_per_req, read_slot, kv_offsets, max_kv_per_req,
 *  out, lse    as for acache_mapped_attention.
 * For bf16 pools with head_dim 128, one query head per KV head and
 * max_q_per_req <= 3072, one plan kernel and one attention kernel run: each
 * request's rows attend to its source rows (read from k_src / v_src) and
 * then to its read list without its src_pos positions (read from the pool),
 * while the row tiles of each (layer, KV head, request) copy its source rows
 * to src_slot, a slice each.  That equals the definition when, as the maps
 * of acache_build_maps arrange for the recompute set, each src_slot[i] is
 * read at position src_pos[i] of request b (read_slot[kv_offsets[b] +
 * src_pos[i]] == src_slot[i]) and at no other position of any request; keys
 * are then summed in another order (fp32 rounding only).  Other pools,
 * grouped query heads (fewer rows to store beside the attention), more query
 * rows per request (each row tile reads every source row of its request), or
 * calls without query rows, run the two calls of the definition, which are
 * faster there, and leave the workspace unused.
 * Workspace: size from acache_store_attend_workspace_bytes (given the same
 * pool, B, max_q_per_req and max_kv_per_req; about 4 * B * max_kv_per_req
 * bytes, or 0 when no call with that pool and max_q_per_req can take the
 * one-kernel path), 16-byte aligned, rewritten by every call (calls sharing
 * it must not overlap).  max_kv_per_req <= 262144 on the one-kernel path.
 * Errors as for the two calls; EWORKSPACE when the workspace is missing or
 * small.  Nothing is enqueued when an error is returned.
 */
int acache_store_attend_workspace_bytes(const acache_kv_pool* pool, int32_t B, int32_t max_q_per_req,
                                        int32_t max_kv_per_req, size_t* bytes /*host*/);

int acache_store_attend(const acache_kv_pool* pool, const void* k_src, const void* v_src,
                        const int32_t* src_pos, const int32_t* src_slot, const int32_t* src_offsets,
                        int32_t n_src, const void* q, const int32_t* q_offsets, int32_t n_q,
                        int32_t max_q_per_req, const int32_t* read_slot, const int32_t* kv_offsets,
                        int32_t max_kv_per_req, int32_t B, int32_t n_q_heads, int32_t layer_begin,
                        int32_t n_layers, float scale, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, acache_stream_t stream);

/*
 * CacheBlend-style HKVD selector scores (Appendix B.5: the alternative anchor
 * selector the paper compares against ranks affix tokens by the KV
 * difference between the affix-only cache and the full-prompt cache):
 *   scores[b][j] += sum over layers, KV heads and head_dim of
 *                   (K_full - K_aff)^2 + (V_full - V_aff)^2,
 * K_aff / V_aff the shared region's rows at slot shared_slots[j] in layer
 * layer_begin + n, and k_full / v_full [n_layers][B][L][n_kv_heads][head_dim]
 * (pool dtype, 16-byte aligned) the full-prompt K and V of the affix tokens.
 * The squared L2 norm of each token's whole KV difference: its Top-K
 * (acache_topk_anchors) is that of the norm.  scores [B][L] fp32 is
 * accumulated (zero it first).  Errors as for acache_probe_scores.
 */
int acache_hkvd_scores(const acache_kv_pool* pool, const int32_t* shared_slots, int32_t L, const void* k_full,
                       const void* v_full, int32_t B, int32_t layer_begin, int32_t n_layers, float* scores,
                       acache_stream_t stream);

/*
 * Merge of two attentions of the same query rows over disjoint key sets, as
 * one softmax over their union.  Used for the full-context reading of the
 * probe normaliser (Eq. (4), Section 3.2): the non-affix rows' attention
 * over the affix (acache_probe_attention) merged with their attention over
 * their own non-affix keys (acache_mapped_attention), whose merged LSE then
 * feeds acache_probe_column_mass.  For every (row, head) pair i:
 *   lse[i] = log(exp(lse_a[i]) + exp(lse_b[i]))            (natural log),
 *   o[i][:] = exp(lse_a[i] - lse[i]) o_a[i][:] + exp(lse_b[i] - lse[i]) o_b[i][:],
 * and o = 0, lse = -inf when both parts are empty (-inf).
 *  o_a, o_b, o  [n_pairs][head_dim] of `dtype` (nullable together: LSE only);
 *  lse_a, lse_b, lse  [n_pairs] fp32.  o may be o_a and lse may be lse_a.
 * EINVAL for NULL LSE pointers, a partial set of O pointers or n_pairs < 0;
 * ESHAPE for head_dim outside {16, 32, 64, 128}; EALIGN for O pointers.
 */
int acache_lse_merge(int32_t dtype, int64_t n_pairs, int32_t head_dim, const void* o_a, const float* lse_a,
                     const void* o_b, const float* lse_b, void* o, float* lse, acache_stream_t stream);

/*
 * KV-cache footprint with every request resident (host arithmetic; all
 * pointers host).  Section 4.1: one shared region holds the affix once and
 * each request's private region holds its recompute set R_b (anchors and
 * request positions, K + seq_len[b] - L slots); Appendix B.2: the regions
 * are allocated at block (page) granularity.  In pages:
 *   shared  = ceil(L / page_size)                     (0 when B = 0),
 *   private = sum_b ceil((K + seq_len[b] - L) / page_size),
 *   dense   = sum_b ceil(seq_len[b] / page_size)      (no sharing: every
 *             request holds its whole context, the baseline cache);
 * each page is page_size * n_layers * n_kv_heads * head_dim * 2 (K and V)
 * elements of `dtype`.  The DropNA cache is the private pages alone.
 * EINVAL for a NULL output or seq_len (with B > 0), negative sizes,
 * K > L or seq_len[b] < L; EDTYPE for an unknown dtype.
 */
int acache_kv_footprint(int32_t B, const int32_t* seq_len /*host*/, int32_t L, int32_t K,
                        int32_t page_size, int32_t n_layers, int32_t n_kv_heads, int32_t head_dim,
                        int32_t dtype, uint64_t* shared_bytes, uint64_t* private_bytes,
                        uint64_t* dense_bytes);

/*
 * Host-side check of slot tables (all pointers host).  page_owner[p] is -1
 * for a shared page, b for a page private to request b, -2 for a free page.
 * Checks every slots[i] is in [0, n_pages*page_size) (ERANGE), lies in a page
 * private to owner[i] (or to any request when owner is NULL) (EREGION), and,
 * when `distinct` is non-zero, that no slot repeats (EDUP).
 * bad_index (host, nullable) receives the first offending i.
 */
int acache_validate_slots(const int32_t* slots, int32_t n, const int32_t* owner,
                          const int32_t* page_owner, int32_t n_pages, int32_t page_size,
                          int32_t distinct, int32_t* bad_index);

/*
 * Checked mode: a device pre-pass over a slot table (Section 4.1: requests
 * read the shared region and their own private slots and write only their
 * own private slots; Appendix C.1: the store writes through the write-side
 * map before the read-slot kernel reads through the read-slot map).
 *
 *  slots       [n] physical slots (device); segment b is
 *              slots[offsets[b] .. offsets[b+1]), request b's entries
 *  offsets     [B+1] (device), nullable with B = 0: one segment with no
 *              request (a table of the shared region, such as shared_slots)
 *  page_owner  [n_pages] (device), nullable: -1 shared page, b private to
 *              request b, -2 free.  Without it only ranges and duplicates
 *              are checked
 *  mode        ACACHE_CHECK_READ: every slot in range and, with page_owner,
 *              in a shared page or a page of its own segment's request (one
 *              segment without offsets: shared pages only);
 *              ACACHE_CHECK_WRITE: every slot in range, with page_owner in a
 *              page of its own segment's request (without offsets: of some
 *              request), and no slot named twice over all segments
 *  bad_index   (host, nullable) receives the smallest failing entry of the
 *              class returned (-1: the offsets table itself)
 *  workspace   >= acache_check_slots_workspace_bytes(n_pages, page_size,
 *              mode) bytes, 256-B aligned (4 bytes per pool slot in write
 *              mode)
 * Returns the first failing class in this order: ERANGE (a slot outside
 * [0, n_pages * page_size), or offsets not rising from 0 to n), EREGION,
 * EDUP; else OK.  The pre-pass reads the tables, offsets and page owners,
 * never the pool.  The call waits for the stream (it reads the result back),
 * so it cannot be captured in a graph.  EINVAL for bad sizes, a NULL table
 * or mode; EWORKSPACE for a missing or short workspace.
 */
enum acache_check_mode { ACACHE_CHECK_READ = 0, ACACHE_CHECK_WRITE = 1 };

int acache_check_slots_workspace_bytes(int32_t n_pages, int32_t page_size, int32_t mode,
                                       size_t* bytes /*host*/);

int acache_check_slots(const int32_t* slots, int32_t n, const int32_t* offsets, int32_t B,
                       const int32_t* page_owner, int32_t n_pages, int32_t page_size, int32_t mode,
                       int32_t* bad_index, void* workspace, size_t workspace_bytes,
                       acache_stream_t stream);

/*
 * acache_scatter_private in checked mode (Section 4.1, Section 4.3,
 * Appendix C.1): the write-mode pre-pass of acache_check_slots over dst_slots
 * (row_offsets [B+1] assigns rows to requests; page_owner as above), then the
 * scatter only when it passes.  On ERANGE, EREGION or EDUP nothing is
 * written to the pool.  Same arguments as acache_scatter_private plus those
 * of the check; waits for the stream like acache_check_slots.
 */
int acache_scatter_private_checked(const acache_kv_pool* pool, const void* k_src, const void* v_src,
                                   const int32_t* dst_slots, int32_t n_rows, const int32_t* row_offsets,
                                   int32_t B, const int32_t* page_owner, int32_t layer_begin,
                                   int32_t n_layers, int32_t* bad_index, void* workspace,
                                   size_t workspace_bytes, acache_stream_t stream);

#if defined(__GNUC__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif /* ACACHE_H */

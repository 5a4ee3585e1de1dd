// Host-side launchers of the ACache kernels (internal to the library; the C
// ABI in acache_api.hip validates arguments and calls these).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "acache_dev.h"

namespace acache {

// Attention over a slot-table key list.  With q_offsets == nullptr every
// query row attends to the single key list kv_table[0 .. n_kv) (the probe
// over the shared affix); otherwise request b's rows q_offsets[b] ..
// q_offsets[b+1] attend to kv_table[kv_offsets[b] .. kv_offsets[b+1]).
struct AttnArgs {
  const void* q;
  const void* pool_k;
  const void* pool_v;
  PoolGeom geo;
  const int32_t* q_offsets;
  int n_q;       // rows of q per layer
  int max_q;     // max rows per request (grid sizing)
  const int32_t* kv_table;
  const int32_t* kv_offsets;
  int n_kv;      // keys when kv_offsets == nullptr
  int max_kv;    // max keys per request
  int B;
  int n_q_heads;
  int layer_begin;
  int n_layers;
  float scale;
  void* out;
  float* lse;
};

// Read-slot attention for decode blocks (at most 32 rows per request) whose
// read tables mostly route the affix to the shared region: every request's
// rows attend to the affix keys shared_slots[0 .. L) minus the keys flagged
// in excl (read once per group of four requests) and to their own list
// priv_slots[b * priv_stride .. + priv_counts[b]), in one softmax.
struct SharedAttnArgs {
  const void* q;
  const void* pool_k;
  const void* pool_v;
  PoolGeom geo;
  const int32_t* q_offsets;
  int n_q;
  int max_q;
  const int32_t* shared_slots;
  int L;
  const uint32_t* excl;
  int excl_words;
  const int32_t* priv_slots;
  const int32_t* priv_counts;
  int priv_stride;
  int B;
  int n_q_heads;
  int layer_begin;
  int n_layers;
  float scale;
  void* out;
  float* lse;
};

// Column mass of the masked rows (Eq. 4 weights summed over heads and rows)
// into partial[n][b][j].
struct ColmassArgs {
  const void* q;
  const void* pool_k;
  PoolGeom geo;
  const int32_t* masked_rows;
  const int32_t* masked_offsets;
  int n_masked;    // entries of masked_rows
  int max_masked;
  const int32_t* shared_slots;
  int L;
  int n_rows;
  int n_q_heads;
  int layer_begin;
  int n_layers;
  int B;
  float scale;
  const float* lse;
  float* partial;
  // MFMA path: each masked row's LSE scaled to -LSE/scale, per (layer, query
  // head), every request's rows padded with -inf to whole 32-row tiles
  // (request b's rows start at masked_offsets[b] + 31 * b); lse_stride floats
  // per (layer, query head)
  float* lse_prep;
  size_t lse_stride;
};

hipError_t launch_topk(const float* scores, int B, int L, int K, int affix_l, int32_t* anchors, hipStream_t st);
hipError_t launch_maps(const int32_t* anchors, const acache_map_args& a, hipStream_t st);
// Per request b: priv_slots[b * stride ..] = read slots of the positions not
// read from the shared region (ascending, padded with the last one to a
// multiple of pad entries), priv_counts[b] their number, and the exclusion
// bits of the affix keys (see SharedAttnArgs).  Positions past max_kv are
// ignored; stride >= max_kv rounded up to a multiple of pad.
hipError_t launch_shared_plan(const int32_t* read_slot, const int32_t* kv_offsets, const int32_t* shared_slots,
                              int B, int affix_l, int L, int max_kv, int stride, int pad, int32_t* priv_slots,
                              int32_t* priv_counts, uint32_t* excl, int excl_words, hipStream_t st);
constexpr int kSharedPrivTile = 32;  // private-list tile of attn_shared_mfma

// Store-then-attend plan: per request, the read list without the positions
// that the call stores (src_pos of src_offsets[b] .. src_offsets[b+1]), in
// position order, into other_slots[b * stride ..], its length into
// other_counts[b].  max_kv <= kStorePlanMaxKv (the position bitmap of one
// request lives in LDS); stride >= max_kv.
constexpr int kStorePlanMaxKv = 1 << 18;
hipError_t launch_store_plan(const int32_t* read_slot, const int32_t* kv_offsets, const int32_t* src_pos,
                             const int32_t* src_offsets, int B, int max_kv, int stride, int32_t* other_slots,
                             int32_t* other_counts, hipStream_t st);
// Checked mode: the pre-pass over a slot table (k_check.hip).  rec[0..2]
// receive the smallest failing entry of ERANGE, EREGION and EDUP (INT32_MAX:
// none); first is n_slots int32 of scratch in write mode.
hipError_t launch_check_slots(const int32_t* slots, int n, const int32_t* offsets, int B,
                              const int32_t* page_owner, int64_t n_slots, int page_shift, int write_mode,
                              int32_t* rec, int32_t* first, hipStream_t stream);

hipError_t launch_block_slots(const int32_t* read_slot, const int32_t* kv_offsets, const int32_t* block_start,
                              int B, int block_len, int32_t* dst, hipStream_t st);
hipError_t launch_scatter(void* pool_k, void* pool_v, const void* k_src, const void* v_src, const int32_t* dst,
                          int n_rows, int layer_begin, int n_layers, const PoolGeom& geo, int elem_bytes,
                          hipStream_t st);

hipError_t launch_lse_merge(int dtype, long long n_pairs, int head_dim, const void* oa, const float* la,
                            const void* ob, const float* lb, void* o, float* l, hipStream_t st);

hipError_t launch_hkvd(const void* pool_k, const void* pool_v, const PoolGeom& geo, const int32_t* shared_slots,
                       const void* kf, const void* vf, int B, int L, int layer_begin, int n_layers, int dtype,
                       float* scores, hipStream_t st);

hipError_t launch_attn_generic(const AttnArgs& a, int dtype, hipStream_t st);
hipError_t launch_colmass_generic(const ColmassArgs& a, int dtype, hipStream_t st);
hipError_t launch_colmass_reduce(const float* partial, int n_rows, int B, int L, float* scores, hipStream_t st);

// bf16, head_dim 128, MFMA kernels (k_attn_mfma.hip)
bool mfma_supported(int dtype, int head_dim);

// Query heads per KV head that the many-query MFMA kernel packs into the rows
// of one unit, or 0 for no packing: packing pays when a KV-head group holds
// several query heads and either the requests have more than 32 rows or the
// group's rows fill a 128-row tile (the K/V tiles then serve every head of
// the group instead of being streamed once per head).
inline int gqa_pack(int n_q_heads, int n_kv_heads, int max_q) {
  const int G = n_kv_heads > 0 ? n_q_heads / n_kv_heads : 1;
  return (G > 1 && (max_q > 32 || (long long)G * max_q >= 128)) ? G : 0;
}
// Units of at least this many query rows (after packing) take the many-query
// kernel with 48 rows per wave on the 16x16x32 MFMA (192-row tiles); smaller
// ones the 32-row tile loop (128-row tiles), where a 192-row tile would leave
// too many waves without rows.
constexpr long long kRows48MinRows = 384;
// The MFMA launches check the sizes their kernels index with 32 bits;
// dry_run = true checks them (same return value) and launches nothing, so
// that a call made of several launches can reject its arguments before it
// enqueues anything.
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t st, bool dry_run = false);
hipError_t launch_attn_mfma_shared(const SharedAttnArgs& a, hipStream_t st, bool dry_run = false);

// Store-then-attend, many-query MFMA path: request b's rows attend to
// other_slots[b * other_stride .. + other_counts[b]) (pool slots) and to rows
// src_offsets[b] .. src_offsets[b+1] of k_src / v_src
// ([n_layers][n_src][n_kv_heads][128]), which are also copied to pool slots
// src_slot[i] of the same layers.
struct StoreAttnArgs {
  const void* q;
  void* pool_k;
  void* pool_v;
  PoolGeom geo;
  const int32_t* q_offsets;
  int n_q;
  int max_q;
  const int32_t* other_slots;
  const int32_t* other_counts;
  int other_stride;
  const void* k_src;
  const void* v_src;
  const int32_t* src_slot;
  const int32_t* src_offsets;
  int n_src;
  int B;
  int n_q_heads;
  int layer_begin;
  int n_layers;
  float scale;
  void* out;
  float* lse;
};
hipError_t launch_attn_mfma_store(const StoreAttnArgs& a, hipStream_t st, bool dry_run = false);
hipError_t launch_colmass_mfma(const ColmassArgs& a, hipStream_t st, bool dry_run = false);

}  // namespace acache

// C ABI of the ACache engine: argument validation, workspace sizing and
// kernel dispatch.  Declarations and semantics: include/acache.h.
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "acache_dev.h"
#include "acache_launch.h"

using namespace acache;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == ACACHE_F32 ? 4 : 2; }

int check_pool(const acache_kv_pool* p) {
  if (!p || !p->k || !p->v) return ACACHE_EINVAL;
  if (p->dtype != ACACHE_F32 && p->dtype != ACACHE_BF16) return ACACHE_EDTYPE;
  if (p->n_layers <= 0 || p->n_pages <= 0 || p->n_kv_heads <= 0) return ACACHE_ESHAPE;
  const int hd = p->head_dim;
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128) return ACACHE_ESHAPE;
  const int ps = p->page_size;
  if (ps <= 0 || ps > 256 || (ps & (ps - 1))) return ACACHE_ESHAPE;
  if ((int64_t)p->n_pages * ps > INT32_MAX) return ACACHE_ESHAPE;
  if (!aligned16(p->k) || !aligned16(p->v)) return ACACHE_EALIGN;
  return ACACHE_OK;
}

int check_layers(const acache_kv_pool* p, int layer_begin, int n_layers) {
  if (layer_begin < 0 || n_layers < 0 || (int64_t)layer_begin + n_layers > p->n_layers) return ACACHE_EINVAL;
  return ACACHE_OK;
}

int check_heads(const acache_kv_pool* p, int n_q_heads) {
  if (n_q_heads <= 0 || n_q_heads % p->n_kv_heads != 0) return ACACHE_ESHAPE;
  if (n_q_heads > 1024) return ACACHE_ESHAPE;
  return ACACHE_OK;
}

PoolGeom geom_of(const acache_kv_pool* p) {
  PoolGeom g;
  g.n_pages = p->n_pages;
  g.page_size = p->page_size;
  int s = 0;
  while ((1 << s) < p->page_size) ++s;
  g.page_shift = s;
  g.n_kv_heads = p->n_kv_heads;
  g.head_dim = p->head_dim;
  return g;
}

int status_of(hipError_t e) { return e == hipSuccess ? ACACHE_OK : ACACHE_EDEVICE; }

// a dry run that rejects the sizes: a limit of the kernels' 32-bit indexing
int limits_of(hipError_t e) { return e == hipSuccess ? ACACHE_OK : ACACHE_ESHAPE; }

int check_map_args(const acache_map_args* m) {
  if (!m) return ACACHE_EINVAL;
  if (m->B < 0 || m->L <= 0 || m->affix_l < 0 || m->K < 0 || m->K > m->L || m->max_seq_len < 0)
    return ACACHE_EINVAL;
  if (m->page_size <= 0 || m->page_size > 256 || (m->page_size & (m->page_size - 1))) return ACACHE_ESHAPE;
  if (m->B > 65535) return ACACHE_ESHAPE;
  if (m->B > 0 && (!m->seq_len || !m->shared_slots || !m->private_pages || !m->private_page_offsets ||
                   !m->kv_offsets || !m->rc_offsets || !m->read_slot))
    return ACACHE_EINVAL;
  return ACACHE_OK;
}

}  // namespace

extern "C" {

int acache_version(void) { return 100; }

const char* acache_status_string(int s) {
  switch (s) {
    case ACACHE_OK: return "ok";
    case ACACHE_EINVAL: return "invalid argument";
    case ACACHE_EDTYPE: return "unsupported dtype";
    case ACACHE_ESHAPE: return "unsupported shape";
    case ACACHE_ERANGE: return "slot or index out of range";
    case ACACHE_EREGION: return "slot outside the request's private region";
    case ACACHE_EDUP: return "duplicate destination slot";
    case ACACHE_EWORKSPACE: return "workspace missing or too small";
    case ACACHE_EDEVICE: return "HIP launch error";
    case ACACHE_EALIGN: return "pointer not 16-byte aligned";
    default: return "unknown status";
  }
}

int acache_anchor_count(int32_t L, double rate, int32_t* K_out) {
  if (!K_out || L < 0 || !(rate >= 0.0 && rate <= 1.0)) return ACACHE_EINVAL;
  double k = ceil(rate * (double)L - 1e-9);
  if (k < 0) k = 0;
  if (k > L) k = L;
  *K_out = (int32_t)k;
  return ACACHE_OK;
}

int acache_probe_column_mass_workspace_bytes(int32_t n_rows, int32_t B, int32_t L, int32_t n_q_heads,
                                             int32_t n_layers, size_t* bytes) {
  if (!bytes || n_rows < 0 || B < 0 || L < 0 || n_q_heads < 0 || n_layers < 0) return ACACHE_EINVAL;
  // partial column masses: one per (layer, query head, request, key) on the
  // MFMA path, one per (layer, request, key) on the vector path; then the
  // masked rows' scaled LSE per (layer, query head), every request padded to
  // whole 32-row tiles (at most n_rows + 31 * B values)
  *bytes = align_up((size_t)n_layers * n_q_heads * B * L * sizeof(float)) +
           align_up((size_t)n_layers * n_q_heads * ((size_t)n_rows + 31 * (size_t)B) * sizeof(float));
  return ACACHE_OK;
}

int acache_probe_workspace_bytes(int32_t n_rows, int32_t B, int32_t L, int32_t n_q_heads, int32_t n_layers,
                                 int32_t lse_given, size_t* bytes) {
  if (!bytes || n_rows < 0 || B < 0 || L < 0 || n_q_heads < 0 || n_layers < 0) return ACACHE_EINVAL;
  size_t ws = 0;
  if (!lse_given) ws += align_up((size_t)n_layers * n_rows * n_q_heads * sizeof(float));
  size_t cm = 0;
  acache_probe_column_mass_workspace_bytes(n_rows, B, L, n_q_heads, n_layers, &cm);
  *bytes = ws + cm;
  return ACACHE_OK;
}

}  // extern "C"

namespace {

int check_probe_common(const acache_kv_pool* pool, const void* q, int32_t n_rows, const int32_t* shared_slots,
                       int32_t L, int32_t n_q_heads, int32_t layer_begin, int32_t n_layers, float scale) {
  int st;
  if ((st = check_pool(pool))) return st;
  if ((st = check_layers(pool, layer_begin, n_layers))) return st;
  if ((st = check_heads(pool, n_q_heads))) return st;
  if (n_rows < 0 || L <= 0) return ACACHE_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ACACHE_EINVAL;
  if (L > (1 << 24)) return ACACHE_ESHAPE;
  if (!shared_slots) return ACACHE_EINVAL;
  if (n_rows > 0 && !q) return ACACHE_EINVAL;
  if (q && !aligned16(q)) return ACACHE_EALIGN;
  return ACACHE_OK;
}

hipError_t probe_attention_launch(const acache_kv_pool* pool, const void* q, int32_t n_rows,
                                  const int32_t* shared_slots, int32_t L, int32_t n_q_heads, int32_t layer_begin,
                                  int32_t n_layers, float scale, void* o_aff, float* lse, hipStream_t s,
                                  bool dry = false) {
  if (n_rows == 0 || n_layers == 0) return hipSuccess;
  AttnArgs a;
  a.q = q;
  a.pool_k = pool->k;
  a.pool_v = pool->v;
  a.geo = geom_of(pool);
  a.q_offsets = nullptr;
  a.n_q = n_rows;
  a.max_q = n_rows;
  a.kv_table = shared_slots;
  a.kv_offsets = nullptr;
  a.n_kv = L;
  a.max_kv = L;
  a.B = 1;
  a.n_q_heads = n_q_heads;
  a.layer_begin = layer_begin;
  a.n_layers = n_layers;
  a.scale = scale;
  a.out = o_aff;
  a.lse = lse;
  if (mfma_supported(pool->dtype, pool->head_dim)) return launch_attn_mfma(a, s, dry);
  return dry ? hipSuccess : launch_attn_generic(a, pool->dtype, s);
}

hipError_t probe_column_mass_launch(const acache_kv_pool* pool, const void* q, int32_t n_rows,
                                    const int32_t* masked_rows, const int32_t* masked_offsets, int32_t n_masked,
                                    int32_t max_masked,
                                    const int32_t* shared_slots, int32_t L, int32_t B, int32_t n_q_heads,
                                    int32_t layer_begin, int32_t n_layers, float scale, const float* lse,
                                    float* scores, float* partial, hipStream_t s, bool dry = false) {
  if (n_layers == 0 || B == 0) return hipSuccess;
  ColmassArgs c;
  c.q = q;
  c.pool_k = pool->k;
  c.geo = geom_of(pool);
  c.masked_rows = masked_rows;
  c.masked_offsets = masked_offsets;
  c.n_masked = n_masked;
  c.max_masked = max_masked;
  c.shared_slots = shared_slots;
  c.L = L;
  c.n_rows = n_rows;
  c.n_q_heads = n_q_heads;
  c.layer_begin = layer_begin;
  c.n_layers = n_layers;
  c.B = B;
  c.scale = scale;
  c.lse = lse;
  c.partial = partial;
  c.lse_stride = (size_t)n_rows + 31 * (size_t)B;
  c.lse_prep = partial + align_up((size_t)n_layers * n_q_heads * B * L * sizeof(float)) / sizeof(float);
  const bool mf = mfma_supported(pool->dtype, pool->head_dim);
  if (dry) return mf ? launch_colmass_mfma(c, s, true) : hipSuccess;
  hipError_t e = mf ? launch_colmass_mfma(c, s) : launch_colmass_generic(c, pool->dtype, s);
  if (e != hipSuccess) return e;
  return launch_colmass_reduce(partial, mf ? n_layers * n_q_heads : n_layers, B, L, scores, s);
}

}  // namespace

extern "C" {

int acache_probe_attention(const acache_kv_pool* pool, const void* q, int32_t n_rows, const int32_t* shared_slots,
                           int32_t L, int32_t n_q_heads, int32_t layer_begin, int32_t n_layers, float scale,
                           void* o_aff, float* lse_aff, acache_stream_t stream) {
  int st;
  if ((st = check_probe_common(pool, q, n_rows, shared_slots, L, n_q_heads, layer_begin, n_layers, scale)))
    return st;
  if (!lse_aff) return ACACHE_EINVAL;
  if (o_aff && !aligned16(o_aff)) return ACACHE_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  if ((st = limits_of(probe_attention_launch(pool, q, n_rows, shared_slots, L, n_q_heads, layer_begin, n_layers,
                                             scale, o_aff, lse_aff, s, true))))
    return st;
  return status_of(probe_attention_launch(pool, q, n_rows, shared_slots, L, n_q_heads, layer_begin, n_layers, scale,
                                          o_aff, lse_aff, s));
}

int acache_probe_column_mass(const acache_kv_pool* pool, const void* q, int32_t n_rows, const int32_t* masked_rows,
                             const int32_t* masked_offsets, int32_t n_masked, int32_t max_masked,
                             const int32_t* shared_slots, int32_t L, int32_t B, int32_t n_q_heads,
                             int32_t layer_begin, int32_t n_layers, float scale, const float* lse_aff,
                             float* scores, void* workspace, size_t workspace_bytes, acache_stream_t stream) {
  int st;
  if ((st = check_probe_common(pool, q, n_rows, shared_slots, L, n_q_heads, layer_begin, n_layers, scale)))
    return st;
  if (B < 0 || n_masked < 0 || n_masked > n_rows || max_masked < 0 || max_masked > n_masked) return ACACHE_EINVAL;
  if (B > 65535) return ACACHE_ESHAPE;
  if (!scores || !lse_aff) return ACACHE_EINVAL;
  if (n_masked > 0 && !masked_rows) return ACACHE_EINVAL;
  if (B > 0 && !masked_offsets) return ACACHE_EINVAL;
  size_t need = 0;
  acache_probe_column_mass_workspace_bytes(n_rows, B, L, n_q_heads, n_layers, &need);
  if (workspace_bytes < need || (need > 0 && !workspace) || ((uintptr_t)workspace & (kAlign - 1)))
    return ACACHE_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if ((st = limits_of(probe_column_mass_launch(pool, q, n_rows, masked_rows, masked_offsets, n_masked, max_masked, shared_slots,
                                               L, B, n_q_heads, layer_begin, n_layers, scale, lse_aff, scores,
                                               (float*)workspace, s, true))))
    return st;
  return status_of(probe_column_mass_launch(pool, q, n_rows, masked_rows, masked_offsets, n_masked, max_masked, shared_slots, L,
                                            B, n_q_heads, layer_begin, n_layers, scale, lse_aff, scores,
                                            (float*)workspace, s));
}

int acache_probe_scores(const acache_kv_pool* pool, const void* q, int32_t n_rows, const int32_t* masked_rows,
                        const int32_t* masked_offsets, int32_t n_masked, int32_t max_masked,
                        const int32_t* shared_slots, int32_t L, int32_t B, int32_t n_q_heads,
                        int32_t layer_begin, int32_t n_layers, float scale, float* scores, void* o_aff,
                        float* lse_aff, void* workspace, size_t workspace_bytes, acache_stream_t stream) {
  int st;
  if ((st = check_probe_common(pool, q, n_rows, shared_slots, L, n_q_heads, layer_begin, n_layers, scale)))
    return st;
  if (B < 0 || n_masked < 0 || n_masked > n_rows || max_masked < 0 || max_masked > n_masked) return ACACHE_EINVAL;
  if (B > 65535) return ACACHE_ESHAPE;
  if (!scores) return ACACHE_EINVAL;
  if (n_masked > 0 && !masked_rows) return ACACHE_EINVAL;
  if (B > 0 && !masked_offsets) return ACACHE_EINVAL;
  if (o_aff && !aligned16(o_aff)) return ACACHE_EALIGN;
  size_t need = 0;
  acache_probe_workspace_bytes(n_rows, B, L, n_q_heads, n_layers, lse_aff != nullptr, &need);
  if (workspace_bytes < need || (need > 0 && !workspace) || ((uintptr_t)workspace & (kAlign - 1)))
    return ACACHE_EWORKSPACE;
  if (n_layers == 0 || B == 0) return ACACHE_OK;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* lse = lse_aff;
  if (!lse) {
    lse = (float*)ws;
    ws += align_up((size_t)n_layers * n_rows * n_q_heads * sizeof(float));
  }
  if ((st = limits_of(probe_attention_launch(pool, q, n_rows, shared_slots, L, n_q_heads, layer_begin, n_layers,
                                             scale, o_aff, lse, s, true))))
    return st;
  if ((st = limits_of(probe_column_mass_launch(pool, q, n_rows, masked_rows, masked_offsets, n_masked, max_masked, shared_slots,
                                               L, B, n_q_heads, layer_begin, n_layers, scale, lse, scores, (float*)ws,
                                               s, true))))
    return st;
  hipError_t e = probe_attention_launch(pool, q, n_rows, shared_slots, L, n_q_heads, layer_begin, n_layers, scale,
                                        o_aff, lse, s);
  if (e != hipSuccess) return ACACHE_EDEVICE;
  return status_of(probe_column_mass_launch(pool, q, n_rows, masked_rows, masked_offsets, n_masked, max_masked, shared_slots, L,
                                            B, n_q_heads, layer_begin, n_layers, scale, lse, scores, (float*)ws, s));
}

int acache_build_maps(const int32_t* anchors, const acache_map_args* maps, acache_stream_t stream) {
  int st;
  if ((st = check_map_args(maps))) return st;
  if (maps->K > 0 && maps->B > 0 && !anchors) return ACACHE_EINVAL;
  return status_of(launch_maps(anchors, *maps, (hipStream_t)stream));
}

int acache_topk_anchors(const float* scores, int32_t B, int32_t L, int32_t K, int32_t affix_l, int32_t* anchors,
                        const acache_map_args* maps, acache_stream_t stream) {
  if (B < 0 || L <= 0 || K < 0 || K > L || affix_l < 0) return ACACHE_EINVAL;
  if (L > 32768 || B > 65535) return ACACHE_ESHAPE;
  if (B > 0 && (!scores || (K > 0 && !anchors))) return ACACHE_EINVAL;
  if (maps) {
    int st;
    if ((st = check_map_args(maps))) return st;
    if (maps->B != B || maps->L != L || maps->K != K || maps->affix_l != affix_l) return ACACHE_EINVAL;
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_topk(scores, B, L, K, affix_l, anchors, s);
  if (e != hipSuccess) return ACACHE_EDEVICE;
  if (maps) return status_of(launch_maps(anchors, *maps, s));
  return ACACHE_OK;
}

int acache_scatter_private(const acache_kv_pool* pool, const void* k_src, const void* v_src,
                           const int32_t* dst_slots, int32_t n_rows, int32_t layer_begin, int32_t n_layers,
                           acache_stream_t stream) {
  int st;
  if ((st = check_pool(pool))) return st;
  if ((st = check_layers(pool, layer_begin, n_layers))) return st;
  if (n_rows < 0) return ACACHE_EINVAL;
  if (n_rows == 0 || n_layers == 0) return ACACHE_OK;
  if (!k_src || !v_src || !dst_slots) return ACACHE_EINVAL;
  if (!aligned16(k_src) || !aligned16(v_src)) return ACACHE_EALIGN;
  if (n_layers > 65535) return ACACHE_ESHAPE;
  return status_of(launch_scatter(pool->k, pool->v, k_src, v_src, dst_slots, n_rows, layer_begin, n_layers,
                                  geom_of(pool), elem_bytes(pool->dtype), (hipStream_t)stream));
}

int acache_block_slots(const int32_t* read_slot, const int32_t* kv_offsets, const int32_t* block_start, int32_t B,
                       int32_t block_len, int32_t* dst_slots, acache_stream_t stream) {
  if (B < 0 || block_len < 0) return ACACHE_EINVAL;
  if ((int64_t)B * block_len > INT32_MAX) return ACACHE_ESHAPE;
  if (B == 0 || block_len == 0) return ACACHE_OK;
  if (!read_slot || !kv_offsets || !block_start || !dst_slots) return ACACHE_EINVAL;
  return status_of(launch_block_slots(read_slot, kv_offsets, block_start, B, block_len, dst_slots,
                                      (hipStream_t)stream));
}

int acache_mapped_attention_workspace_bytes(int32_t B, int32_t n_q, int32_t n_q_heads, int32_t n_layers,
                                            size_t* bytes) {
  if (!bytes || B < 0 || n_q < 0 || n_q_heads < 0 || n_layers < 0) return ACACHE_EINVAL;
  *bytes = 0;
  return ACACHE_OK;
}

}  // extern "C"

namespace {
// acache_mapped_attention: every check, then (dry == false) the launch
int mapped_attention_impl(const acache_kv_pool* pool, const void* q, const int32_t* q_offsets, int32_t n_q,
                          int32_t max_q_per_req, const int32_t* read_slot, const int32_t* kv_offsets,
                          int32_t max_kv_per_req, int32_t B, int32_t n_q_heads, int32_t layer_begin, int32_t n_layers,
                          float scale, void* out, float* lse, hipStream_t s, bool dry) {
  int st;
  if ((st = check_pool(pool))) return st;
  if ((st = check_layers(pool, layer_begin, n_layers))) return st;
  if ((st = check_heads(pool, n_q_heads))) return st;
  if (B < 0 || n_q < 0 || max_q_per_req < 0 || max_q_per_req > n_q || max_kv_per_req < 0) return ACACHE_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ACACHE_EINVAL;
  if (B > 65535) return ACACHE_ESHAPE;
  if (B == 0 || n_q == 0 || n_layers == 0) return ACACHE_OK;
  if (!q || !q_offsets || !kv_offsets || !out) return ACACHE_EINVAL;
  if (max_kv_per_req > 0 && !read_slot) return ACACHE_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return ACACHE_EALIGN;
  AttnArgs a;
  a.q = q;
  a.pool_k = pool->k;
  a.pool_v = pool->v;
  a.geo = geom_of(pool);
  a.q_offsets = q_offsets;
  a.n_q = n_q;
  a.max_q = max_q_per_req;
  a.kv_table = read_slot;
  a.kv_offsets = kv_offsets;
  a.n_kv = 0;
  a.max_kv = max_kv_per_req;
  a.B = B;
  a.n_q_heads = n_q_heads;
  a.layer_begin = layer_begin;
  a.n_layers = n_layers;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  if (!mfma_supported(pool->dtype, pool->head_dim)) return dry ? ACACHE_OK : status_of(launch_attn_generic(a, pool->dtype, s));
  if ((st = limits_of(launch_attn_mfma(a, s, true)))) return st;
  return dry ? ACACHE_OK : status_of(launch_attn_mfma(a, s));
}
}  // namespace

extern "C" {

int acache_mapped_attention(const acache_kv_pool* pool, const void* q, const int32_t* q_offsets, int32_t n_q,
                            int32_t max_q_per_req, const int32_t* read_slot, const int32_t* kv_offsets,
                            int32_t max_kv_per_req, int32_t B, int32_t n_q_heads, int32_t layer_begin,
                            int32_t n_layers, float scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, acache_stream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  return mapped_attention_impl(pool, q, q_offsets, n_q, max_q_per_req, read_slot, kv_offsets, max_kv_per_req, B,
                               n_q_heads, layer_begin, n_layers, scale, out, lse, (hipStream_t)stream, false);
}

}  // extern "C"

namespace {
// workspace of the two-pass shared-affix attention (256-byte aligned parts)
struct SharedWs {
  bool two_pass = false;
  int excl_words = 0, stride = 0;
  size_t priv = 0, counts = 0, excl = 0, total = 0;
};

SharedWs shared_ws_layout(const acache_kv_pool* pool, int32_t B, int32_t n_q, int32_t max_q, int32_t n_q_heads,
                          int32_t n_layers, int32_t max_kv, int32_t L) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  SharedWs w;
  // a decode block whose query-head groups fill a row tile when packed is
  // MFMA-bound: the single-pass call (which packs them) then serves it
  // better than the shared-affix kernel, whose gain is HBM reads.  A batch of
  // one request reads the affix once either way, and the single pass (its
  // keys split over four waves) fills the CU better
  w.two_pass = mfma_supported(pool->dtype, pool->head_dim) && max_q <= 32 && B >= 2 &&
               gqa_pack(n_q_heads, pool->n_kv_heads, max_q) == 0;
  if (!w.two_pass) return w;
  w.excl_words = 2 * ((L + 63) / 64);
  size_t off = 0;
  w.stride = (max_kv + kSharedPrivTile - 1) / kSharedPrivTile * kSharedPrivTile;
  w.priv = off;
  off += up((size_t)B * w.stride * 4);
  w.counts = off;
  off += up((size_t)B * 4);
  w.excl = off;
  off += up((size_t)B * w.excl_words * 4);
  w.total = off;
  return w;
}
}  // namespace

extern "C" {

int acache_mapped_attention_shared_workspace_bytes(const acache_kv_pool* pool, int32_t B, int32_t n_q,
                                                   int32_t max_q_per_req, int32_t n_q_heads, int32_t n_layers,
                                                   int32_t max_kv_per_req, int32_t L, size_t* bytes) {
  int st;
  if (!bytes) return ACACHE_EINVAL;
  if ((st = check_pool(pool))) return st;
  if (B < 0 || n_q < 0 || max_q_per_req < 0 || n_q_heads < 0 || n_layers < 0 || max_kv_per_req < 0 || L < 0)
    return ACACHE_EINVAL;
  *bytes = shared_ws_layout(pool, B, n_q, max_q_per_req, n_q_heads, n_layers, max_kv_per_req, L).total;
  return ACACHE_OK;
}

int acache_mapped_attention_shared(const acache_kv_pool* pool, const void* q, const int32_t* q_offsets, int32_t n_q,
                                   int32_t max_q_per_req, const int32_t* read_slot, const int32_t* kv_offsets,
                                   int32_t max_kv_per_req, const int32_t* shared_slots, int32_t affix_l, int32_t L,
                                   int32_t B, int32_t n_q_heads, int32_t layer_begin, int32_t n_layers, float scale,
                                   void* out, float* lse, void* workspace, size_t workspace_bytes,
                                   acache_stream_t stream) {
  int st;
  if ((st = check_pool(pool))) return st;
  if (affix_l < 0 || L < 0) return ACACHE_EINVAL;
  if (L > 0 && !shared_slots) return ACACHE_EINVAL;
  const SharedWs w = shared_ws_layout(pool, B < 0 ? 0 : B, n_q < 0 ? 0 : n_q, max_q_per_req, n_q_heads < 0 ? 0 : n_q_heads,
                                      n_layers < 0 ? 0 : n_layers, max_kv_per_req < 0 ? 0 : max_kv_per_req, L);
  if (!w.two_pass)
    return acache_mapped_attention(pool, q, q_offsets, n_q, max_q_per_req, read_slot, kv_offsets, max_kv_per_req, B,
                                   n_q_heads, layer_begin, n_layers, scale, out, lse, nullptr, 0, stream);
  if ((st = check_layers(pool, layer_begin, n_layers))) return st;
  if ((st = check_heads(pool, n_q_heads))) return st;
  if (B < 0 || n_q < 0 || max_q_per_req < 0 || max_q_per_req > n_q || max_kv_per_req < 0) return ACACHE_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ACACHE_EINVAL;
  if (B > 65535) return ACACHE_ESHAPE;
  if ((long long)B * (max_kv_per_req + kSharedPrivTile) >= (1ll << 31)) return ACACHE_ESHAPE;
  if (B == 0 || n_q == 0 || n_layers == 0) return ACACHE_OK;
  if (!q || !q_offsets || !kv_offsets || !out) return ACACHE_EINVAL;
  if (max_kv_per_req > 0 && !read_slot) return ACACHE_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return ACACHE_EALIGN;
  if (!workspace || workspace_bytes < w.total) return ACACHE_EWORKSPACE;
  if (!aligned16(workspace)) return ACACHE_EALIGN;
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  SharedAttnArgs a;
  a.q = q;
  a.pool_k = pool->k;
  a.pool_v = pool->v;
  a.geo = geom_of(pool);
  a.q_offsets = q_offsets;
  a.n_q = n_q;
  a.max_q = max_q_per_req;
  a.shared_slots = shared_slots;
  a.L = L;
  a.excl = (const uint32_t*)(ws + w.excl);
  a.excl_words = w.excl_words;
  a.priv_slots = (const int32_t*)(ws + w.priv);
  a.priv_counts = (const int32_t*)(ws + w.counts);
  a.priv_stride = w.stride;
  a.B = B;
  a.n_q_heads = n_q_heads;
  a.layer_begin = layer_begin;
  a.n_layers = n_layers;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  if ((st = limits_of(launch_attn_mfma_shared(a, s, true)))) return st;
  hipError_t e = launch_shared_plan(read_slot, kv_offsets, shared_slots, B, affix_l, L, max_kv_per_req, w.stride,
                                    kSharedPrivTile, (int32_t*)(ws + w.priv), (int32_t*)(ws + w.counts),
                                    (uint32_t*)(ws + w.excl), w.excl_words, s);
  if (e != hipSuccess) return status_of(e);
  return status_of(launch_attn_mfma_shared(a, s));
}

}  // extern "C"

namespace {
// The allocation-free shared-affix call keeps its plan (each request's other
// read slots, their counts, the affix exclusion bits) in this fixed device
// array.  Every GPU the library runs on holds its own copy until the process
// ends; host code reaches it only through the address hipGetSymbolAddress
// reports for the current device, taken once per device.
constexpr size_t kScratchBytes = 8u << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device (set up on its first use there)
int scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ACACHE_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ACACHE_EDEVICE;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ACACHE_OK;
}
}  // namespace

extern "C" {

int acache_mapped_attention_shared_noalloc(const acache_kv_pool* pool, const void* q, const int32_t* q_offsets,
                                           int32_t n_q, int32_t max_q_per_req, const int32_t* read_slot,
                                           const int32_t* kv_offsets, int32_t max_kv_per_req,
                                           const int32_t* shared_slots, int32_t affix_l, int32_t L, int32_t B,
                                           int32_t n_q_heads, int32_t layer_begin, int32_t n_layers, float scale,
                                           void* out, float* lse, acache_stream_t stream) {
  int st;
  if ((st = check_pool(pool))) return st;
  if (B < 0 || n_q < 0 || max_q_per_req < 0 || n_q_heads < 0 || n_layers < 0 || max_kv_per_req < 0 || L < 0)
    return ACACHE_EINVAL;
  const SharedWs w = shared_ws_layout(pool, B, n_q, max_q_per_req, n_q_heads, n_layers, max_kv_per_req, L);
  if (w.total > kScratchBytes) return ACACHE_EWORKSPACE;  // the plan does not fit the fixed scratch
  void* ws = nullptr;
  if (w.total > 0 && (st = scratch_of_current_device(&ws))) return st;
  return acache_mapped_attention_shared(pool, q, q_offsets, n_q, max_q_per_req, read_slot, kv_offsets,
                                        max_kv_per_req, shared_slots, affix_l, L, B, n_q_heads, layer_begin,
                                        n_layers, scale, out, lse, ws, w.total, stream);
}

}  // extern "C"

namespace {
// workspace of the fused store-then-attend path (256-byte aligned parts)
struct StoreWs {
  bool fused = false;
  int stride = 0;
  size_t other = 0, counts = 0, total = 0;
};

// Largest recompute set per request (query rows) that takes the one-kernel
// path.  The one kernel saves the scatter's pass over the rows but reads
// every source row once per row tile of its request.  With the 48-row kernel
// in both forms (from kRows48MinRows rows), the one kernel measured 1.5-3%
// faster than the two calls from 1332 to 2970 rows per request (12 layers,
// stretched affixes of the L=4096 workload, alternated on one box) and 0.85%
// slower at 5683 (L=16384, 32 requests).
constexpr int32_t kStoreOneKernelMaxRows = 3072;

StoreWs store_ws_layout(const acache_kv_pool* pool, int32_t B, int32_t max_q, int32_t max_kv) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  StoreWs w;
  w.fused = mfma_supported(pool->dtype, pool->head_dim) && max_q > 0 && max_q <= kStoreOneKernelMaxRows &&
            max_kv <= kStorePlanMaxKv;
  if (!w.fused) return w;
  w.stride = max_kv;
  w.other = 0;
  w.counts = up((size_t)B * w.stride * 4);
  w.total = w.counts + up((size_t)B * 4);
  return w;
}
}  // namespace

extern "C" {

int acache_store_attend_workspace_bytes(const acache_kv_pool* pool, int32_t B, int32_t max_q_per_req,
                                        int32_t max_kv_per_req, size_t* bytes) {
  int st;
  if (!bytes) return ACACHE_EINVAL;
  if ((st = check_pool(pool))) return st;
  if (B < 0 || max_q_per_req < 0 || max_kv_per_req < 0) return ACACHE_EINVAL;
  *bytes = store_ws_layout(pool, B, max_q_per_req, max_kv_per_req).total;
  return ACACHE_OK;
}

int acache_store_attend(const acache_kv_pool* pool, const void* k_src, const void* v_src, const int32_t* src_pos,
                        const int32_t* src_slot, const int32_t* src_offsets, int32_t n_src, const void* q,
                        const int32_t* q_offsets, int32_t n_q, int32_t max_q_per_req, const int32_t* read_slot,
                        const int32_t* kv_offsets, int32_t max_kv_per_req, int32_t B, int32_t n_q_heads,
                        int32_t layer_begin, int32_t n_layers, float scale, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, acache_stream_t stream) {
  int st;
  if ((st = check_pool(pool))) return st;
  if ((st = check_layers(pool, layer_begin, n_layers))) return st;
  if ((st = check_heads(pool, n_q_heads))) return st;
  if (B < 0 || n_src < 0 || n_q < 0 || max_q_per_req < 0 || max_q_per_req > n_q || max_kv_per_req < 0)
    return ACACHE_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ACACHE_EINVAL;
  if (B > 65535) return ACACHE_ESHAPE;
  if (n_src > 0 && (!k_src || !v_src || !src_pos || !src_slot || !src_offsets)) return ACACHE_EINVAL;
  if (n_src > 0 && (!aligned16(k_src) || !aligned16(v_src))) return ACACHE_EALIGN;
  const StoreWs w = store_ws_layout(pool, B, max_q_per_req, max_kv_per_req);
  // With grouped query heads the rows to store are fewer beside the
  // attention: two query heads per KV head measured 0.7-1.9% slower in one
  // kernel than in the two calls (1332-2970 rows per request), so only
  // one query head per KV head takes the one kernel.
  const bool fused = w.fused && n_q_heads == pool->n_kv_heads;
  if (!fused || B == 0 || n_q == 0 || n_layers == 0) {
    // the definition itself: the scatter, then the attention through
    // read_slot (the attention's arguments are checked before the scatter)
    hipStream_t s = (hipStream_t)stream;
    if ((st = mapped_attention_impl(pool, q, q_offsets, n_q, max_q_per_req, read_slot, kv_offsets, max_kv_per_req, B,
                                    n_q_heads, layer_begin, n_layers, scale, out, lse, s, true)))
      return st;
    if ((st = acache_scatter_private(pool, k_src, v_src, src_slot, n_src, layer_begin, n_layers, stream))) return st;
    return mapped_attention_impl(pool, q, q_offsets, n_q, max_q_per_req, read_slot, kv_offsets, max_kv_per_req, B,
                                 n_q_heads, layer_begin, n_layers, scale, out, lse, s, false);
  }
  if (!q || !q_offsets || !kv_offsets || !out || !src_offsets) return ACACHE_EINVAL;
  if (max_kv_per_req > 0 && !read_slot) return ACACHE_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return ACACHE_EALIGN;
  if (!workspace || workspace_bytes < w.total) return ACACHE_EWORKSPACE;
  if (!aligned16(workspace)) return ACACHE_EALIGN;
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  StoreAttnArgs a;
  a.q = q;
  a.pool_k = pool->k;
  a.pool_v = pool->v;
  a.geo = geom_of(pool);
  a.q_offsets = q_offsets;
  a.n_q = n_q;
  a.max_q = max_q_per_req;
  a.other_slots = (const int32_t*)(ws + w.other);
  a.other_counts = (const int32_t*)(ws + w.counts);
  a.other_stride = w.stride;
  a.k_src = k_src;
  a.v_src = v_src;
  a.src_slot = src_slot;
  a.src_offsets = src_offsets;
  a.n_src = n_src;
  a.B = B;
  a.n_q_heads = n_q_heads;
  a.layer_begin = layer_begin;
  a.n_layers = n_layers;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  if ((st = limits_of(launch_attn_mfma_store(a, s, true)))) return st;
  hipError_t e = launch_store_plan(read_slot, kv_offsets, src_pos, src_offsets, B, max_kv_per_req, w.stride,
                                   (int32_t*)(ws + w.other), (int32_t*)(ws + w.counts), s);
  if (e != hipSuccess) return status_of(e);
  return status_of(launch_attn_mfma_store(a, s));
}

int acache_hkvd_scores(const acache_kv_pool* pool, const int32_t* shared_slots, int32_t L, const void* k_full,
                       const void* v_full, int32_t B, int32_t layer_begin, int32_t n_layers, float* scores,
                       acache_stream_t stream) {
  int st;
  if ((st = check_pool(pool))) return st;
  if ((st = check_layers(pool, layer_begin, n_layers))) return st;
  if (B < 0 || L < 0) return ACACHE_EINVAL;
  if (B == 0 || L == 0 || n_layers == 0) return ACACHE_OK;
  if (!shared_slots || !k_full || !v_full || !scores) return ACACHE_EINVAL;
  if (!aligned16(k_full) || !aligned16(v_full)) return ACACHE_EALIGN;
  return status_of(launch_hkvd(pool->k, pool->v, geom_of(pool), shared_slots, k_full, v_full, B, L, layer_begin,
                               n_layers, pool->dtype, scores, (hipStream_t)stream));
}

int acache_lse_merge(int32_t dtype, int64_t n_pairs, int32_t head_dim, const void* o_a, const float* lse_a,
                     const void* o_b, const float* lse_b, void* o, float* lse, acache_stream_t stream) {
  if (dtype != ACACHE_F32 && dtype != ACACHE_BF16) return ACACHE_EDTYPE;
  if (n_pairs < 0 || !lse_a || !lse_b || !lse) return ACACHE_EINVAL;
  if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128) return ACACHE_ESHAPE;
  const int n_o = (o_a != nullptr) + (o_b != nullptr) + (o != nullptr);
  if (n_o != 0 && n_o != 3) return ACACHE_EINVAL;
  if (n_o == 3 && (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o))) return ACACHE_EALIGN;
  return status_of(launch_lse_merge(dtype, n_pairs, head_dim, o_a, lse_a, o_b, lse_b, o, lse, (hipStream_t)stream));
}

int acache_kv_footprint(int32_t B, const int32_t* seq_len, int32_t L, int32_t K, int32_t page_size,
                        int32_t n_layers, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                        uint64_t* shared_bytes, uint64_t* private_bytes, uint64_t* dense_bytes) {
  if (!shared_bytes || !private_bytes || !dense_bytes) return ACACHE_EINVAL;
  if (B < 0 || L < 0 || K < 0 || K > L || page_size <= 0 || n_layers < 0 || n_kv_heads < 0 || head_dim < 0)
    return ACACHE_EINVAL;
  if (dtype != ACACHE_F32 && dtype != ACACHE_BF16) return ACACHE_EDTYPE;
  if (B > 0 && !seq_len) return ACACHE_EINVAL;
  const uint64_t page = (uint64_t)page_size * (uint64_t)n_layers * (uint64_t)n_kv_heads * (uint64_t)head_dim * 2u *
                        (uint64_t)elem_bytes(dtype);
  auto pages = [&](int64_t n) -> uint64_t { return (uint64_t)((n + page_size - 1) / page_size); };
  uint64_t priv = 0, dense = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (seq_len[b] < L) return ACACHE_EINVAL;
    priv += pages((int64_t)K + seq_len[b] - L);
    dense += pages(seq_len[b]);
  }
  *shared_bytes = B > 0 ? pages(L) * page : 0;
  *private_bytes = priv * page;
  *dense_bytes = dense * page;
  return ACACHE_OK;
}

int acache_check_slots_workspace_bytes(int32_t n_pages, int32_t page_size, int32_t mode, size_t* bytes) {
  if (!bytes || n_pages <= 0 || page_size <= 0 || (page_size & (page_size - 1))) return ACACHE_EINVAL;
  if (mode != ACACHE_CHECK_READ && mode != ACACHE_CHECK_WRITE) return ACACHE_EINVAL;
  const int64_t n_slots = (int64_t)n_pages * page_size;
  if (n_slots > INT32_MAX) return ACACHE_ESHAPE;
  *bytes = kAlign + (mode == ACACHE_CHECK_WRITE ? align_up((size_t)n_slots * sizeof(int32_t)) : 0);
  return ACACHE_OK;
}

int acache_check_slots(const int32_t* slots, int32_t n, const int32_t* offsets, int32_t B,
                       const int32_t* page_owner, int32_t n_pages, int32_t page_size, int32_t mode,
                       int32_t* bad_index, void* workspace, size_t workspace_bytes, acache_stream_t stream) {
  size_t need = 0;
  int st;
  if ((st = acache_check_slots_workspace_bytes(n_pages, page_size, mode, &need))) return st;
  if (n < 0 || B < 0) return ACACHE_EINVAL;
  if ((n > 0 && !slots) || (B > 0 && !offsets)) return ACACHE_EINVAL;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & (kAlign - 1))) return ACACHE_EWORKSPACE;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  int32_t* rec = (int32_t*)workspace;
  int32_t* first = mode == ACACHE_CHECK_WRITE ? (int32_t*)((char*)workspace + kAlign) : nullptr;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_check_slots(slots, n, B > 0 ? offsets : nullptr, B, page_owner,
                                    (int64_t)n_pages * page_size, shift, mode == ACACHE_CHECK_WRITE, rec, first, s);
  if (e != hipSuccess) return ACACHE_EDEVICE;
  int32_t h[3];
  if (hipMemcpyAsync(h, rec, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess) return ACACHE_EDEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return ACACHE_EDEVICE;
  static const int cls[3] = {ACACHE_ERANGE, ACACHE_EREGION, ACACHE_EDUP};
  for (int c = 0; c < 3; ++c)
    if (h[c] != INT32_MAX) {
      if (bad_index) *bad_index = h[c];
      return cls[c];
    }
  return ACACHE_OK;
}

int acache_scatter_private_checked(const acache_kv_pool* pool, const void* k_src, const void* v_src,
                                   const int32_t* dst_slots, int32_t n_rows, const int32_t* row_offsets, int32_t B,
                                   const int32_t* page_owner, int32_t layer_begin, int32_t n_layers,
                                   int32_t* bad_index, void* workspace, size_t workspace_bytes,
                                   acache_stream_t stream) {
  int st;
  if ((st = check_pool(pool))) return st;
  if ((st = check_layers(pool, layer_begin, n_layers))) return st;
  if (n_rows < 0) return ACACHE_EINVAL;
  if (n_rows > 0 && (!k_src || !v_src || !dst_slots)) return ACACHE_EINVAL;
  if (n_rows > 0 && (!aligned16(k_src) || !aligned16(v_src))) return ACACHE_EALIGN;
  if (n_layers > 65535) return ACACHE_ESHAPE;
  if ((st = acache_check_slots(dst_slots, n_rows, row_offsets, B, page_owner, pool->n_pages, pool->page_size,
                               ACACHE_CHECK_WRITE, bad_index, workspace, workspace_bytes, stream)))
    return st;
  return acache_scatter_private(pool, k_src, v_src, dst_slots, n_rows, layer_begin, n_layers, stream);
}

int acache_validate_slots(const int32_t* slots, int32_t n, const int32_t* owner, const int32_t* page_owner,
                          int32_t n_pages, int32_t page_size, int32_t distinct, int32_t* bad_index) {
  if (n < 0 || n_pages <= 0 || page_size <= 0 || (page_size & (page_size - 1))) return ACACHE_EINVAL;
  if (n > 0 && (!slots || !page_owner)) return ACACHE_EINVAL;
  const int64_t n_slots = (int64_t)n_pages * page_size;
  std::vector<uint8_t> seen(distinct ? (size_t)n_slots : 0, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = slots[i];
    if (s < 0 || s >= n_slots) {
      if (bad_index) *bad_index = i;
      return ACACHE_ERANGE;
    }
    const int32_t po = page_owner[s / page_size];
    const bool ok = owner ? (po == owner[i]) : (po >= 0);
    if (!ok) {
      if (bad_index) *bad_index = i;
      return ACACHE_EREGION;
    }
    if (distinct) {
      if (seen[s]) {
        if (bad_index) *bad_index = i;
        return ACACHE_EDUP;
      }
      seen[s] = 1;
    }
  }
  return ACACHE_OK;
}

}  // extern "C"

// Integer and copy kernels of the ACache path (gfx950):
//   * radix-select Top-K of the anchor scores (Eq. 6 of "Affix Cache for
//     Diffusion Large Language Models", Section 3.2),
//   * the write-side recomputation map and the per-request read-slot map
//     (Section 4.1 dual mapping, Section 4.2 admission-time preparation),
//   * the plans of the shared-affix and store-then-attend attentions (each
//     request's read list split by where its keys are read from),
//   * decode-block destination slots (Section 4.3, block decoding),
//   * the private scatter of recomputed K/V rows (Section 4.3 and
//     Appendix C.1: new KV is stored through the write-side map before the
//     read-slot attention runs).
#include "acache_dev.h"
#include "acache_launch.h"

namespace acache {

// ---------------------------------------------------------------------------
// Top-K: exact radix select over order-preserving keys of the fp32 scores.
// ---------------------------------------------------------------------------

// Monotone map fp32 -> uint32 (larger score -> larger key).  NaN maps to 0,
// below every number (the smallest number, -inf, maps to 0x007fffff); -0 and
// +0 both map to the key of +0, so they tie.
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0u;
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Exclusive prefix sum over the block's threads in thread order; also
// returns the block total.  All threads of the block must call it.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = lane < kTopkWaves ? wave_tot[lane] : 0u;
    uint32_t ti = t;
#pragma unroll
    for (int off = 1; off < kTopkWaves; off <<= 1) {
      uint32_t y = __shfl_up(ti, off, 64);
      if (lane >= off) ti += y;
    }
    if (lane < kTopkWaves) wave_tot[lane] = ti - t;  // exclusive wave offsets
    if (lane == kTopkWaves - 1) wave_tot[kTopkWaves] = ti;
  }
  __syncthreads();
  uint32_t res = wave_tot[wave] + incl - v;
  *total = wave_tot[kTopkWaves];
  __syncthreads();
  return res;
}

// One workgroup per request.  Thread t holds scores t*EPT .. t*EPT+EPT-1, so
// thread order is index order and the tie-break scans are plain block scans.
template <int EPT>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores, int L, int K,
                                                             int affix_l, int32_t* __restrict__ anchors) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[kTopkWaves + 1];
  __shared__ uint32_t sh_digit, sh_above;
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* s = scores + (size_t)b * L;
  uint32_t key[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    int i = tid * EPT + e;
    key[e] = i < L ? order_key(s[i]) : 0u;
  }
  // find the K-th largest key, 8 bits at a time from the top
  uint32_t prefix = 0, mask = 0, krem = (uint32_t)K;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (tid * EPT + e < L && (key[e] & mask) == prefix) atomicAdd(&hist[(key[e] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 64) {
      // lane t covers bins 255-4t .. 252-4t (scanning from the top)
      const int top = 255 - 4 * tid;
      uint32_t c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
      uint32_t sum = c0 + c1 + c2 + c3, incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_up(incl, off, 64);
        if (tid >= off) incl += y;
      }
      uint32_t excl = incl - sum;
      if (excl < krem && krem <= incl) {
        uint32_t acc = excl;
        int digit;
        if (acc + c0 >= krem) digit = top;
        else if ((acc += c0) + c1 >= krem) digit = top - 1;
        else if ((acc += c1) + c2 >= krem) digit = top - 2;
        else { acc += c2; digit = top - 3; }
        sh_digit = (uint32_t)digit;
        sh_above = acc;
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    krem -= sh_above;
    __syncthreads();
  }
  const uint32_t thr = prefix, need_eq = krem;  // take the first need_eq keys equal to thr
  uint32_t n_eq = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) n_eq += (tid * EPT + e < L && key[e] == thr);
  uint32_t tot;
  uint32_t eq_before = block_exclusive_scan(n_eq, wave_tot, &tot);
  uint32_t selmask = 0, n_sel = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    bool valid = tid * EPT + e < L;
    bool sel = false;
    if (valid && key[e] > thr) sel = true;
    if (valid && key[e] == thr) {
      sel = eq_before < need_eq;
      ++eq_before;
    }
    if (sel) { selmask |= 1u << e; ++n_sel; }
  }
  uint32_t pos = block_exclusive_scan(n_sel, wave_tot, &tot);
  int32_t* out = anchors + (size_t)b * K;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (selmask & (1u << e)) out[pos++] = affix_l + tid * EPT + e;
}

hipError_t launch_topk(const float* scores, int B, int L, int K, int affix_l, int32_t* anchors,
                       hipStream_t st) {
  if (K == 0 || B == 0) return hipSuccess;
  const int ept = (L + kTopkThreads - 1) / kTopkThreads;
  dim3 grid(B), block(kTopkThreads);
#define ACACHE_TOPK(E) hipLaunchKernelGGL(topk_kernel<E>, grid, block, 0, st, scores, L, K, affix_l, anchors)
  if (ept <= 1) ACACHE_TOPK(1);
  else if (ept <= 2) ACACHE_TOPK(2);
  else if (ept <= 4) ACACHE_TOPK(4);
  else if (ept <= 8) ACACHE_TOPK(8);
  else if (ept <= 16) ACACHE_TOPK(16);
  else ACACHE_TOPK(32);
#undef ACACHE_TOPK
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Maps.  Private index of position p (its rank in R = A u non-affix):
//   p < l        -> p                      (every earlier position is non-affix)
//   p an anchor  -> l + (its rank in A)
//   p > r        -> p - L + K              (l non-affix before, K anchors, p-r-1 after)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void maps_kernel(const int32_t* __restrict__ anchors, acache_map_args a,
                                                   int page_shift) {
  const int b = blockIdx.y;
  const int T = a.seq_len[b];
  const int l = a.affix_l, L = a.L, K = a.K, ps = a.page_size;
  const int kv0 = a.kv_offsets[b], rc0 = a.rc_offsets[b], pp0 = a.private_page_offsets[b];
  const int32_t* A = anchors + (size_t)b * K;
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < T; p += gridDim.x * blockDim.x) {
    int idx;
    if (p < l) {
      idx = p;
    } else if (p < l + L) {
      int lo = 0, hi = K;  // first anchor >= p
      while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (A[mid] < p) lo = mid + 1; else hi = mid;
      }
      idx = (lo < K && A[lo] == p) ? l + lo : -1;
    } else {
      idx = p - L + K;
    }
    int32_t slot;
    if (idx < 0) {
      slot = a.shared_slots[p - l];
    } else {
      slot = a.private_pages[pp0 + (idx >> page_shift)] * ps + (idx & (ps - 1));
      if (a.recompute_pos) a.recompute_pos[rc0 + idx] = p;
      if (a.recompute_slot) a.recompute_slot[rc0 + idx] = slot;
    }
    a.read_slot[kv0 + p] = slot;
  }
}

hipError_t launch_maps(const int32_t* anchors, const acache_map_args& a, hipStream_t st) {
  if (a.B == 0 || a.max_seq_len == 0) return hipSuccess;
  int page_shift = 0;
  while ((1 << page_shift) < a.page_size) ++page_shift;
  int gx = (a.max_seq_len + 255) / 256;
  if (gx > 64) gx = 64;
  hipLaunchKernelGGL(maps_kernel, dim3(gx, a.B), dim3(256), 0, st, anchors, a, page_shift);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plan of the two-pass decode attention: a request's read list (Section 4.3
// read-slot map) is split into the affix positions it reads from the shared
// region, as exclusion bits over the affix, and the ascending list of the
// slots of every other position.  One workgroup per request.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kTopkThreads) void shared_plan_kernel(
    const int32_t* __restrict__ read_slot, const int32_t* __restrict__ kv_offsets,
    const int32_t* __restrict__ shared_slots, int affix_l, int L, int max_kv, int stride, int pad,
    int32_t* __restrict__ priv_slots, int32_t* __restrict__ priv_counts, uint32_t* __restrict__ excl,
    int excl_words) {
  __shared__ uint32_t wave_tot[kTopkWaves + 1];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = kv_offsets[b];
  const int T = min(kv_offsets[b + 1] - k0, max_kv);
  const int32_t* rs = read_slot + k0;
  // affix key j is dropped from the shared pass unless position affix_l + j
  // exists and reads shared_slots[j]; the padding up to a whole 64-key tile
  // is dropped too
  uint32_t* ex = excl + (size_t)b * excl_words;
  for (int j0 = wave * 64; j0 < excl_words * 32; j0 += kTopkThreads) {
    const int j = j0 + lane, pos = affix_l + j;
    const bool drop = j >= L || pos >= T || rs[pos] != shared_slots[j];
    const unsigned long long bits = __ballot(drop);
    if (lane == 0) {
      ex[j0 / 32] = (uint32_t)bits;
      ex[j0 / 32 + 1] = (uint32_t)(bits >> 32);
    }
  }
  int32_t* out = priv_slots + (size_t)b * stride;
  uint32_t base = 0;
  for (int p0 = 0; p0 < T; p0 += kTopkThreads) {
    const int pos = p0 + tid;
    int32_t slot = 0;
    bool keep = false;
    if (pos < T) {
      slot = rs[pos];
      const int j = pos - affix_l;
      keep = j < 0 || j >= L || slot != shared_slots[j];
    }
    uint32_t tot;
    const uint32_t at = block_exclusive_scan(keep ? 1u : 0u, wave_tot, &tot);
    if (keep) out[base + at] = slot;
    base += tot;
  }
  // pad the list to whole tiles of `pad` entries with its last slot, so that
  // tile loads need no bounds (the padded keys are masked by count)
  const uint32_t padded = (base + pad - 1) / pad * pad;
  __syncthreads();  // the last entry is written by another thread
  if (base > 0 && tid < (int)(padded - base)) out[base + tid] = out[base - 1];
  if (tid == 0) priv_counts[b] = (int32_t)base;
}

hipError_t launch_shared_plan(const int32_t* read_slot, const int32_t* kv_offsets, const int32_t* shared_slots,
                              int B, int affix_l, int L, int max_kv, int stride, int pad, int32_t* priv_slots,
                              int32_t* priv_counts, uint32_t* excl, int excl_words, hipStream_t st) {
  if (B == 0) return hipSuccess;
  if (pad < 1 || pad > kTopkThreads || stride < (max_kv + pad - 1) / pad * pad) return hipErrorInvalidValue;
  hipLaunchKernelGGL(shared_plan_kernel, dim3(B), dim3(kTopkThreads), 0, st, read_slot, kv_offsets, shared_slots,
                     affix_l, L, max_kv, stride, pad, priv_slots, priv_counts, excl, excl_words);
  return hipGetLastError();
}

// Store-then-attend plan (Section 4.3: the recomputed rows are stored to
// their private slots and read back by the attention).  Per request b, the
// read list without the positions this call stores: positions src_pos[i]
// (i in src_offsets[b] .. src_offsets[b+1]) are marked in an LDS bitmap and
// every other position p < T_b contributes read_slot[kv_offsets[b] + p], in
// position order, to other_slots[b * stride ..]; other_counts[b] receives
// the count.  Positions past max_kv are ignored.
__global__ __launch_bounds__(kTopkThreads) void store_plan_kernel(
    const int32_t* __restrict__ read_slot, const int32_t* __restrict__ kv_offsets,
    const int32_t* __restrict__ src_pos, const int32_t* __restrict__ src_offsets, int max_kv, int stride,
    int32_t* __restrict__ other_slots, int32_t* __restrict__ other_counts) {
  extern __shared__ uint32_t marked[];  // (max_kv + 31) / 32 words
  __shared__ uint32_t wave_tot[kTopkWaves + 1];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int k0 = kv_offsets[b];
  const int T = min(kv_offsets[b + 1] - k0, max_kv);
  const int words = (T + 31) / 32;
  for (int w = tid; w < words; w += kTopkThreads) marked[w] = 0u;
  __syncthreads();
  for (int i = src_offsets[b] + tid; i < src_offsets[b + 1]; i += kTopkThreads) {
    const int pos = src_pos[i];
    if (pos >= 0 && pos < T) atomicOr(&marked[pos >> 5], 1u << (pos & 31));
  }
  __syncthreads();
  const int32_t* rs = read_slot + k0;
  int32_t* out = other_slots + (size_t)b * stride;
  uint32_t base = 0;
  for (int p0 = 0; p0 < T; p0 += kTopkThreads) {
    const int pos = p0 + tid;
    const bool keep = pos < T && !((marked[pos >> 5] >> (pos & 31)) & 1u);
    const int32_t slot = keep ? rs[pos] : 0;
    uint32_t tot;
    const uint32_t at = block_exclusive_scan(keep ? 1u : 0u, wave_tot, &tot);
    if (keep) out[base + at] = slot;
    base += tot;
  }
  if (tid == 0) other_counts[b] = (int32_t)base;
}

hipError_t launch_store_plan(const int32_t* read_slot, const int32_t* kv_offsets, const int32_t* src_pos,
                             const int32_t* src_offsets, int B, int max_kv, int stride, int32_t* other_slots,
                             int32_t* other_counts, hipStream_t st) {
  if (B == 0) return hipSuccess;
  if (max_kv < 0 || max_kv > kStorePlanMaxKv || stride < max_kv) return hipErrorInvalidValue;
  const size_t lds = (size_t)((max_kv + 31) / 32) * 4;
  hipLaunchKernelGGL(store_plan_kernel, dim3(B), dim3(kTopkThreads), lds, st, read_slot, kv_offsets, src_pos,
                     src_offsets, max_kv, stride, other_slots, other_counts);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void block_slots_kernel(const int32_t* __restrict__ read_slot,
                                                          const int32_t* __restrict__ kv_offsets,
                                                          const int32_t* __restrict__ block_start, int B,
                                                          int block_len, int32_t* __restrict__ dst) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= B * block_len) return;
  int b = t / block_len, i = t - b * block_len;
  dst[t] = read_slot[kv_offsets[b] + block_start[b] + i];
}

hipError_t launch_block_slots(const int32_t* read_slot, const int32_t* kv_offsets, const int32_t* block_start,
                              int B, int block_len, int32_t* dst, hipStream_t st) {
  int n = B * block_len;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(block_slots_kernel, dim3((n + 255) / 256), dim3(256), 0, st, read_slot, kv_offsets,
                     block_start, B, block_len, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Private scatter: 16-byte vector copies.  A (slot, KV head) row of
// head_dim elements is contiguous in the pool; a source row holds all KV
// heads of one position back to back.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void scatter_kernel(char* __restrict__ pool_k, char* __restrict__ pool_v,
                                                      const char* __restrict__ src_k,
                                                      const char* __restrict__ src_v,
                                                      const int32_t* __restrict__ dst, int n_rows,
                                                      int layer_begin, PoolGeom geo, int elem_bytes,
                                                      int vec_shift /* log2(vectors per head row) */,
                                                      int rows_per_block) {
  const int n = blockIdx.y;  // local layer
  const int vpr = 1 << vec_shift;
  const int row_vecs = geo.n_kv_heads * vpr;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(n_rows, r0 + rows_per_block);
  const int items = (r1 - r0) * row_vecs;
  const size_t head_row_bytes = (size_t)geo.head_dim * elem_bytes;
  for (int j = threadIdx.x; j < items; j += blockDim.x) {
    const int rr = j / row_vecs;
    const int v = j - rr * row_vecs;
    const int g = v >> vec_shift, c = v & (vpr - 1);
    const int i = r0 + rr;
    const size_t src_off = ((size_t)n * n_rows + i) * row_vecs * 16 + (size_t)v * 16;
    const size_t dst_off = geo.row(layer_begin + n, dst[i], g) * elem_bytes + (size_t)c * 16;
    u32x4 kx = __builtin_nontemporal_load((const u32x4*)(src_k + src_off));
    u32x4 vx = __builtin_nontemporal_load((const u32x4*)(src_v + src_off));
    __builtin_nontemporal_store(kx, (u32x4*)(pool_k + dst_off));
    __builtin_nontemporal_store(vx, (u32x4*)(pool_v + dst_off));
    (void)head_row_bytes;
  }
}

hipError_t launch_scatter(void* pool_k, void* pool_v, const void* k_src, const void* v_src, const int32_t* dst,
                          int n_rows, int layer_begin, int n_layers, const PoolGeom& geo, int elem_bytes,
                          hipStream_t st) {
  if (n_rows == 0 || n_layers == 0) return hipSuccess;
  const int vpr = geo.head_dim * elem_bytes / 16;
  int vec_shift = 0;
  while ((1 << vec_shift) < vpr) ++vec_shift;
  const int row_vecs = geo.n_kv_heads * vpr;
  int rows_per_block = (2048 + row_vecs - 1) / row_vecs;
  if (rows_per_block < 1) rows_per_block = 1;
  dim3 grid((n_rows + rows_per_block - 1) / rows_per_block, n_layers);
  hipLaunchKernelGGL(scatter_kernel, grid, dim3(256), 0, st, (char*)pool_k, (char*)pool_v, (const char*)k_src,
                     (const char*)v_src, dst, n_rows, layer_begin, geo, elem_bytes, vec_shift, rows_per_block);
  return hipGetLastError();
}

}  // namespace acache

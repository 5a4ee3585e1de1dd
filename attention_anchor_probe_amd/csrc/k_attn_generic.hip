// Vector-ALU attention kernels for every supported (dtype, head_dim): the
// fp32 path and small head dims.  bf16 with head_dim 128 runs on the MFMA
// kernels in k_attn_mfma.hip instead.
//
//   attn_fwd_generic : O = softmax(q K^T * scale) V and LSE over a key list
//                      given by a slot table -- the probe forward over the
//                      shared affix (Eq. 4 of "Affix Cache for Diffusion Large
//                      Language Models", Section 3.2) and the read-slot
//                      attention (Section 4.3, Appendix C.1).
//   colmass_generic  : per-key Eq. (4) weights of the masked rows, summed over
//                      query heads and rows into one partial per (layer,
//                      request, key)  (Eq. 5).
//   colmass_reduce   : scores[b][j] += sum of the partials over their first
//                      index (layers, or layers x query heads), in a fixed
//                      order (deterministic).
#include "acache_dev.h"
#include "acache_launch.h"

namespace acache {

constexpr int kGenRows = 64;   // query rows per workgroup (one per thread)
constexpr int kGenKeys = 32;   // keys per LDS tile

// One thread per (query row, head).  Keys are walked in logical order with an
// online (running max) softmax in the exp2 domain.
template <typename T, int D>
__global__ __launch_bounds__(kGenRows) void attn_fwd_generic(
    const T* __restrict__ q, const T* __restrict__ pool_k, const T* __restrict__ pool_v, PoolGeom geo,
    const int32_t* __restrict__ q_offsets, int n_q, const int32_t* __restrict__ kv_table,
    const int32_t* __restrict__ kv_offsets, int n_kv, int n_q_heads, int layer_begin, float scale,
    T* __restrict__ out, float* __restrict__ lse) {
  __shared__ float ks[kGenKeys][D + 1];
  __shared__ float vs[kGenKeys][D + 1];
  const int b = blockIdx.y;
  const int n = blockIdx.z / n_q_heads, h = blockIdx.z - n * n_q_heads;
  const int g = h / (n_q_heads / geo.n_kv_heads);
  const int layer = layer_begin + n;
  int q0 = 0, q1 = n_q, k0 = 0, k1 = n_kv;
  if (q_offsets) { q0 = q_offsets[b]; q1 = q_offsets[b + 1]; }
  if (kv_offsets) { k0 = kv_offsets[b]; k1 = kv_offsets[b + 1]; }
  const int r = q0 + blockIdx.x * kGenRows + threadIdx.x;
  if (q0 + blockIdx.x * kGenRows >= q1) return;  // whole workgroup idle
  const bool active = r < q1;
  const float c = scale * kLog2e;
  float qv[D], o[D];
  const size_t qrow = (((size_t)n * n_q + (active ? r : q0)) * n_q_heads + h) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) { qv[i] = Elem<T>::load(q + qrow + i); o[i] = 0.f; }
  float m = -INFINITY, l = 0.f;
  const int nk = k1 - k0;
  for (int t0 = 0; t0 < nk; t0 += kGenKeys) {
    __syncthreads();
    for (int e = threadIdx.x; e < kGenKeys * D; e += kGenRows) {
      const int kk = e / D, ci = e - kk * D;
      float kx = 0.f, vx = 0.f;
      if (t0 + kk < nk) {
        const size_t off = geo.row(layer, kv_table[k0 + t0 + kk], g) + ci;
        kx = Elem<T>::load(pool_k + off);
        vx = Elem<T>::load(pool_v + off);
      }
      ks[kk][ci] = kx;
      vs[kk][ci] = vx;
    }
    __syncthreads();
    const int tn = min(kGenKeys, nk - t0);
    for (int kk = 0; kk < tn; ++kk) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) s = fmaf(qv[i], ks[kk][i], s);
      s *= c;
      if (s > m) {
        const float a = exp2f(m - s);
        l *= a;
#pragma unroll
        for (int i = 0; i < D; ++i) o[i] *= a;
        m = s;
      }
      const float p = exp2f(s - m);
      l += p;
#pragma unroll
      for (int i = 0; i < D; ++i) o[i] = fmaf(p, vs[kk][i], o[i]);
    }
  }
  if (!active) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (out) {
#pragma unroll
    for (int i = 0; i < D; ++i) Elem<T>::store(out + qrow + i, o[i] * inv);
  }
  if (lse) lse[((size_t)n * n_q + r) * n_q_heads + h] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

// One thread per affix key j of request b (blockIdx.y) at layer blockIdx.z.
template <typename T, int D>
__global__ __launch_bounds__(64) void colmass_generic(
    const T* __restrict__ q, const T* __restrict__ pool_k, PoolGeom geo, const int32_t* __restrict__ masked_rows,
    const int32_t* __restrict__ masked_offsets, const int32_t* __restrict__ shared_slots, int L, int n_rows,
    int n_q_heads, int layer_begin, float scale, const float* __restrict__ lse, float* __restrict__ partial,
    int B) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y, n = blockIdx.z;
  if (j >= L) return;
  const int layer = layer_begin + n;
  const int m0 = masked_offsets[b], m1 = masked_offsets[b + 1];
  const int grp = n_q_heads / geo.n_kv_heads;
  const float c = scale * kLog2e;
  const int32_t slot = shared_slots[j];
  float acc = 0.f;
  for (int h = 0; h < n_q_heads; ++h) {
    float kv[D];
    const size_t krow = geo.row(layer, slot, h / grp);
#pragma unroll
    for (int i = 0; i < D; ++i) kv[i] = Elem<T>::load(pool_k + krow + i);
    for (int mi = m0; mi < m1; ++mi) {
      const int row = masked_rows[mi];
      const size_t qrow = (((size_t)n * n_rows + row) * n_q_heads + h) * D;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) s = fmaf(Elem<T>::load(q + qrow + i), kv[i], s);
      const float l2 = lse[((size_t)n * n_rows + row) * n_q_heads + h] * kLog2e;
      acc += exp2f(s * c - l2);
    }
  }
  partial[((size_t)n * B + b) * L + j] = acc;
}

// A workgroup owns 32 consecutive (request, key) columns; its eight row
// groups each sum every eighth partial row (four independent accumulators,
// so that each thread keeps four loads in flight), and the group sums are
// added in group order.  The order is fixed, so the result is deterministic.
constexpr int kRedCols = 32, kRedGroups = 8;
__global__ __launch_bounds__(kRedCols * kRedGroups) void colmass_reduce(const float* __restrict__ partial,
                                                                        int n_rows, int BL,
                                                                        float* __restrict__ scores) {
  __shared__ float part[kRedGroups][kRedCols];
  const int c = threadIdx.x % kRedCols, grp = threadIdx.x / kRedCols;
  const int t = blockIdx.x * kRedCols + c;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (t < BL) {
    int n = grp;
    for (; n + 3 * kRedGroups < n_rows; n += 4 * kRedGroups)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] += partial[(size_t)(n + u * kRedGroups) * BL + t];
    for (; n < n_rows; n += kRedGroups) acc[0] += partial[(size_t)n * BL + t];
  }
  part[grp][c] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (grp == 0 && t < BL) {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < kRedGroups; ++k) sum += part[k][c];
    scores[t] += sum;
  }
}

template <typename T>
static hipError_t attn_generic_dispatch(const AttnArgs& a, hipStream_t st) {
  dim3 grid((a.max_q + kGenRows - 1) / kGenRows, a.B, a.n_layers * a.n_q_heads);
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
#define ACACHE_GEN(DD)                                                                                       \
  hipLaunchKernelGGL((attn_fwd_generic<T, DD>), grid, dim3(kGenRows), 0, st, (const T*)a.q,                  \
                     (const T*)a.pool_k, (const T*)a.pool_v, a.geo, a.q_offsets, a.n_q, a.kv_table,          \
                     a.kv_offsets, a.n_kv, a.n_q_heads, a.layer_begin, a.scale, (T*)a.out, a.lse)
  switch (a.geo.head_dim) {
    case 16: ACACHE_GEN(16); break;
    case 32: ACACHE_GEN(32); break;
    case 64: ACACHE_GEN(64); break;
    default: ACACHE_GEN(128); break;
  }
#undef ACACHE_GEN
  return hipGetLastError();
}

hipError_t launch_attn_generic(const AttnArgs& a, int dtype, hipStream_t st) {
  return dtype == ACACHE_F32 ? attn_generic_dispatch<float>(a, st) : attn_generic_dispatch<bf16_t>(a, st);
}

template <typename T>
static hipError_t colmass_generic_dispatch(const ColmassArgs& a, hipStream_t st) {
  dim3 grid((a.L + 63) / 64, a.B, a.n_layers);
  if (grid.y == 0 || grid.z == 0) return hipSuccess;
#define ACACHE_CM(DD)                                                                                   \
  hipLaunchKernelGGL((colmass_generic<T, DD>), grid, dim3(64), 0, st, (const T*)a.q, (const T*)a.pool_k, \
                     a.geo, a.masked_rows, a.masked_offsets, a.shared_slots, a.L, a.n_rows, a.n_q_heads,  \
                     a.layer_begin, a.scale, a.lse, a.partial, a.B)
  switch (a.geo.head_dim) {
    case 16: ACACHE_CM(16); break;
    case 32: ACACHE_CM(32); break;
    case 64: ACACHE_CM(64); break;
    default: ACACHE_CM(128); break;
  }
#undef ACACHE_CM
  return hipGetLastError();
}

hipError_t launch_colmass_generic(const ColmassArgs& a, int dtype, hipStream_t st) {
  return dtype == ACACHE_F32 ? colmass_generic_dispatch<float>(a, st) : colmass_generic_dispatch<bf16_t>(a, st);
}

hipError_t launch_colmass_reduce(const float* partial, int n_rows, int B, int L, float* scores, hipStream_t st) {
  const int BL = B * L;
  if (BL == 0) return hipSuccess;
  hipLaunchKernelGGL(colmass_reduce, dim3((BL + kRedCols - 1) / kRedCols), dim3(kRedCols * kRedGroups), 0, st,
                     partial, n_rows, BL, scores);
  return hipGetLastError();
}

}  // namespace acache

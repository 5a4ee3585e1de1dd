// Elementwise companions of the ACache attention kernels (gfx950).
//
// Merge of two attentions over disjoint key sets: the softmax over
// the union of the sets weights each part's output by its share of the total
// exponential mass.  Used for the full-context reading of the probe
// normaliser of "Affix Cache for Diffusion Large Language Models" (Eq. (4),
// Section 3.2): the attention of the non-affix rows over the affix and over
// their own non-affix keys, combined.
#include "acache_dev.h"
#include "acache_launch.h"

namespace acache {

// Eight consecutive elements of one (row, head) per thread; the threads of a
// pair are consecutive lanes of one wave (head_dim / 8 divides 64), so an
// in-place LSE write by the pair's first lane follows every lane's read.
// o may be oa (and l may be la): those two carry no restrict qualifier.
template <typename T>
__global__ __launch_bounds__(256) void lse_merge_kernel(const T* oa, const float* la,
                                                        const T* __restrict__ ob, const float* __restrict__ lb,
                                                        T* o, float* l, long long n_pairs, int head_dim) {
  const int per = head_dim / 8;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_pairs * per) return;
  const long long pr = t / per;
  const int c = (int)(t - pr * per);
  const float a = la[pr], b = lb[pr];
  const float m = fmaxf(a, b);
  float wa = 0.f, wb = 0.f, lse = -INFINITY;
  if (m != -INFINITY) {
    const float ea = expf(a - m), eb = expf(b - m);
    const float s = ea + eb;
    wa = ea / s;
    wb = eb / s;
    lse = m + logf(s);
  }
  if (o) {
    const size_t base = (size_t)pr * head_dim + (size_t)c * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      Elem<T>::store(o + base + k, wa * Elem<T>::load(oa + base + k) + wb * Elem<T>::load(ob + base + k));
  }
  if (c == 0) l[pr] = lse;
}

hipError_t launch_lse_merge(int dtype, long long n_pairs, int head_dim, const void* oa, const float* la,
                            const void* ob, const float* lb, void* o, float* l, hipStream_t st) {
  if (n_pairs == 0) return hipSuccess;
  const long long threads = n_pairs * (head_dim / 8);
  const long long blocks = (threads + 255) / 256;
  if (blocks > (1ll << 31) - 1) return hipErrorInvalidValue;
  if (dtype == ACACHE_BF16)
    hipLaunchKernelGGL(lse_merge_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, st, (const bf16_t*)oa, la,
                       (const bf16_t*)ob, lb, (bf16_t*)o, l, n_pairs, head_dim);
  else
    hipLaunchKernelGGL(lse_merge_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, (const float*)oa, la,
                       (const float*)ob, lb, (float*)o, l, n_pairs, head_dim);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// CacheBlend-style HKVD selector scores (Appendix B.5 of the same paper): how
// far each affix token's full-prompt K and V lie from the affix-only cache
// in the shared region.  One wave per (request, affix offset); every lane
// sums the squared differences of 8 consecutive elements per step over the
// token's (KV head, d) block of each layer; one reduction per wave at the
// end, so the result is deterministic.
// ---------------------------------------------------------------------------
namespace {
template <typename T> struct Ld8;
template <> struct Ld8<bf16_t> {
  static __device__ __forceinline__ void run(const bf16_t* p, float* x) {
    const uint4 u = *(const uint4*)p;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
};
template <> struct Ld8<float> {
  static __device__ __forceinline__ void run(const float* p, float* x) {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};
}  // namespace

template <typename T>
__global__ __launch_bounds__(256) void hkvd_kernel(const T* __restrict__ pool_k, const T* __restrict__ pool_v,
                                                   PoolGeom geo, const int32_t* __restrict__ shared_slots,
                                                   const T* __restrict__ kf, const T* __restrict__ vf, int B, int L,
                                                   int layer_begin, int n_layers, float* __restrict__ scores) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // j-major: the waves of the B requests of one affix token run together, so
  // that token's shared rows come from HBM once and then from the caches
  const long long tok = (long long)blockIdx.x * 4 + wave;  // j * B + b
  if (tok >= (long long)B * L) return;
  const int j = (int)(tok / B), b = (int)(tok - (long long)j * B);
  const int32_t slot = shared_slots[j];
  const int d = geo.head_dim, hd = geo.n_kv_heads * d;
  float acc = 0.f;
  for (int n = 0; n < n_layers; ++n) {
    const size_t frow = (((size_t)n * B + b) * L + j) * hd;
    // four steps' loads are issued before their arithmetic (more loads in flight)
    for (int e0 = lane * 8; e0 < hd; e0 += 4 * 512) {
      float a[4][16], f[4][16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * 512;
        if (e < hd) {
          const int g = e / d, c = e - g * d;
          const size_t prow = geo.row(layer_begin + n, slot, g) + c;
          Ld8<T>::run(pool_k + prow, a[u]);
          Ld8<T>::run(kf + frow + e, f[u]);
          Ld8<T>::run(pool_v + prow, a[u] + 8);
          Ld8<T>::run(vf + frow + e, f[u] + 8);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + u * 512 < hd) {
#pragma unroll
          for (int k = 0; k < 16; ++k) acc += (f[u][k] - a[u][k]) * (f[u][k] - a[u][k]);
        }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) scores[(size_t)b * L + j] += acc;
}

hipError_t launch_hkvd(const void* pool_k, const void* pool_v, const PoolGeom& geo, const int32_t* shared_slots,
                       const void* kf, const void* vf, int B, int L, int layer_begin, int n_layers, int dtype,
                       float* scores, hipStream_t st) {
  const long long tokens = (long long)B * L;
  if (tokens == 0 || n_layers == 0) return hipSuccess;
  const long long blocks = (tokens + 3) / 4;
  if (blocks > (1ll << 31) - 1) return hipErrorInvalidValue;
  if (dtype == ACACHE_BF16)
    hipLaunchKernelGGL(hkvd_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, st, (const bf16_t*)pool_k,
                       (const bf16_t*)pool_v, geo, shared_slots, (const bf16_t*)kf, (const bf16_t*)vf, B, L,
                       layer_begin, n_layers, scores);
  else
    hipLaunchKernelGGL(hkvd_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, (const float*)pool_k,
                       (const float*)pool_v, geo, shared_slots, (const float*)kf, (const float*)vf, B, L, layer_begin,
                       n_layers, scores);
  return hipGetLastError();
}

}  // namespace acache

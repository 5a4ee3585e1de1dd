// Merge of two attentions over disjoint key sets (gfx950): the softmax over
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
template <typename T>
__global__ __launch_bounds__(256) void lse_merge_kernel(const T* __restrict__ oa, const float* la,
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

}  // namespace acache

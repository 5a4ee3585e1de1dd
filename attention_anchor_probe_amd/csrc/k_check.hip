// Checked mode: a device pre-pass over slot tables (gfx950).
//
// "Affix Cache for Diffusion Large Language Models", Section 4.1 (KV Layout
// and Dual Mapping): the shared region is only read by requests, and each
// request writes only its own private slots; Appendix C.1: new KV is stored
// through the write-side map before the read-slot kernel reads through the
// read-slot map.  The pre-pass reads the tables, the segment offsets and the
// page owners, never the pool: a bad slot id is only compared, never used as
// an address.  It records, per failure class, the smallest failing entry.
#include <algorithm>

#include "acache_dev.h"
#include "acache_launch.h"

namespace acache {

namespace {

constexpr int kCheckThreads = 256;

// Segment of entry i: the b with offsets[b] <= i < offsets[b+1] (offsets
// checked to be non-decreasing from 0 to n by check_offsets_kernel; on a bad
// table the search still stays inside offsets[0 .. B]).
__device__ __forceinline__ int segment_of(const int32_t* offsets, int B, int i) {
  int lo = 0, hi = B;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= i) lo = mid;
    else hi = mid;
  }
  return lo;
}

// rec[0..2]: smallest failing entry of ERANGE, EREGION, EDUP (INT32_MAX =
// none); first[s]: smallest entry naming slot s (WRITE mode)
__global__ __launch_bounds__(kCheckThreads) void check_clear_kernel(int32_t* rec, int32_t* first, int64_t n_first) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < 3) rec[t] = INT32_MAX;
  for (int64_t i = t; i < n_first; i += (int64_t)gridDim.x * blockDim.x) first[i] = INT32_MAX;
}

// The segment table itself: offsets[0] == 0, non-decreasing, offsets[B] == n;
// a bad table is an ERANGE at entry -1
__global__ __launch_bounds__(kCheckThreads) void check_offsets_kernel(const int32_t* offsets, int B, int n,
                                                                       int32_t* rec) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b > B) return;
  bool bad = false;
  if (b == 0) bad = offsets[0] != 0;
  else bad = offsets[b] < offsets[b - 1];
  if (b == B) bad = bad || offsets[B] != n;
  if (bad) atomicMin(&rec[0], -1);
}

// MODE 0 (read): slot in range; with page_owner, its page is shared (-1) or
// the segment's own (b); without segments, shared only.
// MODE 1 (write): slot in range; with page_owner, its page is the segment's
// own (without segments: some request's); the smallest entry of each slot
// is recorded in first[] for the duplicate pass.
template <int MODE>
__global__ __launch_bounds__(kCheckThreads) void check_slots_kernel(const int32_t* slots, int n,
                                                                     const int32_t* offsets, int B,
                                                                     const int32_t* page_owner, int64_t n_slots,
                                                                     int page_shift, int32_t* rec, int32_t* first) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t s = slots[i];
  if (s < 0 || (int64_t)s >= n_slots) {
    atomicMin(&rec[0], i);
    return;
  }
  if (page_owner) {
    const int32_t own = page_owner[(uint32_t)s >> page_shift];
    const int b = offsets ? segment_of(offsets, B, i) : -1;
    bool ok;
    if (MODE == 0) ok = own == -1 || (offsets && own == b);
    else ok = offsets ? own == b : own >= 0;
    if (!ok) atomicMin(&rec[1], i);
  }
  if (MODE == 1) atomicMin(&first[s], i);
}

// entries that repeat a slot named by an earlier entry
__global__ __launch_bounds__(kCheckThreads) void check_dup_kernel(const int32_t* slots, int n, int64_t n_slots,
                                                                   const int32_t* first, int32_t* rec) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t s = slots[i];
  if (s < 0 || (int64_t)s >= n_slots) return;
  if (first[s] != i) atomicMin(&rec[2], i);
}

}  // namespace

hipError_t launch_check_slots(const int32_t* slots, int n, const int32_t* offsets, int B,
                              const int32_t* page_owner, int64_t n_slots, int page_shift, int write_mode,
                              int32_t* rec, int32_t* first, hipStream_t stream) {
  const int64_t n_first = write_mode ? n_slots : 0;
  const int64_t clear_blocks = std::max<int64_t>(1, std::min<int64_t>((n_first + kCheckThreads - 1) / kCheckThreads,
                                                                      4096));
  check_clear_kernel<<<(unsigned)clear_blocks, kCheckThreads, 0, stream>>>(rec, first, n_first);
  if (offsets)
    check_offsets_kernel<<<(B + kCheckThreads) / kCheckThreads, kCheckThreads, 0, stream>>>(offsets, B, n, rec);
  if (n > 0) {
    const unsigned grid = (unsigned)((n + kCheckThreads - 1) / kCheckThreads);
    if (write_mode) {
      check_slots_kernel<1><<<grid, kCheckThreads, 0, stream>>>(slots, n, offsets, B, page_owner, n_slots,
                                                                 page_shift, rec, first);
      check_dup_kernel<<<grid, kCheckThreads, 0, stream>>>(slots, n, n_slots, first, rec);
    } else {
      check_slots_kernel<0><<<grid, kCheckThreads, 0, stream>>>(slots, n, offsets, B, page_owner, n_slots,
                                                                 page_shift, rec, first);
    }
  }
  return hipGetLastError();
}

}  // namespace acache

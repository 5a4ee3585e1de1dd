// bf16 MFMA kernels for head_dim 128 on gfx950 (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation).
//
//   softmax(q K^T * scale) V and LSE over a key list read through a slot
//   table: the probe forward of the non-affix rows over the shared affix
//   (Eq. 4 of "Affix Cache for Diffusion Large Language Models", Section 3.2)
//   and the read-slot attention of Section 4.3 / Appendix C.1, in two shapes:
//     attn_rows48_mfma a workgroup owns 192 query rows (48 per wave, three
//                      16-row blocks on the 16x16x32 MFMA) and every wave
//                      walks every key: units of at least 384 rows (probe,
//                      recompute-sized sets, packed grouped query heads);
//     attn_rows_mfma   the same with 128 query rows (32 per wave) for smaller
//                      units (a decode block's packed query-head group);
//     attn_store_rows_mfma  the same over a request's freshly recomputed
//                      rows, read from their source while the same launch
//                      stores them, and then its other keys
//                      (store-then-attend);
//     attn_split_mfma  a workgroup owns 32 query rows and its four waves split
//                      each 128-key tile into four 32-key slices; the partial
//                      (max, sum, O) of the waves are merged at the end
//                      (decode blocks of 32 queries);
//     attn_shared_mfma decode blocks of four requests that share the affix:
//                      the affix tiles are loaded once for the four, each
//                      wave then streams its own request's other keys.
//   colmass_mfma   the Eq. (4) weights of the masked rows recomputed as
//       exp(q.k * scale - LSE) and summed over the rows of each request: one
//       partial per (layer, query head, request, key); the partials are
//       summed in a fixed order afterwards (Eq. 5), so no atomics are used.
//
// MFMA 32x32x16 operand mapping used throughout (lane l, g = l / 32):
//   A (M x K): lane holds row l % 32, eight K-slots (g, j), j = 0..7
//   B (K x N): lane holds column l % 32, the same eight K-slots
//   C (M x N): lane holds column l % 32, rows 8*(i/4) + 4*g + i%4, i = 0..15
// A contraction only needs A and B to agree on what each K-slot means, so
// the head dimension is split as d = 16*c + 8*g + j for MFMA step c, and the
// key slots of the P.V product follow the C layout of the score tile.
#include <type_traits>

#include "acache_dev.h"
#include "acache_launch.h"

namespace acache {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int D = 128;
constexpr int KS = D + 8;  // LDS row stride (bf16) of K and Q tiles: 272 B, spreads rows over banks

struct AttnP {
  const bf16_t* q;
  const bf16_t* pool_k;
  const bf16_t* pool_v;
  PoolGeom geo;
  const int32_t* q_offsets;
  int n_q;
  int q_tiles;
  const int32_t* kv_table;
  const int32_t* kv_offsets;
  int n_kv;
  size_t layer_bytes;  // bytes of one layer of the K (or V) pool, < 4 GiB
  int B;
  int n_q_heads;
  int layer_begin;
  float c2;  // scale * log2(e)
  bf16_t* out;
  float* lse;
  int n_units;
  int per_xcd;
  // attn_shared_mfma only: bit j of excl[b * excl_words + j / 32] set = affix
  // key j is not read from the shared region by request b (the padding up to
  // whole 64-key tiles is set too); request b's other read slots are
  // priv_table[b * kv_stride .. + kv_counts[b])
  const uint32_t* excl;
  int excl_words;
  const int32_t* priv_table;
  const int32_t* kv_counts;
  int kv_stride;
  // attn_store_rows_mfma only: request b's fresh K/V rows are rows
  // src_offsets[b] .. src_offsets[b+1] of src_k / src_v
  // ([layers][n_src][n_kv_heads][128]); they are attended before its other keys
  // (priv_table / kv_counts / kv_stride) and copied to pool slots src_slot[i]
  const char* src_k;
  const char* src_v;
  const int32_t* src_slot;
  const int32_t* src_offsets;
  int n_src;
  char* pool_kw;  // the pool, written by the copy
  char* pool_vw;
  // attn_rows_mfma only: gpack > 1 packs the query heads of a KV-head group
  // into the rows of a unit (a unit is then a (layer, KV head, request, row
  // tile); its rows are the pairs (head g*gpack + j, query i), j-major), so
  // that every K/V tile serves all heads of the group
  int gpack;
};

struct ColP {
  const bf16_t* q;
  const bf16_t* pool_k;
  PoolGeom geo;
  const int32_t* masked_rows;
  const int32_t* masked_offsets;
  int n_masked;
  const int32_t* shared_slots;
  int L;
  int n_rows;
  int n_q_heads;
  int layer_begin;
  int B;
  float c2;
  const float* lse;
  float* partial;  // [n_layers][n_q_heads][B][L]
  const float* lse_prep;  // per (layer, query head): -LSE/scale of the masked rows, padded
  size_t lse_stride;
  int key_blocks;
  int n_units;
  int per_xcd;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ u32x4 ld16(const bf16_t* p) { return *(const u32x4*)p; }

// 2^x on the hardware exp unit (v_exp_f32): results below 2^-126 flush
// toward zero, which is harmless for softmax weights; exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// two floats to packed bf16 (round to nearest even, one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum of lanes l and l ^ 32 (the two halves of a score column), on the
// VALU: permlane32_swap leaves lane l's partner value in one of its two results
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous run of logical units so that units sharing K/V (or Q) run on
// the same XCD and hit its L2.
__device__ __forceinline__ int xcd_unit(int per_xcd) {
  const int i = blockIdx.x;
  return (i & 7) * per_xcd + (i >> 3);
}


}  // namespace

// 16-byte chunk swizzle of a 256-byte V row: conflict-free for row-wise
// 16-byte writes and for the transposing reads (4 rows x 2 chunks per 16 lanes)
__device__ __forceinline__ uint32_t vswz_rows(uint32_t row, uint32_t chunk) { return chunk ^ ((row & 3u) << 2); }

// bf16x4 view of LDS for the transposing reads
typedef __bf16 bf16x4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4s lds_bf16x4s;

__global__ __launch_bounds__(256, 2) void attn_split_mfma(AttnP p) {
  constexpr int BN = 128;                // keys per LDS tile; wave w computes keys 32w .. 32w+31
  constexpr int KLD = BN * 16 / 256;     // 16-byte K (and V) row pieces per thread per tile
  constexpr int KS_BYTES = BN * KS * 2;
  constexpr int VR_BYTES = BN * D * 2;
  constexpr int MERGE_BYTES = 4 * 4 * 16 * 64 * 4 + 2 * 4 * 64 * 4;
  constexpr int LDS_BYTES = (KS_BYTES + VR_BYTES) > MERGE_BYTES ? (KS_BYTES + VR_BYTES) : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  bf16_t* Ks = (bf16_t*)smem;
  char* Vr = smem + KS_BYTES;  // V rows as stored in the pool, 16-byte chunks swizzled by row

  const int unit = xcd_unit(p.per_xcd);
  if (unit >= p.n_units) return;
  int r = unit;
  const int t = r % p.q_tiles;
  r /= p.q_tiles;
  const int b = r % p.B;
  r /= p.B;
  const int h = r % p.n_q_heads;
  const int n = r / p.n_q_heads;
  const int g = h / (p.n_q_heads / p.geo.n_kv_heads);
  const int layer = p.layer_begin + n;
  int q0 = 0, q1 = p.n_q, k0 = 0, k1 = p.n_kv;
  if (p.q_offsets) { q0 = p.q_offsets[b]; q1 = p.q_offsets[b + 1]; }
  if (p.kv_offsets) { k0 = p.kv_offsets[b]; k1 = p.kv_offsets[b + 1]; }
  const int rbase = q0 + t * 32;
  if (rbase >= q1) return;
  const int nk = k1 - k0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g2 = lane >> 5, l32 = lane & 31;
  const int qrow = rbase + l32;
  const bool qvalid = qrow < q1;

  // Q as the B operand of S^T = K Q^T
  bf16x8 qf[8];
  {
    const bf16_t* qp = p.q + (((size_t)n * p.n_q + (qvalid ? qrow : q0)) * p.n_q_heads + h) * D + g2 * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = qvalid ? as_bf16x8(ld16(qp + c * 16)) : as_bf16x8(u32x4{0, 0, 0, 0});
  }

  float m = -INFINITY, lsum = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};

  u32x4 kreg[KLD], vreg[KLD];
  uint32_t koff[KLD];
  const int ntiles = (nk + BN - 1) / BN;
  // one layer of the pool is addressed from a scalar base with 32-bit byte offsets
  const char* kbase = (const char*)p.pool_k + (size_t)layer * p.layer_bytes;
  const char* vbase = (const char*)p.pool_v + (size_t)layer * p.layer_bytes;
  const uint32_t page_bytes = (uint32_t)p.geo.n_kv_heads * p.geo.page_size * D * 2;
  const uint32_t head_off = (uint32_t)g * p.geo.page_size * D * 2 + (uint32_t)(tid & 15) * 16;
  auto slot_off = [&](int32_t slot) -> uint32_t {
    return ((uint32_t)slot >> p.geo.page_shift) * page_bytes + head_off +
           ((uint32_t)slot & (uint32_t)(p.geo.page_size - 1)) * (D * 2);
  };

  // Thread tid moves 16-byte piece tid%16 of rows tid/16 + 16e of the tile,
  // for K and for V.  Slots of a tile are loaded one tile ahead of its rows,
  // so a row load never waits on the table load that names it.  Keys past the
  // end are clamped to the last key (their scores are masked to -inf below,
  // so their rows only ever meet a zero weight).
  auto sload = [&](int tile) {
    const int kb = tile * BN;
#pragma unroll
    for (int e = 0; e < KLD; ++e) koff[e] = (uint32_t)p.kv_table[k0 + min(kb + (tid >> 4) + 16 * e, nk - 1)];
  };
  auto dload = [&]() {
#pragma unroll
    for (int e = 0; e < KLD; ++e) {
      const uint32_t off = slot_off((int32_t)koff[e]);
      kreg[e] = *(const u32x4*)(kbase + off);
      vreg[e] = *(const u32x4*)(vbase + off);
    }
  };
  auto lstore = [&]() {
    const uint32_t dc = tid & 15;
#pragma unroll
    for (int e = 0; e < KLD; ++e) {
      const uint32_t key = (tid >> 4) + 16 * e;
      *(u32x4*)(Ks + key * KS + dc * 8) = kreg[e];
      *(u32x4*)(Vr + key * (D * 2) + vswz_rows(key, dc) * 16) = vreg[e];
    }
  };

  // per-lane offsets of the transposing V reads (keys 4*g + 0..3 and
  // 8 + 4*g + 0..3 of each 16-key block, d column a*32 + lane%32)
  const uint32_t i16 = lane & 15;
  uint32_t vrd[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint32_t row = wave * 32 + 4 * g2 + (i16 >> 2);
    const uint32_t dcol = a * 32 + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
    vrd[a] = row * (D * 2) + vswz_rows(row, dcol >> 3) * 16 + (dcol & 7) * 2;
  }

  if (ntiles > 0) {
    sload(0);
    dload();
    if (ntiles > 1) sload(1);
  }
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();
    lstore();
    __syncthreads();
    if (tile + 1 < ntiles) {
      dload();
      if (tile + 2 < ntiles) sload(tile + 2);
    }
    const int kb = tile * BN;
    f32x16 s = f32x16{};
    {
      const bf16_t* kp = Ks + (wave * 32 + l32) * KS + g2 * 8;
#pragma unroll
      for (int c = 0; c < 8; ++c) s = mfma(as_bf16x8(*(const u32x4*)(kp + c * 16)), qf[c], s);
    }
    // keys past the end (tail tile only) get -inf; the running max m lives in
    // the scaled log2 domain, c2 > 0, so max(s) * c2 is the scaled tile max
    if (kb + BN > nk) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb + wave * 32 + 8 * (i >> 2) + 4 * g2 + (i & 3) >= nk) s[i] = -INFINITY;
    }
    float mr = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mr = fmaxf(mr, s[i]);
    mr = half_max(mr);
    const float mt = mr * p.c2;
    // rescale only when the running max grows by more than 2^8 (exact either
    // way: O and the row sum carry the same factor)
    if (mt > m + 8.f) {
      const float alpha = exp2f(m - mt);
      lsum *= alpha;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[a][i] *= alpha;
      m = mt;
    }
    const float nm = (m == -INFINITY) ? 0.f : -m;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x8 pb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pv = fast_exp2(fmaf(s[8 * hh + j], p.c2, nm));
        lsum += pv;
        pb[j] = (__bf16)pv;
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const char* vp = Vr + vrd[a] + 16 * hh * (D * 2);
        const bf16x4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4s*)vp);
        const bf16x4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4s*)(vp + 8 * (D * 2)));
        o[a] = mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, o[a]);
      }
    }
  }

  // merge the four waves' partial results through LDS
  float* red = (float*)smem;                      // [wave][a][i][lane]
  float* mw = red + 4 * 4 * 16 * 64;              // [wave][lane]
  float* lw = mw + 4 * 64;                        // [wave][lane]
  const float lt = half_sum(lsum);
  __syncthreads();  // every wave is done with the K/V tiles
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) red[((wave * 4 + a) * 16 + i) * 64 + lane] = o[a][i];
  mw[wave * 64 + lane] = m;
  lw[wave * 64 + lane] = lt;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, mw[w * 64 + lane]);
  float f[4], Lt = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mwv = mw[w * 64 + lane];
    f[w] = mwv == -INFINITY ? 0.f : exp2f(mwv - M);
    Lt += f[w] * lw[w * 64 + lane];
  }
  if (!qvalid) return;
  const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
  const int a = wave;  // each wave finishes one 32-wide slice of the head dimension
  if (p.out) {
    bf16_t* op = p.out + (((size_t)n * p.n_q + qrow) * p.n_q_heads + h) * D;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      float v4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = 4 * i4 + k;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) acc += red[((w * 4 + a) * 16 + i) * 64 + lane] * f[w];
        v4[k] = acc * inv;
      }
      const int d = a * 32 + 8 * i4 + 4 * g2;
      u32x2 wv;
      wv[0] = pack_bf16x2(v4[0], v4[1]);
      wv[1] = pack_bf16x2(v4[2], v4[3]);
      *(u32x2*)(op + d) = wv;
    }
  }
  if (p.lse && wave == 0 && g2 == 0)
    p.lse[((size_t)n * p.n_q + qrow) * p.n_q_heads + h] = Lt > 0.f ? (M + log2f(Lt)) * kLn2 : -INFINITY;
}

// Many-query attention (probe forward over the shared affix; read-slot
// attention of recompute-sized query sets).  A workgroup owns 128 query rows
// (32 per wave) and walks the key list in tiles of 64.  K and V tiles are
// gathered through the slot table straight into LDS (two K and two V
// stages) by direct-to-LDS loads (no register staging); rows are stored as
// they sit in the pool with their 16-byte chunks XOR-swizzled by row, and the
// V^T operands of P.V come from transposing LDS reads.  Slot numbers arrive
// through buffer loads a tile ahead; the next tile's loads are in flight while
// the current one is computed, with one barrier per tile.
namespace {
constexpr int RB = 64;                   // keys per tile
constexpr int RSTAGES = 2;
constexpr int ROWB = D * 2;              // bytes of one K or V row
constexpr int RSTAGE_BYTES = RB * ROWB * 2;
constexpr int PTILE = kSharedPrivTile;   // keys per private tile of attn_shared_mfma (per wave)
static_assert(4 * PTILE * ROWB * 2 <= RSTAGES * RSTAGE_BYTES, "private regions fit the tile ring");

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Workgroup barrier without the full memory drain __syncthreads() implies:
// the direct-to-LDS tile loads are waited for explicitly (vmcnt) before it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Direct-to-LDS loads.  Lane i's bytes land at LDS byte address
// lds_base + size * i; M0 holds lds_base, passed to the instruction as an
// operand (the compiler sets it).  They are issued as asm: the compiler's
// wait insertion would treat a load into one LDS stage as a store that every
// later LDS read must wait for, also the reads of the other stage.  The
// kernels wait for these loads on vmcnt explicitly (a stage is read only
// after the wait and barrier that follow its loads), and every load whose
// result they consume is waited for after such an explicit wait.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_base) : "memory");
}

// the same with a scalar base and a 32-bit per-lane byte offset (saddr form:
// no 64-bit address arithmetic per lane)
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_base) : "memory");
}

// 4 bytes per lane from a per-lane global address
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(gptr), "{m0}"(lds_base) : "memory");
}

// A wave-uniform pointer, asserted to the compiler so that it stays in scalar
// registers (the scalar base of dma16s).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// x on the lanes whose bit of `lanes` is clear, y on the others: one
// v_cndmask with a scalar lane mask (the mask is built on the scalar unit;
// the compiler keeps the wait states a matrix-unit result needs before it)
__device__ __forceinline__ float select_lanes(float x, float y, uint64_t lanes) {
  return __builtin_amdgcn_inverse_ballot_w64(lanes) ? y : x;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// 16-byte chunk swizzles of a 256-byte K or V row: conflict-free for the
// MFMA operand reads of K (16 rows x one chunk) and the transposing reads of
// V (4 rows x 2 chunks per 16 lanes)
__device__ __forceinline__ uint32_t kswz(uint32_t row, uint32_t chunk) { return chunk ^ (row & 15u); }
__device__ __forceinline__ uint32_t vswz2(uint32_t row, uint32_t chunk) { return chunk ^ ((row & 3u) << 2); }
}  // namespace

// Key-list source of tile_loop: key j of the list is slot table[j] of the
// (layer, KV head) whose rows start at kbase / vbase.  A mixed source
// (tile_loop<_, true>) puts nf rows of a contiguous buffer first: keys
// 0 .. nf-1 are rows 0 .. nf-1 at byte offset j * fstride from fkbase /
// fvbase, and keys nf .. nk-1 are slots table[0 .. nk-nf-1].
struct TileSrc {
  const char* kbase;
  const char* vbase;
  uint32_t page_bytes;  // bytes of one page of one layer (all KV heads)
  uint32_t head_off;    // byte offset of the KV head within a page
  int page_shift;
  uint32_t page_mask;
  const int32_t* table;
  int nk;
  const uint32_t* excl;  // EXCL only: bit j of excl[j / 32] set drops key j (padded to 64-key tiles)
  const char* fkbase;    // MIXED only
  const char* fvbase;
  uint32_t fstride;
  int nf;
};

// Streams a key list through the workgroup's LDS in 64-key tiles into the
// online softmax (running max m in scaled log2 units, row sum lsum, O
// accumulators o) of this wave's 32 query rows, whose Q fragments are qf.
// Every wave of the workgroup calls it: the tile loads are shared, and
// waves with live == false only help load.
template <bool EXCL, bool MIXED = false>
__device__ __forceinline__ void tile_loop(char* smem, const TileSrc& src, float c2, const bf16x8 (&qf)[8],
                                          bool live, int wave, int lane, float& m, float& lsum, f32x16 (&o)[4]) {
  const int nk = src.nk;
  const int ntiles = (nk + RB - 1) / RB;
  const int g2 = lane >> 5, l32 = lane & 31;

  // Tile t's K rows sit in K stage t%2 and its V rows in V stage t%2; this
  // wave loads rows 16*wave .. 16*wave+15 of each: DMA instruction i covers
  // rows 16*wave + 4i + lane/16, one 16-byte chunk per lane.  Iteration t
  // computes the scores of tile t+1 while it takes the softmax and P.V of
  // tile t (scores computed one iteration earlier), and starts the loads of
  // K(t+2) and V(t+1): every load has a whole iteration to land.
  constexpr uint32_t KSTAGE = RB * ROWB;
  // per-lane parts of the DMA addresses: lane/16 picks the row of the 4-row
  // group, lane%16 the LDS chunk; the global chunk is its swizzle
  const int sel = lane >> 4;
  // slot of the row this lane moves in DMA instruction i of the next K tile
  // (row 16*wave + 4i + lane/16), loaded a tile ahead of its use
  // Full tiles read their four slots through a buffer resource (lane part
  // in the vector offset, tile and row-group parts in the scalar offset).  The last, partial tile clamps
  // its rows to the last key of the list instead, so that every V row it
  // loads is one of the list's rows (finite; its weight is zero).  MIXED:
  // key j below nf is row j of the contiguous buffer; the others read
  // table[j - nf] through a buffer resource sized to the table (the loads of
  // keys below nf read its first entry and are not used).
  const int nf = MIXED ? src.nf : 0;
  const int32_t* vtable = src.table;
  const __amdgpu_buffer_rsrc_t trs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vtable, (short)0, (nk - nf) * 4, 0x00020000);
  const uint32_t trow = (uint32_t)(16 * wave + sel) * 4;
  int32_t vs[4];
  // the list position of the row this lane moves in DMA instruction i
  auto key_of = [&](int tile, int i) { return min(tile * RB + 16 * wave + sel + 4 * i, nk - 1); };
  auto sload = [&](int tile, int32_t* vs) {
    if constexpr (MIXED) {
      // contiguous rows need no table read; whole table tiles read it as
      // below, shifted by nf; the tile across nf and the last partial tile
      // read it per lane.  A loaded value is used a tile later (selecting
      // between it and the row index here would wait for the load)
      if (tile * RB + RB <= nf) {
      } else if (tile * RB >= nf && tile * RB + RB <= nk) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vs[i] = __builtin_amdgcn_raw_buffer_load_b32(trs, trow, (tile * RB - nf) * 4 + 16 * i, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vs[i] = __builtin_amdgcn_raw_buffer_load_b32(trs, (uint32_t)max(key_of(tile, i) - nf, 0) * 4, 0, 0);
      }
    } else if (tile * RB + RB <= nk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vs[i] = __builtin_amdgcn_raw_buffer_load_b32(trs, trow, tile * (RB * 4) + 16 * i, 0);
    } else {
      const int r0 = tile * RB + 16 * wave + sel;
#pragma unroll
      for (int i = 0; i < 4; ++i) vs[i] = vtable[min(r0 + 4 * i, nk - 1)];
    }
  };
  // global chunk offsets (bits 4..7 of a row offset) of the K and V rows
  // this lane moves; kvx turns a K offset into the V offset of the same row
  uint32_t kchunk[4], kvx[4];
  const uint32_t vchunk = vswz2(sel, lane & 15) * 16;  // row & 3 == sel
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kchunk[i] = kswz(4 * i + sel, lane & 15) * 16;  // row & 15 == (4i + sel)
    kvx[i] = kchunk[i] ^ vchunk;
  }
  const uint32_t lds0 = lds_addr(smem) + 16 * wave * ROWB;
  const char* kbase_s = uniform_ptr(src.kbase + src.head_off);
  const char* vbase_s = uniform_ptr(src.vbase + src.head_off);
  const uint32_t rmask = src.page_mask << 8;
  const char* fkbase_s = MIXED ? uniform_ptr(src.fkbase) : nullptr;
  const char* fvbase_s = MIXED ? uniform_ptr(src.fvbase) : nullptr;
  // K loads of a tile also record its row offsets (off, with the K chunk),
  // which its V loads reuse one iteration later.  MIXED: a lane whose key
  // is below nf loads from the contiguous buffer; only the tile across nf
  // has lanes of both kinds
  auto pool_off = [&](const int32_t* vs, int i) {
    const uint32_t slot = (uint32_t)vs[i];
    // page index and page bytes are below 2^24, their product plus the row
    // offset below 2^32; the row part (bits 8..) and the chunk part (bits
    // 4..7) do not overlap
    return __umul24(slot >> src.page_shift, src.page_bytes) + (((slot << 8) & rmask) | kchunk[i]);
  };
  // row bytes and row count below 2^24, their product below 2^32; a whole
  // tile of contiguous rows splits the offset into a tile part (scalar) and
  // this lane's row and chunk
  auto fresh_off = [&](int tile, int i) { return __umul24((uint32_t)key_of(tile, i), src.fstride) + kchunk[i]; };
  const uint32_t frow0 = MIXED ? __umul24((uint32_t)(16 * wave + sel), src.fstride) : 0u;
  auto fresh_off_full = [&](int tile, int i) {
    return __umul24((uint32_t)(tile * RB + 4 * i), src.fstride) + frow0 + kchunk[i];
  };
  // a K tile's row offsets from its slots (koff), then its loads (kissue)
  auto koff = [&](int tile, uint32_t* off, const int32_t* vs) {
    if (!MIXED || tile * RB >= nf) {  // only table keys (uniform)
#pragma unroll
      for (int i = 0; i < 4; ++i) off[i] = pool_off(vs, i);
    } else if (tile * RB + RB <= nf) {  // only contiguous rows (uniform)
#pragma unroll
      for (int i = 0; i < 4; ++i) off[i] = fresh_off_full(tile, i);
    } else {  // the one tile across nf: per lane
#pragma unroll
      for (int i = 0; i < 4; ++i) off[i] = key_of(tile, i) < nf ? fresh_off(tile, i) : pool_off(vs, i);
    }
  };
  auto kissue = [&](int tile, const uint32_t* off) {
    const uint32_t st = lds0 + (tile & 1) * KSTAGE;
    if (!MIXED || tile * RB >= nf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16s(kbase_s, off[i], st + 4 * i * ROWB);
    } else if (tile * RB + RB <= nf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16s(fkbase_s, off[i], st + 4 * i * ROWB);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (key_of(tile, i) < nf) dma16s(fkbase_s, off[i], st + 4 * i * ROWB);
        else dma16s(kbase_s, off[i], st + 4 * i * ROWB);
      }
    }
  };
  auto dma_k = [&](int tile, uint32_t* off, const int32_t* vs) {
    koff(tile, off, vs);
    kissue(tile, off);
  };
  auto dma_v = [&](int tile, const uint32_t* off) {
    const uint32_t st = lds0 + (2 + (tile & 1)) * KSTAGE;
    if (!MIXED || tile * RB >= nf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16s(vbase_s, off[i] ^ kvx[i], st + 4 * i * ROWB);
    } else if (tile * RB + RB <= nf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16s(fvbase_s, off[i] ^ kvx[i], st + 4 * i * ROWB);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (key_of(tile, i) < nf) dma16s(fvbase_s, off[i] ^ kvx[i], st + 4 * i * ROWB);
        else dma16s(vbase_s, off[i] ^ kvx[i], st + 4 * i * ROWB);
      }
    }
  };

  // per-lane LDS read offsets within a stage (row and swizzle parts; the tile
  // sub-block adds compile-time multiples of 16 rows, which keep the swizzle)
  uint32_t krd[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) krd[c] = l32 * ROWB + kswz(l32, 2 * c + g2) * 16;
  const uint32_t i16 = lane & 15;
  uint32_t vrd[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint32_t row = 4 * g2 + (i16 >> 2);
    const uint32_t dcol = a * 32 + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
    vrd[a] = row * ROWB + vswz2(row, dcol >> 3) * 16 + (dcol & 7) * 2;
  }

  auto scores = [&](f32x16* s, int tile) {
    const char* st = smem + (tile & 1) * KSTAGE;
    s[0] = s[1] = f32x16{};
    // the two 32-key halves alternate, so that two independent accumulation
    // chains share the matrix pipe.  In the shared-affix decode (EXCL), where
    // workgroups in the memory-bound private phase share the CU, the shared
    // phase runs at wave priority 1 and its score block at 2; in the
    // many-query kernels, where every wave is matrix-bound, raising the
    // priority was slower
    if constexpr (EXCL) __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        s[sub] = mfma(as_bf16x8(*(const u32x4*)(st + krd[c] + sub * 32 * ROWB)), qf[c], s[sub]);
      }
    if constexpr (EXCL) __builtin_amdgcn_s_setprio(1);
  };
  // A tile's scores become its softmax weights as soon as they are computed,
  // at the end of the iteration before the one that takes P.V: the body of an
  // iteration (next scores, this tile's P.V, the next tile's exponentials) is
  // then free of data-dependent branches, so the matrix and vector work of
  // one wave can interleave.
  // EXCL: the tile's two exclusion words (one per 32-key half) are loaded
  // with vector loads two tiles ahead (a scalar load would have to wait for
  // every LDS read in flight) and taken into scalar registers after the wait
  // that opens the iteration
  auto xload = [&](int tile, uint32_t* x) {
    if constexpr (EXCL) {
      if (tile < ntiles) {
        x[0] = src.excl[2 * tile];
        x[1] = src.excl[2 * tile + 1];
      }
    }
  };
  // Keys a tile must not count: EXCL, the dropped keys and the padding past
  // the list (exclusion bits; applied to the scores on every tile, without a
  // branch: most affix tiles hold an anchor); otherwise the keys of the last,
  // partial tile past the end of the list (their rows repeat the list's last
  // key, so their scores are finite).  Lane half g2 holds keys
  // 8*(i/4) + 4*g2 + i%4 of each 32-key half.
  auto excl_mask = [&](f32x16* s, uint32_t e0, uint32_t e1) {
    // element i of lane half g2 is key 8*(i/4) + 4*g2 + i%4: its bit for
    // lanes 0..31 and lanes 32..63 forms a 64-bit lane mask
    const float ninf = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const uint32_t w = sub ? e1 : e0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t k = 8 * (i >> 2) + (i & 3);
        const uint32_t lo = 0u - ((w >> k) & 1u), hi = 0u - ((w >> (k + 4)) & 1u);
        s[sub][i] = select_lanes(s[sub][i], ninf, ((uint64_t)hi << 32) | lo);
      }
    }
  };
  auto past_end = [&](int tile, int sub, int i) { return tile * RB + sub * 32 + 8 * (i >> 2) + 4 * g2 + (i & 3) >= nk; };
  auto mask = [&](f32x16* s, int tile, uint32_t e0, uint32_t e1) {
    if constexpr (EXCL) {
      excl_mask(s, e0, e1);
    } else if (tile * RB + RB > nk) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (past_end(tile, sub, i)) s[sub][i] = -INFINITY;
    }
  };
  // weights P = 2^(s * c2 + nm) in place and this lane's sum of them (its 32
  // keys of the tile), in four short chains
  auto lane_sum = [&](const f32x16* s) -> float {
    float ls[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = sub ? 0 : 4; i < 16; ++i) ls[i & 3] += s[sub][i];
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  auto expsum = [&](f32x16* s, float nm) -> float {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[sub][i] = fast_exp2(fmaf(s[sub][i], c2, nm));
    return lane_sum(s);
  };
  // The exact step: the tile's max (both lane halves of a query), the
  // running max raised to it when it is larger (O and the row sum rescaled
  // by the same factor, so the result is exact either way), then the weights.
  auto weigh_exact = [&](f32x16* s) -> float {
    float mr = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 16; ++i) mr = fmaxf(mr, s[sub][i]);
    const float mt = half_max(mr) * c2;
    if (mt > m) {
      const float alpha = exp2f(m - mt);  // 0 while m is -inf (O and the sum are still 0)
      lsum *= alpha;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[a][i] *= alpha;
      m = mt;
    }
    return expsum(s, m == -INFINITY ? 0.f : -m);
  };
  // Weights of a freshly scored tile against the running max as it stands
  // (weigh_fast, in the iteration body) and their check (weigh_check).  When every
  // lane's sum stays at most 2^8 (so every weight does, as with a running max
  // within 8 of the true one), the weights are kept; otherwise (a key above
  // the running max by more than a factor 8 on average, or no finite running
  // max yet: weights inf or NaN) the wave takes the exact step on scores
  // recomputed from the tile, which is still in LDS.  No tile max is needed
  // on the common path, and no branch stands before the exponentials: the
  // last tile's keys past the end are zeroed after them.
  // the weights in bf16, the operand of P.V: pw[sub][hh] holds keys
  // 16*hh + (the C layout's eight per lane) of 32-key half sub
  auto to_bf16 = [&](const f32x16* s, bf16x8 (*pw)[2]) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int j = 0; j < 8; ++j) pw[sub][hh][j] = (__bf16)s[sub][8 * hh + j];
  };
  auto weigh_fast = [&](f32x16* s, bf16x8 (*pw)[2], float& ls, uint32_t e0, uint32_t e1) {
    if constexpr (EXCL) excl_mask(s, e0, e1);
    ls = expsum(s, -m);
    asm volatile("" ::"v"(ls));  // the weights and their sum belong to the iteration body
    to_bf16(s, pw);
  };
  auto weigh_check = [&](f32x16* s, bf16x8 (*pw)[2], int tile, float ls, uint32_t e0, uint32_t e1) {
    if constexpr (!EXCL) {
      if (tile * RB + RB > nk) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (past_end(tile, sub, i)) s[sub][i] = 0.f;
        ls = lane_sum(s);
        to_bf16(s, pw);
      }
    }
    if (__builtin_amdgcn_ballot_w64(!(ls <= 256.f)) != 0) {
      scores(s, tile);
      mask(s, tile, e0, e1);
      ls = weigh_exact(s);
      to_bf16(s, pw);
    }
    lsum += ls;
  };
  // The matrix work of an iteration: the scores of tile t+1 (K fragments,
  // accumulated from zero) and P.V of tile t (V^T fragments from transposing
  // reads, P rounded to bf16 as the other operand), one MFMA of each in
  // turn, so that the K and the V reads are spread evenly over the MFMAs.
  // The V^T operand's key slots follow the score tile's C layout (keys
  // 4*g + 0..3 and 8 + 4*g + 0..3 of each 16-key block).
  auto score_absorb = [&](f32x16* s, int stile, const bf16x8 (*pw)[2], int vtile) {
    const char* st = smem + (stile & 1) * KSTAGE;
    const char* vst = smem + (2 + (vtile & 1)) * KSTAGE;
    s[0] = s[1] = f32x16{};
    if constexpr (EXCL) __builtin_amdgcn_s_setprio(2);  // see scores()
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = i >> 1, sub = i & 1;
      s[sub] = mfma(as_bf16x8(*(const u32x4*)(st + krd[c] + sub * 32 * ROWB)), qf[c], s[sub]);
      const int vsub = i >> 3, hh = (i >> 2) & 1, a = i & 3;
      const char* vp = vst + vrd[a] + (vsub * 32 + 16 * hh) * ROWB;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vp);
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 8 * ROWB));
      o[a] = mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pw[vsub][hh], o[a]);
    }
  };
  // Instruction order of that block (the compiler keeps each LDS read next
  // to the MFMA that takes it, so every MFMA would wait out a whole LDS
  // latency): reads two MFMA pairs ahead, the V pair after each score MFMA
  // and the K fragment after each P.V MFMA.  The tile's weights follow.
  auto pipeline = [&]() {
    constexpr int kMfma = 0x008, kDsRead = 0x100;
    __builtin_amdgcn_sched_group_barrier(kDsRead, 6, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      if (i < 14) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      if (i < 14) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
    }
  };
  // one iteration: pc holds the bf16 weights of tile t, pn receives those of
  // t+1; oc holds the row offsets of tile t+1, on receives those of t+2;
  // xc holds the exclusion words of tile t+1, xn receives those of t+2
  f32x16 sn[2];
  auto step = [&](int tile, const bf16x8 (*pc)[2], bf16x8 (*pn)[2], const uint32_t* oc, uint32_t* on,
                  const uint32_t* xc, uint32_t* xn) {
    __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): K(t+1) and V(t) have landed
    wg_barrier();                        // ... in every wave; K(t) and V(t-1) are no longer read
    uint32_t f0 = 0, f1 = 0;
    if constexpr (EXCL) {
      f0 = __builtin_amdgcn_readfirstlane(xc[0]);
      f1 = __builtin_amdgcn_readfirstlane(xc[1]);
      xload(tile + 2, xn);
    }
    if (tile + 2 < ntiles) {
      dma_k(tile + 2, on, vs);
      if (tile + 3 < ntiles) sload(tile + 3, vs);
    }
    if (tile + 1 < ntiles) dma_v(tile + 1, oc);
    if (!live) return;
    score_absorb(sn, tile + 1, pc, tile);
    pipeline();
    // back to the phase's priority only after the scheduling groups: an
    // s_setprio bounds a scheduling region, and one inside the block would
    // leave its MFMAs and LDS reads outside the groups
    if constexpr (EXCL) __builtin_amdgcn_s_setprio(1);
    float ls;
    weigh_fast(sn, pn, ls, f0, f1);
    weigh_check(sn, pn, tile + 1, ls, f0, f1);
  };

  // the last iteration: P.V of the last tile only (there is no next tile to
  // score, so its body is the absorb half of score_absorb)
  auto last_step = [&](int tile, const bf16x8 (*pc)[2]) {
    __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): V(t) has landed
    wg_barrier();                        // ... in every wave
    if (!live) return;
    const char* vst = smem + (2 + (tile & 1)) * KSTAGE;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int vsub = i >> 3, hh = (i >> 2) & 1, a = i & 3;
      const char* vp = vst + vrd[a] + (vsub * 32 + 16 * hh) * ROWB;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vp);
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 8 * ROWB));
      o[a] = mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pc[vsub][hh], o[a]);
    }
  };

  bf16x8 pa[2][2], pb[2][2];
  uint32_t oa[4], ob[4];
  uint32_t xa[2] = {0u, 0u}, xb[2] = {0u, 0u};
  if (ntiles > 0) {
    // the slots of tiles 0 and 1 in one round trip, both tiles' offsets
    // (the one wait for them, before any tile load: the compiler does not
    // count the tile loads, and a wait for a slot load issued before one of
    // them would drain it too), then the loads of K0, V0 and K1
    int32_t v1[4];
    sload(0, vs);
    if (ntiles > 1) sload(1, v1);
    koff(0, ob, vs);
    if (ntiles > 1) koff(1, oa, v1);
    kissue(0, ob);
    dma_v(0, ob);
    if (ntiles > 1) kissue(1, oa);
    xload(0, xb);
    xload(1, xa);
    if (ntiles > 2) sload(2, vs);
    __builtin_amdgcn_s_waitcnt(0x3F70);
    wg_barrier();
    if (live) {
      scores(sn, 0);
      mask(sn, 0, __builtin_amdgcn_readfirstlane(xb[0]), __builtin_amdgcn_readfirstlane(xb[1]));
      lsum += weigh_exact(sn);
      to_bf16(sn, pa);
    }
  }
  for (int tile = 0; tile < ntiles - 1; tile += 2) {
    step(tile, pa, pb, oa, ob, xa, xb);
    if (tile + 2 < ntiles) step(tile + 1, pb, pa, ob, oa, xb, xa);
  }
  if (ntiles > 0) {
    if (ntiles & 1) last_step(ntiles - 1, pa);
    else last_step(ntiles - 1, pb);
  }
}

// Many-query attention (attn_rows_mfma and attn_store_rows_mfma): a
// workgroup owns 128 query rows (32 per wave) of one (layer, head or packed
// head group, request) and walks the whole key list with tile_loop.  STORE:
// the key list is the request's fresh rows (src_k / src_v) followed by its
// other keys (priv_table), and the units of one query head per KV head copy
// those rows of their (layer, KV head) to the pool, a slice per row tile; the
// call reads no slot it writes, so the copy needs no ordering against the
// attention.
template <bool STORE>
__device__ __forceinline__ void rows_body(const AttnP& p, char* smem) {
  const int unit = xcd_unit(p.per_xcd);
  if (unit >= p.n_units) return;
  const bool packed = p.gpack > 1;
  const int n_uh = packed ? p.geo.n_kv_heads : p.n_q_heads;  // heads that index units
  int r = unit;
  const int t = r % p.q_tiles;
  r /= p.q_tiles;
  const int b = r % p.B;
  r /= p.B;
  const int hu = r % n_uh;
  const int n = r / n_uh;
  const int g = packed ? hu : hu / (p.n_q_heads / p.geo.n_kv_heads);
  const int layer = p.layer_begin + n;
  const int tid = threadIdx.x, lane = tid & 63;
  if constexpr (STORE) {
    // the q_tiles units of one query head per KV head copy the rows of their
    // (layer, KV head, request) to the pool, one slice each, 16 bytes a
    // thread and four rows' loads in flight before their stores
    if (packed || hu % (p.n_q_heads / p.geo.n_kv_heads) == 0) {
      const int s0 = p.src_offsets[b], s1 = p.src_offsets[b + 1];
      const int per = (s1 - s0 + p.q_tiles - 1) / p.q_tiles;
      const int c0 = s0 + t * per, c1 = min(s1, c0 + per);
      const size_t row_stride = (size_t)p.geo.n_kv_heads * ROWB;
      const size_t sbase = (size_t)n * p.n_src * row_stride + (size_t)g * ROWB;
      const size_t dbase = (size_t)layer * p.layer_bytes + (size_t)g * p.geo.page_size * ROWB;
      const size_t page_bytes = (size_t)p.geo.n_kv_heads * p.geo.page_size * ROWB;
      const int c = tid & 15;
      for (int i0 = c0 + (tid >> 4); i0 < c1; i0 += 4 * 16) {
        u32x4 kx[4], vx[4];
        size_t dof[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = min(i0 + 16 * u, c1 - 1);  // rows past c1 repeat the last row's copy
          const uint32_t slot = (uint32_t)p.src_slot[i];
          const size_t so = sbase + (size_t)i * row_stride + c * 16;
          dof[u] = dbase + (size_t)(slot >> p.geo.page_shift) * page_bytes +
                   (size_t)(slot & (p.geo.page_size - 1)) * ROWB + c * 16;
          kx[u] = __builtin_nontemporal_load((const u32x4*)(p.src_k + so));
          vx[u] = __builtin_nontemporal_load((const u32x4*)(p.src_v + so));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          __builtin_nontemporal_store(kx[u], (u32x4*)(p.pool_kw + dof[u]));
          __builtin_nontemporal_store(vx[u], (u32x4*)(p.pool_vw + dof[u]));
        }
      }
    }
  }
  int q0 = 0, q1 = p.n_q, k0 = 0, k1 = p.n_kv;
  if (p.q_offsets) { q0 = p.q_offsets[b]; q1 = p.q_offsets[b + 1]; }
  if constexpr (STORE) {
    k1 = p.kv_counts[b];
  } else if (p.kv_offsets) {
    k0 = p.kv_offsets[b];
    k1 = p.kv_offsets[b + 1];
  }
  const int nq = q1 - q0;
  const int rows = packed ? p.gpack * nq : nq;  // rows of this (request, head or group)
  const int rbase = t * 128;
  if (rbase >= rows) return;
  const int nk = k1 - k0;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g2 = lane >> 5, l32 = lane & 31;
  // this wave holds rows rbase + 32 * wave + l32
  const int wrow = rbase + 32 * wave;
  const bool wave_live = wrow < rows;
  const int lrow = wrow + l32;
  const bool qvalid = lrow < rows;
  // this lane's query row and head (rows >= 1 here, so nq >= 1); lanes past
  // the rows take the first row and head of the unit, whose Q they load but
  // whose results they never store
  int qrow = q0 + (qvalid ? lrow : 0), h = hu;
  if (packed) {
    const int j = qvalid ? lrow / nq : 0;
    qrow = q0 + (qvalid ? lrow - j * nq : 0);
    h = g * p.gpack + j;
  }
  // Q as the B operand of S^T = K Q^T
  bf16x8 qf[8];
  {
    const bf16_t* qp = p.q + (((size_t)n * p.n_q + qrow) * p.n_q_heads + h) * D + g2 * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = qvalid ? as_bf16x8(ld16(qp + c * 16)) : as_bf16x8(u32x4{0, 0, 0, 0});
  }
  // no wait here: the Q loads overlap the first tile loads, and the vmcnt(0)
  // that closes the tile loop's prologue covers both

  float m = -INFINITY, lsum = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) o[a] = f32x16{};

  TileSrc src;
  src.kbase = (const char*)p.pool_k + (size_t)layer * p.layer_bytes;
  src.vbase = (const char*)p.pool_v + (size_t)layer * p.layer_bytes;
  src.page_bytes = (uint32_t)p.geo.n_kv_heads * p.geo.page_size * ROWB;
  src.head_off = (uint32_t)g * p.geo.page_size * ROWB;
  src.page_shift = p.geo.page_shift;
  src.page_mask = (uint32_t)(p.geo.page_size - 1);
  src.table = STORE ? p.priv_table + (size_t)b * p.kv_stride : p.kv_table + k0;
  src.nk = nk;
  src.excl = nullptr;
  if constexpr (!STORE) {
    tile_loop<false>(smem, src, p.c2, qf, wave_live, wave, lane, m, lsum, o);
  } else {
    // one list: the request's fresh rows first, read from the source (rows
    // s0 .. s1 of this layer and KV head, one row stride apart), then its
    // other keys.  The fresh rows hold the anchors, the keys of largest
    // attention mass, so the running max is near its final value before
    // the other keys come and the exact step is rare
    const int s0 = p.src_offsets[b], s1 = p.src_offsets[b + 1];
    const size_t row_stride = (size_t)p.geo.n_kv_heads * ROWB;
    const size_t off = ((size_t)n * p.n_src + s0) * row_stride + (size_t)g * ROWB;
    src.fkbase = p.src_k + off;
    src.fvbase = p.src_v + off;
    src.fstride = (uint32_t)row_stride;
    src.nf = s1 - s0;
    src.nk = src.nf + nk;
    tile_loop<false, true>(smem, src, p.c2, qf, wave_live, wave, lane, m, lsum, o);
  }
  const float lt = half_sum(lsum);
  if (!qvalid) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const size_t row = ((size_t)n * p.n_q + qrow) * p.n_q_heads + h;
  if (p.out) {
    bf16_t* op = p.out + row * D;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = a * 32 + 8 * i4 + 4 * g2;
        u32x2 w;
        w[0] = pack_bf16x2(o[a][4 * i4 + 0] * inv, o[a][4 * i4 + 1] * inv);
        w[1] = pack_bf16x2(o[a][4 * i4 + 2] * inv, o[a][4 * i4 + 3] * inv);
        *(u32x2*)(op + d) = w;
      }
  }
  if (p.lse && g2 == 0) p.lse[row] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
}

__global__ __launch_bounds__(256, 2) void attn_rows_mfma(AttnP p) {
  __shared__ __attribute__((aligned(1024))) char smem[RSTAGES * RSTAGE_BYTES];
  rows_body<false>(p, smem);
}

__global__ __launch_bounds__(256, 2) void attn_store_rows_mfma(AttnP p) {
  __shared__ __attribute__((aligned(1024))) char smem[RSTAGES * RSTAGE_BYTES];
  rows_body<true>(p, smem);
}

// Many-query attention on the 16x16x32 MFMA with 48 query rows per wave
// (three 16-row blocks), 192 rows per workgroup (attn_rows48_mfma).  Every K
// fragment read from LDS (16 keys x 32 dims) feeds the score MFMAs of the
// three row blocks, and every V^T fragment (16 dims x 32 keys) their three
// P.V MFMAs, so a 32-key tile takes two thirds of the LDS fragment reads and
// two thirds of the tile loads per FLOP of the 32-row tile loop, at 2 waves
// per SIMD.
//
// MFMA 16x16x32 operand mapping (lane l, r = l % 16, q = l / 16):
//   A (16 x 32): lane holds row r, eight K-slots (q, j), j = 0..7
//   B (32 x 16): lane holds column r, the same eight K-slots
//   C (16 x 16): lane holds column r, rows 4*q + i, i = 0..3
// Scores are computed transposed (S^T = K Q^T, head dim d = 32c + 8q + j for
// MFMA step c), so a lane holds one query row and keys 16*kb + 4q + i of key
// block kb; the P.V product takes those eight weights as its B operand, with
// K-slot j meaning key 4q + j (j < 4) or 16 + 4q + j - 4 of the tile.
namespace {
constexpr int T48 = 32;                      // keys per tile
constexpr uint32_t T48_BYTES = T48 * ROWB;   // one K or V tile: 8 KiB
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16-byte chunk swizzle of a V row in this kernel's tiles: a transposing
// read of one 32-lane half covers rows 8h .. 8h+7 at two chunks each, which
// this spreads over all 64 banks (the second read of a fragment, 16 rows on,
// keeps the swizzle)
__device__ __forceinline__ uint32_t vswz48(uint32_t row, uint32_t chunk) { return chunk ^ ((row & 7u) << 1); }
// max / sum over the four lanes of a query row (l, l^16, l^32, l^48)
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
}  // namespace

// STORE: the key list is the request's fresh rows (src_k / src_v) followed
// by its other keys (priv_table), and the units of one query head per KV
// head copy those rows of their (layer, KV head, request) to the pool, a
// slice per row tile, as in rows_body<true>
template <bool STORE>
__device__ __forceinline__ void rows48_body(const AttnP& p, char* smem) {
  const int unit = xcd_unit(p.per_xcd);
  if (unit >= p.n_units) return;
  const bool packed = p.gpack > 1;
  const int n_uh = packed ? p.geo.n_kv_heads : p.n_q_heads;  // heads that index units
  int r = unit;
  const int t = r % p.q_tiles;
  r /= p.q_tiles;
  const int b = r % p.B;
  r /= p.B;
  const int hu = r % n_uh;
  const int n = r / n_uh;
  const int g = packed ? hu : hu / (p.n_q_heads / p.geo.n_kv_heads);
  const int layer = p.layer_begin + n;
  const int tid = threadIdx.x, lane = tid & 63;
  if constexpr (STORE) {
    // the q_tiles units of one query head per KV head copy the rows of their
    // (layer, KV head, request) to the pool, one slice each, 16 bytes a
    // thread and four rows' loads in flight before their stores
    if (packed || hu % (p.n_q_heads / p.geo.n_kv_heads) == 0) {
      const int s0 = p.src_offsets[b], s1 = p.src_offsets[b + 1];
      const int per = (s1 - s0 + p.q_tiles - 1) / p.q_tiles;
      const int c0 = s0 + t * per, c1 = min(s1, c0 + per);
      const size_t row_stride = (size_t)p.geo.n_kv_heads * ROWB;
      const size_t sbase = (size_t)n * p.n_src * row_stride + (size_t)g * ROWB;
      const size_t dbase = (size_t)layer * p.layer_bytes + (size_t)g * p.geo.page_size * ROWB;
      const size_t pg_bytes = (size_t)p.geo.n_kv_heads * p.geo.page_size * ROWB;
      const int c = tid & 15;
      for (int i0 = c0 + (tid >> 4); i0 < c1; i0 += 4 * 16) {
        u32x4 kx[4], vx[4];
        size_t dof[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = min(i0 + 16 * u, c1 - 1);  // rows past c1 repeat the last row's copy
          const uint32_t slot = (uint32_t)p.src_slot[i];
          const size_t so = sbase + (size_t)i * row_stride + c * 16;
          dof[u] = dbase + (size_t)(slot >> p.geo.page_shift) * pg_bytes +
                   (size_t)(slot & (p.geo.page_size - 1)) * ROWB + c * 16;
          kx[u] = __builtin_nontemporal_load((const u32x4*)(p.src_k + so));
          vx[u] = __builtin_nontemporal_load((const u32x4*)(p.src_v + so));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          __builtin_nontemporal_store(kx[u], (u32x4*)(p.pool_kw + dof[u]));
          __builtin_nontemporal_store(vx[u], (u32x4*)(p.pool_vw + dof[u]));
        }
      }
    }
  }
  int q0 = 0, q1 = p.n_q, k0 = 0, k1 = p.n_kv;
  if (p.q_offsets) { q0 = p.q_offsets[b]; q1 = p.q_offsets[b + 1]; }
  if constexpr (STORE) {
    k1 = p.kv_counts[b];
  } else if (p.kv_offsets) {
    k0 = p.kv_offsets[b];
    k1 = p.kv_offsets[b + 1];
  }
  const int nq = q1 - q0;
  const int rows = packed ? p.gpack * nq : nq;
  const int rbase = t * 192;
  if (rbase >= rows) return;
  // STORE: keys 0 .. nf-1 are the fresh rows, keys nf .. nk-1 the table's
  const int nf = STORE ? p.src_offsets[b + 1] - p.src_offsets[b] : 0;
  const int nk = nf + k1 - k0;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, qd = lane >> 4;
  // this wave holds rows rbase + 48 * wave + 16 * rb + r16 (rb = 0..2)
  const int wrow = rbase + 48 * wave;
  const bool live = wrow < rows;
  int qrow[3], qhead[3];
  bool qvalid[3];
  bf16x8 qf[3][4];
#pragma unroll
  for (int rb = 0; rb < 3; ++rb) {
    const int lrow = wrow + 16 * rb + r16;
    qvalid[rb] = lrow < rows;
    // lanes past the rows take the first row and head of the unit (loaded,
    // never stored)
    qrow[rb] = q0 + (qvalid[rb] ? lrow : 0);
    qhead[rb] = hu;
    if (packed) {
      const int j = qvalid[rb] ? lrow / nq : 0;
      qrow[rb] = q0 + (qvalid[rb] ? lrow - j * nq : 0);
      qhead[rb] = g * p.gpack + j;
    }
    // streaming loads: Q is read once, and the L2 is better kept for the
    // affix tiles that every row tile of the head reads
    const bf16_t* qp = p.q + (((size_t)n * p.n_q + qrow[rb]) * p.n_q_heads + qhead[rb]) * D + 8 * qd;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qf[rb][c] = qvalid[rb] ? as_bf16x8(__builtin_nontemporal_load((const u32x4*)(qp + 32 * c)))
                             : as_bf16x8(u32x4{0, 0, 0, 0});
  }

  float m[3] = {-INFINITY, -INFINITY, -INFINITY}, lsum[3] = {0.f, 0.f, 0.f};
  f32x4 o[8][3];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) o[db][rb] = f32x4{};

  const float c2 = p.c2;
  const int ntiles = (nk + T48 - 1) / T48;
  // tile loads: this wave moves rows 8*wave .. 8*wave+7 of each K and V tile;
  // DMA instruction i covers rows 8*wave + 4i + lane/16, one 16-byte chunk
  // per lane
  const int sel = lane >> 4;
  const int32_t* vtable = STORE ? p.priv_table + (size_t)b * p.kv_stride : p.kv_table + k0;
  const __amdgpu_buffer_rsrc_t trs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vtable, (short)0, (nk - nf) * 4, 0x00020000);
  const uint32_t trow = (uint32_t)(8 * wave + sel) * 4;
  // the list position of the row this lane moves in DMA instruction i
  auto key_of = [&](int tile, int i) { return min(tile * T48 + 8 * wave + sel + 4 * i, nk - 1); };
  auto sload = [&](int tile, int32_t* vs) {
    if constexpr (STORE) {
      // fresh rows need no slot; whole table tiles read it through the
      // buffer resource shifted by nf; the tile across nf and the last
      // partial tile read it per lane (keys below nf read entry 0, unused)
      if (tile * T48 + T48 <= nf) {
      } else if (tile * T48 >= nf && tile * T48 + T48 <= nk) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          vs[i] = __builtin_amdgcn_raw_buffer_load_b32(trs, trow, (tile * T48 - nf) * 4 + 16 * i, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          vs[i] = __builtin_amdgcn_raw_buffer_load_b32(trs, (uint32_t)max(key_of(tile, i) - nf, 0) * 4, 0, 0);
      }
      return;
    }
    if (tile * T48 + T48 <= nk) {
#pragma unroll
      for (int i = 0; i < 2; ++i) vs[i] = __builtin_amdgcn_raw_buffer_load_b32(trs, trow, tile * (T48 * 4) + 16 * i, 0);
    } else {
      // the last partial tile repeats the list's last key (finite rows;
      // their scores are masked)
      const int r0 = tile * T48 + 8 * wave + sel;
#pragma unroll
      for (int i = 0; i < 2; ++i) vs[i] = vtable[min(r0 + 4 * i, nk - 1)];
    }
  };
  uint32_t kchunk[2], kvx[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // the row is 8*wave + 4i + sel: row & 15 == 8*(wave & 1) + 4i + sel, row & 7 == 4i + sel
    kchunk[i] = kswz(8 * (wave & 1) + 4 * i + sel, lane & 15) * 16;
    kvx[i] = kchunk[i] ^ (vswz48(4 * i + sel, lane & 15) * 16);
  }
  const uint32_t lds0 = lds_addr(smem) + 8 * wave * ROWB;
  const char* kbase_s =
      uniform_ptr((const char*)p.pool_k + (size_t)layer * p.layer_bytes + (size_t)g * p.geo.page_size * ROWB);
  const char* vbase_s =
      uniform_ptr((const char*)p.pool_v + (size_t)layer * p.layer_bytes + (size_t)g * p.geo.page_size * ROWB);
  const uint32_t page_bytes = (uint32_t)p.geo.n_kv_heads * p.geo.page_size * ROWB;
  const int page_shift = p.geo.page_shift;
  const uint32_t rmask = (uint32_t)(p.geo.page_size - 1) << 8;
  auto pool_off = [&](const int32_t* vs, int i) {
    const uint32_t slot = (uint32_t)vs[i];
    return __umul24(slot >> page_shift, page_bytes) + (((slot << 8) & rmask) | kchunk[i]);
  };
  // STORE: a fresh row's offset in the source (row bytes and row count below
  // 2^24, their product below 2^32)
  const char* fkbase_s = STORE ? uniform_ptr(p.src_k + ((size_t)n * p.n_src + p.src_offsets[b]) *
                                                           p.geo.n_kv_heads * ROWB + (size_t)g * ROWB)
                               : nullptr;
  const char* fvbase_s = STORE ? uniform_ptr(p.src_v + ((size_t)n * p.n_src + p.src_offsets[b]) *
                                                           p.geo.n_kv_heads * ROWB + (size_t)g * ROWB)
                               : nullptr;
  const uint32_t fstride = (uint32_t)p.geo.n_kv_heads * ROWB;
  auto fresh_off = [&](int tile, int i) { return __umul24((uint32_t)key_of(tile, i), fstride) + kchunk[i]; };
  auto koff = [&](int tile, uint32_t* off, const int32_t* vs) {
    if (!STORE || tile * T48 >= nf) {  // only table keys (uniform)
#pragma unroll
      for (int i = 0; i < 2; ++i) off[i] = pool_off(vs, i);
    } else if (tile * T48 + T48 <= nf) {  // only fresh rows (uniform)
#pragma unroll
      for (int i = 0; i < 2; ++i) off[i] = fresh_off(tile, i);
    } else {  // the one tile across nf: per lane
#pragma unroll
      for (int i = 0; i < 2; ++i) off[i] = key_of(tile, i) < nf ? fresh_off(tile, i) : pool_off(vs, i);
    }
  };
  auto kissue = [&](int tile, const uint32_t* off) {
    const uint32_t st = lds0 + (tile & 1) * T48_BYTES;
    if (!STORE || tile * T48 >= nf) {
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16s(kbase_s, off[i], st + 4 * i * ROWB);
    } else if (tile * T48 + T48 <= nf) {
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16s(fkbase_s, off[i], st + 4 * i * ROWB);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (key_of(tile, i) < nf) dma16s(fkbase_s, off[i], st + 4 * i * ROWB);
        else dma16s(kbase_s, off[i], st + 4 * i * ROWB);
      }
    }
  };
  auto vissue = [&](int tile, const uint32_t* off) {
    const uint32_t st = lds0 + (2 + (tile & 1)) * T48_BYTES;
    if (!STORE || tile * T48 >= nf) {
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16s(vbase_s, off[i] ^ kvx[i], st + 4 * i * ROWB);
    } else if (tile * T48 + T48 <= nf) {
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16s(fvbase_s, off[i] ^ kvx[i], st + 4 * i * ROWB);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (key_of(tile, i) < nf) dma16s(fvbase_s, off[i] ^ kvx[i], st + 4 * i * ROWB);
        else dma16s(vbase_s, off[i] ^ kvx[i], st + 4 * i * ROWB);
      }
    }
  };

  // LDS read offsets within a stage: K fragment of step c (row r16 of key
  // block kb, 16-byte chunk 4c + q; key block 1 adds 16 rows, which keep the
  // swizzle); V^T fragment of dim block db (rows 4q + r16/4, 8 bytes at dim
  // 16*db + 4*(r16 % 4); the second read adds 16 rows)
  uint32_t krd[4], vrd[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) krd[c] = r16 * ROWB + kswz(r16, 4 * c + qd) * 16;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const uint32_t row = 4 * qd + (r16 >> 2);
    const uint32_t dcol = 16 * db + 4 * (r16 & 3);
    vrd[db] = row * ROWB + vswz48(row, dcol >> 3) * 16 + (dcol & 7) * 2;
  }

  // scores of a tile: s[kb][rb], keys 16*kb + 4q + i of the tile for query
  // row r16 of row block rb
  auto scores = [&](f32x4 (*s)[3], int tile) {
    const char* st = smem + (tile & 1) * T48_BYTES;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rb = 0; rb < 3; ++rb) s[kb][rb] = f32x4{};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = as_bf16x8(*(const u32x4*)(st + krd[c] + kb * 16 * ROWB));
#pragma unroll
        for (int rb = 0; rb < 3; ++rb) s[kb][rb] = mfma16(kf, qf[rb][c], s[kb][rb]);
      }
  };
  auto past_end = [&](int tile, int kb, int i) { return tile * T48 + 16 * kb + 4 * qd + i >= nk; };
  auto mask = [&](f32x4 (*s)[3], int tile, float v) {
    if (tile * T48 + T48 > nk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rb = 0; rb < 3; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (past_end(tile, kb, i)) s[kb][rb][i] = v;
    }
  };
  auto lane_sum = [&](f32x4 (*s)[3], int rb) -> float {
    return ((s[0][rb][0] + s[0][rb][1]) + (s[0][rb][2] + s[0][rb][3])) +
           ((s[1][rb][0] + s[1][rb][1]) + (s[1][rb][2] + s[1][rb][3]));
  };
  auto expsum = [&](f32x4 (*s)[3], int rb, float nm) -> float {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[kb][rb][i] = fast_exp2(fmaf(s[kb][rb][i], c2, nm));
    return lane_sum(s, rb);
  };
  auto to_bf16 = [&](f32x4 (*s)[3], bf16x8* pw) {
#pragma unroll
    for (int rb = 0; rb < 3; ++rb)
#pragma unroll
      for (int j = 0; j < 8; ++j) pw[rb][j] = (__bf16)s[j >> 2][rb][j & 3];
  };
  // exact step for row block rb: the tile's max of each row, the running max
  // raised to it when larger (O and the row sum rescaled), then the weights
  auto weigh_exact = [&](f32x4 (*s)[3], int rb) -> float {
    float mr = fmaxf(fmaxf(fmaxf(s[0][rb][0], s[0][rb][1]), fmaxf(s[0][rb][2], s[0][rb][3])),
                     fmaxf(fmaxf(s[1][rb][0], s[1][rb][1]), fmaxf(s[1][rb][2], s[1][rb][3])));
    const float mt = quad_max(mr) * c2;
    if (mt > m[rb]) {
      const float alpha = exp2f(m[rb] - mt);  // 0 while m is -inf (O and the sum are still 0)
      lsum[rb] *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db][rb] *= alpha;
      m[rb] = mt;
    }
    return expsum(s, rb, m[rb] == -INFINITY ? 0.f : -m[rb]);
  };
  // Weights of a freshly scored tile against the running max as it stands
  // are kept when every lane's sum of them stays at most 2^8 (every weight
  // does: a running max within 8 of the true one); otherwise the wave takes
  // the exact step on scores recomputed from the tile, still in LDS.  Keys
  // past the end of the list are zeroed after the exponentials.
  auto weigh = [&](f32x4 (*s)[3], bf16x8* pw, int tile) {
    float ls[3];
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) ls[rb] = expsum(s, rb, -m[rb]);
    if (tile * T48 + T48 > nk) {
      mask(s, tile, 0.f);
#pragma unroll
      for (int rb = 0; rb < 3; ++rb) ls[rb] = lane_sum(s, rb);
    }
    if (__builtin_amdgcn_ballot_w64(!(ls[0] <= 256.f) || !(ls[1] <= 256.f) || !(ls[2] <= 256.f)) != 0) {
      scores(s, tile);
      mask(s, tile, -INFINITY);
#pragma unroll
      for (int rb = 0; rb < 3; ++rb) ls[rb] = weigh_exact(s, rb);
    }
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) lsum[rb] += ls[rb];
    to_bf16(s, pw);
  };
  // the matrix work of an iteration: scores of tile t+1 (three MFMAs per K
  // fragment) and P.V of tile t (three MFMAs per V^T fragment), a group of
  // each in turn; reads two groups ahead
  auto absorb_group = [&](const char* vst, const bf16x8* pc, int db) {
    const char* vp = vst + vrd[db];
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vp);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 16 * ROWB));
    const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) o[db][rb] = mfma16(vf, pc[rb], o[db][rb]);
  };
  auto score_absorb = [&](f32x4 (*s)[3], int stile, const bf16x8* pc, int vtile) {
    const char* st = smem + (stile & 1) * T48_BYTES;
    const char* vst = smem + (2 + (vtile & 1)) * T48_BYTES;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rb = 0; rb < 3; ++rb) s[kb][rb] = f32x4{};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i >> 1, kb = i & 1;
      const bf16x8 kf = as_bf16x8(*(const u32x4*)(st + krd[c] + kb * 16 * ROWB));
#pragma unroll
      for (int rb = 0; rb < 3; ++rb) s[kb][rb] = mfma16(kf, qf[rb][c], s[kb][rb]);
      absorb_group(vst, pc, i);
    }
    constexpr int kMfma = 0x008, kDsRead = 0x100;
    __builtin_amdgcn_sched_group_barrier(kDsRead, 6, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 3, 0);
      if (i < 6) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kMfma, 3, 0);
      if (i < 6) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
    }
  };
  f32x4 sn[2][3];
  // iteration t: pc = P(t); pn receives P(t+1); oc = row offsets of tile t+1
  // (its V load is issued here), on receives those of t+2; vs = slots of t+2
  int32_t vs[2];
  auto step = [&](int tile, const bf16x8* pc, bf16x8* pn, const uint32_t* oc, uint32_t* on) {
    __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): K(t+1), V(t) and the slots of t+2 have landed
    wg_barrier();                        // ... in every wave; K(t) and V(t-1) are no longer read
    if (tile + 2 < ntiles) {
      koff(tile + 2, on, vs);
      kissue(tile + 2, on);
      if (tile + 3 < ntiles) sload(tile + 3, vs);
    }
    if (tile + 1 < ntiles) vissue(tile + 1, oc);
    if (!live) return;
    score_absorb(sn, tile + 1, pc, tile);
    weigh(sn, pn, tile + 1);
  };
  auto last_step = [&](int tile, const bf16x8* pc) {
    __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): V(t) has landed
    wg_barrier();
    if (!live) return;
    const char* vst = smem + (2 + (tile & 1)) * T48_BYTES;
#pragma unroll
    for (int db = 0; db < 8; ++db) absorb_group(vst, pc, db);
  };

  bf16x8 pa[3], pb[3];
  uint32_t oa[2], ob[2];
  if (ntiles > 0) {
    // the slots of tiles 0 and 1 in one round trip, both tiles' offsets,
    // then the loads of K0, V0, K1 and the slots of tile 2
    int32_t v1[2];
    sload(0, vs);
    if (ntiles > 1) sload(1, v1);
    koff(0, ob, vs);
    if (ntiles > 1) koff(1, oa, v1);
    kissue(0, ob);
    vissue(0, ob);
    if (ntiles > 1) kissue(1, oa);
    if (ntiles > 2) sload(2, vs);
    __builtin_amdgcn_s_waitcnt(0x3F70);
    wg_barrier();
    if (live) {
      scores(sn, 0);
      mask(sn, 0, -INFINITY);
#pragma unroll
      for (int rb = 0; rb < 3; ++rb) lsum[rb] += weigh_exact(sn, rb);
      to_bf16(sn, pa);
    }
  }
  for (int tile = 0; tile < ntiles - 1; tile += 2) {
    step(tile, pa, pb, oa, ob);
    if (tile + 2 < ntiles) step(tile + 1, pb, pa, ob, oa);
  }
  if (ntiles > 0) {
    if (ntiles & 1) last_step(ntiles - 1, pa);
    else last_step(ntiles - 1, pb);
  }

#pragma unroll
  for (int rb = 0; rb < 3; ++rb) {
    const float lt = quad_sum(lsum[rb]);
    if (!qvalid[rb]) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const size_t row = ((size_t)n * p.n_q + qrow[rb]) * p.n_q_heads + qhead[rb];
    if (p.out) {
      bf16_t* op = p.out + row * D + 4 * qd;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        u32x2 w;
        w[0] = pack_bf16x2(o[db][rb][0] * inv, o[db][rb][1] * inv);
        w[1] = pack_bf16x2(o[db][rb][2] * inv, o[db][rb][3] * inv);
        *(u32x2*)(op + 16 * db) = w;
      }
    }
    if (p.lse && qd == 0) p.lse[row] = lt > 0.f ? (m[rb] + log2f(lt)) * kLn2 : -INFINITY;
  }
}

__global__ __launch_bounds__(256, 2) void attn_rows48_mfma(AttnP p) {
  // two K stages then two V stages of 32-key tiles
  __shared__ __attribute__((aligned(1024))) char smem[4 * T48_BYTES];
  rows48_body<false>(p, smem);
}

__global__ __launch_bounds__(256, 2) void attn_store_rows48_mfma(AttnP p) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * T48_BYTES];
  rows48_body<true>(p, smem);
}

// Read-slot attention of decode blocks whose requests share one affix
// (Section 4.3 and Appendix C.1, with the single shared region of
// Section 4.1).  A workgroup owns one (layer, query head) and four requests;
// wave w owns the (at most 32) query rows of request 4t + w.  Two phases feed
// one online softmax per row:
//   shared   the affix keys as one tile list for the four requests, loaded
//            once per workgroup (tile_loop, as in attn_rows_mfma); each wave
//            drops the keys its request does not read from the shared region;
//   private  then each wave streams the rest of its request's read slots
//            through its own 16 KB of LDS in 32-key tiles, refilling K and V
//            separately so the next tile's loads overlap this tile's math.
__global__ __launch_bounds__(256, 2) void attn_shared_mfma(AttnP p) {
  __shared__ __attribute__((aligned(1024))) char smem[RSTAGES * RSTAGE_BYTES];
  typedef const __attribute__((address_space(4))) int32_t* sc_i32;
  typedef const __attribute__((address_space(4))) uint32_t* sc_u32;
  const int unit = xcd_unit(p.per_xcd);
  if (unit >= p.n_units) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g2 = lane >> 5, l32 = lane & 31;
  int r = unit;
  const int t = r % p.q_tiles;
  r /= p.q_tiles;
  const int h = r % p.n_q_heads;
  const int n = r / p.n_q_heads;
  const int g = h / (p.n_q_heads / p.geo.n_kv_heads);
  const int layer = p.layer_begin + n;
  const int b = 4 * t + wave;  // wave-uniform
  int q0 = 0, q1 = 0;
  if (b < p.B) {
    q0 = p.q_offsets[b];
    q1 = min(p.q_offsets[b + 1], q0 + 32);
  }
  const int qrow = q0 + l32;
  const bool qvalid = qrow < q1;
  const bool wave_live = q1 > q0;

  // Q as the B operand of S^T = K Q^T (one row block per wave)
  bf16x8 qf[8];
  {
    const bf16_t* qp = p.q + (((size_t)n * p.n_q + (qvalid ? qrow : 0)) * p.n_q_heads + h) * D + g2 * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = qvalid ? as_bf16x8(ld16(qp + c * 16)) : as_bf16x8(u32x4{0, 0, 0, 0});
  }
  // no wait here: the Q loads overlap the first tile loads; the waits of
  // either phase cover them (loads complete in order)

  float m = -INFINITY, lsum = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) o[a] = f32x16{};

  const char* kbase = (const char*)p.pool_k + (size_t)layer * p.layer_bytes;
  const char* vbase = (const char*)p.pool_v + (size_t)layer * p.layer_bytes;
  const uint32_t page_bytes = (uint32_t)p.geo.n_kv_heads * p.geo.page_size * ROWB;
  const uint32_t head_off = (uint32_t)g * p.geo.page_size * ROWB;
  // byte offset of a slot's row from the head's first row (page index and
  // page bytes are below 2^24, the layer below 2^32: checked at launch)
  const uint32_t row_mask = (uint32_t)(p.geo.page_size - 1) << 8;
  auto slot_off = [&](int32_t slot) -> uint32_t {
    return __umul24((uint32_t)slot >> p.geo.page_shift, page_bytes) + (((uint32_t)slot << 8) & row_mask);
  };
  // ---- shared phase: the affix keys, loaded once for the four requests
  auto shared_phase = [&]() {
    if (p.n_kv <= 0) return;
    TileSrc src;
    src.kbase = kbase;
    src.vbase = vbase;
    src.page_bytes = page_bytes;
    src.head_off = head_off;
    src.page_shift = p.geo.page_shift;
    src.page_mask = (uint32_t)(p.geo.page_size - 1);
    src.table = p.kv_table;
    src.nk = p.n_kv;
    src.excl = p.excl + (size_t)min(b, p.B - 1) * p.excl_words;
    __builtin_amdgcn_s_setprio(1);  // ahead of the private phase's waves on the CU
    tile_loop<true>(smem, src, p.c2, qf, wave_live, wave, lane, m, lsum, o);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- private phase: this wave's own 32-key tiles, no workgroup barriers
  auto private_phase = [&]() {
    if (!wave_live) return;
    const int cnt = ((sc_i32)p.kv_counts)[b];
    if (cnt <= 0) return;
    // every load issued before this phase (the Q rows among them) is waited
    // for here, at no cost after the shared phase's own final wait; without
    // it the compiler waits for them inside the loop, where the wait would
    // also drain the tile's V loads
    __builtin_amdgcn_s_waitcnt(0x3F70);
    // per-lane constants of this phase, computed here from a lane index the
    // compiler cannot trace back, so that none of them is held in registers
    // through the shared phase
    int lane_p;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane_p) : "v"(lane));
    // DMA instruction i moves rows 4i + lane/16 (of a 16- or 32-row block),
    // one 16-byte chunk per lane; the global chunk is the swizzle of the LDS one
    const int sel = lane_p >> 4;
    uint32_t kchunk[4];
  #pragma unroll
    for (int i = 0; i < 4; ++i) kchunk[i] = kswz(4 * i + sel, lane_p & 15) * 16;
    const uint32_t vchunk = vswz2(sel, lane_p & 15) * 16;
    auto pick = [&](int32_t s0, int32_t s1, int32_t s2, int32_t s3) {
      return (sel & 2) ? ((sel & 1) ? s3 : s2) : ((sel & 1) ? s1 : s0);
    };
    uint32_t krd[8];
  #pragma unroll
    for (int c = 0; c < 8; ++c) krd[c] = (lane_p & 31) * ROWB + kswz(lane_p & 31, 2 * c + (lane_p >> 5)) * 16;
    const uint32_t i16 = lane_p & 15;
    uint32_t vrd[4];
  #pragma unroll
    for (int a = 0; a < 4; ++a) {
      const uint32_t row = 4 * (lane_p >> 5) + (i16 >> 2);
      const uint32_t dcol = a * 32 + 16 * ((lane_p >> 4) & 1) + 4 * (i16 & 3);
      vrd[a] = row * ROWB + vswz2(row, dcol >> 3) * 16 + (dcol & 7) * 2;
    }

    // online-softmax update with NS 32-key score blocks (C layout) and the
    // P.V product with V^T read from the V rows at vst
    auto update = [&](auto ns, f32x16* s, const char* vst) {
      constexpr int NS = decltype(ns)::value;
      float mr = -INFINITY;
  #pragma unroll
      for (int sub = 0; sub < NS; ++sub)
  #pragma unroll
        for (int i = 0; i < 16; ++i) mr = fmaxf(mr, s[sub][i]);
      mr = half_max(mr);
      const float mt = mr * p.c2;
      if (mt > m + 8.f) {  // lazy rescale, exact either way
        const float alpha = exp2f(m - mt);
        lsum *= alpha;
  #pragma unroll
        for (int a = 0; a < 4; ++a)
  #pragma unroll
          for (int i = 0; i < 16; ++i) o[a][i] *= alpha;
        m = mt;
      }
      const float nm = (m == -INFINITY) ? 0.f : -m;
  #pragma unroll
      for (int sub = 0; sub < NS; ++sub)
  #pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8 pb;
  #pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float pv = fast_exp2(fmaf(s[sub][8 * hh + j], p.c2, nm));
            lsum += pv;
            pb[j] = (__bf16)pv;
          }
  #pragma unroll
          for (int a = 0; a < 4; ++a) {
            const char* vp = vst + vrd[a] + (sub * 32 + 16 * hh) * ROWB;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vp);
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 8 * ROWB));
            o[a] = mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, o[a]);
          }
        }
    };

    sc_i32 ptab = (sc_i32)(p.priv_table + (size_t)b * p.kv_stride);
    const char* reg = smem + wave * (PTILE * ROWB * 2);  // K rows, then V rows
    const uint32_t kdst = lds_addr(reg), vdst = kdst + PTILE * ROWB;
    const int nt = (cnt + PTILE - 1) / PTILE;
    int32_t ps[PTILE];
    // the lists are padded with valid slots to whole tiles
    auto pload = [&](int tile) {
      const int kb = tile * PTILE;
#pragma unroll
      for (int i = 0; i < PTILE; ++i) ps[i] = ptab[kb + i];
    };
    // a tile's K loads record its row offsets, which its V loads reuse
    const char* kbase_s = uniform_ptr(kbase + head_off);
    const char* vbase_s = uniform_ptr(vbase + head_off);
    uint32_t po[PTILE / 4];
    auto dma_k = [&]() {
#pragma unroll
      for (int i = 0; i < PTILE / 4; ++i) {
        po[i] = slot_off(pick(ps[4 * i], ps[4 * i + 1], ps[4 * i + 2], ps[4 * i + 3]));
        dma16s(kbase_s, po[i] + kchunk[i & 3], kdst + 4 * i * ROWB);
      }
    };
    auto dma_v = [&]() {
#pragma unroll
      for (int i = 0; i < PTILE / 4; ++i) dma16s(vbase_s, po[i] + vchunk, vdst + 4 * i * ROWB);
    };
    pload(0);
    dma_k();
    dma_v();
    for (int tile = 0; tile < nt; ++tile) {
      const bool more = tile + 1 < nt;
      if (more) pload(tile + 1);
      __builtin_amdgcn_s_waitcnt(0x3F78);  // vmcnt(8): K of this tile has landed (its V may not have)
      f32x16 s[1] = {f32x16{}};
#pragma unroll
      for (int c = 0; c < 8; ++c) s[0] = mfma(as_bf16x8(*(const u32x4*)(reg + krd[c])), qf[c], s[0]);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): K reads (and the next slots) are done
      if (more) dma_k();
      const int kb = tile * PTILE;
      if (kb + PTILE > cnt) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb + 8 * (i >> 2) + 4 * g2 + (i & 3) >= cnt) s[0][i] = -INFINITY;
      }
      if (more) __builtin_amdgcn_s_waitcnt(0x3F78);  // vmcnt(8): V of this tile has landed
      else __builtin_amdgcn_s_waitcnt(0x3F70);
      update(std::integral_constant<int, 1>{}, s, reg + PTILE * ROWB);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): V reads are done
      if (more) dma_v();
    }
  };

  shared_phase();
  wg_barrier();  // every wave is done with the shared tiles before its private loads land
  private_phase();

  const float lt = half_sum(lsum);
  if (!qvalid) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const size_t row = ((size_t)n * p.n_q + qrow) * p.n_q_heads + h;
  bf16_t* op = p.out + row * D;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = a * 32 + 8 * i4 + 4 * g2;
      u32x2 w;
      w[0] = pack_bf16x2(o[a][4 * i4 + 0] * inv, o[a][4 * i4 + 1] * inv);
      w[1] = pack_bf16x2(o[a][4 * i4 + 2] * inv, o[a][4 * i4 + 3] * inv);
      *(u32x2*)(op + d) = w;
    }
  if (p.lse && g2 == 0) p.lse[row] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
}

// Column mass of the masked rows.  A workgroup owns 256 affix keys (64 per
// wave, held as two B-operand tiles in registers) of one (layer, query head)
// and streams every request's masked rows through LDS in tiles of 32.  The
// tiles of all requests are walked as one list.  Q rows go straight from
// global memory to LDS (direct-to-LDS loads, the same swizzled 256-byte row
// layout as the K tiles of the attention), two stages deep: right after the
// barrier of iteration t the loads of tile t+2 start, and they land during
// the iteration.  The loop is software pipelined: while a wave takes the
// exponentials of tile t, it computes the scores of tile t+1.  Each score
// accumulator starts at -LSE/scale of its row, so that the weight is
// exp2(c2 * accumulator); those values come prepared by colmass_lse_prep
// (padded with -inf to whole tiles) and reach LDS by direct loads too.  The
// kernel fits three workgroups (three waves per SIMD) on a CU.
__global__ __launch_bounds__(256, 2) void colmass_mfma(ColP p) {
  __shared__ __attribute__((aligned(1024))) char Qs[2][32 * ROWB];
  __shared__ __attribute__((aligned(16))) float lse2[2][32];
  const int unit = xcd_unit(p.per_xcd);
  if (unit >= p.n_units) return;
  const int kblk = unit % p.key_blocks;
  const int r = unit / p.key_blocks;
  const int h = r % p.n_q_heads;
  const int n = r / p.n_q_heads;
  const int g = h / (p.n_q_heads / p.geo.n_kv_heads);
  const int layer = p.layer_begin + n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g2 = lane >> 5, l32 = lane & 31;
  const int kw = kblk * 256 + wave * 64;  // this wave's first key

  // K as the B operand of S = Q K^T (two 32-key tiles)
  bf16x8 kf[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int j = min(kw + nt * 32 + l32, p.L - 1);
    const bf16_t* kp = p.pool_k + p.geo.row(layer, p.shared_slots[j], g) + g2 * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) kf[nt][c] = as_bf16x8(ld16(kp + c * 16));
  }

  // request offsets are the same for every lane: read them as scalars
  const __attribute__((address_space(4))) int32_t* moff =
      (const __attribute__((address_space(4))) int32_t*)p.masked_offsets;
  float* part = p.partial + ((size_t)n * p.n_q_heads + h) * p.B * p.L;
  const int j0 = kw + l32, j1 = kw + 32 + l32;
  // requests without masked rows contribute zero
  for (int b = 0; b < p.B; ++b)
    if (moff[b + 1] == moff[b] && g2 == 0) {
      if (j0 < p.L) part[(size_t)b * p.L + j0] = 0.f;
      if (j1 < p.L) part[(size_t)b * p.L + j1] = 0.f;
    }

  // tile iterator over (request, first masked row) of all non-empty requests;
  // past the last request it points at row 0 of the masked list (which
  // exists whenever a tile does), so that loads issued ahead stay in bounds
  struct It { int b, r0, m1; };
  auto first_from = [&](int b) -> It {
    while (b < p.B && moff[b + 1] == moff[b]) ++b;
    if (b >= p.B) return It{p.B, 0, 1};
    return It{b, moff[b], moff[b + 1]};
  };
  auto next = [&](It t) -> It {
    if (t.b >= p.B) return t;
    if (t.r0 + 32 < t.m1) return It{t.b, t.r0 + 32, t.m1};
    return first_from(t.b + 1);
  };
  It t0 = first_from(0);
  if (t0.b >= p.B) return;  // no masked rows anywhere (uniform over the workgroup)

  // Direct-to-LDS loads: instruction i of wave w fills tile rows 8w+4i ..
  // 8w+4i+3, lane/16 picking the row and lane%16 the LDS chunk, which holds
  // the row's global chunk kswz(row, lane%16).
  const int ra = 8 * wave + (lane >> 4);  // tile rows this lane moves: ra, ra + 4
  const uint32_t gchunk0 = kswz(ra, lane & 15) * 16, gchunk1 = kswz(ra + 4, lane & 15) * 16;
  // one layer and head of Q from a scalar base: a row's bytes start at
  // row * qrow_bytes (below 2^32, rows and row bytes below 2^24: checked at launch)
  const char* qhead = uniform_ptr((const char*)(p.q + ((size_t)n * p.n_rows * p.n_q_heads + h) * D));
  const uint32_t qrow_bytes = (uint32_t)p.n_q_heads * D * sizeof(bf16_t);
  const uint32_t lds_q = lds_addr(&Qs[0][0]) + 8 * wave * ROWB;
  // masked-row indices of a tile: the two rows this lane moves, read through
  // a buffer over masked_rows (the tile's first row in the scalar offset).
  // Rows past the request's last masked row take whatever row follows (the
  // next request's, or row 0 past the end of the list, where the buffer
  // reads zero): a valid row whose accumulator start is -inf, weight 0.
  const __amdgpu_buffer_rsrc_t mrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.masked_rows, (short)0, p.n_masked * 4, 0x00020000);
  struct RowIdx { int ra, rb; };
  auto rows_load = [&](It t) -> RowIdx {
    RowIdx ix;
    ix.ra = __builtin_amdgcn_raw_buffer_load_b32(mrs, ra * 4, t.r0 * 4, 0);
    ix.rb = __builtin_amdgcn_raw_buffer_load_b32(mrs, ra * 4 + 16, t.r0 * 4, 0);
    return ix;
  };
  auto dma_q = [&](int stage, const RowIdx& ix) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_q + stage * (32 * ROWB));
    dma16s(qhead, __umul24((uint32_t)ix.ra, qrow_bytes) + gchunk0, dst);
    dma16s(qhead, __umul24((uint32_t)ix.rb, qrow_bytes) + gchunk1, dst + 4 * ROWB);
  };
  // the tile's 32 prepared accumulator starts (-inf past the request's
  // rows, so they add exp2(-inf) = 0), moved by lanes 0..31 of wave 0
  const float* lprep = p.lse_prep + (size_t)(n * p.n_q_heads + h) * p.lse_stride;
  auto dma_lse = [&](int stage, It t) {
    if (wave == 0 && lane < 32)
      dma4(lprep + t.r0 + 31 * (size_t)t.b + lane, __builtin_amdgcn_readfirstlane(lds_addr(&lse2[stage][0])));
  };
  // scores of the tile in stage st, from accumulators that start at its
  // rows' -LSE/scale
  uint32_t qrd[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) qrd[c] = l32 * ROWB + kswz(l32, 2 * c + g2) * 16;
  auto scores = [&](f32x16* s, int st) {
    const char* qs = &Qs[st][0];
    f32x16 init;
#pragma unroll
    for (int i = 0; i < 16; ++i) init[i] = lse2[st][8 * (i >> 2) + 4 * g2 + (i & 3)];
    bf16x8 qv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) qv[c] = as_bf16x8(*(const u32x4*)(qs + qrd[c]));
    s[0] = init;
    s[1] = init;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      s[0] = mfma(qv[c], kf[0][c], s[0]);
      s[1] = mfma(qv[c], kf[1][c], s[1]);
    }
  };

  // prologue: tiles t0 and t1 loading into stages 0 and 1, t2's row indices
  It t1 = next(t0), t2 = next(t1), t3 = next(t2);
  dma_q(0, rows_load(t0));
  dma_lse(0, t0);
  RowIdx in = rows_load(t1);
  if (t1.b < p.B) {
    dma_q(1, in);
    dma_lse(1, t1);
  }
  in = rows_load(t2);
  __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): tile t0 (and t1) in LDS, t2's indices in registers
  __syncthreads();
  f32x16 sa[2], sb[2];
  scores(sa, 0);
  int st = 0;  // stage of tile t0
  float acc0 = 0.f, acc1 = 0.f;

  // one tile: sc holds the scores of t0, sn receives those of t1
  auto step = [&](f32x16* sc, f32x16* sn) {
    __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): this wave's loads of t1 (and t2's indices) landed
    __syncthreads();  // t1 is in stage st^1 for every wave; no wave still reads stage st
    // tile t2 into stage st, and the indices of t3, while this iteration computes
    if (t2.b < p.B) {
      dma_q(st, in);
      dma_lse(st, t2);
    }
    const It t4 = next(t3);
    in = rows_load(t3);
    // keep those loads here, at the top of the iteration: the compiler
    // would sink them to its end, where its wait for them at the loop edge
    // would then stall
    asm volatile("" ::: "memory");
    // past the last tile the scores read a stale stage and are never used;
    // computing them keeps this block branch-free
    scores(sn, st ^ 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc0 += fast_exp2(sc[0][i] * p.c2);
      acc1 += fast_exp2(sc[1][i] * p.c2);
    }
    // Instruction order: the accumulator starts and three Q fragments read
    // ahead, then each MFMA pair (one fragment, both key tiles) with the next
    // fragment read and a share of tile t0's exponentials and sums, so that
    // the LDS reads spread over the tile instead of arriving in one burst
    {
      constexpr int kMfma = 0x008, kValu = 0x002, kDsRead = 0x100;
      __builtin_amdgcn_sched_group_barrier(kDsRead, 7, 0);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kValu, 6, 0);
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        if (c < 5) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kValu, 6, 0);
      }
    }
    if (t1.b != t0.b) {  // last tile of this request: write its partial column masses
      const float a0 = half_sum(acc0);
      const float a1 = half_sum(acc1);
      if (g2 == 0) {
        if (j0 < p.L) part[(size_t)t0.b * p.L + j0] = a0;
        if (j1 < p.L) part[(size_t)t0.b * p.L + j1] = a1;
      }
      acc0 = acc1 = 0.f;
    }
    t0 = t1;
    t1 = t2;
    t2 = t3;
    t3 = t4;
    st ^= 1;
  };
  while (true) {
    step(sa, sb);
    if (t0.b >= p.B) break;
    step(sb, sa);
    if (t0.b >= p.B) break;
  }
}

// The column mass's accumulator starts: for every (layer, query head) and
// request b, -LSE/scale of the request's masked rows in order, then -inf up to
// a whole number of 32-row tiles, starting at masked_offsets[b] + 31 * b.
__global__ __launch_bounds__(256) void colmass_lse_prep(const float* __restrict__ lse,
                                                        const int32_t* __restrict__ masked_rows,
                                                        const int32_t* __restrict__ masked_offsets, int n_rows,
                                                        int n_q_heads, int x_tiles, float neg_inv_scale,
                                                        float* __restrict__ out, size_t stride) {
  const int nh = blockIdx.x / x_tiles;  // layer * n_q_heads + query head
  const int i = (blockIdx.x - nh * x_tiles) * 256 + threadIdx.x;
  const int b = blockIdx.y;
  const int n = nh / n_q_heads, h = nh - n * n_q_heads;
  const int m0 = masked_offsets[b], m = masked_offsets[b + 1] - m0;
  if (i >= ((m + 31) & ~31)) return;
  float v = -INFINITY;
  if (i < m) v = lse[((size_t)n * n_rows + masked_rows[m0 + i]) * n_q_heads + h] * neg_inv_scale;
  out[(size_t)nh * stride + m0 + 31 * (size_t)b + i] = v;
}

bool mfma_supported(int dtype, int head_dim) { return dtype == ACACHE_BF16 && head_dim == D; }

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t st, bool dry_run) {
  const int B = a.q_offsets ? a.B : 1;
  const int G = gqa_pack(a.n_q_heads, a.geo.n_kv_heads, a.max_q);
  const bool split = G == 0 && a.max_q <= 32;
  if (G > 0 && (long long)G * a.n_q >= (1ll << 31)) return hipErrorInvalidValue;
  const long long rows = G > 0 ? (long long)G * a.max_q : a.max_q;
  const bool r48 = !split && rows >= kRows48MinRows;
  const int RT = split ? 32 : (r48 ? 192 : 128);
  AttnP p{};
  p.q = (const bf16_t*)a.q;
  p.pool_k = (const bf16_t*)a.pool_k;
  p.pool_v = (const bf16_t*)a.pool_v;
  p.geo = a.geo;
  p.q_offsets = a.q_offsets;
  p.n_q = a.n_q;
  const long long q_tiles = (rows + RT - 1) / RT;
  if (q_tiles > (1ll << 30)) return hipErrorInvalidValue;
  p.q_tiles = (int)q_tiles;
  p.gpack = G;
  p.kv_table = a.kv_table;
  p.kv_offsets = a.kv_offsets;
  p.n_kv = a.n_kv;
  p.layer_bytes = (size_t)a.geo.n_pages * a.geo.n_kv_heads * a.geo.page_size * D * 2;
  if (p.layer_bytes >= (1ull << 32)) return hipErrorInvalidValue;
  // tile row offsets are 24-bit products of page index and page bytes
  if ((size_t)a.geo.n_kv_heads * a.geo.page_size * D * 2 >= (1u << 24)) return hipErrorInvalidValue;
  p.B = B;
  p.n_q_heads = a.n_q_heads;
  p.layer_begin = a.layer_begin;
  p.c2 = a.scale * kLog2e;
  p.out = (bf16_t*)a.out;
  p.lse = a.lse;
  const long long units = (long long)a.n_layers * (G > 0 ? a.geo.n_kv_heads : a.n_q_heads) * B * q_tiles;
  if (units == 0) return hipSuccess;
  if (units > (1ll << 30)) return hipErrorInvalidValue;
  p.n_units = (int)units;
  p.per_xcd = (int)((units + 7) / 8);
  if (dry_run) return hipSuccess;
  dim3 grid(8 * p.per_xcd), block(256);
  if (split) hipLaunchKernelGGL(attn_split_mfma, grid, block, 0, st, p);
  else if (r48) hipLaunchKernelGGL(attn_rows48_mfma, grid, block, 0, st, p);
  else hipLaunchKernelGGL(attn_rows_mfma, grid, block, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_attn_mfma_store(const StoreAttnArgs& a, hipStream_t st, bool dry_run) {
  const int G = gqa_pack(a.n_q_heads, a.geo.n_kv_heads, a.max_q);
  if (G > 0 && (long long)G * a.n_q >= (1ll << 31)) return hipErrorInvalidValue;
  const long long rows = G > 0 ? (long long)G * a.max_q : a.max_q;
  const bool r48 = rows >= kRows48MinRows;
  const int RT = r48 ? 192 : 128;
  AttnP p{};
  p.q = (const bf16_t*)a.q;
  p.pool_k = (const bf16_t*)a.pool_k;
  p.pool_v = (const bf16_t*)a.pool_v;
  p.pool_kw = (char*)a.pool_k;
  p.pool_vw = (char*)a.pool_v;
  p.geo = a.geo;
  p.q_offsets = a.q_offsets;
  p.n_q = a.n_q;
  const long long q_tiles = (rows + RT - 1) / RT;
  if (q_tiles > (1ll << 30)) return hipErrorInvalidValue;
  p.q_tiles = (int)q_tiles;
  p.gpack = G;
  p.priv_table = a.other_slots;
  p.kv_counts = a.other_counts;
  p.kv_stride = a.other_stride;
  p.src_k = (const char*)a.k_src;
  p.src_v = (const char*)a.v_src;
  p.src_slot = a.src_slot;
  p.src_offsets = a.src_offsets;
  p.n_src = a.n_src;
  p.layer_bytes = (size_t)a.geo.n_pages * a.geo.n_kv_heads * a.geo.page_size * D * 2;
  if (p.layer_bytes >= (1ull << 32)) return hipErrorInvalidValue;
  // tile row offsets are 24-bit products of page index and page bytes
  if ((size_t)a.geo.n_kv_heads * a.geo.page_size * D * 2 >= (1u << 24)) return hipErrorInvalidValue;
  // byte offsets of source rows within a layer are 32-bit in the tile loads
  if ((size_t)a.n_src * a.geo.n_kv_heads * D * 2 >= (1ull << 32)) return hipErrorInvalidValue;
  p.B = a.B;
  p.n_q_heads = a.n_q_heads;
  p.layer_begin = a.layer_begin;
  p.c2 = a.scale * kLog2e;
  p.out = (bf16_t*)a.out;
  p.lse = a.lse;
  const long long units = (long long)a.n_layers * (G > 0 ? a.geo.n_kv_heads : a.n_q_heads) * a.B * q_tiles;
  if (units == 0) return hipSuccess;
  if (units > (1ll << 30)) return hipErrorInvalidValue;
  p.n_units = (int)units;
  p.per_xcd = (int)((units + 7) / 8);
  if (dry_run) return hipSuccess;
  if (r48) hipLaunchKernelGGL(attn_store_rows48_mfma, dim3(8 * p.per_xcd), dim3(256), 0, st, p);
  else hipLaunchKernelGGL(attn_store_rows_mfma, dim3(8 * p.per_xcd), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_attn_mfma_shared(const SharedAttnArgs& a, hipStream_t st, bool dry_run) {
  if (a.max_q > 32) return hipErrorInvalidValue;
  AttnP p{};
  p.q = (const bf16_t*)a.q;
  p.pool_k = (const bf16_t*)a.pool_k;
  p.pool_v = (const bf16_t*)a.pool_v;
  p.geo = a.geo;
  p.q_offsets = a.q_offsets;
  p.n_q = a.n_q;
  p.q_tiles = (a.B + 3) / 4;
  p.kv_table = a.shared_slots;
  p.n_kv = a.L;
  p.layer_bytes = (size_t)a.geo.n_pages * a.geo.n_kv_heads * a.geo.page_size * D * 2;
  if (p.layer_bytes >= (1ull << 32)) return hipErrorInvalidValue;
  // tile row offsets are 24-bit products of page index and page bytes
  if ((size_t)a.geo.n_kv_heads * a.geo.page_size * D * 2 >= (1u << 24)) return hipErrorInvalidValue;
  p.B = a.B;
  p.n_q_heads = a.n_q_heads;
  p.layer_begin = a.layer_begin;
  p.c2 = a.scale * kLog2e;
  p.out = (bf16_t*)a.out;
  p.lse = a.lse;
  p.excl = a.excl;
  p.excl_words = a.excl_words;
  p.priv_table = a.priv_slots;
  p.kv_counts = a.priv_counts;
  p.kv_stride = a.priv_stride;
  const long long units = (long long)a.n_layers * a.n_q_heads * p.q_tiles;
  if (units == 0) return hipSuccess;
  if (units > (1ll << 30)) return hipErrorInvalidValue;
  p.n_units = (int)units;
  p.per_xcd = (int)((units + 7) / 8);
  if (dry_run) return hipSuccess;
  hipLaunchKernelGGL(attn_shared_mfma, dim3(8 * p.per_xcd), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_colmass_mfma(const ColmassArgs& a, hipStream_t st, bool dry_run) {
  ColP p;
  p.q = (const bf16_t*)a.q;
  p.pool_k = (const bf16_t*)a.pool_k;
  p.geo = a.geo;
  p.masked_rows = a.masked_rows;
  p.masked_offsets = a.masked_offsets;
  p.n_masked = a.n_masked;
  p.shared_slots = a.shared_slots;
  p.L = a.L;
  p.n_rows = a.n_rows;
  p.n_q_heads = a.n_q_heads;
  p.layer_begin = a.layer_begin;
  p.B = a.B;
  p.c2 = a.scale * kLog2e;
  p.lse = a.lse;
  p.partial = a.partial;
  p.lse_prep = a.lse_prep;
  p.lse_stride = a.lse_stride;
  p.key_blocks = (a.L + 255) / 256;
  // Q rows are addressed with 32-bit offsets and 24-bit products
  const long long qrow_bytes = (long long)a.n_q_heads * D * 2;
  if (a.n_rows >= (1 << 24) || qrow_bytes >= (1 << 24) || (long long)a.n_rows * qrow_bytes >= (1ll << 32))
    return hipErrorInvalidValue;
  const long long units = (long long)a.n_layers * a.n_q_heads * p.key_blocks;
  if (units == 0) return hipSuccess;
  if (units > (1ll << 30)) return hipErrorInvalidValue;
  p.n_units = (int)units;
  p.per_xcd = (int)((units + 7) / 8);
  const int x_tiles = (((a.max_masked + 31) & ~31) + 255) / 256;
  if ((long long)x_tiles * a.n_layers * a.n_q_heads > (1ll << 31) - 1 || a.B > 65535) return hipErrorInvalidValue;
  if (dry_run) return hipSuccess;
  if (x_tiles > 0 && a.B > 0) {
    hipLaunchKernelGGL(colmass_lse_prep, dim3(x_tiles * a.n_layers * a.n_q_heads, a.B), dim3(256), 0, st, a.lse,
                       a.masked_rows, a.masked_offsets, a.n_rows, a.n_q_heads, x_tiles, -1.0f / a.scale,
                       a.lse_prep, a.lse_stride);
  }
  hipLaunchKernelGGL(colmass_mfma, dim3(8 * p.per_xcd), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace acache

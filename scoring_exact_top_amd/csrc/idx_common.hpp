// Device building blocks shared by the prefill and decode kernels (gfx950).
//
// Scoring (Fused Indexer Top-k page, "1.1 The problem" equation):
//   I[t,s] = k_scale[s] * sum_j w'[t,j] * max(dot8(q8[t,j], k8[s]), 0),
//   w'[t,j] = w[t,j] * q_scale[t,j]
// Positive scales commute with ReLU, so both scales leave the dot product and
// the 128-deep FP8 contraction is one v_mfma_f32_16x16x128_f8f6f4 per 16 heads
// x 16 keys.  A (16 heads x 128) lives in registers for the whole key loop;
// B (128 x 16 keys) comes straight from global memory, each lane holding the
// 32 contiguous bytes [32*(lane/16), +32) of key lane%16.  Operand lane maps
// for A and B are the same, so any consistent split of the 128-byte vectors
// gives the same dot product.
//
// The 16x16 f32 result puts head 4*(lane/16)+r of a 16-head block in register
// r of the lane that owns key lane%16.  Each lane therefore ReLUs and weights
// its 16 heads of a key, and four partial sums of the same key sit in lanes
// that differ in bits 4 and 5.  Four 16-key sub-tiles are combined by a
// reduce-scatter built on v_permlane32_swap / v_permlane16_swap so that after
// three adds lane l owns the complete score of key l of the 64-key tile, with
// the same addition tree (g0+g2)+(g1+g3) for every key: identical keys give
// bit-identical scores wherever they sit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idxk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kH = 64;
constexpr int kD = 128;
constexpr int kKmax = 2048;
constexpr int kWG = 256;     // threads per workgroup
constexpr int kWaves = 4;    // waves per workgroup (one per SIMD)
constexpr int kTile = 64;    // keys per wave-iteration (4 MFMA sub-tiles of 16)

// Sub-tile c of a 64-key tile covers keys [kSubOff[c], +16).  This order makes
// the reduce-scatter below land key l in lane l.
__device__ __forceinline__ int sub_off(int c) { return c == 0 ? 0 : c == 1 ? 32 : c == 2 ? 16 : 48; }

// Order-preserving map of an FP32 score to uint32 ("3.2 Sampled threshold":
// radix passes run on order-preserving 32-bit integers).  -0 maps like +0.
__device__ __forceinline__ uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Number of set bits of `ball` below this lane.
__device__ __forceinline__ uint32_t rank_in(uint64_t ball) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(ball >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ball, 0u));
}

__device__ __forceinline__ v8i ld32(const uint8_t* p) {
  const uint4* v = reinterpret_cast<const uint4*>(p);
  uint4 x = v[0], y = v[1];
  v8i r;
  r[0] = (int)x.x; r[1] = (int)x.y; r[2] = (int)x.z; r[3] = (int)x.w;
  r[4] = (int)y.x; r[5] = (int)y.y; r[6] = (int)y.z; r[7] = (int)y.w;
  return r;
}

// One query row as held by a lane: A operands of the four 16-head blocks and
// the folded weights w' of the 16 heads whose results land in this lane.
struct QOp {
  v8i a[4];
  float wq[16];
};

__device__ __forceinline__ void load_q(QOp& o, const uint8_t* q, const float* q_scale, const float* w,
                                       int64_t t, uint32_t lane) {
  const uint8_t* base = q + t * (kH * kD);
  const uint32_t g = lane >> 4, i = lane & 15;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    o.a[b] = ld32(base + (16 * b + i) * kD + 32 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * b + 4 * g + r;
      const float qs = q_scale ? q_scale[t * kH + j] : 1.0f;
      o.wq[4 * b + r] = w[t * kH + j] * qs;
    }
  }
}

// Partial weighted-ReLU sum over this lane's 16 heads for key lane%16 of the
// sub-tile whose B operand is kb.
__device__ __forceinline__ float partial16(const QOp& o, const v8i& kb) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  v4f c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.a[0], kb, z, 0, 0, 0, 0, 0, 0);
  v4f c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.a[1], kb, z, 0, 0, 0, 0, 0, 0);
  v4f c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.a[2], kb, z, 0, 0, 0, 0, 0, 0);
  v4f c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.a[3], kb, z, 0, 0, 0, 0, 0, 0);
  float p = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) p = fmaf(o.wq[r], fmaxf(c0[r], 0.f), p);
#pragma unroll
  for (int r = 0; r < 4; ++r) p = fmaf(o.wq[4 + r], fmaxf(c1[r], 0.f), p);
#pragma unroll
  for (int r = 0; r < 4; ++r) p = fmaf(o.wq[8 + r], fmaxf(c2[r], 0.f), p);
#pragma unroll
  for (int r = 0; r < 4; ++r) p = fmaf(o.wq[12 + r], fmaxf(c3[r], 0.f), p);
  return p;
}

// p0..p3: partials of sub-tiles 0..3 (keys 0-15, 32-47, 16-31, 48-63).
// Returns the full head sum of key `lane` of the 64-key tile.
__device__ __forceinline__ float reduce_scatter4(float p0, float p1, float p2, float p3) {
  auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  const float A = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
  const float B = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(A), __float_as_uint(B), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// Scores (before k_scale) of the 64 keys whose B operands are kb[0..3]; lane
// l receives key l.
__device__ __forceinline__ float tile_sum(const QOp& o, const v8i (&kb)[4]) {
  const float p0 = partial16(o, kb[0]);
  const float p1 = partial16(o, kb[1]);
  const float p2 = partial16(o, kb[2]);
  const float p3 = partial16(o, kb[3]);
  return reduce_scatter4(p0, p1, p2, p3);
}

// ------------------------------------------------------------- histograms

// Add 1 to hist[d] for every lane with m set.  The first active lane's digit
// is counted with one atomic for all lanes that share it (candidate scores
// crowd into few buckets in the high passes); other lanes add directly.
// Must be called by all 64 lanes of the wave.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t d, bool m) {
  const uint64_t act = __ballot(m);
  if (act == 0) return;
  const int leader = __ffsll((unsigned long long)act) - 1;
  const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
  const bool same = m && d == dl;
  const uint64_t sb = __ballot(same);
  if ((int)lane_id() == leader) atomicAdd(&hist[dl], (uint32_t)__popcll(sb));
  if (m && !same) atomicAdd(&hist[d], 1u);
}

// Wave-aggregated slot reservation on an LDS or global counter ("3.4
// Instruction-level optimizations": one atomic per group, positions from a
// ballot).  Returns this lane's position (valid where `take`).  All lanes call.
template <typename CounterT>
__device__ __forceinline__ uint32_t reserve(CounterT* counter, bool take) {
  const uint64_t ball = __ballot(take);
  if (ball == 0) return 0;
  uint32_t base = 0;
  if (lane_id() == 0) base = atomicAdd(counter, (uint32_t)__popcll(ball));
  base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
  return base + rank_in(ball);
}

// ------------------------------------------------------------- radix select

// Shared state for one workgroup-wide selection.
struct SelShared {
  uint32_t hist[256];
  uint32_t bucket, above, inbucket, pad0;
  uint32_t gt_count, eq_count, pad1, pad2;
};

// Result of the digit passes: every key with (key & mask) > prefix is in the
// top-K; `rem` more are taken among keys with (key & mask) == prefix.
struct SelResult {
  uint32_t prefix, mask;
  int rem;
};

// From a complete 256-bin histogram in sh.hist, find the bucket that holds
// the rem-th largest element (wave 0 scans, result broadcast through LDS).
__device__ __forceinline__ void find_bucket(SelShared& sh, int rem, int tid) {
  if (tid < 64) {
    const uint32_t lane = tid;
    const uint32_t h0 = sh.hist[4 * lane + 0], h1 = sh.hist[4 * lane + 1];
    const uint32_t h2 = sh.hist[4 * lane + 2], h3 = sh.hist[4 * lane + 3];
    const uint32_t s = h0 + h1 + h2 + h3;
    uint32_t suf = s;  // inclusive suffix sum over lanes >= lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(suf, off, 64);
      if (lane + off < 64) suf += o;
    }
    const uint32_t above_lane = suf - s;
    const uint32_t r = (uint32_t)rem;
    if (above_lane < r && r <= suf) {
      uint32_t acc = above_lane;
      uint32_t b, hb;
      if (acc + h3 >= r) { b = 4 * lane + 3; hb = h3; }
      else if ((acc += h3) + h2 >= r) { b = 4 * lane + 2; hb = h2; }
      else if ((acc += h2) + h1 >= r) { b = 4 * lane + 1; hb = h1; }
      else { acc += h1; b = 4 * lane; hb = h0; }
      sh.bucket = b;
      sh.above = acc;
      sh.inbucket = hb;
    }
  }
}

// Exact K-th-largest search by four 8-bit radix passes from the high byte
// down ("3.2 Sampled threshold", select step).  `src.key(i)` gives element
// i's order-preserving key.  If first_hist_ready, sh.hist already holds the
// top-byte histogram of all n elements (built during scoring).  Stops early
// once the chosen bucket is taken whole (allow_early).  Requires 1 <= rem <= n.
// All threads of the workgroup call this.
template <typename Src>
__device__ SelResult radix_select(const Src& src, int n, int rem, SelShared& sh, int tid,
                                  bool first_hist_ready, bool allow_early) {
  uint32_t prefix = 0, mask = 0;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (!(shift == 24 && first_hist_ready)) {
      for (int i = tid; i < 256; i += kWG) sh.hist[i] = 0;
      __syncthreads();
      for (int base = 0; base < n; base += kWG) {
        const int i = base + tid;
        const bool v = i < n;
        const uint32_t key = v ? src.key(i) : 0u;
        hist_add(sh.hist, (key >> shift) & 255u, v && ((key & mask) == prefix));
      }
      __syncthreads();
    }
    find_bucket(sh, rem, tid);
    __syncthreads();
    const uint32_t b = sh.bucket, above = sh.above, inb = sh.inbucket;
    __syncthreads();
    prefix |= b << shift;
    mask |= 0xFFu << shift;
    rem -= (int)above;
    if (allow_early && (int)inb == rem) break;
  }
  return SelResult{prefix, mask, rem};
}

// Write the selection into out[0..kr): ids of keys above the boundary first,
// then `rem` ids from the boundary group, then -1 up to K.
template <typename Src>
__device__ void emit_selection(const Src& src, int n, const SelResult& sel, int kr, int K,
                               int32_t* out, SelShared& sh, int tid) {
  if (tid == 0) { sh.gt_count = 0; sh.eq_count = 0; }
  __syncthreads();
  const int gt_base = 0, eq_base = kr - sel.rem;
  for (int base = 0; base < n; base += kWG) {
    const int i = base + tid;
    const bool v = i < n;
    const uint32_t key = v ? src.key(i) : 0u;
    const uint32_t mk = key & sel.mask;
    const bool gt = v && mk > sel.prefix;
    const bool eq = v && mk == sel.prefix;
    const uint32_t pg = reserve(&sh.gt_count, gt);
    if (gt) out[gt_base + pg] = src.id(i);
    const uint32_t pe = reserve(&sh.eq_count, eq);
    if (eq && (int)pe < sel.rem) out[eq_base + pe] = src.id(i);
  }
  for (int i = kr + tid; i < K; i += kWG) out[i] = -1;
}

}  // namespace idxk

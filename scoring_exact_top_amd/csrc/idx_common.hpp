// Device building blocks shared by the prefill and decode kernels (gfx950).
//
// Score of query row t against key s (Fusing Indexer Scoring and Exact Top-k page, "1.1 The
// problem" equation, with the FP8 operands dequantised by their scales as in
// "2.3 Problem definition"):
//
//   I[t,s] = k_scale[s] * sum_j w'_j * max(c_j, 0),   w'_j = w[t,j] * q_scale[t,j],
//   c_j    = dot(e4m3(q8[t,j,:]), e4m3(k8[s,:]))      (both scales are > 0)
//
// The ReLU is evaluated as max(c,0) = (c + |c|)/2, so that
//
//   sum_j w'_j max(c_j,0) = sum_j (w'_j/2)|c_j|  +  (1/2) u.k,   u = sum_j w'_j q_j.
//
// The first sum costs one VALU op per head (an FMA with an |x| source
// modifier); the linear term u.k goes to the matrix core: u is split into
// eight e4m3 vectors with FP32 scales, u ~= sum_m sigma_m e4m3(u8_m), residual
// below 27^-7 * 16/448 |u|_max, and these eight rows form half of a fifth
// 16-row A block, shared by two query rows (u_slot below).
//
// Every 128-deep FP8 contraction is one v_mfma_f32_16x16x128_f8f6f4 per 16
// rows x 16 keys.  A (rows x 128) lives in registers for the whole key loop;
// B (128 x 16 keys) comes from global memory through a buffer resource, lane l
// holding the 32 contiguous bytes [32*(l/16), +32) of key l%16 (A uses the
// same lane map, so any consistent split of the 128 bytes gives the same dot
// product).  The 16x16 f32 result puts row 4*(l/16)+r of a block in register r
// of the lane that owns key l%16: each lane weights its 16 heads and its 4
// rows of the u block, and the four partial sums of a key sit in lanes that
// differ in bits 4 and 5.  Four 16-key sub-tiles are combined by a
// reduce-scatter on v_permlane32_swap / v_permlane16_swap so that lane l ends
// with key l of the 64-key tile, through the same addition tree
// (g0+g2)+(g1+g3) for every key: identical keys give bit-identical scores
// wherever they sit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idxk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kH = 64;
constexpr int kD = 128;
constexpr int kKmax = 2048;
constexpr int kWG = 256;     // threads per workgroup of the 4-wave kernels
constexpr int kWaves = 4;
constexpr int kMaxWaves = 16;  // the register select's largest workgroup (1024 threads)
constexpr int kTile = 64;    // keys per tile (4 MFMA sub-tiles of 16)
constexpr int kUTerms = 8;   // e4m3 terms of the linear vector u

// Sub-tile c of a 64-key tile covers keys [sub_off(c), +16).  This order makes
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

// Make this wave's LDS writes visible to all its lanes before they read.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ v8i ld32(const uint8_t* p) {
  const uint4* v = reinterpret_cast<const uint4*>(p);
  uint4 x = v[0], y = v[1];
  v8i r;
  r[0] = (int)x.x; r[1] = (int)x.y; r[2] = (int)x.z; r[3] = (int)x.w;
  r[4] = (int)y.x; r[5] = (int)y.y; r[6] = (int)y.z; r[7] = (int)y.w;
  return r;
}

__device__ __forceinline__ v8i cat8(v4i x, v4i y) {
  v8i r;
  r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
  r[4] = y[0]; r[5] = y[1]; r[6] = y[2]; r[7] = y[3];
  return r;
}

// OCP e4m3fn conversions on gfx950's own FP8 converters (OCP formats on
// this architecture; checked against a bit-field codec over every non-NaN
// code, all rounding midpoints and the subnormal range).
// Bytes 2H and 2H+1 of w as floats:
template <bool H>
__device__ __forceinline__ float2 e4m3x2_dec(uint32_t w) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, H);
  return make_float2(f[0], f[1]);
}
// Nearest codes (ties to even) of a and b in bytes 0 and 1; the inputs are
// clamped to [-448, 448] because the converter does not saturate.
__device__ __forceinline__ uint32_t e4m3x2_enc(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.f, 448.f);
  b = __builtin_amdgcn_fmed3f(b, -448.f, 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Layout of the shared u block: row 4*(m/2) + 2p + (m%2) carries term m of
// slot p (p = 0, 1: the first or second row of a pair).  Result rows
// 4g..4g+3 of a block land in lane group g, so every lane holds two terms of
// each slot (terms 2g and 2g+1, in registers 2p and 2p+1): each row of a pair
// adds two u partials per lane, none of them zero.

// One query row as held by a lane: A operands of the four 16-head blocks and
// of the u block, the halved weights w'/2 of the 16 heads whose results land in
// this lane, and the halved scales sigma/2 of the 4 u-block rows it holds
// (zero for the rows of the other slot).
struct QOp {
  v8i a[4];
  v8i au;
  float wh[16];
  float sh[4];
};

// Two query rows as held by a lane, sharing one u block in that layout:
// sh[p][i] is sigma/2 of u-block row 4g+2p+i, whose result is register 2p+i
// of this lane's u accumulator.
struct QOp2 {
  v8i a[2][4];
  v8i au;
  float wh[2][16];
  float sh[2][2];
};

// Per-head query scales, all ones, for calls without q_scale.
__constant__ float kOnes[kH] = {
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f,
    1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};

__device__ __forceinline__ const float* row_qscale(const float* q_scale, int64_t t) {
  return q_scale ? q_scale + t * kH : kOnes;
}

// Linear vector u[d] = sum_j w_j q_scale_j dec(q[t,j,d]) of row t, split
// into kUTerms e4m3 terms written to codes[m*128 + d]; the scales go to sig.
// Lane l reads dims 16*(l&7) .. +15 of heads j = (l>>3) + 8i, i < 8, all
// eight 16-byte loads in flight together; the eight lanes that share a dim
// slice then add their partials with shuffles (tree xor 8, 16, 32).  The
// sum u goes through `codes` (512 bytes of FP32) to lanes d and d+64.
// Term m takes the nearest e4m3 codes of r_m / sigma_m, then
// r_{m+1} = r_m - sigma_m * dec(code), with sigma_0 = max|u| / 448 and
// sigma_{m+1} = sigma_m / 27.  That ratio needs no further max-reduction:
// a code within [-448, 448] is within 16 units of its value (half the
// largest e4m3 spacing, 32), so |r_{m+1}| <= 16 sigma_m = (16*27/448)
// sigma_{m+1} <= 448 sigma_{m+1}, and the next quotient needs no clamp.
// The loads of split_u: lane l's eight 16-byte code slices (heads
// (l>>3) + 8i) and those heads' weights w_j q_scale_j.
struct URaw {
  uint4 x[8];
  float wj[8];
};

__device__ __forceinline__ void split_u_codes(URaw& r, const uint8_t* q, int64_t t, uint32_t lane) {
  const uint8_t* base = q + t * (kH * kD) + 16 * (lane & 7u);
  const uint32_t h0 = lane >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.x[i] = *reinterpret_cast<const uint4*>(base + (h0 + 8 * i) * kD);
}

__device__ __forceinline__ void split_u_core(const URaw& r, uint32_t lane, uint8_t* codes, float (&sig)[kUTerms]);

__device__ __forceinline__ void split_u(const uint8_t* q, const float* q_scale, const float* w, int64_t t,
                                        uint32_t lane, uint8_t* codes, float (&sig)[kUTerms]) {
  const float* qs = row_qscale(q_scale, t);
  const uint32_t h0 = lane >> 3;
  URaw r;
  split_u_codes(r, q, t, lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) r.wj[i] = w[t * kH + h0 + 8 * i] * qs[h0 + 8 * i];
  split_u_core(r, lane, codes, sig);
}

__device__ __forceinline__ void split_u_core(const URaw& r, uint32_t lane, uint8_t* codes, float (&sig)[kUTerms]) {
  const uint4 (&x)[8] = r.x;
  const float (&wj)[8] = r.wj;
  float acc[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t wd[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2 lo = e4m3x2_dec<false>(wd[k]), hi = e4m3x2_dec<true>(wd[k]);
      acc[4 * k] = fmaf(wj[i], lo.x, acc[4 * k]);
      acc[4 * k + 1] = fmaf(wj[i], lo.y, acc[4 * k + 1]);
      acc[4 * k + 2] = fmaf(wj[i], hi.x, acc[4 * k + 2]);
      acc[4 * k + 3] = fmaf(wj[i], hi.y, acc[4 * k + 3]);
    }
  }
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    acc[d] += __shfl_xor(acc[d], 8, 64);
    acc[d] += __shfl_xor(acc[d], 16, 64);
    acc[d] += __shfl_xor(acc[d], 32, 64);
  }
  float* uf = reinterpret_cast<float*>(codes);
  if (lane < 8u) {
#pragma unroll
    for (int d = 0; d < 16; d += 4)
      *reinterpret_cast<float4*>(uf + 16 * lane + d) = make_float4(acc[d], acc[d + 1], acc[d + 2], acc[d + 3]);
  }
  wave_sync();
  float u0 = uf[lane], u1 = uf[64 + lane];
  wave_sync();
  float amax = fmaxf(fabsf(u0), fabsf(u1));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  float s = amax / 448.f;
#pragma unroll
  for (int m = 0; m < kUTerms; ++m) {
    const float inv = 1.0f / s;
    const uint32_t c = s > 0.f ? e4m3x2_enc(u0 * inv, u1 * inv) : 0u;
    codes[m * kD + lane] = (uint8_t)c;
    codes[m * kD + 64 + lane] = (uint8_t)(c >> 8);
    const float2 d = e4m3x2_dec<false>(c);
    u0 = fmaf(-s, d.x, u0);
    u1 = fmaf(-s, d.y, u1);
    sig[m] = s;
    s *= (1.0f / 27.0f);
  }
}

__device__ __forceinline__ void head_ops(v8i (&a)[4], float (&wh)[16], const uint8_t* q, const float* q_scale,
                                         const float* w, int64_t t, uint32_t lane) {
  const uint8_t* base = q + t * (kH * kD);
  const float* qs = row_qscale(q_scale, t);
  const uint32_t g = lane >> 4, i = lane & 15;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    a[b] = ld32(base + (16 * b + i) * kD + 32 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * b + 4 * g + r;
      wh[4 * b + r] = 0.5f * (w[t * kH + j] * qs[j]);
    }
  }
}

// Prepare rows t0 and t1 (all 64 lanes; scratch = 16*128 bytes of LDS).
__device__ __forceinline__ void prepare_q2(QOp2& o, const uint8_t* q, const float* q_scale, const float* w,
                                           int64_t t0, int64_t t1, uint32_t lane, uint8_t* scratch) {
  head_ops(o.a[0], o.wh[0], q, q_scale, w, t0, lane);
  head_ops(o.a[1], o.wh[1], q, q_scale, w, t1, lane);
  float s0[kUTerms], s1[kUTerms];
  split_u(q, q_scale, w, t0, lane, scratch, s0);
  split_u(q, q_scale, w, t1, lane, scratch + kUTerms * kD, s1);
  wave_sync();
  const uint32_t g = lane >> 4, i = lane & 15;
  // A row i of the u block: slot (i & 3) >> 1, term 2 (i >> 2) + (i & 1)
  const uint32_t urow = ((i & 3u) >> 1) * kUTerms + 2u * (i >> 2) + (i & 1u);
  const uint32_t* src = reinterpret_cast<const uint32_t*>(scratch + urow * kD + 32 * g);
#pragma unroll
  for (int k = 0; k < 8; ++k) o.au[k] = (int)src[k];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int m = 2 * (int)g + x;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < kUTerms; ++j) {
      a0 = m == j ? s0[j] : a0;
      a1 = m == j ? s1[j] : a1;
    }
    o.sh[0][x] = 0.5f * a0;
    o.sh[1][x] = 0.5f * a1;
  }
  wave_sync();
}

// Prepare query row t (all 64 lanes; scratch = 8*128 bytes of LDS).  slot
// (0 or 1) places the u terms where prepare_q2 puts them for the first or
// the second row of a pair, so that a row scored alone adds exactly
// the same nonzero partial sums in the same lanes and order as in its pair
// and gets bit-identical scores (the other slot's rows are zero codes with
// zero scales, and adding 0*0 leaves a sum unchanged).
__device__ __forceinline__ void prepare_q_tail(QOp& o, const float (&sig)[kUTerms], uint32_t lane, uint8_t* scratch,
                                               int slot);

__device__ __forceinline__ void prepare_q(QOp& o, const uint8_t* q, const float* q_scale, const float* w,
                                          int64_t t, uint32_t lane, uint8_t* scratch, int slot) {
  head_ops(o.a, o.wh, q, q_scale, w, t, lane);
  float sig[kUTerms];
  split_u(q, q_scale, w, t, lane, scratch, sig);
  prepare_q_tail(o, sig, lane, scratch, slot);
}

// prepare_q in two steps, for a caller that issues other loads between
// them: prepare_q_load issues every load (the operand codes of head_ops,
// the code slices of split_u, one weight w_j q_scale_j per lane), and
// prepare_q_finish does the arithmetic with no memory access besides LDS.
// The weights reach other lanes by shuffles; every value is computed as in
// prepare_q, so the two give bit-identical operands.
struct QRaw {
  v8i a[4];
  URaw u;
  float wq;  // lane j: w_j * q_scale_j
};

__device__ __forceinline__ void prepare_q_load(QRaw& r, const uint8_t* q, const float* q_scale, const float* w,
                                               int64_t t, uint32_t lane) {
  const uint8_t* base = q + t * (kH * kD);
  const uint32_t g = lane >> 4, i = lane & 15;
#pragma unroll
  for (int b = 0; b < 4; ++b) r.a[b] = ld32(base + (16 * b + i) * kD + 32 * g);
  split_u_codes(r.u, q, t, lane);
  r.wq = w[t * kH + lane] * row_qscale(q_scale, t)[lane];
}

__device__ __forceinline__ void prepare_q_finish(QOp& o, QRaw& r, uint32_t lane, uint8_t* scratch, int slot) {
  const uint32_t g = lane >> 4;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    o.a[b] = r.a[b];
#pragma unroll
    for (int k = 0; k < 4; ++k) o.wh[4 * b + k] = 0.5f * __shfl(r.wq, 16 * b + 4 * (int)g + k, 64);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) r.u.wj[i] = __shfl(r.wq, (int)(lane >> 3) + 8 * i, 64);
  float sig[kUTerms];
  split_u_core(r.u, lane, scratch, sig);
  prepare_q_tail(o, sig, lane, scratch, slot);
}

__device__ __forceinline__ void prepare_q_tail(QOp& o, const float (&sig)[kUTerms], uint32_t lane, uint8_t* scratch,
                                               int slot) {
  wave_sync();
  const uint32_t g = lane >> 4, i = lane & 15;
  if (((i & 3u) >> 1) == (uint32_t)slot) {  // A row i carries term 2 (i >> 2) + (i & 1) of slot (i & 3) >> 1
    const uint32_t term = 2u * (i >> 2) + (i & 1u);
    const uint32_t* src = reinterpret_cast<const uint32_t*>(scratch + term * kD + 32 * g);
#pragma unroll
    for (int k = 0; k < 8; ++k) o.au[k] = (int)src[k];
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) o.au[k] = 0;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 2 * (int)g + (r & 1);  // result row 4g + r: slot r >> 1, term m
    float sr = 0.f;
#pragma unroll
    for (int j = 0; j < kUTerms; ++j) sr = m == j ? sig[j] : sr;
    o.sh[r] = (r >> 1) == slot ? 0.5f * sr : 0.f;
  }
  wave_sync();
}

// Keys of one 64-key tile as B operands plus the scale of this lane's key.
struct KeyTile {
  v8i kb[4];
  float ks;
};

// Buffer resources over the key codes and key scales of `nkeys` keys.  Reads
// past the end return 0 (and are masked by the callers).
struct KeyBuf {
  rsrc_t k, ks;
};
__device__ __forceinline__ KeyBuf make_keybuf(const uint8_t* k, const float* k_scale, int64_t nkeys) {
  const int64_t nk = nkeys < 0 ? 0 : nkeys;
  const int kb = (int)(nk * kD > 0x7fffffffLL ? 0x7fffffffLL : nk * kD);
  const int sb = (int)(nk * 4 > 0x7fffffffLL ? 0x7fffffffLL : nk * 4);
  return KeyBuf{__builtin_amdgcn_make_buffer_rsrc((void*)k, (short)0, kb, 0x00020000),
                __builtin_amdgcn_make_buffer_rsrc((void*)k_scale, (short)0, sb, 0x00020000)};
}

// Tile of 64 consecutive keys starting at key index `base` (wave-uniform).
// Lane offsets are loop invariant; the tile offset is a scalar.
__device__ __forceinline__ void load_tile(KeyTile& t, const KeyBuf& kbuf, int base, uint32_t lane) {
  const int voff = (int)(lane & 15) * kD + 32 * (int)(lane >> 4);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int soff = (base + sub_off(c)) * kD;
    const v4i x = __builtin_amdgcn_raw_buffer_load_b128(kbuf.k, voff, soff, 0);
    const v4i y = __builtin_amdgcn_raw_buffer_load_b128(kbuf.k, voff + 16, soff, 0);
    t.kb[c] = cat8(x, y);
  }
  t.ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(kbuf.ks, (int)lane * 4, base * 4, 0));
}

// Relaid keys: tile j occupies bytes [8192 j, 8192 (j+1)) as eight 1 KiB
// blocks, block 2c+h holding, for lane l = 0..63, the 16 bytes that lane l
// loads as the h-th half of its B operand of sub-tile c (key sub_off(c) +
// l%16, bytes 32*(l/16) + 16h .. +16).  A load instruction then reads one
// contiguous KiB instead of 64 lanes striding 128 bytes apart.
__device__ __forceinline__ int relaid_src_offset(int tile, int blk, int l) {
  const int c = blk >> 1, h = blk & 1;
  return ((tile << 6) + sub_off(c) + (l & 15)) * kD + 32 * (l >> 4) + 16 * h;
}

// Tile index used for a refill of tile `tile` (scalar) of `ntiles` >= 1: a
// refill past the last tile, whose data is never scored, reloads the last
// tile instead, so every load's address stays inside the buffers and every
// offset fits in 31 bits.
__device__ __forceinline__ int refill_tile(int tile, int ntiles) { return tile < ntiles ? tile : ntiles - 1; }

// Tile of 64 arbitrary keys: key_of(i) gives the key index of tile slot i.
template <class F>
__device__ __forceinline__ void load_tile_gather(KeyTile& t, const KeyBuf& kbuf, const F& key_of, uint32_t lane) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int voff = key_of(sub_off(c) + (int)(lane & 15)) * kD + 32 * (int)(lane >> 4);
    const v4i x = __builtin_amdgcn_raw_buffer_load_b128(kbuf.k, voff, 0, 0);
    const v4i y = __builtin_amdgcn_raw_buffer_load_b128(kbuf.k, voff + 16, 0, 0);
    t.kb[c] = cat8(x, y);
  }
  t.ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(kbuf.ks, key_of((int)lane) * 4, 0, 0));
}

// MFMA part of a tile: 4 sub-tiles x 5 blocks into separate accumulators.
__device__ __forceinline__ void tile_mfma(const QOp& o, const v8i (&kb)[4], v4f (&acc)[20]) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
      acc[5 * c + b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.a[b], kb[c], z, 0, 0, 0, 0, 0, 0);
    acc[5 * c + 4] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.au, kb[c], z, 0, 0, 0, 0, 0, 0);
  }
}

// p0..p3: partials of sub-tiles 0..3 (keys 0-15, 32-47, 16-31, 48-63).
// Returns the full sum of key `lane` of the 64-key tile.
__device__ __forceinline__ float reduce_scatter4(float p0, float p1, float p2, float p3) {
  auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  const float A = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
  const float B = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(A), __float_as_uint(B), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// Epilogue of tile_mfma: per lane and sub-tile, sum over its 16 heads of
// (w'/2)|c| then over its 4 u-block rows of (sigma/2) d, in this fixed order;
// then the reduce-scatter.  Lane l returns key l's sum (before k_scale).
__device__ __forceinline__ float tile_epilogue(const QOp& o, const v4f (&acc)[20]) {
  float p[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float x = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) x = fmaf(o.wh[4 * b + r], fabsf(acc[5 * c + b][r]), x);
#pragma unroll
    for (int r = 0; r < 4; ++r) x = fmaf(o.sh[r], acc[5 * c + 4][r], x);
    p[c] = x;
  }
  return reduce_scatter4(p[0], p[1], p[2], p[3]);
}

// Score of the tile (lane l: key l), k_scale applied.  Same arithmetic as
// tile_mfma + tile_epilogue, pipelined by sub-tile: the MFMAs of sub-tile
// c+1 are issued before the epilogue of sub-tile c, so only two sub-tiles'
// accumulators (40 VGPRs instead of 80) are live at once.
__device__ __forceinline__ float tile_score(const QOp& o, const KeyTile& t) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  v4f acc[2][5];
  const auto issue = [&](v4f (&a)[5], const v8i& kb) {
#pragma unroll
    for (int b = 0; b < 4; ++b) a[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.a[b], kb, z, 0, 0, 0, 0, 0, 0);
    a[4] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.au, kb, z, 0, 0, 0, 0, 0, 0);
  };
  float p[4];
  issue(acc[0], t.kb[0]);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c < 3) issue(acc[(c + 1) & 1], t.kb[c + 1]);
    const v4f (&a)[5] = acc[c & 1];
    float x = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) x = fmaf(o.wh[4 * b + r], fabsf(a[b][r]), x);
#pragma unroll
    for (int r = 0; r < 4; ++r) x = fmaf(o.sh[r], a[4][r], x);
    p[c] = x;
  }
  return reduce_scatter4(p[0], p[1], p[2], p[3]) * t.ks;
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
  uint32_t wsum[3][kMaxWaves];  // per-wave minima, maxima and key counts of range_select_regs
  uint32_t ring[2][256];     // range_select_regs: with hist, one histogram per pass in rotation
  uint32_t trash[64];        // range_select_regs: where the keys outside a pass's range are counted
};

// Result of the digit passes: every key with (key & mask) > prefix is in the
// top-K; `rem` more are taken among the `group` keys with (key & mask) ==
// prefix.  rem < group only where the group is one value (all digits
// fixed): a tie at the K-th score, resolved toward the lowest positions.
struct SelResult {
  uint32_t prefix, mask;
  int rem, group;
};

// ------------------------------------------------- wave-wide DPP primitives

// Lane-to-lane moves inside the VALU (DPP) instead of LDS permutes: each
// step of a wave scan or reduction costs one VALU operation rather than an
// LDS round trip.  Every lane of the wave must be active.
namespace dpp {
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;  // GFX9 row broadcasts
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;      // quad_perm [1,0,3,2], [2,3,0,1]
constexpr int kRowHalfMirror = 0x141, kRowMirror = 0x140;
// lane value moved by `ctrl`; lanes whose source lies outside the row (or
// whose row is masked off) get `fill`
template <int ctrl, int row_mask = 0xf>
__device__ __forceinline__ uint32_t mov(uint32_t fill, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, ctrl, row_mask, 0xf, false);
}
}  // namespace dpp

// Inclusive prefix sum over the wave's 64 lanes in lane order: a scan
// within each row of 16 lanes by shifts of 1, 2, 4 and 8, then the row
// totals carried by broadcasting lane 15 into rows 1 and 3 and lane 31
// into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
  x += dpp::mov<dpp::kRowShr1>(0u, x);
  x += dpp::mov<dpp::kRowShr2>(0u, x);
  x += dpp::mov<dpp::kRowShr4>(0u, x);
  x += dpp::mov<dpp::kRowShr8>(0u, x);
  x += dpp::mov<dpp::kRowBcast15, 0xa>(0u, x);
  x += dpp::mov<dpp::kRowBcast31, 0xc>(0u, x);
  return x;
}

// Reduction over the wave's 64 lanes, returned wave-uniform: within each
// row of 16 by two quad exchanges and the half-row and row mirrors, then
// the four row results read on the scalar unit.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, const Op& op) {
  x = op(x, dpp::mov<dpp::kQuadXor1>(x, x));
  x = op(x, dpp::mov<dpp::kQuadXor2>(x, x));
  x = op(x, dpp::mov<dpp::kRowHalfMirror>(x, x));
  x = op(x, dpp::mov<dpp::kRowMirror>(x, x));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return op(op(a, b), op(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return wave_reduce(x, [](uint32_t p, uint32_t q) { return p < q ? p : q; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return wave_reduce(x, [](uint32_t p, uint32_t q) { return p > q ? p : q; });
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return wave_reduce(x, [](uint32_t p, uint32_t q) { return p + q; });
}

// From a complete 256-bin histogram in sh.hist, find the bucket that holds
// the rem-th largest element (wave 0 scans, result broadcast through LDS).
__device__ __forceinline__ void find_bucket(SelShared& sh, int rem, int tid) {
  if (tid < 64) {
    const uint32_t lane = tid;
    const uint32_t h0 = sh.hist[4 * lane + 0], h1 = sh.hist[4 * lane + 1];
    const uint32_t h2 = sh.hist[4 * lane + 2], h3 = sh.hist[4 * lane + 3];
    const uint32_t s = h0 + h1 + h2 + h3;
    const uint32_t inc = wave_inclusive_sum(s);
    const uint32_t above_lane = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63) - inc;  // lanes above this one
    const uint32_t suf = above_lane + s;
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

// The same search run by one wave on its own over a complete 256-bin
// histogram in LDS (no barrier, no broadcast): the bucket, the count above
// it and the count in it, wave-uniform.
__device__ __forceinline__ void wave_find_bucket(const uint32_t* hist, int rem, uint32_t lane, uint32_t& bucket,
                                                 uint32_t& above, uint32_t& inbucket) {
  const uint32_t h0 = hist[4 * lane + 0], h1 = hist[4 * lane + 1];
  const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
  const uint32_t s = h0 + h1 + h2 + h3;
  const uint32_t inc = wave_inclusive_sum(s);
  const uint32_t above_lane = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63) - inc;  // lanes above this one
  const uint32_t suf = above_lane + s;
  const uint32_t r = (uint32_t)rem;
  const bool owner = above_lane < r && r <= suf;
  uint32_t acc = above_lane, b = 4 * lane, hb = h0;
  if (acc + h3 >= r) { b = 4 * lane + 3; hb = h3; }
  else if ((acc += h3) + h2 >= r) { b = 4 * lane + 2; hb = h2; }
  else if ((acc += h2) + h1 >= r) { b = 4 * lane + 1; hb = h1; }
  else { acc += h1; }
  const int ol = __ffsll((unsigned long long)__ballot(owner)) - 1;
  bucket = (uint32_t)__builtin_amdgcn_readlane((int)b, ol);
  above = (uint32_t)__builtin_amdgcn_readlane((int)acc, ol);
  inbucket = (uint32_t)__builtin_amdgcn_readlane((int)hb, ol);
}

// Exact K-th-largest search by four 8-bit radix passes from the high byte
// down ("3.2 Sampled threshold", select step).  `src.key(i)` gives element
// i's order-preserving key.  If first_hist_ready, sh.hist already holds the
// top-byte histogram of all n elements (built during scoring).  Stops early
// once the chosen bucket is taken whole (allow_early).  Requires 1 <= rem <= n.
// All threads of the workgroup (NW waves) call this.
template <int NW = kWaves, typename Src>
__device__ SelResult radix_select(const Src& src, int n, int rem, SelShared& sh, int tid,
                                  bool first_hist_ready, bool allow_early) {
  constexpr int NT = 64 * NW;
  uint32_t prefix = 0, mask = 0;
  int group = n;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (!(shift == 24 && first_hist_ready)) {
      for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
      __syncthreads();
      for (int base = 0; base < n; base += NT) {
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
    group = (int)inb;
    if (allow_early && (int)inb == rem) break;
  }
  return SelResult{prefix, mask, rem, group};
}

// Exclusive prefix sum over the workgroup (NW waves) of one per-thread
// count, in thread order; also returns the total.  All threads call this.
template <int NW = kWaves>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t a, SelShared& sh, int tid, uint32_t& total) {
  const uint32_t lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t inc = wave_inclusive_sum(a);
  if (lane == 63) sh.wsum[0][wave] = inc;
  __syncthreads();
  uint32_t before = 0u;
  total = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = sh.wsum[0][w];
    before += w < wave ? c : 0u;
    total += c;
  }
  __syncthreads();
  return before + inc - a;
}

// Write the selection into out[0..kr): ids of keys above the boundary first,
// then `rem` ids from the boundary group (the lowest positions first where
// the group is a tie larger than rem), then -1 up to K.  NW waves.
template <int NW = kWaves, typename Src>
__device__ void emit_selection(const Src& src, int n, const SelResult& sel, int kr, int K,
                               int32_t* out, SelShared& sh, int tid) {
  constexpr int NT = 64 * NW;
  if (tid == 0) { sh.gt_count = 0; sh.eq_count = 0; }
  __syncthreads();
  const int eq_base = kr - sel.rem;
  const bool ordered = sel.rem < sel.group;  // a tie: take its lowest positions
  uint32_t eq_done = 0u;                     // group members before this pass (ordered)
  for (int base = 0; base < n; base += NT) {
    const int i = base + tid;
    const bool v = i < n;
    const uint32_t key = v ? src.key(i) : 0u;
    const uint32_t mk = key & sel.mask;
    const bool gt = v && mk > sel.prefix;
    const bool eq = v && mk == sel.prefix;
    const uint32_t pg = reserve(&sh.gt_count, gt);
    if (gt) out[pg] = src.id(i);
    if (!ordered) {
      const uint32_t pe = reserve(&sh.eq_count, eq);
      if (eq && (int)pe < sel.rem) out[eq_base + pe] = src.id(i);
    } else if (eq_done < (uint32_t)sel.rem) {  // workgroup-uniform
      uint32_t tot;
      const uint32_t pe = eq_done + block_exclusive_scan<NW>(eq ? 1u : 0u, sh, tid, tot);
      if (eq && pe < (uint32_t)sel.rem) out[eq_base + pe] = src.id(i);
      eq_done += tot;
    }
  }
  for (int i = kr + tid; i < K; i += NT) out[i] = -1;
}

// ------------------------------------------ register-resident selection

// Where a thread's register keys come from: key[j] is list element
// base + j*step, valid when that is below n.  jmax is wave-uniform: no lane
// of the wave holds a valid key[j] for j >= jmax.
struct RegLayout {
  uint32_t base, step, n, jmax;
  __device__ uint32_t at(int j) const { return base + (uint32_t)j * step; }
  __device__ bool valid(int j) const { return at(j) < n; }
};

// The workgroup (NW waves) holds one list of n elements, element
// j*64*NW + tid in key[j].
template <int NW = kWaves>
__device__ __forceinline__ RegLayout block_list_layout(uint32_t n, uint32_t tid) {
  constexpr uint32_t nt = 64u * NW;
  return RegLayout{tid, nt, n, (n + nt - 1u) / nt};
}

// Loads of one list of (key bits, id) pairs into registers, key[j] and
// id[j] = element lay.at(j): one 8-byte buffer load per element, whose
// out-of-range reads return 0, so all of them are issued back to back
// without a branch per element; invalid slots get key 0 and read nothing
// (their offset lies past every buffer, so the bounds check answers them
// without a memory access).  `extent` (uniform) bounds the list; lay.valid
// masks the entries; dec maps the stored key bits to the key.
template <int M, class Dec>
__device__ __forceinline__ void load_list_regs(uint32_t (&key)[M], int32_t (&id)[M], const uint2* list,
                                               uint32_t extent, const RegLayout& lay, const Dec& dec) {
  const rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)list, (short)0, (int)(extent * 8u), 0x00020000);
  v2i raw[M];
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const int off = lay.valid(j) ? (int)(lay.at(j) * 8u) : 0x7FFFFFF0;
    raw[j] = __builtin_amdgcn_raw_buffer_load_b64(rl, off, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < M; ++j) {
    key[j] = lay.valid(j) ? dec((uint32_t)raw[j].x) : 0u;
    id[j] = raw[j].y;
  }
}

// Selection over keys held in registers: every key above `last` is in the
// top-K, and `rem` of the `group` keys in [lo, last] complete it.  rem <
// group only where lo == last (a tie at the K-th score).
struct RangeSel {
  uint32_t lo, last;
  int rem, group;
};

// Register lists for the functions below hold nonzero keys, with 0 in
// unused slots (load_list_regs stores 0 there).  Candidate keys qualify: a
// candidate passed score >= tau, which no NaN does, and only a NaN maps to
// key 0.  So no per-slot validity mask is kept.  A list is read through a
// functor kf(j) returning slot j's key, so that derived keys (the tie-break
// below) need no second register array.

// The K-th-largest search ("3.2 Sampled threshold", select step) with digits
// taken relative to the list's own range: the first pass cuts [min, max]
// into 256 equal power-of-two bins, so a candidate list (scores between tau
// and the row maximum) spreads over the bins and the search usually ends
// after two passes, when the bin that holds the K-th key is taken whole.
// Each further pass splits the chosen bin 256 ways; a bin of width one ends
// the search.  Requires 1 <= rem < number of keys.  All threads of the
// workgroup call this.
// One barrier per pass: the passes take three histograms in rotation
// (sh.ring[0], sh.ring[1], sh.hist, ...), every wave finds the bucket
// itself, and each pass clears the histogram of the pass after it, which
// was last read two passes before (so behind this pass's barrier for every
// wave).  sh.hist is first written in the second pass, behind two
// barriers, so that a caller's earlier use of it has ended.  NW waves (4 to
// 16) per workgroup; the first 256 threads clear the 256 bins.  A list of
// one value (massive ties) needs no pass.
// kScores: the keys are f2key images of scores.  Where they lie on both
// sides of zero, equal key bins would hold nearly all of them in one or two
// bins (the key range between two scores of opposite sign is mostly taken
// by tiny magnitudes), and the atomics of that pass would queue on those
// bins; the first pass then cuts the score range [min, max] itself into 256
// equal bins (monotone in the key, so each bin is a key range), and one
// reduction finds the key range of the chosen bin for the passes after it.
template <int M, int NW = kWaves, bool kScores = true, class KF>
__device__ __forceinline__ RangeSel range_select_regs(const KF& kf, const RegLayout& lay, int rem, SelShared& sh, int tid) {
  static_assert(NW >= 4 && NW <= kMaxWaves, "256 bins cleared by the first 256 threads");
  const uint32_t lane = tid & 63;
  const int wave = tid >> 6;
  const bool clears = NW == 4 || tid < 256;
  const auto ring = [&](int i) { return i == 2 ? sh.hist : sh.ring[i]; };
  if (clears) sh.ring[0][tid] = 0u;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u, mn2 = 0xFFFFFFFFu, mx2 = 0u;  // two chains
  uint32_t cnt = 0u;  // keys held (nonzero)
#pragma unroll
  for (int j = 0; j < M; ++j) {
    if ((uint32_t)j < lay.jmax) {
      const uint32_t k = kf(j);
      cnt += k ? 1u : 0u;
      if (j & 1) {
        mn2 = min(mn2, k ? k : 0xFFFFFFFFu);
        mx2 = max(mx2, k);
      } else {
        mn = min(mn, k ? k : 0xFFFFFFFFu);
        mx = max(mx, k);
      }
    }
  }
  mn = wave_min_u32(min(mn, mn2));
  mx = wave_max_u32(max(mx, mx2));
  cnt = wave_sum_u32(cnt);
  if (lane == 0) { sh.wsum[0][wave] = mn; sh.wsum[1][wave] = mx; sh.wsum[2][wave] = cnt; }
  __syncthreads();
  cnt = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mn = min(mn, sh.wsum[0][w]);
    mx = max(mx, sh.wsum[1][w]);
    cnt += sh.wsum[2][w];
  }
  if (mx == mn) {  // every key is one value (massive ties): no pass to run
    __syncthreads();  // the minima are read before sh is used again
    return RangeSel{mn, mn, rem, (int)cnt};
  }
  const uint32_t span = mx - mn;
  const int bits = span ? 32 - __clz((int)span) : 0;
  int s = bits > 8 ? bits - 8 : 0;
  uint32_t lo = mn, width = span;  // the range is [lo, lo + width]
  int group = (int)cnt;
  int cur = 0;
  bool done = false;
  if (kScores && mn < 0x80000000u && mx >= 0x80000000u && bits > 24) {  // scores of both signs
    const float vlo = key2f(mn);
    const float scale = 256.0f / (key2f(mx) - vlo);
    // bin of a key: 0..255, nondecreasing in the key (a NaN product, which
    // finite scores do not make, would land in the top bin)
    const auto vbin = [&](uint32_t k) { return (uint32_t)fminf((key2f(k) - vlo) * scale, 255.0f); };
    uint32_t* const h = ring(0);
    if (clears) ring(1)[tid] = 0u;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      if ((uint32_t)j < lay.jmax) {
        const uint32_t k = kf(j);
        atomicAdd(k ? &h[vbin(k)] : &sh.trash[lane], 1u);
      }
    }
    __syncthreads();
    uint32_t b, above, inb;
    wave_find_bucket(h, rem, lane, b, above, inb);
    rem -= (int)above;
    group = (int)inb;
    // the chosen bin's smallest and largest keys (the minima above were read
    // before this pass's barrier, so sh.wsum is free)
    uint32_t bmn = 0xFFFFFFFFu, bmx = 0u;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      if ((uint32_t)j < lay.jmax) {
        const uint32_t k = kf(j);
        const bool in = k != 0u && vbin(k) == b;
        bmn = in ? min(bmn, k) : bmn;
        bmx = in ? max(bmx, k) : bmx;
      }
    }
    bmn = wave_min_u32(bmn);
    bmx = wave_max_u32(bmx);
    if (lane == 0) { sh.wsum[0][wave] = bmn; sh.wsum[1][wave] = bmx; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      bmn = min(bmn, sh.wsum[0][w]);
      bmx = max(bmx, sh.wsum[1][w]);
    }
    lo = bmn;
    width = bmx - bmn;
    const int wb = width ? 32 - __clz((int)width) : 0;
    s = wb > 8 ? wb - 8 : 0;
    cur = 1;  // ring(1) was cleared by this pass
    done = (int)inb == rem || width == 0u;  // taken whole, or one value (a tie)
  }
#pragma unroll 1
  while (!done) {
    const int nxt = cur == 2 ? 0 : cur + 1;
    uint32_t* const h = ring(cur);
    if (clears) ring(nxt)[tid] = 0u;
    // branch-free: a key outside the range is counted in this lane's trash
    // bin (no exec-mask change per slot, no conflicts among those lanes)
#pragma unroll
    for (int j = 0; j < M; ++j) {
      if ((uint32_t)j < lay.jmax) {  // wave-uniform guard; keeps the keys in registers
        const uint32_t d = kf(j) - lo;  // key 0 wraps above any width (lo >= 1)
        atomicAdd(d <= width ? &h[d >> s] : &sh.trash[lane], 1u);
      }
    }
    __syncthreads();
    uint32_t b, above, inb;
    wave_find_bucket(h, rem, lane, b, above, inb);
    rem -= (int)above;
    group = (int)inb;
    const uint32_t off = b << s;
    lo += off;
    width = min(width - off, (1u << s) - 1u);  // s <= 24
    if ((int)inb == rem || s == 0) break;
    s = s > 8 ? s - 8 : 0;
    cur = nxt;
  }
  __syncthreads();  // every wave has read the histograms before sh is used again
  return RangeSel{lo, lo + width, rem, group};
}

// Smallest key in [sel.lo, sel.last]: the smallest key selected by `sel`
// when the boundary range is taken whole or holds one value.  All threads
// of the workgroup call this.
template <int M, int NW = kWaves, class KF>
__device__ __forceinline__ uint32_t range_min_regs(const KF& kf, const RegLayout& lay, const RangeSel& sel, SelShared& sh,
                                   int tid) {
  const uint32_t lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t width = sel.last - sel.lo;
  uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < M; ++j)
    if ((uint32_t)j < lay.jmax && kf(j) - sel.lo <= width) mn = min(mn, kf(j));
  mn = wave_min_u32(mn);
  if (lane == 0) sh.wsum[0][wave] = mn;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) mn = min(mn, sh.wsum[0][w]);
  __syncthreads();
  return mn;
}

// Which boundary keys to take: all of [lo, last] when rem == group, else
// (a tie at one value) the rem with the lowest ids, found by a second
// range select over ~id of the tied keys (ids are >= 0 and distinct, so
// ~id is nonzero and the select ends with the rem largest ~id taken whole).
// Returns the smallest ~id taken (0: no tie-break, every boundary key).
template <int NW = kWaves, int M>
__device__ __forceinline__ uint32_t tie_bound_regs(const uint32_t (&key)[M], const int32_t (&id)[M], const RegLayout& lay,
                                   const RangeSel& sel, SelShared& sh, int tid) {
  if (sel.rem >= sel.group) return 0u;
  const uint32_t v = sel.lo;
  // recomputed at every use (the empty asm hides the value from common
  // subexpression elimination): a precomputed copy of all M values would
  // stay live across the whole kernel and cost M registers where ties are
  // rare
  const auto tk = [&](int j) {
    uint32_t x = (uint32_t)id[j];
    asm volatile("" : "+v"(x));
    return key[j] == v ? ~x : 0u;
  };
  return range_select_regs<M, NW, false>(tk, lay, sel.rem, sh, tid).lo;
}

// Emit for range_select_regs: keys above `last` fill out[0, kr - rem), the
// boundary keys taken (those in [lo, last] with ~id >= idlo: exactly rem of
// them) fill out[kr - rem, kr), -1 up to K; idmap(id[j]) is written.  Each
// thread counts its winners of both kinds, one workgroup scan turns the
// counts into the thread's first output slots, and the thread writes its
// winners there in slot order, so the result does not depend on timing.
// At most 65535 keys per list (two 16-bit counts share a word).  NW waves.
template <int NW = kWaves, int M, class IdMap>
__device__ __forceinline__ void emit_range_regs(const uint32_t (&key)[M], const int32_t (&id)[M], const RegLayout& lay,
                                const RangeSel& sel, uint32_t idlo, int kr, int K, int32_t* out,
                                const IdMap& idmap, SelShared& sh, int tid) {
  const uint32_t width = sel.last - sel.lo;
  // every slot's output id first, all loads of a map that reads memory (one
  // page-table entry per slot for paged rows) issued together and waited
  // for after the counting below; translated inside the stores' branches,
  // each load was waited for alone
  int32_t mid[M];
#pragma unroll
  for (int j = 0; j < M; ++j) mid[j] = idmap(id[j]);
  const auto gt = [&](int j) { return key[j] > sel.last; };
  const auto eq = [&](int j) {  // recomputed at every use, as in tie_bound_regs
    uint32_t x = (uint32_t)id[j];
    asm volatile("" : "+v"(x));
    return key[j] - sel.lo <= width && ~x >= idlo;
  };
  uint32_t mine = 0u, mine2 = 0u;  // this thread's winners: above | boundary << 16 (two chains)
#pragma unroll
  for (int j = 0; j < M; ++j) {
    if ((uint32_t)j < lay.jmax) {
      const uint32_t c = (gt(j) ? 1u : 0u) + (eq(j) ? 0x10000u : 0u);
      if (j & 1) mine2 += c; else mine += c;
    }
  }
  mine += mine2;
  uint32_t total;
  const uint32_t first = block_exclusive_scan<NW>(mine, sh, tid, total);
  uint32_t pg = first & 0xFFFFu;
  uint32_t pe = (uint32_t)(kr - sel.rem) + (first >> 16);
  // branch-free stores through a resource bounded at out[kr]: a lane that
  // stores nothing in a slot gets an offset past every buffer, and a
  // boundary key past kr (none where the tie-break ran) is dropped the same
  // way
  const rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)out, (short)0, kr * 4, 0x00020000);
#pragma unroll
  for (int j = 0; j < M; ++j) {
    if ((uint32_t)j < lay.jmax) {
      const bool g = gt(j), e = eq(j);
      __builtin_amdgcn_raw_buffer_store_b32(mid[j], ro, g ? (int)(pg * 4u) : 0x7FFFFFF0, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(mid[j], ro, e ? (int)(pe * 4u) : 0x7FFFFFF0, 0, 0);
      pg += g ? 1u : 0u;
      pe += e ? 1u : 0u;
    }
  }
  for (int i = kr + tid; i < K; i += 64 * NW) out[i] = -1;
  __syncthreads();
}

// ------------------------------------------------- wave-level selection


// Radix select run by ONE wave over its own 256-bin LDS histogram, so that
// several rows of a workgroup are selected concurrently without workgroup
// barriers.  Same contract as radix_select (1 <= rem <= n).
template <typename Src>
__device__ SelResult wave_radix_select(const Src& src, int n, int rem, uint32_t* hist, uint32_t lane,
                                       bool allow_early) {
  uint32_t prefix = 0, mask = 0;
  int group = n;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[lane + 64 * i] = 0u;
    wave_sync();
    for (int base = 0; base < n; base += 64) {
      const int i = base + (int)lane;
      const bool v = i < n;
      const uint32_t key = v ? src.key(i) : 0u;
      hist_add(hist, (key >> shift) & 255u, v && ((key & mask) == prefix));
    }
    wave_sync();
    uint32_t bb, above, inb;
    wave_find_bucket(hist, rem, lane, bb, above, inb);
    prefix |= bb << shift;
    mask |= 0xFFu << shift;
    rem -= (int)above;
    group = (int)inb;
    wave_sync();  // histogram reads done before the next pass clears it
    if (allow_early && (int)inb == rem) break;
  }
  return SelResult{prefix, mask, rem, group};
}

}  // namespace idxk

// BF16 stream scan (page "Deleting the key transpose puts the DSA indexer scan on its streaming
// floor"): B independent streams (decode sequences), each with its own N unquantised BF16 keys
// [N][128] and one 64-head BF16 query; every key is scored,
//
//   I[b,i] = sum_{j<64} w[b,j] * ReLU( q[b,j] . k[b,i] ),   i in [0, lens[b]),
//
// and each stream keeps its exact top-K.  Bound by HBM: a key is 256 bytes and
// costs 2*64*128 FLOP, far below the BF16 MFMA ridge.
//
//   k_scan_bf16      G workgroups per stream sweep it together: workgroup g
//                    takes the groups of 4 consecutive 64-key tiles g, g+G,
//                    ..., one tile per wave, so that a stream is read as one
//                    advancing front (separate per-workgroup chunks read
//                    about 20% slower); per 16-key sub-tile 16 MFMAs
//                    (v_mfma_f32_16x16x32_bf16: 4 head blocks x 4 K-steps of
//                    32 dims), keys as the B operand read straight from their
//                    [N][128] rows (each load a 64-byte piece of each of 16
//                    keys): both MFMA operands take K-contiguous rows, so
//                    the transpose that the page removes by swapping the
//                    operands' roles never arises; one tile of lead refilled
//                    sub-tile by sub-tile in place;
//                    ReLU and head weights in registers, the same 4-group
//                    reduce-scatter as the FP8 path; one FP32 score per key
//                    written to the stream's score row.
//   k_rows_gather / k_topk_rows (idx_rows.hip): per stream a sampled cut, a
//                    gather over many workgroups, an exact register select.
//   k_stream_floor   the page's floor: read every 256-byte key record, write
//                    one 4-byte value per record, no arithmetic of the method.
#include <hip/hip_ext.h>
#include <string.h>

#include "idx_internal.hpp"
#include "idx_rows.hpp"
#include "idx_scan.hpp"

namespace idxk {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct ScanArgs {
  const uint16_t* q;  // [B][64][128] BF16 patterns
  const float* w;     // [B][64]
  const uint16_t* k;  // [B][N][128]
  const int32_t* lens;
  int32_t B, N, K, G;
  uint32_t* ctrl;
  float* scores;      // [B][N]
};

__device__ __forceinline__ v8bf as_bf(v4i x) {
  v8bf r;
  __builtin_memcpy(&r, &x, sizeof r);
  return r;
}

// Lane l = 16g + i holds, for K-step s (0..3) of a 128-dim row, the 8 dims
// 32s + 8g .. +7 (bytes 64s + 16g .. +15 of the row): one load instruction
// reads a whole 64-byte piece of each of its 16 rows (a piece split over 4
// instructions reads about 15% slower), and both operands (keys as B, heads
// as A) use the same dim permutation, so every dot product is over all 128
// dims.
__global__ __launch_bounds__(kWG, 2) void k_scan_bf16(ScanArgs A) {
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x, b = blockIdx.y;
  if (g == 0 && b == 0) clear_ctrl(A.ctrl, tid);  // first kernel of the call
  const int L = A.lens[b];
  if (L <= A.K || L > A.N) return;  // remap or invalid: the selection kernel handles the row
  const int tstep = kWaves * A.G;
  const int tile0 = kWaves * g + wave, tile_end = (L + 63) >> 6;
  if (tile0 >= tile_end) return;

  const uint32_t gi = lane >> 4, li = lane & 15;
  // query operands: head block hb, K-step s; the lane's 16 weights (heads
  // 16hb + 4gi + r, where its accumulator rows land)
  v8bf qa[4][4];
  float wl[16];
  const uint16_t* qb = A.q + (int64_t)b * kH * kD;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qa[hb][s] = as_bf(*reinterpret_cast<const v4i*>(qb + (16 * hb + li) * kD + 32 * s + 8 * gi));
#pragma unroll
    for (int r = 0; r < 4; ++r) wl[4 * hb + r] = A.w[(int64_t)b * kH + 16 * hb + 4 * gi + r];
  }
  // keys of this stream through a buffer resource: rows past L read as 0,
  // and scores past L are dropped
  const rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)(A.k + (int64_t)b * A.N * kD), (short)0,
                                                      L * (kD * 2), 0x00020000);
  const rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc((void*)(A.scores + (int64_t)b * A.N), (short)0,
                                                      L * 4, 0x00020000);
  const int voff = (int)li * (kD * 2) + 16 * (int)gi;
  v8bf kb[4][4];  // sub-tile c, K-step s: the current tile, refilled in place with the next one
  // a refill runs up to tstep tiles past the stream's end: such tiles take
  // an offset past any key buffer (2^31 bytes; the bounds check drops their
  // loads), so no offset is computed beyond the stream
  const auto load_sub = [&](int tile, int c) {
    const int soff = tile < tile_end ? (tile * kTile + sub_off(c)) * (kD * 2) : (int)0x80000000u;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kb[c][s] = as_bf(__builtin_amdgcn_raw_buffer_load_b128(kr, voff, soff + 64 * s, 0));
  };
#pragma unroll
  for (int c = 0; c < 4; ++c) load_sub(tile0, c);
  const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int T = tile0; T < tile_end; T += tstep) {
    float p[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v4f acc[4] = {z, z, z, z};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[hb][s], kb[c][s], acc[hb], 0, 0, 0);
      load_sub(T + tstep, c);  // reads past the stream's keys return 0
      float x = 0.f;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int r = 0; r < 4; ++r) x = fmaf(wl[4 * hb + r], fmaxf(acc[hb][r], 0.f), x);
      p[c] = x;
    }
    const float sc = reduce_scatter4(p[0], p[1], p[2], p[3]);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), sr, ((T << 6) + (int)lane) * 4, 0, 0);
  }
}

// Read n records of 256 bytes, write one float per record (the sum of its
// first and last words, so that every byte is loaded and nothing folds away):
// the streaming floor the scan is measured against.  The waves of the grid
// sweep the records as one front, each load a contiguous 1 KiB per wave
// (lane l: 16 bytes of record 4*(wave's group) + l/16), read non-temporally
// (nothing is read twice); lanes l%16 == 0 write.  Deeper unrolling and
// per-wave chunks measured slower.
__global__ __launch_bounds__(kWG) void k_stream_floor(const uint4* src, int64_t n, float* dst) {
  const uint32_t lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kWG + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kWG) >> 6;
  for (int64_t r0 = wave * 4; r0 < n; r0 += nwaves * 4) {
    const int64_t r = r0 + (lane >> 4);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < n) {
      const v4i t = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src) + r * 16 + (lane & 15));
      v = make_uint4((uint32_t)t[0], (uint32_t)t[1], (uint32_t)t[2], (uint32_t)t[3]);
    }
    float x = __uint_as_float(v.x) + __uint_as_float(v.w);
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    if ((lane & 15) == 0 && r < n) dst[r] = x;
  }
}

// ------------------------------------------------------------------ host

static inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

static int scan_split(int32_t B, int32_t N) {
  // about 1024 workgroups (three per CU are resident at 168 VGPRs; 512, 768,
  // 1536 and 2048 measured 1-4% slower), at least 4096 keys per workgroup
  int g = B > 0 ? 1024 / B : 1;
  const int by_len = N / 4096;
  if (g > by_len) g = by_len;
  return g < 1 ? 1 : (g > 4096 ? 4096 : g);
}

static int scan_gather_split(int32_t B) {
  int g = 1;  // a power of two
  while (2 * g <= kMaxGatherSplit && 2 * g * B <= 512) g *= 2;
  return g;
}

struct ScanLayout {
  size_t ctrl, scores, gcnt, gkey, gid, total;
};

static ScanLayout scan_layout(int32_t B, int32_t N) {
  ScanLayout L;
  size_t o = 0;
  const size_t b = (size_t)(B > 0 ? B : 0);
  L.ctrl = o; o = a256(o + 4 * kCtrlWords);
  L.scores = o; o = a256(o + 4 * b * (size_t)(N > 0 ? N : 0));
  L.gcnt = o; o = a256(o + 4 * b * (size_t)scan_gather_split(B));
  L.gkey = o; o = a256(o + 4 * b * 6144);
  L.gid = o; o = a256(o + 4 * b * 6144);
  L.total = o;
  return L;
}

size_t scan_bf16_workspace_bytes(int32_t B, int32_t N, int32_t K) {
  if (B < 0 || N < 0 || K < 1 || K > kKmax) return 0;
  return scan_layout(B, N).total;
}

int scan_bf16(const uint16_t* q, const float* w, const uint16_t* k, const int32_t* lens, int32_t B, int32_t N,
              int32_t K, int32_t* out_idx, void* workspace, size_t workspace_bytes, hipStream_t stream,
              const idx_topk_opts* opts) {
  if (B < 0 || N < 0 || K < 1 || K > kKmax) return IDX_EINVAL;
  if (B > kMaxGridY) return IDX_EUNSUPPORTED;  // streams index the grid's y dimension
  // one stream's keys per buffer resource (the last tile's rows included)
  if (((int64_t)N + kTile) * kD * 2 > 0x7fffffffLL) return IDX_EUNSUPPORTED;
  if (opts && (opts->force_tau || opts->cand_cap || opts->row_status || opts->clock_out || opts->math_only ||
               opts->main_reps < 0 || opts->main_reps > 1000))
    return IDX_EINVAL;
  if (B == 0) return IDX_OK;
  if (!q || !w || !k || !lens || !out_idx) return IDX_EINVAL;
  if (((uintptr_t)q & 15u) || ((uintptr_t)k & 15u)) return IDX_EINVAL;
  const ScanLayout L = scan_layout(B, N);
  if (!workspace || workspace_bytes < L.total) return IDX_EWORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return IDX_EINVAL;
  char* ws = static_cast<char*>(workspace);
  ScanArgs A{q, w, k, lens, B, N, K, scan_split(B, N), reinterpret_cast<uint32_t*>(ws + L.ctrl),
             reinterpret_cast<float*>(ws + L.scores)};
  hipEvent_t ev0 = opts ? static_cast<hipEvent_t>(opts->ev_main_start) : nullptr;
  hipEvent_t ev1 = opts ? static_cast<hipEvent_t>(opts->ev_main_stop) : nullptr;
  // the timing events, when given, are recorded by the launches themselves
  // (main_reps > 1 repeats the idempotent scan for timing)
  const int reps = opts && opts->main_reps > 1 ? opts->main_reps : 1;
  for (int r = 0; r < reps; ++r) {
    hipEvent_t e0 = r == 0 ? ev0 : nullptr, e1 = r == reps - 1 ? ev1 : nullptr;
    if (e0 || e1)
      hipExtLaunchKernelGGL(k_scan_bf16, dim3(A.G, B), dim3(kWG), 0, stream, e0, e1, 0, A);
    else
      hipLaunchKernelGGL(k_scan_bf16, dim3(A.G, B), dim3(kWG), 0, stream, A);
  }
  if (hipGetLastError() != hipSuccess) return IDX_EHIP;
  const int gs = scan_gather_split(B);
  RowsArgs R{A.scores, (int64_t)N, nullptr, lens, B, N, K, out_idx, A.ctrl, nullptr, 0, 0,
             reinterpret_cast<uint32_t*>(ws + L.gkey), reinterpret_cast<int32_t*>(ws + L.gid),
             reinterpret_cast<uint32_t*>(ws + L.gcnt), 6144 / gs, gs};
  return launch_topk_rows_gathered(R, stream);
}

const float* scan_bf16_scores(const void* workspace, int32_t B, int32_t N) {
  if (!workspace || B < 0 || N < 0) return nullptr;
  return reinterpret_cast<const float*>(static_cast<const char*>(workspace) + scan_layout(B, N).scores);
}

int stream_floor(const void* src, int64_t n_records, float* dst, hipStream_t stream) {
  if (n_records < 0) return IDX_EINVAL;
  if (n_records == 0) return IDX_OK;
  if (!src || !dst || ((uintptr_t)src & 15u)) return IDX_EINVAL;
  hipLaunchKernelGGL(k_stream_floor, dim3(2048), dim3(kWG), 0, stream, static_cast<const uint4*>(src),
                     n_records, dst);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;
}

}  // namespace idxk

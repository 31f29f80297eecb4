// Shared device helpers for the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lfm {

constexpr int kHidden = 2048;   // d
constexpr int kExperts = 64;    // E
constexpr int kTopK = 4;        // k
constexpr int kFF = 1536;       // expert intermediate width
constexpr int kWave = 64;       // CDNA wavefront width
constexpr float kRouterEps = 1e-6f;
constexpr float kRmsEps = 1e-6f;
// Largest N taken by the weight-streaming (decode) kernels, which group
// their own tokens in LDS (capacity kStreamMaxTokens).  Measured against the
// grouped kernels with 32- and 64-row token tiles (layer us, first N tokens
// of one layer, streaming / grouped): bf16 N = 1: 31.0-32.0 / 38.2-40.2;
// 8: 68.5 / 64.7-65.4; 64 (the 64-token decode workload): 143.4-146.5 /
// 136.6-137.7.  FP8 experts: N = 1: 30.8-31.2 / 36.1-36.6; 8: 52.3 / 47.6.
constexpr int kDecodeMaxTokens = 4;    // both layers: weight-streaming kernels up to here
constexpr int kStreamMaxTokens = 256;  // tokens the weight-streaming kernels can group

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 16 bytes of bf16 values as loaded from memory.
struct alignas(16) Pack8 {
  uint4 u;
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Widening a bf16 bit pattern to fp32 is exact.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (the gfx950 conversion
// instruction; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats to two bf16 in one word, lo in the low half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// D = A * B + C on a 16x16 tile with K = 32 (bf16 in, fp32 accumulate).
// Lane l supplies row (l % 16) of A and column (l % 16) of B, eight K
// elements each; the accumulator of lane l holds column (l % 16), rows
// 4 * (l / 16) + r for r = 0..3.
__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// D = A * B + C on a 32x32 tile with K = 16 (bf16 in, fp32 accumulate).
// Lane l supplies row (l % 32) of A and column (l % 32) of B, K elements
// 8 (l / 32) .. 8 (l / 32) + 7 each; accumulator value r of lane l is
// column (l % 32), row 8 (r / 4) + 4 (l / 32) + (r % 4).  On gfx950 this
// form runs at twice the bf16 rate of the 16x16x32 one.
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Row of the 32-row tile held by accumulator value r of lane l.
__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
}

// Packed expert weights: 1 KB fragments of 32 rows x 16 K, lane-major
// (bytes [16 l, 16 l + 16) hold row l % 32, K 8 (l / 32) .. + 7), ordered
// (expert, 32-row block, K step) with the K steps of a block contiguous.
// Gate/up: block b has W_gate rows 16 b .. 16 b + 15 as rows 0..15 and the
// W_up rows 16 b .. 16 b + 15 as rows 16..31 (96 blocks, 128 K steps);
// down: block b has W_down rows 32 b .. 32 b + 31 (64 blocks, 96 K steps).
constexpr int kGateupBlocks = kFF / 16;
constexpr int kGateupSteps = kHidden / 16;
constexpr int kDownBlocks = kHidden / 32;
constexpr int kDownSteps = kFF / 16;
constexpr uint32_t kFragBytes = 1024;

__device__ __forceinline__ float silu(float g) {
  // The hardware reciprocal (1 ulp) in place of an IEEE divide: the product
  // is rounded to bf16 right after.
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer loads: a uniform base (SGPRs) plus a 32-bit per-lane byte offset,
// so that a wavefront's many loads share one address register.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16 bytes at byte offset voff + soff.  NT: read once, non-temporal.
template <bool NT>
__device__ __forceinline__ uint4 buf_ld(Rsrc r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT ? 2 : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A value that is the same in every lane, made known to be so (kept in a
// scalar register).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Maps a linear m-tile id to (expert, first row) given the expert row
// offsets: expert e owns ceil(count_e / tile_rows) consecutive m-tiles.
// Returns false when the id is past the last tile.  Every lane of the wave
// must call it (it uses cross-lane operations).
struct MTile {
  int expert;
  int row_begin;  // first grouped row of the tile
  int rows;       // valid rows in the tile (<= tile_rows)
};

__device__ __forceinline__ bool map_mtile(const int* __restrict__ offsets, int mt, int tile_rows,
                                          MTile& t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int beg = offsets[lane];
  const int cnt = offsets[lane + 1] - beg;
  const int nt = (cnt + tile_rows - 1) / tile_rows;
  const int incl = wave_inclusive_scan(nt, lane);
  const int total = __shfl(incl, kWave - 1, kWave);
  if (mt >= total) return false;
  const unsigned long long ball = __ballot(incl > mt);
  const int e = __ffsll(static_cast<long long>(ball)) - 1;
  const int excl_e = __shfl(incl - nt, e, kWave);
  const int beg_e = __shfl(beg, e, kWave);
  const int cnt_e = __shfl(cnt, e, kWave);
  const int m0 = (mt - excl_e) * tile_rows;
  t.expert = e;
  t.row_begin = beg_e + m0;
  t.rows = min(tile_rows, cnt_e - m0);
  return true;
}

// FP8 (OCP E4M3) helpers.  Four floats to four codes, round to nearest
// even (the gfx950 conversion instruction; a value rounding to zero keeps its
// sign).  The callers scale by 448 / amax first, so no input exceeds 448.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// Eight E4M3 codes (bytes of lo, then hi) as eight bf16 values (exact: every
// E4M3 value is a bf16 value).
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  using bf16x2 = __bf16 __attribute__((ext_vector_type(2)));
  const bf16x2 v[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false),
                       __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true),
                       __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false),
                       __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true)};
  uint4 r;
  __builtin_memcpy(&r, v, sizeof(r));
  return r;
}

}  // namespace lfm

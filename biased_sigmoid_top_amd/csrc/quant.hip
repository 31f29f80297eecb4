// Per-row, per-128-group FP8 quantisation of bf16 rows, for the FP8 layer's
// grouped path (token rows of X before gate/up, hidden rows H before down).
//
// Method: the inferencekey.com page on the 24B reasoning MoE (German
// edition, "Für Engineers" part, the quantisation entry) gives the FP8
// checkpoint's activations as FP8 (E4M3) quantised dynamically per group of
// 128.  A group with largest magnitude amax is coded as E4M3(x * (448 /
// amax)) in fp32 (round to nearest even, the sign of a zero kept) with the
// scale amax / 448; amax = 0 gives zero codes and scale 0 -- the same
// arithmetic as the weight-streaming FP8 kernels, which quantise in
// registers.
//
// Code layout (one byte per value, row pitch K bytes): within each 32-wide
// piece of a row the 8-code runs are stored in the order 0, 2, 1, 3, so
// that 16-byte chunk 2p + h of the row holds columns 32p + 8h .. + 7 and
// 32p + 16 + 8h .. + 7 -- the columns that lane half h of an FP8 matrix-core
// operand meets in the packed weight fragments (pack_fp8.hip).  The grouped
// kernels stage these chunks exactly as they stage 16-byte chunks of bf16
// rows.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kQGroup = 128;
constexpr int kQLanesPerGroup = kQGroup / 8;               // 8 values (16 bytes) per lane
constexpr int kQGroupsPerWave = kWave / kQLanesPerGroup;   // 4
constexpr int kQWavesPerBlock = 4;

// Four consecutive (row, group) items per wavefront, 16 lanes per item, 8
// values per lane.  Rows have a multiple of four groups (K = 2048 or 1536),
// so a wavefront's items share one row.
__global__ __launch_bounds__(kQWavesPerBlock * kWave) void quantize_groups_kernel(
    const uint16_t* __restrict__ A, int64_t rows, int K, uint8_t* __restrict__ Q,
    float* __restrict__ S) {
  const int groups = K / kQGroup;
  const int lane = threadIdx.x % kWave;
  const int64_t item = (static_cast<int64_t>(blockIdx.x) * kQWavesPerBlock + threadIdx.x / kWave) *
                           kQGroupsPerWave + lane / kQLanesPerGroup;
  if (item >= rows * groups) return;
  const int64_t row = item / groups;
  const int g = static_cast<int>(item % groups);
  const int run = lane % kQLanesPerGroup;  // 8-value run of the group
  const size_t at = static_cast<size_t>(row) * K + g * kQGroup;
  const uint4 v = *reinterpret_cast<const uint4*>(A + at + 8 * run);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  // Largest magnitude of the group on the bf16 bit patterns (finite values
  // order as their bits), then over the group's 16 lanes.
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) m = max(m, max(w[k] & 0x7fffu, (w[k] >> 16) & 0x7fffu));
  float amax = __uint_as_float(m << 16);
#pragma unroll
  for (int off = kQLanesPerGroup / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  const float inv = amax > 0.f ? 448.f / amax : 0.f;
  auto q4 = [&](uint32_t lo, uint32_t hi) {
    return e4m3x4(__uint_as_float(lo << 16) * inv, __uint_as_float(lo & 0xffff0000u) * inv,
                  __uint_as_float(hi << 16) * inv, __uint_as_float(hi & 0xffff0000u) * inv);
  };
  // Run r of a 32-wide piece (r = run % 4) goes to 8-byte slot 0, 2, 1, 3.
  const int slot = (run & ~3) | ((run & 1) << 1) | ((run >> 1) & 1);
  *reinterpret_cast<uint2*>(Q + at + 8 * slot) = make_uint2(q4(w[0], w[1]), q4(w[2], w[3]));
  if (run == 0) S[static_cast<size_t>(row) * groups + g] = amax / 448.f;
}

}  // namespace

hipError_t launch_quantize_groups(const uint16_t* A, int64_t rows, int K, uint8_t* Q, float* S,
                                  hipStream_t stream) {
  const int64_t items = rows * (K / kQGroup);
  const int64_t per_block = static_cast<int64_t>(kQWavesPerBlock) * kQGroupsPerWave;
  const int64_t blocks = (items + per_block - 1) / per_block;
  hipLaunchKernelGGL(quantize_groups_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(kQWavesPerBlock * kWave), 0, stream, A, rows, K, Q, S);
  return hipGetLastError();
}

}  // namespace lfm

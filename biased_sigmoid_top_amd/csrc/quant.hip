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
// registers.  The codes are stored as their bf16 values (every E4M3 value is
// a bf16 value), so the grouped kernels stage them as they stage bf16 rows.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kQGroup = 128;
constexpr int kQWavesPerBlock = 4;

// One wavefront per (row, group): lane l holds values 2l and 2l + 1.
__global__ __launch_bounds__(kQWavesPerBlock * kWave) void quantize_groups_kernel(
    const uint16_t* __restrict__ A, int64_t rows, int K, uint16_t* __restrict__ Q,
    float* __restrict__ S) {
  const int groups = K / kQGroup;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kQWavesPerBlock + threadIdx.x / kWave;
  if (item >= rows * groups) return;
  const int lane = threadIdx.x % kWave;
  const int64_t row = item / groups;
  const int g = static_cast<int>(item % groups);
  const size_t at = static_cast<size_t>(row) * K + g * kQGroup + 2 * lane;
  const uint32_t v = *reinterpret_cast<const uint32_t*>(A + at);
  // Largest magnitude on the bf16 bit patterns (finite values order as their bits).
  float amax = __uint_as_float(max(v & 0x7fffu, (v >> 16) & 0x7fffu) << 16);
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  const float inv = amax > 0.f ? 448.f / amax : 0.f;
  const float lo = __uint_as_float(v << 16) * inv, hi = __uint_as_float(v & 0xffff0000u) * inv;
  const uint32_t codes = e4m3x4(lo, hi, 0.f, 0.f);
  const uint4 vals = e4m3x8_to_bf16(codes, 0u);
  *reinterpret_cast<uint32_t*>(Q + at) = vals.x;
  if (lane == 0) S[static_cast<size_t>(row) * groups + g] = amax / 448.f;
}

}  // namespace

hipError_t launch_quantize_groups(const uint16_t* A, int64_t rows, int K, uint16_t* Q, float* S,
                                  hipStream_t stream) {
  const int64_t items = rows * (K / kQGroup);
  const int64_t blocks = (items + kQWavesPerBlock - 1) / kQWavesPerBlock;
  hipLaunchKernelGGL(quantize_groups_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(kQWavesPerBlock * kWave), 0, stream, A, rows, K, Q, S);
  return hipGetLastError();
}

}  // namespace lfm

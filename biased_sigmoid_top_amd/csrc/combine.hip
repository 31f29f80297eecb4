// Weighted combine back to token order, and the RMS normalisation that
// precedes the feed-forward network.
//
// Method: flozi.net guide "LFM2.5-24B-A2B: Biased Routing, Short
// Convolutions and Ten KV Caches":
//  - section "What to verify in a deployment": the expert path accumulates
//    the weighted expert outputs;
//  - section "The exact checkpoint": RMS normalisation before the
//    feed-forward network and a residual add after it.
//
// The combine reads the four expert rows of a token (stored in slot order)
// and accumulates them in the fixed order j = 0..3 in fp32 (no atomics), so
// the result is the same on every run.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kRowThreads = 256;  // one token row of 2048 values per workgroup

// out[t] = (resid[t] +) sum_j w[t, j] * Y[t*4 + j]; resid may alias out.
// Y rows are in slot order, so a token's four rows are contiguous.
__global__ __launch_bounds__(kRowThreads) void combine_kernel(const float* __restrict__ Y,
                                                              const float* __restrict__ w,
                                                              const float* resid, float* out) {
  const size_t t = blockIdx.x;
  const float4 wt = *reinterpret_cast<const float4*>(w + t * kTopK);
  const float* y0 = Y + t * kTopK * kHidden;
  const float* y1 = y0 + kHidden;
  const float* y2 = y1 + kHidden;
  const float* y3 = y2 + kHidden;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col = (h * kRowThreads + threadIdx.x) * 4;
    const float4 a = *reinterpret_cast<const float4*>(y0 + col);
    const float4 b = *reinterpret_cast<const float4*>(y1 + col);
    const float4 c = *reinterpret_cast<const float4*>(y2 + col);
    const float4 d = *reinterpret_cast<const float4*>(y3 + col);
    float4 acc;
    acc.x = fmaf(wt.w, d.x, fmaf(wt.z, c.x, fmaf(wt.y, b.x, wt.x * a.x)));
    acc.y = fmaf(wt.w, d.y, fmaf(wt.z, c.y, fmaf(wt.y, b.y, wt.x * a.y)));
    acc.z = fmaf(wt.w, d.z, fmaf(wt.z, c.z, fmaf(wt.y, b.z, wt.x * a.z)));
    acc.w = fmaf(wt.w, d.w, fmaf(wt.z, c.w, fmaf(wt.y, b.w, wt.x * a.w)));
    float* dst = out + t * kHidden + col;
    if (resid != nullptr) {
      const float4 x = *reinterpret_cast<const float4*>(resid + t * kHidden + col);
      acc.x = x.x + acc.x;
      acc.y = x.y + acc.y;
      acc.z = x.z + acc.z;
      acc.w = x.w + acc.w;
    }
    *reinterpret_cast<float4*>(dst) = acc;
  }
}

// X[t] = bf16(x[t] / sqrt(mean(x[t]^2) + eps)), unit weight.
__global__ __launch_bounds__(kRowThreads) void rmsnorm_kernel(const float* __restrict__ x,
                                                              uint16_t* __restrict__ X) {
  __shared__ float wave_ss[kRowThreads / kWave];
  const size_t t = blockIdx.x;
  const float* row = x + t * kHidden;
  float4 v[2];
  float ss = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v[h] = *reinterpret_cast<const float4*>(row + (h * kRowThreads + threadIdx.x) * 4);
    ss = fmaf(v[h].x, v[h].x, ss);
    ss = fmaf(v[h].y, v[h].y, ss);
    ss = fmaf(v[h].z, v[h].z, ss);
    ss = fmaf(v[h].w, v[h].w, ss);
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) wave_ss[threadIdx.x / kWave] = ss;
  __syncthreads();
  const float tot = (wave_ss[0] + wave_ss[1]) + (wave_ss[2] + wave_ss[3]);
  const float inv = 1.0f / sqrtf(tot * (1.0f / kHidden) + kRmsEps);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = pack_bf16x2(v[h].x * inv, v[h].y * inv);
    const uint32_t hi = pack_bf16x2(v[h].z * inv, v[h].w * inv);
    *reinterpret_cast<uint2*>(X + t * kHidden + (h * kRowThreads + threadIdx.x) * 4) =
        make_uint2(lo, hi);
  }
}

}  // namespace

hipError_t launch_combine(const float* Y, const float* w, const float* resid, float* out,
                          int64_t N, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(N), dim3(kRowThreads), 0, stream, Y, w, resid, out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, uint16_t* X, int64_t N, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(N), dim3(kRowThreads), 0, stream, x, X);
  return hipGetLastError();
}

}  // namespace lfm

// Router: skinny bf16 MFMA GEMM (X W_r^T), sigmoid per logit, biased top-4
// selection on a wavefront (one lane per expert), unbiased weights
// normalised by sum + eps, and the per-block expert histogram used by the
// dispatch step.
//
// Method: flozi.net guide "LFM2.5-24B-A2B: Biased Routing, Short
// Convolutions and Ten KV Caches", section "The router has two different
// scores" -- sigmoid on each logit, the stored bias added after the
// activation takes part in the selection only, weights from the unbiased
// scores, normalised with an epsilon, routed scale 1.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kRouteThreads = 512;  // 8 wavefronts
constexpr int kRouteWaves = kRouteThreads / kWave;

// Orders floats like their values as unsigned integers.
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup routes TM tokens.  Wave w multiplies token tile
// (w % (TM/16)) against all 64 router rows over K range number
// (w / (TM/16)); the K partials are summed in LDS in a fixed order.
template <int TM>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wr,
    const float* __restrict__ bias, int32_t* __restrict__ idx_out, float* __restrict__ w_out,
    int32_t* __restrict__ blockcounts, int N) {
  constexpr int kTileT = TM / 16;            // token tiles per workgroup
  constexpr int kSplits = kRouteWaves / kTileT;
  constexpr int kChunk = kHidden / kSplits;  // K elements per wave
  static_assert(kChunk % 128 == 0, "K chunk must be a multiple of 128");

  __shared__ float part[kSplits][TM][kExperts + 1];
  __shared__ int wave_counts[kRouteWaves][kExperts];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int tt = wave % kTileT;
  const int ks = wave / kTileT;
  const int t0 = blockIdx.x * TM;

  // ---- logits: 16 tokens x 64 experts per wave over its K chunk ----
  const int r16 = lane & 15;
  const int g = lane >> 4;
  int tok = t0 + tt * 16 + r16;
  tok = tok < N ? tok : N - 1;  // rows past N are computed and discarded
  const uint16_t* xrow = X + static_cast<size_t>(tok) * kHidden;
  f32x4 acc[4] = {};
  for (int kb = ks * kChunk; kb < (ks + 1) * kChunk; kb += 128) {
    uint4 a[4], b[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = ld16(xrow + kb + (4 * i + g) * 8);
#pragma unroll
    for (int et = 0; et < 4; ++et) {
      const uint16_t* wrow = Wr + static_cast<size_t>(et * 16 + r16) * kHidden + kb;
#pragma unroll
      for (int i = 0; i < 4; ++i) b[et][i] = ld16(wrow + (4 * i + g) * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int et = 0; et < 4; ++et) acc[et] = mfma16(a[i], b[et][i], acc[et]);
  }
#pragma unroll
  for (int et = 0; et < 4; ++et)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[ks][tt * 16 + 4 * g + r][et * 16 + r16] = acc[et][r];
  __syncthreads();

  // ---- selection: one wavefront per token, lane e holds expert e ----
  const float b_e = bias[lane];
  int my_count = 0;
  for (int t = wave; t < TM; t += kRouteWaves) {
    float l = 0.0f;
#pragma unroll
    for (int s = 0; s < kSplits; ++s) l += part[s][t][lane];
    const float s_e = 1.0f / (1.0f + expf(-l));
    const float c_e = s_e + b_e;
    const uint64_t key = (static_cast<uint64_t>(orderable(c_e)) << 32) |
                         static_cast<uint32_t>(kExperts - 1 - lane);
    bool taken = false;
    int sel[kTopK];
    float sel_s[kTopK];
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
      uint64_t k = taken ? 0ull : key;
#pragma unroll
      for (int off = kWave / 2; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(k, off, kWave);
        k = o > k ? o : k;
      }
      const int win = kExperts - 1 - static_cast<int>(k & 0xffffffffu);
      taken = taken || (lane == win);
      sel[j] = win;
      sel_s[j] = __shfl(s_e, win, kWave);
      sum += sel_s[j];
    }
    const int tg = t0 + t;
    if (tg < N) {
      my_count += taken ? 1 : 0;
      if (lane < kTopK) {
        const float denom = sum + kRouterEps;
        int e_out = sel[0];
        float s_out = sel_s[0];
#pragma unroll
        for (int j = 1; j < kTopK; ++j)
          if (lane == j) { e_out = sel[j]; s_out = sel_s[j]; }
        idx_out[static_cast<size_t>(tg) * kTopK + lane] = e_out;
        w_out[static_cast<size_t>(tg) * kTopK + lane] = s_out / denom;
      }
    }
  }
  if (blockcounts != nullptr) {
    wave_counts[wave][lane] = my_count;
    __syncthreads();
    if (wave == 0) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < kRouteWaves; ++w) c += wave_counts[w][lane];
      blockcounts[static_cast<size_t>(blockIdx.x) * kExperts + lane] = c;
    }
  }
}

}  // namespace

int route_block_tokens(int64_t N) { return N <= 2048 ? 16 : 64; }

hipError_t launch_route(const uint16_t* X, const uint16_t* Wr, const float* bias, int32_t* idx,
                        float* w, int32_t* blockcounts, int N, hipStream_t stream) {
  const int tm = route_block_tokens(N);
  const int grid = (N + tm - 1) / tm;
  if (tm == 16)
    hipLaunchKernelGGL(route_kernel<16>, dim3(grid), dim3(kRouteThreads), 0, stream, X, Wr, bias,
                       idx, w, blockcounts, N);
  else
    hipLaunchKernelGGL(route_kernel<64>, dim3(grid), dim3(kRouteThreads), 0, stream, X, Wr, bias,
                       idx, w, blockcounts, N);
  return hipGetLastError();
}

}  // namespace lfm

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
//
// Two forms, the same arithmetic.  Every 16-token tile is split into 16
// K slices of 128; a wavefront multiplies the tile's 16 token rows by all 64
// router rows over one slice (16 MFMAs) into a 16 x 64 fp32 partial.  A
// wavefront per token then adds the 16 partials of each logit in slice
// order, applies the sigmoid and the bias, takes the top 4 and normalises
// the weights.
//  * Split (up to 2048 tokens): route_partial runs one wavefront per (tile,
//    slice) and stores the partials to the workspace, route_select reduces
//    them.  With N = 64 that is 64 wavefronts on 64 CUs, so the router
//    matrix is pulled through many CUs at once.
//  * Fused (above 2048 tokens): a 16-wavefront workgroup per tile, the
//    partials staged in LDS -- one launch, no scratch traffic.  Each
//    workgroup's CU reads the whole 256 KB router matrix, which costs about
//    12 us however few tiles run (the rate at which one CU's misses are
//    served), so it pays only once the split form's partial traffic is
//    larger.  Measured per call: N = 1024 split 9.2 us, fused 11.9; N = 4096
//    split 18.6, fused 12.3.  Beyond 256 tiles (4,096 tokens) a workgroup
//    takes several tiles in turn with its wavefronts' router slices kept in
//    registers, so that each CU reads the router matrix once: at N = 16,384
//    four tiles per workgroup.
// For the FP8 layer's grouped path the router also writes X's E4M3 codes
// and group scales: a K slice of 128 is one activation group (the
// inferencekey.com page on the 24B reasoning MoE, "Für Engineers" part, the
// quantisation entry: FP8 activations quantised dynamically per group of
// 128), and the slice's wavefront already holds the group's 128 values of
// each of its 16 rows, so no separate quantisation launch reads X again.
// The codes and scales are those of quantize_groups_kernel (quant.hip):
// the same fp32 decisions and the same byte order.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kRouteTokens = 16;
constexpr int kSlices = kHidden / 128;                // 16 K slices
constexpr int kSelectThreads = kRouteTokens * kWave;  // one wavefront per token
constexpr int kFusedThreads = kSlices * kWave;        // one wavefront per slice
constexpr int kPartStride = kExperts + 4;             // LDS row pitch: conflict-free partial stores
constexpr int64_t kSplitMaxTokens = 2048;
constexpr int kFusedMaxWorkgroups = 256;              // one per CU
static_assert(kSlices == kRouteTokens, "the fused kernel's wavefronts serve as slices, then tokens");

// Orders floats like their values as unsigned integers.
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// E4M3 codes and scale of the 128-value group (row tok, group slice) whose
// runs 4i + g (8 values each, i = 0..3) lane holds in a[i], g = lane / 16;
// the four lanes of a row (lane % 16) hold the whole group.  Q: rows of 2048
// codes, in every 32-wide piece the 8-code runs in the order 0, 2, 1, 3;
// S: 16 scales per row.
__device__ __forceinline__ void quantize_slice(const uint4 (&a)[4], int tok, bool real, int slice,
                                               int lane, uint8_t* __restrict__ Q, float* __restrict__ S) {
  const int g = lane >> 4;
  // Largest magnitude on the bf16 bit patterns (finite values order as
  // their bits), then over the row's four lanes.
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {a[i].x, a[i].y, a[i].z, a[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max(w[k] & 0x7fffu, (w[k] >> 16) & 0x7fffu));
  }
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 16, kWave)));
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 32, kWave)));
  const float amax = __uint_as_float(m << 16);
  const float inv = amax > 0.f ? 448.f / amax : 0.f;
  auto q4 = [&](uint32_t lo, uint32_t hi) {
    return e4m3x4(__uint_as_float(lo << 16) * inv, __uint_as_float(lo & 0xffff0000u) * inv,
                  __uint_as_float(hi << 16) * inv, __uint_as_float(hi & 0xffff0000u) * inv);
  };
  if (!real) return;
  uint8_t* row = Q + static_cast<size_t>(tok) * kHidden + slice * 128;
  // Run 4i + g is run g of 32-wide piece i: 8-byte slot 0, 2, 1, 3 of it.
  const int slot = ((g & 1) << 1) | (g >> 1);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint2*>(row + 8 * (4 * i + slot)) = make_uint2(q4(a[i].x, a[i].y), q4(a[i].z, a[i].w));
  if (g == 0) S[static_cast<size_t>(tok) * kSlices + slice] = amax / 448.f;
}

// Router rows of K slice `slice` as the B operands of slice_product.
__device__ __forceinline__ void slice_weights(const uint16_t* __restrict__ Wr, int slice, int lane,
                                              uint4 (&b)[4][4]) {
  const int r16 = lane & 15;
  const int g = lane >> 4;
#pragma unroll
  for (int et = 0; et < 4; ++et) {
    const uint16_t* wrow = Wr + static_cast<size_t>(et * 16 + r16) * kHidden + slice * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[et][i] = ld16(wrow + (4 * i + g) * 8);
  }
}

// The products of slice_partial on router rows already loaded by
// slice_weights; the token row pieces are left in a (row tok of X).
__device__ __forceinline__ void slice_product(const uint16_t* __restrict__ X, const uint4 (&b)[4][4],
                                              int tok, int slice, int lane, uint4 (&a)[4], f32x4 (&acc)[4]) {
  const int g = lane >> 4;
  const uint16_t* xrow = X + static_cast<size_t>(tok) * kHidden + slice * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = ld16(xrow + (4 * i + g) * 8);
#pragma unroll
  for (int et = 0; et < 4; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int et = 0; et < 4; ++et) acc[et] = mfma16(a[i], b[et][i], acc[et]);
}

// Partial logits of token tile `tile` over K slice `slice`.  acc[et][r] of
// a lane is expert et*16 + lane % 16, token 4 * (lane / 16) + r of the tile.
// With Q (QUANT) the slice's group of each real token row is quantised too.
template <bool QUANT>
__device__ __forceinline__ void slice_partial(const uint16_t* __restrict__ X,
                                              const uint16_t* __restrict__ Wr, int tile, int slice,
                                              int N, int lane, f32x4 (&acc)[4],
                                              uint8_t* __restrict__ Q, float* __restrict__ S) {
  const int r16 = lane & 15;
  const int g = lane >> 4;
  int tok = tile * kRouteTokens + r16;
  const bool real = tok < N;
  tok = real ? tok : N - 1;  // rows past N are computed and discarded
  const int kb = slice * 128;
  const uint16_t* xrow = X + static_cast<size_t>(tok) * kHidden + kb;
  uint4 a[4], b[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = ld16(xrow + (4 * i + g) * 8);
#pragma unroll
  for (int et = 0; et < 4; ++et) {
    const uint16_t* wrow = Wr + static_cast<size_t>(et * 16 + r16) * kHidden + kb;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[et][i] = ld16(wrow + (4 * i + g) * 8);
  }
  // Keep every load above this point: one memory round trip.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int et = 0; et < 4; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int et = 0; et < 4; ++et) acc[et] = mfma16(a[i], b[et][i], acc[et]);
  if constexpr (QUANT) quantize_slice(a, tok, real, slice, lane, Q, S);
}

// Selection for one token on one wavefront (lane = expert), from the logit
// l of the lane's expert.  Writes the token's 4 experts and weights when tg
// is a real token; returns whether the lane's expert was selected.
__device__ __forceinline__ bool select_token(float l, float b_e, int lane, int tg, int N,
                                             int32_t* __restrict__ idx_out,
                                             float* __restrict__ w_out) {
  const float s_e = 1.0f / (1.0f + expf(-l));
  const float c_e = s_e + b_e;
  const uint32_t key = orderable(c_e);
  bool taken = false;
  int sel[kTopK];
  float sel_s[kTopK];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kTopK; ++j) {
    const uint32_t m = wave_max_u32(taken ? 0u : key);
    // Equal scores: the lowest expert id among them wins.
    const unsigned long long ball = __ballot(!taken && key == m);
    const int win = __ffsll(static_cast<long long>(ball)) - 1;
    taken = taken || (lane == win);
    sel[j] = win;
    sel_s[j] = __shfl(s_e, win, kWave);
    sum += sel_s[j];
  }
  if (tg < N && lane < kTopK) {
    int e_out = sel[0];
    float s_out = sel_s[0];
#pragma unroll
    for (int j = 1; j < kTopK; ++j)
      if (lane == j) { e_out = sel[j]; s_out = sel_s[j]; }
    idx_out[static_cast<size_t>(tg) * kTopK + lane] = e_out;
    w_out[static_cast<size_t>(tg) * kTopK + lane] = s_out / (sum + kRouterEps);
  }
  return tg < N && taken;
}

// Per-tile expert histogram: counts[t][lane] holds whether token t chose the
// lane's expert; wavefront 0 adds them up after the barrier.
__device__ __forceinline__ void store_histogram(int (&counts)[kRouteTokens][kExperts], int t, int lane,
                                                bool chosen, int tile, int32_t* __restrict__ blockcounts) {
  counts[t][lane] = chosen ? 1 : 0;
  __syncthreads();
  if (t == 0) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kRouteTokens; ++w) c += counts[w][lane];
    blockcounts[static_cast<size_t>(tile) * kExperts + lane] = c;
  }
}

// part layout: [token tile][slice][16 tokens][64 experts] fp32.
template <bool QUANT>
__global__ __launch_bounds__(kWave) void route_partial_kernel(const uint16_t* __restrict__ X,
                                                              const uint16_t* __restrict__ Wr,
                                                              float* __restrict__ part, int N,
                                                              uint8_t* __restrict__ Q, float* __restrict__ S) {
  const int lane = threadIdx.x;
  f32x4 acc[4];
  slice_partial<QUANT>(X, Wr, blockIdx.x / kSlices, blockIdx.x % kSlices, N, lane, acc, Q, S);
  float* dst = part + static_cast<size_t>(blockIdx.x) * kRouteTokens * kExperts;
#pragma unroll
  for (int et = 0; et < 4; ++et)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(4 * (lane >> 4) + r) * kExperts + et * 16 + (lane & 15)] = acc[et][r];
}

__global__ __launch_bounds__(kSelectThreads) void route_select_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, int32_t* __restrict__ blockcounts, int N) {
  __shared__ int counts[kRouteTokens][kExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int t = threadIdx.x / kWave;  // token of this wavefront within the tile
  const float* src = part + static_cast<size_t>(blockIdx.x) * kSlices * kRouteTokens * kExperts +
                     t * kExperts + lane;
  float p[kSlices];
#pragma unroll
  for (int s = 0; s < kSlices; ++s) p[s] = src[s * kRouteTokens * kExperts];
  float l = 0.0f;
#pragma unroll
  for (int s = 0; s < kSlices; ++s) l += p[s];
  const bool chosen = select_token(l, bias[lane], lane, blockIdx.x * kRouteTokens + t, N, idx_out, w_out);
  if (blockcounts != nullptr) store_histogram(counts, t, lane, chosen, blockIdx.x, blockcounts);
}

// Tiles blockIdx.x * tiles_per_wg ... + tiles_per_wg - 1 (those below N),
// one after the other.  Wavefront w multiplies K slice w of every tile with
// the router rows of that slice, loaded once; the partials of a tile go
// through LDS to the wavefront of each token, in slice order.
template <bool QUANT>
__global__ __launch_bounds__(kFusedThreads) void route_fused_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ blockcounts, int N,
    uint8_t* __restrict__ Q, float* __restrict__ S, int tiles_per_wg) {
  __shared__ float part[kSlices][kRouteTokens][kPartStride];
  __shared__ int counts[kRouteTokens][kExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int tiles = (N + kRouteTokens - 1) / kRouteTokens;
  uint4 b[4][4];
  slice_weights(Wr, wave, lane, b);
  for (int k = 0; k < tiles_per_wg; ++k) {
    const int tile = blockIdx.x * tiles_per_wg + k;
    if (tile >= tiles) break;  // the same in every wavefront
    {
      int tok = tile * kRouteTokens + (lane & 15);
      const bool real = tok < N;
      tok = real ? tok : N - 1;  // rows past N are computed and discarded
      uint4 a[4];
      f32x4 acc[4];
      slice_product(X, b, tok, wave, lane, a, acc);
#pragma unroll
      for (int et = 0; et < 4; ++et)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wave][4 * (lane >> 4) + r][et * 16 + (lane & 15)] = acc[et][r];
      if constexpr (QUANT) quantize_slice(a, tok, real, wave, lane, Q, S);
    }
    __syncthreads();
    const int t = wave;  // now: the token of this wavefront within the tile
    float l = 0.0f;
#pragma unroll
    for (int s = 0; s < kSlices; ++s) l += part[s][t][lane];
    const bool chosen = select_token(l, bias[lane], lane, tile * kRouteTokens + t, N, idx_out, w_out);
    if (blockcounts != nullptr) store_histogram(counts, t, lane, chosen, tile, blockcounts);
    __syncthreads();  // part and counts are rewritten by the next tile
  }
}

}  // namespace

int route_block_tokens(int64_t) { return kRouteTokens; }

size_t route_partial_bytes(int64_t N) {
  if (N > kSplitMaxTokens) return 0;  // the fused router keeps its partials in LDS
  const size_t tiles = static_cast<size_t>((N + kRouteTokens - 1) / kRouteTokens);
  return tiles * kSlices * kRouteTokens * kExperts * sizeof(float);
}

hipError_t launch_route(const uint16_t* X, const uint16_t* Wr, const float* bias, int32_t* idx,
                        float* w, int32_t* blockcounts, float* part, int N, hipStream_t stream,
                        uint8_t* Xq, float* Xs) {
  const int tiles = (N + kRouteTokens - 1) / kRouteTokens;
  const bool quant = Xq != nullptr;
  if (N > kSplitMaxTokens) {
    const int per_wg = (tiles + kFusedMaxWorkgroups - 1) / kFusedMaxWorkgroups;
    const int wgs = (tiles + per_wg - 1) / per_wg;
    hipLaunchKernelGGL(quant ? route_fused_kernel<true> : route_fused_kernel<false>, dim3(wgs),
                       dim3(kFusedThreads), 0, stream, X, Wr, bias, idx, w, blockcounts, N, Xq, Xs, per_wg);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(quant ? route_partial_kernel<true> : route_partial_kernel<false>,
                     dim3(tiles * kSlices), dim3(kWave), 0, stream, X, Wr, part, N, Xq, Xs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_select_kernel, dim3(tiles), dim3(kSelectThreads), 0, stream, part, bias,
                     idx, w, blockcounts, N);
  return hipGetLastError();
}

}  // namespace lfm

// Grouped expert GEMMs for few tokens per expert (decode-shaped batches).
//
// Method: each selected expert is a gated SiLU MLP with three matrices
// (flozi.net guide "LFM2.5-24B-A2B: Biased Routing, Short Convolutions and
// Ten KV Caches", section "The router has two different scores"):
//   H = silu(X_e W_gate_e^T) * (X_e W_up_e^T)    (bf16 out, fp32 accumulate)
//   Y = H_e W_down_e^T                           (fp32 out)
//
// With a handful of tokens per expert the work is bound by reading each
// active expert's weights from HBM once.  Weights are in the packed
// fragment layout (pack.hip), so each wavefront load is one contiguous 1 KB
// non-temporal read that lands directly in the MFMA A-operand registers;
// every weight fragment is read by exactly one wavefront.  The token rows
// (B operand: few rows, shared by all workgroups of an expert) come through
// the caches.  Loads for the next K step are issued before the MFMAs of the
// current one.
//
// Workgroups walk a linear (m-tile, column block) grid; the m-tile list is
// derived on the device from the expert row offsets, and workgroups past
// the last m-tile exit at once, so no host readback is needed.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kFrag = 512;                         // bf16 elements per 16x32 fragment
constexpr int kGateUpBlocks = kFF / 64;            // 24: 4 waves x 16 H columns
constexpr int kDownBlocks = kHidden / 128;         // 16: 4 waves x 32 features
constexpr int kStepFrags = 2;                      // K fragments (of 32) per pipeline step

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming read: used once, so marked non-temporal.
__device__ __forceinline__ uint4 ld_stream(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int TT>
__global__ __launch_bounds__(kStreamThreads) void gateup_stream_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wgu,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row2tok,
    uint16_t* __restrict__ H) {
  constexpr int kSteps = (kHidden / 32) / kStepFrags;
  const int nb = blockIdx.x % kGateUpBlocks;
  const int mt = blockIdx.x / kGateUpBlocks;
  MTile tile;
  if (!map_mtile(offsets, mt, 16 * TT, tile)) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int hb = nb * 4 + wave;  // 16-column block of H
  const int ntt = __builtin_amdgcn_readfirstlane((tile.rows + 15) / 16);

  const uint16_t* wg =
      Wgu + (static_cast<size_t>(tile.expert) * (kFF / 16) + hb) * 2 * (kHidden / 32) * kFrag +
      lane * 8;
  const uint16_t* wu = wg + (kHidden / 32) * kFrag;
  const uint16_t* xr[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int r = tt * 16 + r16;
    const int tok = row2tok[tile.row_begin + (r < tile.rows ? r : 0)];
    xr[tt] = X + static_cast<size_t>(tok) * kHidden + g * 8;
  }

  f32x4 accg[TT], accu[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) { accg[tt] = f32x4{0, 0, 0, 0}; accu[tt] = accg[tt]; }

  uint4 cg[kStepFrags], cu[kStepFrags], cx[TT][kStepFrags];
  auto load = [&](int s, uint4 (&ag)[kStepFrags], uint4 (&au)[kStepFrags],
                  uint4 (&bx)[TT][kStepFrags]) {
#pragma unroll
    for (int f = 0; f < kStepFrags; ++f) {
      const int kf = s * kStepFrags + f;
      ag[f] = ld_stream(wg + kf * kFrag);
      au[f] = ld_stream(wu + kf * kFrag);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        bx[tt][f] = (tt == 0 || tt < ntt) ? ld16(xr[tt] + kf * 32) : make_uint4(0, 0, 0, 0);
    }
  };
  auto compute = [&](const uint4 (&ag)[kStepFrags], const uint4 (&au)[kStepFrags],
                     const uint4 (&bx)[TT][kStepFrags]) {
#pragma unroll
    for (int f = 0; f < kStepFrags; ++f)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        if (tt == 0 || tt < ntt) {
          accg[tt] = mfma16(ag[f], bx[tt][f], accg[tt]);
          accu[tt] = mfma16(au[f], bx[tt][f], accu[tt]);
        }
  };

  load(0, cg, cu, cx);
  for (int s = 0; s < kSteps - 1; ++s) {
    uint4 ng[kStepFrags], nu[kStepFrags], nx[TT][kStepFrags];
    load(s + 1, ng, nu, nx);
    compute(cg, cu, cx);
#pragma unroll
    for (int f = 0; f < kStepFrags; ++f) {
      cg[f] = ng[f];
      cu[f] = nu[f];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) cx[tt][f] = nx[tt][f];
    }
  }
  compute(cg, cu, cx);

  // Lane holds token (tt*16 + r16) and H columns hb*16 + 4g + r, r = 0..3.
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int r = tt * 16 + r16;
    if (r < tile.rows) {
      uint32_t p[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float h0 = silu(accg[tt][2 * q]) * accu[tt][2 * q];
        const float h1 = silu(accg[tt][2 * q + 1]) * accu[tt][2 * q + 1];
        p[q] = static_cast<uint32_t>(f32_to_bf16(h0)) | (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
      }
      uint16_t* dst = H + static_cast<size_t>(tile.row_begin + r) * kFF + hb * 16 + 4 * g;
      *reinterpret_cast<uint2*>(dst) = make_uint2(p[0], p[1]);
    }
  }
}

template <int TT>
__global__ __launch_bounds__(kStreamThreads) void down_stream_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,
    const int32_t* __restrict__ offsets, float* __restrict__ Y) {
  constexpr int kSteps = (kFF / 32) / kStepFrags;
  const int nb = blockIdx.x % kDownBlocks;
  const int mt = blockIdx.x / kDownBlocks;
  MTile tile;
  if (!map_mtile(offsets, mt, 16 * TT, tile)) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int rt0 = nb * 8 + wave * 2;  // two 16-row tiles of output features
  const int ntt = __builtin_amdgcn_readfirstlane((tile.rows + 15) / 16);

  const uint16_t* wr[2];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
    wr[ft] = Wd + (static_cast<size_t>(tile.expert) * (kHidden / 16) + rt0 + ft) * (kFF / 32) * kFrag +
             lane * 8;
  const uint16_t* hr[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int r = tt * 16 + r16;
    hr[tt] = H + static_cast<size_t>(tile.row_begin + (r < tile.rows ? r : 0)) * kFF + g * 8;
  }

  f32x4 acc[2][TT];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[ft][tt] = f32x4{0, 0, 0, 0};

  uint4 cw[2][kStepFrags], ch[TT][kStepFrags];
  auto load = [&](int s, uint4 (&aw)[2][kStepFrags], uint4 (&bh)[TT][kStepFrags]) {
#pragma unroll
    for (int f = 0; f < kStepFrags; ++f) {
      const int kf = s * kStepFrags + f;
#pragma unroll
      for (int ft = 0; ft < 2; ++ft) aw[ft][f] = ld_stream(wr[ft] + kf * kFrag);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        bh[tt][f] = (tt == 0 || tt < ntt) ? ld16(hr[tt] + kf * 32) : make_uint4(0, 0, 0, 0);
    }
  };
  auto compute = [&](const uint4 (&aw)[2][kStepFrags], const uint4 (&bh)[TT][kStepFrags]) {
#pragma unroll
    for (int f = 0; f < kStepFrags; ++f)
#pragma unroll
      for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          if (tt == 0 || tt < ntt) acc[ft][tt] = mfma16(aw[ft][f], bh[tt][f], acc[ft][tt]);
  };

  load(0, cw, ch);
  for (int s = 0; s < kSteps - 1; ++s) {
    uint4 nw[2][kStepFrags], nh[TT][kStepFrags];
    load(s + 1, nw, nh);
    compute(cw, ch);
#pragma unroll
    for (int f = 0; f < kStepFrags; ++f) {
#pragma unroll
      for (int ft = 0; ft < 2; ++ft) cw[ft][f] = nw[ft][f];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) ch[tt][f] = nh[tt][f];
    }
  }
  compute(cw, ch);

  // Lane holds token (tt*16 + r16) and features (rt0 + ft)*16 + 4g + r.
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int r = tt * 16 + r16;
    if (r < tile.rows) {
      float* dst = Y + static_cast<size_t>(tile.row_begin + r) * kHidden + rt0 * 16 + 4 * g;
#pragma unroll
      for (int ft = 0; ft < 2; ++ft)
        *reinterpret_cast<float4*>(dst + ft * 16) =
            make_float4(acc[ft][tt][0], acc[ft][tt][1], acc[ft][tt][2], acc[ft][tt][3]);
    }
  }
}

}  // namespace

int64_t max_mtiles(int64_t N, int tile_rows) {
  const int64_t rows = N * kTopK;
  const int64_t a = (rows + static_cast<int64_t>(kExperts) * (tile_rows - 1)) / tile_rows;
  const int64_t b = static_cast<int64_t>(kExperts) * ((N + tile_rows - 1) / tile_rows);
  return a < b ? a : b;
}

hipError_t launch_gateup_stream(const uint16_t* X, const uint16_t* Wgu, const int32_t* offsets,
                                const int32_t* row2tok, uint16_t* H, int64_t N, int tile_rows,
                                hipStream_t stream) {
  const int64_t grid = max_mtiles(N, tile_rows) * kGateUpBlocks;
  if (tile_rows == 16)
    hipLaunchKernelGGL(gateup_stream_kernel<1>, dim3(grid), dim3(kStreamThreads), 0, stream, X,
                       Wgu, offsets, row2tok, H);
  else
    hipLaunchKernelGGL(gateup_stream_kernel<2>, dim3(grid), dim3(kStreamThreads), 0, stream, X,
                       Wgu, offsets, row2tok, H);
  return hipGetLastError();
}

hipError_t launch_down_stream(const uint16_t* H, const uint16_t* Wd, const int32_t* offsets,
                              float* Y, int64_t N, int tile_rows, hipStream_t stream) {
  const int64_t grid = max_mtiles(N, tile_rows) * kDownBlocks;
  if (tile_rows == 16)
    hipLaunchKernelGGL(down_stream_kernel<1>, dim3(grid), dim3(kStreamThreads), 0, stream, H, Wd,
                       offsets, Y);
  else
    hipLaunchKernelGGL(down_stream_kernel<2>, dim3(grid), dim3(kStreamThreads), 0, stream, H, Wd,
                       offsets, Y);
  return hipGetLastError();
}

}  // namespace lfm

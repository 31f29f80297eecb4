// Grouped expert GEMMs for few tokens per expert (decode-shaped batches).
//
// Method: each selected expert is a gated SiLU MLP with three matrices
// (flozi.net guide "LFM2.5-24B-A2B: Biased Routing, Short Convolutions and
// Ten KV Caches", section "The router has two different scores"):
//   H = silu(X_e W_gate_e^T) * (X_e W_up_e^T)    (bf16 out, fp32 accumulate)
//   Y = H_e W_down_e^T                           (fp32 out)
//
// With a handful of tokens per expert the work is bound by streaming each
// active expert's weights from HBM exactly once.  Weights therefore go
// straight from global memory into MFMA operand registers (no LDS), each
// weight row is read by exactly one wavefront, the loads for the next
// 128-wide K step are issued before the MFMAs of the current one, and the
// token rows (few, shared by every workgroup of the expert) come through
// the caches.  The weight rows are the MFMA A operand (16 rows) and the
// tokens the B operand (16 columns); the K dimension inside a 128-wide step
// is visited in an order that lets every lane read 16 contiguous bytes per
// load (the same order on both operands, so the dot products are
// unchanged).
//
// Workgroups walk a linear (m-tile, column block) grid; the m-tile list is
// derived on the device from the expert row offsets, and workgroups past
// the last m-tile exit at once, so no host readback is needed.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kGateUpCols = 64;                    // H columns per workgroup (16 per wave)
constexpr int kGateUpBlocks = kFF / kGateUpCols;   // 24
constexpr int kDownRowsPerWave = 32;               // output features per wave
constexpr int kDownCols = 4 * kDownRowsPerWave;    // 128 per workgroup
constexpr int kDownBlocks = kHidden / kDownCols;   // 16

// Loads the 16-byte pieces a lane needs for one 128-wide K step of a row.
__device__ __forceinline__ void load_step(const uint16_t* row, int kb, int g, uint4 (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ld16(row + kb + (4 * i + g) * 8);
}

template <int TT>
__global__ __launch_bounds__(kStreamThreads) void gateup_stream_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wgu,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row2tok,
    uint16_t* __restrict__ H) {
  const int nb = blockIdx.x % kGateUpBlocks;
  const int mt = blockIdx.x / kGateUpBlocks;
  MTile tile;
  if (!map_mtile(offsets, mt, 16 * TT, tile)) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int n = nb * kGateUpCols + wave * 16;  // first H column of this wave

  const uint16_t* wg = Wgu + (static_cast<size_t>(tile.expert) * 2 * kFF + n + r16) * kHidden;
  const uint16_t* wu = wg + static_cast<size_t>(kFF) * kHidden;
  const uint16_t* xr[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int r = tt * 16 + r16;
    const int tok = row2tok[tile.row_begin + (r < tile.rows ? r : 0)];
    xr[tt] = X + static_cast<size_t>(tok) * kHidden;
  }

  f32x4 accg[TT], accu[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) { accg[tt] = f32x4{0, 0, 0, 0}; accu[tt] = accg[tt]; }

  uint4 cg[4], cu[4], cx[TT][4];
  load_step(wg, 0, g, cg);
  load_step(wu, 0, g, cu);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) load_step(xr[tt], 0, g, cx[tt]);

  for (int kb = 0; kb < kHidden; kb += 128) {
    uint4 ng[4], nu[4], nx[TT][4];
    const int kn = kb + 128 < kHidden ? kb + 128 : kb;  // last step reloads (cached) data
    load_step(wg, kn, g, ng);
    load_step(wu, kn, g, nu);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) load_step(xr[tt], kn, g, nx[tt]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        accg[tt] = mfma16(cg[i], cx[tt][i], accg[tt]);
        accu[tt] = mfma16(cu[i], cx[tt][i], accu[tt]);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cg[i] = ng[i];
      cu[i] = nu[i];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) cx[tt][i] = nx[tt][i];
    }
  }

  // Lane holds token (tt*16 + r16) and H columns n + 4g + r, r = 0..3.
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
      uint16_t* dst = H + static_cast<size_t>(tile.row_begin + r) * kFF + n + 4 * g;
      *reinterpret_cast<uint2*>(dst) = make_uint2(p[0], p[1]);
    }
  }
}

template <int TT>
__global__ __launch_bounds__(kStreamThreads) void down_stream_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,
    const int32_t* __restrict__ offsets, float* __restrict__ Y) {
  const int nb = blockIdx.x % kDownBlocks;
  const int mt = blockIdx.x / kDownBlocks;
  MTile tile;
  if (!map_mtile(offsets, mt, 16 * TT, tile)) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int f0 = nb * kDownCols + wave * kDownRowsPerWave;  // first output feature

  const uint16_t* wr[2];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
    wr[ft] = Wd + (static_cast<size_t>(tile.expert) * kHidden + f0 + ft * 16 + r16) * kFF;
  const uint16_t* hr[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int r = tt * 16 + r16;
    hr[tt] = H + static_cast<size_t>(tile.row_begin + (r < tile.rows ? r : 0)) * kFF;
  }

  f32x4 acc[2][TT];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[ft][tt] = f32x4{0, 0, 0, 0};

  uint4 cw[2][4], ch[TT][4];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft) load_step(wr[ft], 0, g, cw[ft]);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) load_step(hr[tt], 0, g, ch[tt]);

  for (int kb = 0; kb < kFF; kb += 128) {
    uint4 nw[2][4], nh[TT][4];
    const int kn = kb + 128 < kFF ? kb + 128 : kb;
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) load_step(wr[ft], kn, g, nw[ft]);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) load_step(hr[tt], kn, g, nh[tt]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[ft][tt] = mfma16(cw[ft][i], ch[tt][i], acc[ft][tt]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int ft = 0; ft < 2; ++ft) cw[ft][i] = nw[ft][i];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) ch[tt][i] = nh[tt][i];
    }
  }

  // Lane holds token (tt*16 + r16) and features f0 + ft*16 + 4g + r.
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int r = tt * 16 + r16;
    if (r < tile.rows) {
      float* dst = Y + static_cast<size_t>(tile.row_begin + r) * kHidden + f0 + 4 * g;
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

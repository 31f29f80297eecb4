// Grouped expert GEMMs for many tokens per expert (prefill-shaped batches):
// LDS-tiled bf16 MFMA kernels over the expert-grouped rows of the dispatch
// step.
//
// Method: each selected expert is a gated SiLU MLP with three matrices
// (flozi.net guide "LFM2.5-24B-A2B: Biased Routing, Short Convolutions and
// Ten KV Caches", section "The router has two different scores"):
//   H = silu(X_e W_gate_e^T) * (X_e W_up_e^T)    (bf16 out, fp32 accumulate)
//   Y = H_e W_down_e^T                           (fp32 out)
// over the tokens grouped by expert (section "What to verify in a
// deployment").
//
// Tile: 128 grouped rows (tokens of one expert) x 128 weight rows, K step
// 64, double-buffered in LDS (2 x 32 KB, so two workgroups share a CU).
// Four wavefronts in a 2 x 2 arrangement each own 64 rows x 64 weight rows
// (4 x 4 tiles of the 16x16x32 MFMA).  For gate/up the 128 weight rows are
// 64 gate rows and the 64 matching up rows, so the SiLU product happens in
// registers; for down they are 128 output features.
//
// Both operands sit in LDS in MFMA-fragment order (1 KB per 16 x 32
// fragment, lane-major), so every LDS read and write by a wavefront is one
// contiguous, conflict-free 1 KB access.  The packed weights are already in
// that order (16 KB contiguous per K step and workgroup); token rows are
// gathered from their slot (X row t for gate/up, H row t*4 + j for down)
// straight into fragment positions.
//
// Grid: m-tile major, column block minor.  The 24 (gate/up) or 16 (down)
// workgroups of an m-tile are adjacent and share its token rows through L2;
// workgroups of one column block recur every 24 / 16 ids, which keeps them
// on one XCD (ids are dealt to the 8 XCDs round-robin) where they share the
// expert's weight block in L2.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kTileThreads = 256;
constexpr int kBM = 128;                 // grouped rows per tile
constexpr int kBK = 64;                  // K per stage (two 32-wide fragments)
constexpr int kFragU4 = 64;              // uint4 per 1 KB fragment
constexpr int kStageU4 = 2 * 1024;       // A (8 x 2 fragments) + B (2 x 8 fragments)

template <bool GATEUP>
__global__ __launch_bounds__(kTileThreads) void expert_tiled_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Wp,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row2slot,
    uint16_t* __restrict__ H, float* __restrict__ Y) {
  constexpr int K = GATEUP ? kHidden : kFF;
  constexpr int kBlocks = GATEUP ? kFF / 64 : kHidden / 128;  // column blocks
  constexpr int kStages = K / kBK;
  __shared__ uint4 lds[2][kStageU4];

  MTile tile;
  if (!map_mtile(offsets, blockIdx.x / kBlocks, kBM, tile)) return;
  const int nb = blockIdx.x % kBlocks;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int wm = wave >> 1;  // 64-row half of the tile
  const int wn = wave & 1;   // 64-row half of the weight block

  // Global -> register staging.  Token operand: load u of this thread is
  // fragment (tt = (wave + 4u) / 2, kf = wave % 2), lane position `lane`,
  // i.e. row tt*16 + r16, K offset kf*32 + 8g of the stage.
  const uint16_t* arow[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = ((wave + 4 * u) >> 1) * 16 + r16;
    const int slot = row2slot[tile.row_begin + (row < tile.rows ? row : 0)];
    const int src = GATEUP ? slot / kTopK : slot;
    arow[u] = A + static_cast<size_t>(src) * K + (wave & 1) * 32 + g * 8;
  }
  // Weight operand: the stage's 16 fragments are 16 KB contiguous.
  const uint16_t* wblk =
      Wp + static_cast<size_t>(tile.expert * kBlocks + nb) * (K / 32) * 8 * 512 + tid * 8;

  uint4 ra[4], rb[4];
  auto load_stage = [&](int s) {
#pragma unroll
    for (int u = 0; u < 4; ++u) ra[u] = ld16(arow[u] + s * kBK);
#pragma unroll
    for (int u = 0; u < 4; ++u) rb[u] = ld16(wblk + (static_cast<size_t>(s) * 1024 + u * 256) * 8);
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) lds[buf][(wave + 4 * u) * kFragU4 + lane] = ra[u];
#pragma unroll
    for (int u = 0; u < 4; ++u) lds[buf][1024 + u * 256 + tid] = rb[u];
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int s = 0; s < kStages; ++s) {
    const int buf = s & 1;
    if (s + 1 < kStages) load_stage(s + 1);
#pragma unroll
    for (int kf = 0; kf < 2; ++kf) {
      uint4 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = lds[buf][((wm * 4 + i) * 2 + kf) * kFragU4 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = lds[buf][1024 + (kf * 8 + wn * 4 + j) * kFragU4 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(fb[j], fa[i], acc[i][j]);
    }
    if (s + 1 < kStages) store_stage(buf ^ 1);
    __syncthreads();
  }

  // Lane holds token row (wm*4 + i)*16 + r16 of the tile and rows 4g + r of
  // weight fragment j.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wm * 4 + i) * 16 + r16;
    if (row >= tile.rows) continue;
    const int slot = row2slot[tile.row_begin + row];
    if (GATEUP) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {  // fragments (gate, up) of column block wn*2 + c
        const f32x4 gt = acc[i][2 * c], up = acc[i][2 * c + 1];
        const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(silu(gt[0]) * up[0])) |
                            (static_cast<uint32_t>(f32_to_bf16(silu(gt[1]) * up[1])) << 16);
        const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(silu(gt[2]) * up[2])) |
                            (static_cast<uint32_t>(f32_to_bf16(silu(gt[3]) * up[3])) << 16);
        uint16_t* dst = H + static_cast<size_t>(slot) * kFF + nb * 64 + (wn * 2 + c) * 16 + 4 * g;
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
      }
    } else {
      float* dst = Y + static_cast<size_t>(slot) * kHidden + nb * 128 + wn * 64 + 4 * g;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(dst + j * 16) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
  }
}

}  // namespace

hipError_t launch_gateup_tiled(const uint16_t* X, const uint16_t* Wgu, const int32_t* offsets,
                               const int32_t* row2slot, uint16_t* H, int64_t N,
                               hipStream_t stream) {
  const int64_t grid = max_mtiles(N, kBM) * (kFF / 64);
  hipLaunchKernelGGL(expert_tiled_kernel<true>, dim3(grid), dim3(kTileThreads), 0, stream, X, Wgu,
                     offsets, row2slot, H, nullptr);
  return hipGetLastError();
}

hipError_t launch_down_tiled(const uint16_t* H, const uint16_t* Wd, const int32_t* offsets,
                             const int32_t* row2slot, float* Y, int64_t N, hipStream_t stream) {
  const int64_t grid = max_mtiles(N, kBM) * (kHidden / 128);
  hipLaunchKernelGGL(expert_tiled_kernel<false>, dim3(grid), dim3(kTileThreads), 0, stream, H, Wd,
                     offsets, row2slot, nullptr, Y);
  return hipGetLastError();
}

}  // namespace lfm

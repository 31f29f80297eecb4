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
constexpr bool kWideTiles = false;       // 128 x 256 tiles (expert_tiled_wide_kernel)

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

  // Two register sets: the global loads of stage s + 2 are in flight while
  // stage s is multiplied and stage s + 1 goes from registers into LDS.
  uint4 ra[2][4], rb[2][4];
  auto load_stage = [&](int s, int set) {
#pragma unroll
    for (int u = 0; u < 4; ++u) ra[set][u] = ld16(arow[u] + s * kBK);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      rb[set][u] = ld16(wblk + (static_cast<size_t>(s) * 1024 + u * 256) * 8);
  };
  auto store_stage = [&](int buf, int set) {
#pragma unroll
    for (int u = 0; u < 4; ++u) lds[buf][(wave + 4 * u) * kFragU4 + lane] = ra[set][u];
#pragma unroll
    for (int u = 0; u < 4; ++u) lds[buf][1024 + u * 256 + tid] = rb[set][u];
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  auto compute = [&](int buf) {
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
  };

  static_assert(kStages % 2 == 0 && kStages >= 4, "pipeline assumes an even stage count");
  load_stage(0, 0);
  load_stage(1, 1);
  store_stage(0, 0);
  __syncthreads();
  // Iteration s: loads of s + 2 into set s % 2, compute s, stage s + 1 (set
  // (s + 1) % 2) into LDS.  Unrolled by two so the register sets are static.
  for (int s = 0; s < kStages; s += 2) {
    if (s + 2 < kStages) load_stage(s + 2, 0);
    compute(0);
    store_stage(1, 1);
    __syncthreads();
    if (s + 3 < kStages) load_stage(s + 3, 1);
    compute(1);
    if (s + 2 < kStages) store_stage(0, 0);
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

// Wide variant: 128 rows x 256 weight rows per workgroup (two column
// blocks), one column block per wavefront column, so each wavefront owns
// 64 rows x 128 weight rows (4 x 8 MFMA tiles, 128 accumulator registers).
// Per 32-wide K step a wavefront reads 12 fragments from LDS for 32 MFMAs
// (0.375 KB per MFMA instead of 0.5).  96 KB of LDS: one workgroup per CU.
template <bool GATEUP>
__global__ __launch_bounds__(kTileThreads) void expert_tiled_wide_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Wp,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row2slot,
    uint16_t* __restrict__ H, float* __restrict__ Y) {
  constexpr int K = GATEUP ? kHidden : kFF;
  constexpr int kBlocks = GATEUP ? kFF / 64 : kHidden / 128;  // column blocks
  constexpr int kPairs = kBlocks / 2;                          // workgroups per m-tile
  constexpr int kStages = K / kBK;
  constexpr int kStageWide = 3 * 1024;  // uint4: A 1024, B 2 x 1024
  __shared__ uint4 lds[2][kStageWide];

  MTile tile;
  if (!map_mtile(offsets, blockIdx.x / kPairs, kBM, tile)) return;
  const int pair = blockIdx.x % kPairs;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int wm = wave >> 1;  // 64-row half of the tile
  const int wn = wave & 1;   // column block of the pair

  const uint16_t* arow[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = ((wave + 4 * u) >> 1) * 16 + r16;
    const int slot = row2slot[tile.row_begin + (row < tile.rows ? row : 0)];
    const int src = GATEUP ? slot / kTopK : slot;
    arow[u] = A + static_cast<size_t>(src) * K + (wave & 1) * 32 + g * 8;
  }
  const uint16_t* wblk[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
    wblk[b] = Wp + static_cast<size_t>(tile.expert * kBlocks + pair * 2 + b) * (K / 32) * 8 * 512 +
              tid * 8;

  uint4 ra[2][4], rb[2][8];
  auto load_stage = [&](int s, int set) {
#pragma unroll
    for (int u = 0; u < 4; ++u) ra[set][u] = ld16(arow[u] + s * kBK);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        rb[set][b * 4 + u] = ld16(wblk[b] + (static_cast<size_t>(s) * 1024 + u * 256) * 8);
  };
  auto store_stage = [&](int buf, int set) {
#pragma unroll
    for (int u = 0; u < 4; ++u) lds[buf][(wave + 4 * u) * kFragU4 + lane] = ra[set][u];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int u = 0; u < 4; ++u) lds[buf][1024 + b * 1024 + u * 256 + tid] = rb[set][b * 4 + u];
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  auto compute = [&](int buf) {
#pragma unroll
    for (int kf = 0; kf < 2; ++kf) {
      uint4 fa[4], fb[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = lds[buf][((wm * 4 + i) * 2 + kf) * kFragU4 + lane];
#pragma unroll
      for (int j = 0; j < 8; ++j) fb[j] = lds[buf][1024 + wn * 1024 + (kf * 8 + j) * kFragU4 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(fb[j], fa[i], acc[i][j]);
    }
  };

  static_assert(kStages % 2 == 0 && kStages >= 4, "pipeline assumes an even stage count");
  load_stage(0, 0);
  load_stage(1, 1);
  store_stage(0, 0);
  __syncthreads();
  for (int s = 0; s < kStages; s += 2) {
    if (s + 2 < kStages) load_stage(s + 2, 0);
    compute(0);
    store_stage(1, 1);
    __syncthreads();
    if (s + 3 < kStages) load_stage(s + 3, 1);
    compute(1);
    if (s + 2 < kStages) store_stage(0, 0);
    __syncthreads();
  }

  const int blk = pair * 2 + wn;  // this wavefront's column block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wm * 4 + i) * 16 + r16;
    if (row >= tile.rows) continue;
    const int slot = row2slot[tile.row_begin + row];
    if (GATEUP) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {  // fragments (gate, up) of 16-column group cb
        const f32x4 gt = acc[i][2 * cb], up = acc[i][2 * cb + 1];
        const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(silu(gt[0]) * up[0])) |
                            (static_cast<uint32_t>(f32_to_bf16(silu(gt[1]) * up[1])) << 16);
        const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(silu(gt[2]) * up[2])) |
                            (static_cast<uint32_t>(f32_to_bf16(silu(gt[3]) * up[3])) << 16);
        uint16_t* dst = H + static_cast<size_t>(slot) * kFF + blk * 64 + cb * 16 + 4 * g;
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
      }
    } else {
      float* dst = Y + static_cast<size_t>(slot) * kHidden + blk * 128 + 4 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<float4*>(dst + j * 16) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
  }
}

}  // namespace

hipError_t launch_gateup_tiled(const uint16_t* X, const uint16_t* Wgu, const int32_t* offsets,
                               const int32_t* row2slot, uint16_t* H, int64_t N,
                               hipStream_t stream) {
  if (kWideTiles) {
    const int64_t grid = max_mtiles(N, kBM) * (kFF / 128);
    hipLaunchKernelGGL(expert_tiled_wide_kernel<true>, dim3(grid), dim3(kTileThreads), 0, stream,
                       X, Wgu, offsets, row2slot, H, nullptr);
  } else {
    const int64_t grid = max_mtiles(N, kBM) * (kFF / 64);
    hipLaunchKernelGGL(expert_tiled_kernel<true>, dim3(grid), dim3(kTileThreads), 0, stream, X,
                       Wgu, offsets, row2slot, H, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_down_tiled(const uint16_t* H, const uint16_t* Wd, const int32_t* offsets,
                             const int32_t* row2slot, float* Y, int64_t N, hipStream_t stream) {
  if (kWideTiles) {
    const int64_t grid = max_mtiles(N, kBM) * (kHidden / 256);
    hipLaunchKernelGGL(expert_tiled_wide_kernel<false>, dim3(grid), dim3(kTileThreads), 0, stream,
                       H, Wd, offsets, row2slot, nullptr, Y);
  } else {
    const int64_t grid = max_mtiles(N, kBM) * (kHidden / 128);
    hipLaunchKernelGGL(expert_tiled_kernel<false>, dim3(grid), dim3(kTileThreads), 0, stream, H,
                       Wd, offsets, row2slot, nullptr, Y);
  }
  return hipGetLastError();
}

}  // namespace lfm

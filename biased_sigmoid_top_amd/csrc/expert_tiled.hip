// Grouped expert GEMMs for many tokens per expert (prefill-shaped batches),
// over the expert-grouped rows of the dispatch step.
//
// Method: each selected expert is a gated SiLU MLP with three matrices
// (flozi.net guide "LFM2.5-24B-A2B: Biased Routing, Short Convolutions and
// Ten KV Caches", section "The router has two different scores"):
//   H = silu(X_e W_gate_e^T) * (X_e W_up_e^T)    (bf16 out, fp32 accumulate)
//   Y = H_e W_down_e^T                           (fp32 out)
// over the tokens grouped by expert (section "What to verify in a
// deployment").
//
// Tile: 128 grouped rows (tokens of one expert) x 256 weight rows, 32x32x16
// bf16 MFMAs (on gfx950 twice the rate of the 16x16x32 form).  Each of the
// four wavefronts owns 64 weight rows (two packed row blocks) for all 128
// tokens: 4 x 2 accumulator tiles.  Because no two wavefronts share weight
// rows, the weights need no LDS: every wavefront streams its own packed
// fragments (one contiguous 1 KB load each) straight into its MFMA
// registers, three K stages ahead.  The token rows, which all four
// wavefronts share, are gathered from their slots (X row t for gate/up, H
// row t*4 + j for down) two stages ahead into registers and stored into a
// double-buffered LDS tile in fragment order, so every LDS access is a
// contiguous, conflict-free 1 KB wavefront access.  Two workgroups share a
// CU.  For gate/up the 32 rows of a packed block are 16 gate rows and the
// matching 16 up rows, so the SiLU product is formed in registers.
//
// Grid: m-tile major, 16 (gate/up, 12 used) or 8 (down) column slots per
// m-tile.  Workgroup ids are dealt to the 8 XCDs round-robin, so the
// m-tiles of one expert that use the same weight block sit on one XCD and
// start together, and share the block through that XCD's L2.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kTileThreads = 256;
constexpr int kBM = 128;                  // grouped rows per tile
constexpr int kBlocksPerTile = 8;         // packed 32-row blocks per tile (256 weight rows)
constexpr int kKS = 2;                    // 16-wide K steps per stage
constexpr int kBK = 16 * kKS;             // K per stage
constexpr int kWSlots = 4;                // weight register ring: three stages ahead
constexpr int kChunks = kBM * (kBK / 8) / kTileThreads;  // 16-byte token pieces per thread per stage

template <bool GATEUP>
struct TileShape {
  static constexpr int K = GATEUP ? kHidden : kFF;
  static constexpr int kSteps = GATEUP ? kGateupSteps : kDownSteps;
  static constexpr int kBlocks = GATEUP ? kGateupBlocks : kDownBlocks;
  static constexpr int kColTiles = kBlocks / kBlocksPerTile;  // 12 or 8
  static constexpr int kColSlots = GATEUP ? 16 : 8;           // multiple of the XCD count
  static constexpr int kStages = K / kBK;
};

template <bool GATEUP>
__global__ __launch_bounds__(kTileThreads, 2) void expert_tiled_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Wp,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row2slot,
    uint16_t* __restrict__ H, float* __restrict__ Y) {
  using T = TileShape<GATEUP>;
  static_assert(T::kStages % kWSlots == 0, "the stage loop is unrolled by the ring size");
  __shared__ uint4 tok[2][4 * kKS][kWave];  // 2 stages x (4 token blocks x kKS steps) fragments

  const int nb = blockIdx.x % T::kColSlots;
  if (nb >= T::kColTiles) return;
  MTile tile;
  if (!map_mtile(offsets, blockIdx.x / T::kColSlots, kBM, tile)) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  // Token pieces of this thread: piece q = tid + 256 i is row q / 4, 16-byte
  // chunk q % 4 of the stage's 64 bytes; in LDS it is lane (c % 2) * 32 +
  // row % 32 of fragment (row / 32, c / 2).
  const uint16_t* arow[kChunks];
  int lds_f[kChunks], lds_l[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int q = tid + kTileThreads * i, r = q / 4, c = q % 4;
    const int slot = row2slot[tile.row_begin + (r < tile.rows ? r : 0)];
    arow[i] = A + static_cast<size_t>(GATEUP ? slot / kTopK : slot) * T::K + c * 8;
    lds_f[i] = (r / 32) * kKS + c / 2;
    lds_l[i] = (c % 2) * 32 + r % 32;
  }
  // This wavefront's two packed row blocks; K steps of a block are contiguous.
  const uint16_t* wblk = Wp + (static_cast<size_t>(tile.expert) * T::kBlocks + nb * kBlocksPerTile +
                               wave * 2) * T::kSteps * (kFragBytes / 2) + lane * 8;
  constexpr size_t kBlockElems = static_cast<size_t>(T::kSteps) * (kFragBytes / 2);

  uint4 wring[kWSlots][2][kKS];
  // Stages past the end reload the last stage (in bounds, never used).
  auto load_w = [&](int s, uint4 (&w)[2][kKS]) {
    const int sc = s < T::kStages ? s : T::kStages - 1;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int j = 0; j < kKS; ++j)
        w[f][j] = ld16(wblk + f * kBlockElems + static_cast<size_t>(sc * kKS + j) * (kFragBytes / 2));
  };
  uint4 stg[2][kChunks];
  auto load_x = [&](int s, uint4 (&g)[kChunks]) {
    const int sc = s < T::kStages ? s : T::kStages - 1;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) g[i] = ld16(arow[i] + sc * kBK);
  };
  auto store_x = [&](int buf, const uint4 (&g)[kChunks]) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) tok[buf][lds_f[i]][lds_l[i]] = g[i];
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tb][f][r] = 0.f;

#pragma unroll
  for (int s = 0; s < kWSlots - 1; ++s) load_w(s, wring[s]);
  {
    uint4 g0[kChunks];
    load_x(0, g0);
    store_x(0, g0);
  }
  load_x(1, stg[0]);
  load_x(2, stg[1]);
  __syncthreads();

  // Stage s: multiplies LDS buffer s % 2 with ring slot s % 4, loads the
  // weights of stage s + 3 into the free slot, stores the tokens of stage
  // s + 1 (loaded two stages ago, in g) into the other buffer and loads
  // those of stage s + 3 into g.
  auto stage = [&](int s, int buf, uint4 (&wc)[2][kKS], uint4 (&wn)[2][kKS], uint4 (&g)[kChunks]) {
    load_w(s + kWSlots - 1, wn);
#pragma unroll
    for (int j = 0; j < kKS; ++j) {
      uint4 t[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) t[tb] = tok[buf][tb * kKS + j][lane];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int f = 0; f < 2; ++f) acc[tb][f] = mfma32(wc[f][j], t[tb], acc[tb][f]);
    }
    store_x(buf ^ 1, g);
    load_x(s + 3, g);
    __syncthreads();
  };
  for (int s = 0; s < T::kStages; s += kWSlots) {
#pragma unroll
    for (int q = 0; q < kWSlots; ++q)
      stage(s + q, q % 2, wring[q], wring[(q + kWSlots - 1) % kWSlots], stg[q % 2]);
  }

  // acc[tb][f]: token row tb*32 + lane % 32 of the tile; rows
  // mfma32_row(r, lane) of packed block nb*8 + wave*2 + f.
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int row = tb * 32 + lane % 32;
    if (row >= tile.rows) continue;
    const int slot = row2slot[tile.row_begin + row];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int blk = nb * kBlocksPerTile + wave * 2 + f;
      if (GATEUP) {
        // Values r < 8 are gate rows, r + 8 the up rows of the same H column.
        uint16_t* dst = H + static_cast<size_t>(slot) * kFF + blk * 16 + 4 * (lane / 32);
#pragma unroll
        for (int g8 = 0; g8 < 2; ++g8) {
          uint32_t p[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int r = g8 * 4 + h * 2;
            p[h] = static_cast<uint32_t>(f32_to_bf16(silu(acc[tb][f][r]) * acc[tb][f][r + 8])) |
                   (static_cast<uint32_t>(f32_to_bf16(silu(acc[tb][f][r + 1]) * acc[tb][f][r + 9])) << 16);
          }
          *reinterpret_cast<uint2*>(dst + g8 * 8) = make_uint2(p[0], p[1]);
        }
      } else {
        float* dst = Y + static_cast<size_t>(slot) * kHidden + blk * 32 + 4 * (lane / 32);
#pragma unroll
        for (int g8 = 0; g8 < 4; ++g8)
          *reinterpret_cast<float4*>(dst + g8 * 8) =
              make_float4(acc[tb][f][g8 * 4], acc[tb][f][g8 * 4 + 1], acc[tb][f][g8 * 4 + 2],
                          acc[tb][f][g8 * 4 + 3]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gateup_tiled(const uint16_t* X, const uint16_t* Wgu, const int32_t* offsets,
                               const int32_t* row2slot, uint16_t* H, int64_t N,
                               hipStream_t stream) {
  const int64_t grid = max_mtiles(N, kBM) * TileShape<true>::kColSlots;
  hipLaunchKernelGGL(expert_tiled_kernel<true>, dim3(grid), dim3(kTileThreads), 0, stream, X, Wgu,
                     offsets, row2slot, H, nullptr);
  return hipGetLastError();
}

hipError_t launch_down_tiled(const uint16_t* H, const uint16_t* Wd, const int32_t* offsets,
                             const int32_t* row2slot, float* Y, int64_t N, hipStream_t stream) {
  const int64_t grid = max_mtiles(N, kBM) * TileShape<false>::kColSlots;
  hipLaunchKernelGGL(expert_tiled_kernel<false>, dim3(grid), dim3(kTileThreads), 0, stream, H, Wd,
                     offsets, row2slot, nullptr, Y);
  return hipGetLastError();
}

}  // namespace lfm

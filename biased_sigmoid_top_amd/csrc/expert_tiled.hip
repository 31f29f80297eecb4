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
// Tile: 128 grouped rows (tokens of one expert) x 64 weight rows per
// wavefront, 32x32x16 bf16 MFMAs (on gfx950 twice the rate of the 16x16x32
// form).  Gate/up runs 8 wavefronts per workgroup (512 weight rows), one
// workgroup per CU; down runs 4 (256 rows), two per CU, or 8 (256 or 512
// rows) depending on the batch size (see the shape selection).  Each wavefront
// owns 64 weight rows (two packed row blocks) for all 128 tokens: 4 x 2
// accumulator tiles.  Because no two wavefronts share weight rows, the
// weights need no LDS: every wavefront streams its own packed fragments
// (one contiguous 1 KB buffer load each) straight into its MFMA registers,
// three K stages ahead.  The token rows, which all wavefronts share, are
// gathered from their slots (X row t for gate/up, H row t*4 + j for down)
// as whole 128-byte lines, one per row per pair of K stages, so that no L2
// request carries half a line.  They are stored into a double-buffered,
// XOR-swizzled LDS tile (one barrier per stage pair), and the MFMA operands
// of each K step are read from it one step ahead.  The more wavefronts
// share a token tile, the fewer bytes a CU pulls through its L1 per MFMA,
// which is what bounds these kernels.  For gate/up the 32 rows of a packed
// block are 16 gate rows and the matching 16 up rows, so the SiLU product
// is formed in registers.
//
// FP8 mode (the FP8 layer above 256 tokens): the weights are the FP8 codes
// of pack_fp8.hip, one 1 KB fragment per 32-row block and K stage, widened
// to bf16 in registers before each MFMA; the token rows are the bf16 values
// of their E4M3 codes (quant.hip).  Each 128-wide K group -- one pass of the
// four-stage loop -- adds its products of codes (exact, summed in fp32)
// times weight block scale x the token row's scale, as the block-scaled
// format defines, through one accumulator set kept in units of the current
// group's scale product (see the kernel), so the FP8 mode takes the same
// tile shapes as the bf16 one.
//
// Grid: workgroup ids are dealt to the 8 XCDs round-robin.  Tiles are
// launched in groups of m-tiles x column tiles that hold a multiple of 8
// tiles, each XCD taking a run of consecutive (column-major) tiles of the
// group: every XCD gets the same share, and a column tile -- read by every
// m-tile of its expert -- stays on one XCD (down: 8 column tiles) or two
// (gate/up: 6 column tiles over groups of four m-tiles) and is shared
// through their L2.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kKS = 2;                    // 16-wide K steps per stage
constexpr int kBK = 16 * kKS;             // K per stage
constexpr int kWSlots = 4;                // weight register ring: three stages ahead
constexpr int kPairBytes = 2 * kBK * 2;   // token bytes per row per stage pair: one 128-byte line
constexpr int kXcds = 8;

// LDS position of a token piece: 16-byte chunk c (0..7) of row r's line for a
// stage pair goes to stage c / 4, K step (c / 2) % 2, K half c % 2 of that
// step's fragment, at fragment lane (c % 2) * 32 + (r % 32 ^ swz(c)).  The XOR
// keeps both the stores (eight chunks of one row, or of two rows, at once)
// and the MFMA operand reads (32 rows of one K half) free of bank conflicts.
__device__ __forceinline__ int swz(int c) { return c + 8 * (c & 1); }

// Gate/up: 8 wavefronts (128 x 512 tiles), one workgroup per CU.  Down
// from 2049 to 6144 tokens: 4 wavefronts (128 x 256), two per CU -- its 8
// column tiles then deal evenly over the CUs where 4 wide ones would leave a
// half-empty last round (N = 4096: down 159 us against 164; gate/up 256
// against 267 with 4); the other batch sizes take other shapes (below).
template <bool GATEUP, int FB_, int WAVES_ = (GATEUP ? 8 : 4), int TB_ = 4>
struct TileShape {
  static constexpr int FB = FB_;  // packed 32-row blocks per wavefront
  static constexpr int kTB = TB_;  // 32-row token blocks per tile
  static constexpr int kBM = 32 * kTB;  // grouped rows per tile
  static constexpr int kWaves = WAVES_;
  static constexpr int kThreads = kWaves * kWave;
  // Workgroups per CU the register budget is set for: one for 8 wavefronts
  // or for 256-token tiles (whose accumulators take a whole register file).
  static constexpr int kPerCu = (kWaves == 8 || kTB == 8) ? 1 : 2;
  static constexpr int kChunks = kBM * (kPairBytes / 16) / kThreads;  // 16-byte token pieces per thread per pair
  static constexpr int kRowStep = kThreads / 8;  // tile rows one pass of the workgroup loads
  static constexpr int K = GATEUP ? kHidden : kFF;
  static constexpr int kSteps = GATEUP ? kGateupSteps : kDownSteps;
  static constexpr int kBlocks = GATEUP ? kGateupBlocks : kDownBlocks;
  static constexpr int kBlocksPerTile = kWaves * FB;
  static constexpr int kColTiles = kBlocks / kBlocksPerTile;
  // m-tiles per launch group: a group holds a multiple of kXcds tiles.
  static constexpr int kGroup =
      kXcds / (kColTiles % kXcds == 0 ? kXcds : kColTiles % 4 == 0 ? 4 : kColTiles % 2 == 0 ? 2 : 1);
  static constexpr int kStages = K / kBK;
  static_assert(kBlocks % kBlocksPerTile == 0, "column tiles cover the weight rows");
  static_assert(kGroup * kColTiles % kXcds == 0, "a launch group deals evenly over the XCDs");
};

// FP8: Wp holds the FP8 codes of the experts (pack_fp8.hip layout: 1 KB
// fragments of 32 rows x 32 K, one per K stage), Ws their fp32 block scales,
// A the bf16 values of the token rows' E4M3 codes and As the rows' scales per
// 128-wide K group.  A group of four stages (128 K) adds its products times
// weight scale x token scale.  One accumulator set serves all groups: it
// holds the sum so far in units of the current group's scale product (one
// per token column and, for gate/up, per gate or up half), so before each
// group it is multiplied by old unit / new unit, and at the end by the last
// unit.  (Where a scale is 0 the group's codes are all 0, and the unit
// stays.)  The products are exact and the sums fp32, as with a second
// accumulator set per group, up to the rounding of the unit changes (a few
// fp32 ulps per group; the ratio uses the hardware reciprocal).
template <bool GATEUP, int FB_, int WAVES_, int TB_, bool FP8 = false, bool NTW = false>
__global__ __launch_bounds__((TileShape<GATEUP, FB_, WAVES_, TB_>::kThreads),
                             (TileShape<GATEUP, FB_, WAVES_, TB_>::kPerCu))
void expert_tiled_kernel(
    const uint16_t* __restrict__ A, const void* __restrict__ Wp,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row2slot,
    uint16_t* __restrict__ H, float* __restrict__ Y, const float* __restrict__ Ws,
    const float* __restrict__ As) {
  using T = TileShape<GATEUP, FB_, WAVES_, TB_>;
  constexpr int FB = T::FB;
  constexpr int TB = T::kTB;
  constexpr int kWK = FP8 ? 1 : kKS;  // 16-byte weight loads per block and stage
  static_assert(!FP8 || kWSlots * kBK == 128, "an FP8 scale group is one pass of the stage loop");
  static_assert(T::kStages % kWSlots == 0, "the stage loop is unrolled by the ring size");
  // Token fragments: 2 pair buffers x (2 stages x 4 token blocks x kKS steps).
  __shared__ uint4 tok[2][2 * TB * kKS * kWave];

  // Launch groups of kGroup m-tiles x kColTiles column tiles; workgroup ids
  // are dealt to the XCDs round-robin, so id w of a group runs on XCD w % 8.
  // Tile t = c * kGroup + m of the group (column tile c, m-tile m) goes to
  // XCD t / (tiles per XCD): each XCD takes a run of consecutive tiles, so a
  // column tile, read by every m-tile of its expert, stays on one or two
  // XCDs and is shared through their L2.
  constexpr int kPerXcd = T::kGroup * T::kColTiles / kXcds;
  const int w = blockIdx.x % (T::kGroup * T::kColTiles);
  const int t = (w % kXcds) * kPerXcd + w / kXcds;
  const int nb = t / T::kGroup;
  const int mt = blockIdx.x / (T::kGroup * T::kColTiles) * T::kGroup + t % T::kGroup;
  MTile tile;
  if (!map_mtile(offsets, mt, T::kBM, tile)) return;
  const int live_rows = uniform(tile.rows);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  // Token pieces of this thread: row r0 + kRowStep * i of the tile, 16-byte
  // chunk c of the row's 128-byte line of a stage pair; eight consecutive
  // lanes read one whole line.  All the pieces share c and r0 % 32, so their
  // LDS positions differ by whole token-block fragments.
  const int r0 = tid / 8, c = tid % 8;
  const uint16_t* arow[T::kChunks];
#pragma unroll
  for (int i = 0; i < T::kChunks; ++i) {
    const int r = r0 + T::kRowStep * i;
    const int slot = row2slot[tile.row_begin + (r < tile.rows ? r : 0)];
    arow[i] = A + static_cast<size_t>(GATEUP ? slot / kTopK : slot) * T::K + c * 8;
  }
  const int st_pos = ((c / 4) * TB * kKS + (c / 2) % 2) * kWave + (c % 2) * 32 + ((r0 % 32) ^ swz(c)) +
                     (r0 / 32) * kKS * kWave;
  static_assert(T::kRowStep % 32 == 0, "a thread's pieces share their row within a token block");
  // MFMA operand position of this lane for stage sp of a pair, K step j.
  int rd_pos[2][kKS];
#pragma unroll
  for (int sp = 0; sp < 2; ++sp)
#pragma unroll
    for (int j = 0; j < kKS; ++j)
      rd_pos[sp][j] = (sp * TB * kKS + j) * kWave + (lane & 32) + ((lane & 31) ^ swz(sp * 4 + j * 2 + lane / 32));

  // This wavefront's FB packed row blocks, K steps of a block contiguous,
  // read as buffer loads: the expert's packed matrix (12 MB at most) is the
  // buffer, the wavefront's first block a scalar offset, the lane's 16 bytes
  // of a fragment the only per-lane offset.
  constexpr uint32_t kBlockBytes = static_cast<uint32_t>(T::kStages * kWK) * kFragBytes;
  const Rsrc wr = make_rsrc(static_cast<const uint8_t*>(Wp) +
                                static_cast<size_t>(uniform(tile.expert)) * T::kBlocks * kBlockBytes,
                            T::kBlocks * kBlockBytes);
  const uint32_t wbase = uniform(static_cast<uint32_t>((nb * T::kBlocksPerTile + wave * FB) * kBlockBytes));
  const uint32_t wlane = lane * 16;

  uint4 wring[kWSlots][FB][kWK];
  // Stages past the end reload the last stage (in bounds, never used).
  auto load_w = [&](int s, uint4 (&wv)[FB][kWK]) {
    const uint32_t sc = s < T::kStages ? s : T::kStages - 1;
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
      for (int j = 0; j < kWK; ++j)
        wv[f][j] = buf_ld<NTW>(wr, wlane, wbase + f * kBlockBytes + (sc * kWK + j) * kFragBytes);
  };
  constexpr int kPairs = T::kStages / 2;
  uint4 stg[T::kChunks];
  auto load_x = [&](int pair) {
    const int pc = pair < kPairs ? pair : kPairs - 1;
#pragma unroll
    for (int i = 0; i < T::kChunks; ++i) stg[i] = ld16(arow[i] + pc * (kPairBytes / 2));
  };
  auto store_x = [&](int pb) {
#pragma unroll
    for (int i = 0; i < T::kChunks; ++i) tok[pb][st_pos + i * (T::kRowStep / 32) * kKS * kWave] = stg[i];
  };

  f32x16 acc[TB][FB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tb][f][r] = 0.f;

  // FP8 scales: this wavefront's weight row blocks (128 rows) and the
  // tile rows' token rows (padding rows take row 0's; their results are
  // dropped).
  int srow[FP8 ? TB : 1];
  if constexpr (FP8) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int row = tb * 32 + lane % 32;
      const int slot = row2slot[tile.row_begin + (row < tile.rows ? row : 0)];
      srow[tb] = GATEUP ? slot / kTopK : slot;
    }
  }
  // FP8 scales of one K group, and the units of the accumulators.
  constexpr int kG = T::K / 128;
  constexpr float kFltMin = 1.17549435e-38f;  // smallest normal fp32
  float xs[FP8 ? TB : 1], wsa[FP8 ? FB : 1], wsb[FP8 ? FB : 1];
  float unit[FP8 ? TB : 1][FP8 ? FB : 1][2];
  auto load_scales = [&](int g) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) xs[tb] = As[static_cast<size_t>(srow[tb]) * kG + g];
    const int e = uniform(tile.expert);
#pragma unroll
    for (int f = 0; f < FB; ++f) {
      const int blk = nb * T::kBlocksPerTile + wave * FB + f;
      if (GATEUP) {  // gate rows (values r < 8 of a tile) and up rows
        wsa[f] = Ws[((e * 2 + 0) * (kFF / 128) + blk / 8) * kG + g];
        wsb[f] = Ws[((e * 2 + 1) * (kFF / 128) + blk / 8) * kG + g];
      } else {
        wsa[f] = wsb[f] = Ws[(e * (kHidden / 128) + blk / 4) * kG + g];
      }
    }
  };
  // Re-expresses the sums in units of the scales last loaded.
  auto rebase = [&] {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        const float sc[2] = {wsa[f] * xs[tb], wsb[f] * xs[tb]};
        float k[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          k[h] = sc[h] != 0.f ? unit[tb][f][h] * __builtin_amdgcn_rcpf(sc[h]) : 1.f;
          // A subnormal scale product would overflow the reciprocal: there
          // (rarely, per lane) the ratio is an IEEE division.
          if (sc[h] != 0.f && !(sc[h] >= kFltMin)) k[h] = unit[tb][f][h] / sc[h];
          unit[tb][f][h] = sc[h] != 0.f ? sc[h] : unit[tb][f][h];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tb][f][r] *= (r < 8 ? k[0] : k[1]);
      }
  };
  // Group 0's scales go first, so that waiting for them leaves the ring's
  // loads in flight.
  if constexpr (FP8) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int f = 0; f < FB; ++f) unit[tb][f][0] = unit[tb][f][1] = 1.f;
    load_scales(0);
  }
#pragma unroll
  for (int s = 0; s < kWSlots - 1; ++s) load_w(s, wring[s]);
  load_x(0);
  store_x(0);
  load_x(1);
  __syncthreads();

  // Token operands, double-buffered: tk[x] holds the four token-block
  // fragments of one K step.
  uint4 tk[2][TB];
  auto read_tk = [&](int pb, int sp, int j, uint4 (&d)[TB]) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) d[tb] = tok[pb][rd_pos[sp][j] + tb * kKS * kWave];
  };
  // Gate/up skips the MFMAs of 32-row token blocks that are all padding
  // (the last m-tile of an expert); in the down kernel the branches cost
  // more registers than it has.
  auto mma = [&](const uint4 (&wj)[FB][kWK], int j, const uint4 (&d)[TB]) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
      if (!GATEUP || tb == 0 || tb * 32 < live_rows)
#pragma unroll
        for (int f = 0; f < FB; ++f) {
          if constexpr (FP8) {
            // Lane bytes 0..7: K step 0 of the stage, 8..15: K step 1.
            const uint4 wbf = j == 0 ? e4m3x8_to_bf16(wj[f][0].x, wj[f][0].y)
                                     : e4m3x8_to_bf16(wj[f][0].z, wj[f][0].w);
            acc[tb][f] = mfma32(wbf, d[tb], acc[tb][f]);
          } else {
            acc[tb][f] = mfma32(wj[f][j], d[tb], acc[tb][f]);
          }
        }
  };
  // The fences keep the issue order written here, which the wait counts
  // below rely on: weight loads, then the next LDS operands, then MFMAs.
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  read_tk(0, 0, 0, tk[0]);

  // Stage s of pair p (LDS buffer pb = p % 2) multiplies with ring slot
  // s % 4 and loads the weights of stage s + 3 into the free slot; the LDS
  // operands of each K step are read one step ahead.  The first stage of a
  // pair stores the next pair's tokens (loaded one pair ago) into the other
  // buffer, whose last readers passed the previous barrier, and loads the
  // pair after that.  The second stage's barrier comes once its own LDS
  // reads are done, before its last MFMAs: it publishes the stored tokens
  // and frees buffer pb for the next store.
  auto stage = [&](int s, int sp, int pb, uint4 (&wc)[FB][kWK], uint4 (&wn)[FB][kWK]) {
    static_assert(kKS == 2, "two K steps per stage");
    load_w(s + kWSlots - 1, wn);
    read_tk(pb, sp, 1, tk[1]);
    fence();
    mma(wc, 0, tk[0]);
    fence();
    if (sp == 0) {
      read_tk(pb, 1, 0, tk[0]);
      fence();
      mma(wc, 1, tk[1]);
      fence();
      store_x(pb ^ 1);
      load_x(s / 2 + 2);
      fence();
    } else {
      __syncthreads();
      read_tk(pb ^ 1, 0, 0, tk[0]);
      fence();
      mma(wc, 1, tk[1]);
      fence();
    }
  };
  if constexpr (FP8) rebase();  // the sums are 0: this sets the units of group 0
  for (int s = 0; s < T::kStages; s += kWSlots) {
    // The next group's scales are loaded a group ahead (the last group loads
    // its own again: the rebase is then exact, old unit / same unit = 1).
    if constexpr (FP8) load_scales(min(s / kWSlots + 1, kG - 1));
#pragma unroll
    for (int q = 0; q < kWSlots; ++q)
      stage(s + q, q % 2, q / 2, wring[q], wring[(q + kWSlots - 1) % kWSlots]);
    if constexpr (FP8) rebase();
  }
  if constexpr (FP8) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tb][f][r] *= unit[tb][f][r < 8 ? 0 : 1];
  }

  // acc[tb][f]: token row tb*32 + lane % 32 of the tile; rows
  // mfma32_row(r, lane) of packed block nb * kBlocksPerTile + wave * FB + f.
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int row = tb * 32 + lane % 32;
    if (row >= tile.rows) continue;
    const int slot = row2slot[tile.row_begin + row];
#pragma unroll
    for (int f = 0; f < FB; ++f) {
      const int blk = nb * T::kBlocksPerTile + wave * FB + f;
      if (GATEUP) {
        // Values r < 8 are gate rows, r + 8 the up rows of the same H column.
        uint16_t* dst = H + static_cast<size_t>(slot) * kFF + blk * 16 + 4 * (lane / 32);
        const f32x16& v = acc[tb][f];
#pragma unroll
        for (int g8 = 0; g8 < 2; ++g8) {
          uint32_t p[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int r = g8 * 4 + h * 2;
            p[h] = pack_bf16x2(silu(v[r]) * v[r + 8], silu(v[r + 1]) * v[r + 9]);
          }
          *reinterpret_cast<uint2*>(dst + g8 * 8) = make_uint2(p[0], p[1]);
        }
        fence();  // one tile at a time: bounds the registers the SiLU needs
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

template <bool GATEUP, int FB, int WAVES, int TB>
int64_t tiled_grid(int64_t N) {
  using T = TileShape<GATEUP, FB, WAVES, TB>;
  const int64_t groups = (max_mtiles(N, T::kBM) + T::kGroup - 1) / T::kGroup;
  return groups * T::kGroup * T::kColTiles;
}

// Column tiles by batch size.  With few tokens per expert the kernels are
// bound by the weight stream, each expert has one or two m-tiles, and the
// tile count barely exceeds what the device holds, so the last round of
// tiles runs on a fraction of the CUs; narrower tiles make that tail
// shorter.  Gate/up: 512 weight rows (8 wavefronts x two blocks) by
// default, 128 rows (4 wavefronts x one block, two workgroups per CU) for
// 193-512 tokens, 256 rows (8 x one) for 513-2048.  Down: 128 rows (4 x
// one) up to 512 tokens, 256 rows (8 x one) for 513-2048, 256 rows (4 x
// two) for 2049-6144, 512 rows (8 x two) above.  Measured (layer of seed
// 4, first N tokens; gate/up 512 / 128 / 256 rows, us): N = 160: 92 / 97 /
// -; 256: 132 / 112 / -; 320: - / 112 / 117; 512: - / 119 / 121; 640: - /
// 130 / 126; 1024: - / 140 / 133; earlier, 4096: 245 / - / 261.  Down 256 /
// 128 rows: N = 128: 61 / 52; 320: 71 / 61; 512: 77 / 69; 640: 74 / 75;
// 2048: 104 / 108.  Down by N (us, same box, mean of two runs for the
// 256-row form; 256 rows as 4 x two / 256 rows as 8 x one / 512 rows as 8 x
// two): N = 1024: 83.1 / 78.6 / 83.8; 2048: 112.3 / 104.5 / 115.8; 4096:
// 157.3 / 160.3 / 165.7; 6144: 210.6 / 217.6 / 209.9; 8192: 277.6 / 299.0 /
// 264.8; 16384: 497.2 / 541.0 / 470.8.  With eight wavefronts a workgroup
// has a CU to itself and its token tile feeds twice the weight rows.
// Weight loads: up to kOneTouchTokens tokens most experts have a single
// m-tile, so each weight byte is read once and the loads are non-temporal
// (layer us, same box, plain / non-temporal: N = 160: 149.5-152.9 /
// 141.8-144.3; 320: 174.1-177.9 / 164.5-168.5; 640: 219-220 both); above,
// the m-tiles of an expert share its weight tiles through the L2 and
// non-temporal loads cost (N = 2048: 333 / 362-368; 4096: 465-476 / 532-535).
// The FP8 grouped kernels (from 257 tokens) follow the same rule (FP8 layer
// us: N = 300: 141.1-141.6 / 138.0-138.9; 400: 156.1-156.3 / 152.3-152.4;
// 512: 166.4-167.0 / 165.5-165.9).
constexpr int64_t kOneTouchTokens = 512;
enum class GateupTiles { kWide, kNarrow4, kNarrow8 };
GateupTiles gateup_tiles(int64_t N) {
  if (N > 192 && N <= 512) return GateupTiles::kNarrow4;
  if (N > 512 && N <= 2048) return GateupTiles::kNarrow8;
  return GateupTiles::kWide;
}
enum class DownTiles { kNarrow4, kNarrow8, kMid, kWide8 };
DownTiles down_tiles(int64_t N) {
  if (N <= 512) return DownTiles::kNarrow4;
  if (N <= 2048) return DownTiles::kNarrow8;
  if (N <= 6144) return DownTiles::kMid;
  return DownTiles::kWide8;
}

template <bool GATEUP, int FB, int WAVES = (GATEUP ? 8 : 4), int TB = 4, bool FP8 = false,
          bool NTW = false, typename Out>
hipError_t launch_tiled(const uint16_t* A, const void* W, const int32_t* offsets,
                        const int32_t* row2slot, Out* out, int64_t N, hipStream_t stream,
                        const float* Ws = nullptr, const float* As = nullptr) {
  uint16_t* H = nullptr;
  float* Y = nullptr;
  if constexpr (GATEUP) H = out; else Y = out;
  hipLaunchKernelGGL((expert_tiled_kernel<GATEUP, FB, WAVES, TB, FP8, NTW>),
                     dim3(tiled_grid<GATEUP, FB, WAVES, TB>(N)),
                     dim3(TileShape<GATEUP, FB, WAVES, TB>::kThreads), 0, stream, A, W, offsets,
                     row2slot, H, Y, Ws, As);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup_tiled(const uint16_t* X, const uint16_t* Wgu, const int32_t* offsets,
                               const int32_t* row2slot, uint16_t* H, int64_t N,
                               hipStream_t stream) {
  switch (gateup_tiles(N)) {
    case GateupTiles::kNarrow4:
      return launch_tiled<true, 1, 4, 4, false, true>(X, Wgu, offsets, row2slot, H, N, stream);
    case GateupTiles::kNarrow8:
      return launch_tiled<true, 1>(X, Wgu, offsets, row2slot, H, N, stream);
    default:
      return N <= kOneTouchTokens ? launch_tiled<true, 2, 8, 4, false, true>(X, Wgu, offsets, row2slot, H, N, stream)
                                  : launch_tiled<true, 2>(X, Wgu, offsets, row2slot, H, N, stream);
  }
}

hipError_t launch_down_tiled(const uint16_t* H, const uint16_t* Wd, const int32_t* offsets,
                             const int32_t* row2slot, float* Y, int64_t N, hipStream_t stream) {
  switch (down_tiles(N)) {
    case DownTiles::kNarrow4:
      return launch_tiled<false, 1, 4, 4, false, true>(H, Wd, offsets, row2slot, Y, N, stream);
    case DownTiles::kNarrow8:
      return launch_tiled<false, 1, 8>(H, Wd, offsets, row2slot, Y, N, stream);
    case DownTiles::kWide8:
      return launch_tiled<false, 2, 8>(H, Wd, offsets, row2slot, Y, N, stream);
    default:
      return launch_tiled<false, 2>(H, Wd, offsets, row2slot, Y, N, stream);
  }
}

hipError_t launch_gateup_tiled_fp8(const uint16_t* Xq, const uint8_t* Wq, const float* Ws,
                                   const float* Xs, const int32_t* offsets, const int32_t* row2slot,
                                   uint16_t* H, int64_t N, hipStream_t stream) {
  switch (gateup_tiles(N)) {
    case GateupTiles::kNarrow4:
      return launch_tiled<true, 1, 4, 4, true, true>(Xq, Wq, offsets, row2slot, H, N, stream, Ws, Xs);
    case GateupTiles::kNarrow8:
      return launch_tiled<true, 1, 8, 4, true>(Xq, Wq, offsets, row2slot, H, N, stream, Ws, Xs);
    default:
      return N <= kOneTouchTokens ? launch_tiled<true, 2, 8, 4, true, true>(Xq, Wq, offsets, row2slot, H, N, stream, Ws, Xs)
                                  : launch_tiled<true, 2, 8, 4, true>(Xq, Wq, offsets, row2slot, H, N, stream, Ws, Xs);
  }
}

hipError_t launch_down_tiled_fp8(const uint16_t* Hq, const uint8_t* Wq, const float* Ws,
                                 const float* Hs, const int32_t* offsets, const int32_t* row2slot,
                                 float* Y, int64_t N, hipStream_t stream) {
  switch (down_tiles(N)) {
    case DownTiles::kNarrow4:
      return launch_tiled<false, 1, 4, 4, true, true>(Hq, Wq, offsets, row2slot, Y, N, stream, Ws, Hs);
    case DownTiles::kNarrow8:
      return launch_tiled<false, 1, 8, 4, true>(Hq, Wq, offsets, row2slot, Y, N, stream, Ws, Hs);
    default:  // the 4-wavefront form of two blocks would spill in FP8 mode
      return launch_tiled<false, 2, 8, 4, true>(Hq, Wq, offsets, row2slot, Y, N, stream, Ws, Hs);
  }
}

}  // namespace lfm

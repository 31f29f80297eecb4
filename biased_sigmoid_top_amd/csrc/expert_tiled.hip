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
// FP8 mode (the FP8 layer above 256 tokens): the products run on the gfx950
// FP8 matrix core (32x32x64 E4M3).  The weights are the FP8 codes of
// pack_fp8.hip (two 1 KB fragments per 32-row block and 64-wide K stage),
// the token rows their E4M3 codes from quant.hip, whose byte order makes a
// stage's 64 code bytes of a row land in LDS exactly where 32 bf16 columns
// land in bf16 mode, so staging, swizzle and operand reads are shared.  A
// stage pair is one 128-wide K group, which adds its products of codes
// times weight block scale x the token row's scale, as the block-scaled
// format defines, through one accumulator set kept in units of the current
// group's scales (see the kernel), so the FP8 mode takes the bf16 mode's
// tile shapes with half the stages.  The core's sums are not fp32 sums of
// the exact products: it aligns a step's 64 products and drops the bits
// below the alignment (measured: within 2^-11.6 of the sum of their
// magnitudes).
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
  static_assert(kBlocks % kBlocksPerTile == 0, "column tiles cover the weight rows");
  static_assert(kGroup * kColTiles % kXcds == 0, "a launch group deals evenly over the XCDs");
};

// D = A * B + C on a 32x32 tile with K = 64 on the FP8 matrix core (E4M3
// codes in, fp32 out).  Lane l supplies 32 codes of row l % 32 of A (a0, then
// a1) and 32 codes of column l % 32 of B (b0, then b1); byte i of a lane's A
// and byte i of B in a lane of the same half (l / 32) meet the same K, so
// both operands only need their bytes in one common order.  Accumulator
// layout as mfma32.  (Zero scale operands select the unscaled instruction.)
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma32_fp8(const uint4& a0, const uint4& a1, const uint4& b0,
                                             const uint4& b1, f32x16 c) {
  const i32x8 a = {static_cast<int>(a0.x), static_cast<int>(a0.y), static_cast<int>(a0.z),
                   static_cast<int>(a0.w), static_cast<int>(a1.x), static_cast<int>(a1.y),
                   static_cast<int>(a1.z), static_cast<int>(a1.w)};
  const i32x8 b = {static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z),
                   static_cast<int>(b0.w), static_cast<int>(b1.x), static_cast<int>(b1.y),
                   static_cast<int>(b1.z), static_cast<int>(b1.w)};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// FP8 mode: Wp holds the FP8 codes of the experts (pack_fp8.hip layout: 1 KB
// fragments of 32 rows x 32 K, lane l's 16 bytes columns 8h..8h+7 and
// 16+8h..16+8h+7 of row l % 32, h = l / 32), Ws their fp32 block scales, A
// the token rows' E4M3 codes (quant.hip, whose byte order puts those same
// columns in 16-byte chunk 2p + h of each 32-wide piece p) and As the rows'
// scales per 128-wide K group.  A stage is 64 K: two fragments per block and
// the 64 code bytes of each token row, which the LDS tile holds exactly as it
// holds 32 bf16 columns, so one FP8 MFMA takes the stage's two K halves at
// once.  A stage pair is one 128-wide K group, whose products of codes must
// be multiplied by weight block scale x token scale.  One accumulator set
// serves all groups: it holds the sum so far in units of the current group's
// scales -- a token unit per token column and a weight unit per block (and
// gate or up half) -- so at the start of each group the sums are multiplied
// by old unit / new unit, and at the end by the last units.  Where a scale
// is 0 the group's codes are all 0, and that unit stays.  The scales of a
// tile are staged in LDS once, before the stage loop.
// Slots of at most 32 * kSelfWords tokens grouped by expert, as the dispatch
// step groups them (offsets: exclusive prefix of the per-expert counts;
// rows: slots t * 4 + j of each expert in token order), computed in LDS by
// one workgroup of at least kExperts threads, token t on thread t %
// nthreads: per-expert token bitmasks, a word prefix per expert, a prefix
// over the experts, then each slot's rank from one popcount.  A token's four experts
// are distinct, so each (expert, token) bit is set once.  scratch holds at
// least 2 * kExperts * kSelfWords words and is free again on return.
// Capacity: 512 tokens in the 128-row token tiles, 256 in the shorter ones
// (whose LDS token tile holds the masks of 256).
constexpr int kSelfTokens = 512;
constexpr int kSelfShortTokens = 256;
template <int kSelfWords>
__device__ __forceinline__ void group_slots_lds(const int32_t* __restrict__ idx, int N, int* off,
                                                int* rows, uint32_t* scratch, int nthreads) {
  uint32_t (*mask)[kSelfWords] = reinterpret_cast<uint32_t (*)[kSelfWords]>(scratch);
  int (*wbase)[kSelfWords] = reinterpret_cast<int (*)[kSelfWords]>(scratch + kExperts * kSelfWords);
  const int tid = threadIdx.x;
  for (int i = tid; i < kExperts * kSelfWords; i += nthreads) (&mask[0][0])[i] = 0u;
  __syncthreads();
  for (int t = tid; t < N; t += nthreads) {
    const int4 v = *reinterpret_cast<const int4*>(idx + static_cast<size_t>(t) * kTopK);
    const int e4[kTopK] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < kTopK; ++j) atomicOr(&mask[e4[j]][t / 32], 1u << (t % 32));
  }
  __syncthreads();
  if (tid < kExperts) {  // wavefront 0, lane = expert
    int run = 0;
#pragma unroll
    for (int w = 0; w < kSelfWords; ++w) {
      wbase[tid][w] = run;
      run += __popc(mask[tid][w]);
    }
    const int incl = wave_inclusive_scan(run, tid);
    off[tid] = incl - run;
    if (tid == kExperts - 1) off[kExperts] = incl;
  }
  __syncthreads();
  for (int t = tid; t < N; t += nthreads) {
    const int4 v = *reinterpret_cast<const int4*>(idx + static_cast<size_t>(t) * kTopK);
    const int e4[kTopK] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
      const int e = e4[j];
      const int rank = wbase[e][t / 32] + __popc(mask[e][t / 32] & ((1u << (t % 32)) - 1u));
      rows[off[e] + rank] = t * kTopK + j;
    }
  }
  __syncthreads();
}

template <bool GATEUP, int FB_, int WAVES_, int TB_, bool FP8 = false, bool NTW = false, bool SELF = false,
          bool OFF32 = true>
__global__ __launch_bounds__((TileShape<GATEUP, FB_, WAVES_, TB_>::kThreads),
                             (TileShape<GATEUP, FB_, WAVES_, TB_>::kPerCu))
void expert_tiled_kernel(
    const void* __restrict__ A, const void* __restrict__ Wp, const int32_t* __restrict__ idx, int ntok,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row2slot,
    uint16_t* __restrict__ H, float* __restrict__ Y, const float* __restrict__ Ws,
    const float* __restrict__ As) {
  using T = TileShape<GATEUP, FB_, WAVES_, TB_>;
  constexpr int FB = T::FB;
  constexpr int TB = T::kTB;
  // K per stage: 32 bf16 or 64 E4M3 columns, 64 bytes of a token row either way.
  constexpr int kStageK = FP8 ? 2 * kBK : kBK;
  constexpr int kStages = T::K / kStageK;
  constexpr int kRowBytes = T::K * (FP8 ? 1 : 2);
  static_assert(kStages % kWSlots == 0, "the stage loop is unrolled by the ring size");
  static_assert(!FP8 || 2 * kStageK == 128, "an FP8 scale group is one stage pair");
  static_assert(!FP8 || TB % 2 == 0, "FP8 token operands alternate between two slots per stage");
  // Token fragments: 2 pair buffers x (2 stages x 4 token blocks x kKS steps).
  __shared__ uint4 tok[2][2 * TB * kKS * kWave];
  // FP8 scales of the tile: the token rows' ([group][tile row]) and the
  // weight blocks' ([wavefront][block][gate | up][group]).
  constexpr int kG = T::K / 128;
  constexpr int kH = GATEUP ? 2 : 1;
  constexpr int kWsPerWave = FB * kH * kG;
  __shared__ float xs_lds[FP8 ? kG * T::kBM : 1];
  __shared__ float ws_lds[FP8 ? T::kWaves * kWsPerWave : 1];
  static_assert(!FP8 || (T::kThreads % T::kBM == 0 && kWsPerWave <= kWave), "scale staging");

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
  // SELF (gate/up of small batches): the workgroup groups the slots itself
  // from the selections, and workgroup 0 publishes the grouping for the
  // down kernel; otherwise the dispatch step's grouping is read.
  __shared__ int self_off[SELF ? kExperts + 1 : 1];
  constexpr int kSelfCap = TB >= 4 ? kSelfTokens : kSelfShortTokens;
  constexpr int kSelfWords = kSelfCap / 32;
  __shared__ int self_rows[SELF ? kSelfCap * kTopK : 1];
  const int32_t* grp_off = offsets;
  const int32_t* grp_rows = row2slot;
  if constexpr (SELF) {
    static_assert(GATEUP && T::kThreads >= kExperts &&
                      sizeof(tok) >= 2 * kExperts * kSelfWords * sizeof(uint32_t),
                  "a wavefront of experts; the masks fit in the token tile");
    group_slots_lds<kSelfWords>(idx, ntok, self_off, self_rows, reinterpret_cast<uint32_t*>(&tok[0][0]), T::kThreads);
    if (blockIdx.x == 0) {
      for (int i = threadIdx.x; i <= kExperts; i += T::kThreads) offsets[i] = self_off[i];
      for (int i = threadIdx.x; i < ntok * kTopK; i += T::kThreads) row2slot[i] = self_rows[i];
    }
    grp_off = self_off;
    grp_rows = self_rows;
  }
  MTile tile;
  if (!map_mtile(grp_off, mt, T::kBM, tile)) return;
  const int live_rows = uniform(tile.rows);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  // Token pieces of this thread: row r0 + kRowStep * i of the tile, 16-byte
  // chunk c of the row's 128-byte line of a stage pair; eight consecutive
  // lanes read one whole line.  With 32 or more rows per pass the pieces
  // share r0 % 32, so their LDS positions differ by whole token-block
  // fragments (the 2-wavefront shapes take 16 rows per pass).
  // OFF32 (token matrices below 2 GB; the host picks it): the rows are read
  // through a buffer resource over the token matrix with 32-bit offsets,
  // and a padding row of the tile takes an offset past its end, which the
  // range check turns into zeros with no memory read.  A CU's L1 request
  // rate bounds these kernels, so the padding rows' bytes cost time
  // (measured, layer us, 64-bit row pointers with padding rows reading row
  // 0 / this form: N = 1,024 256.8-259.4 / 249.9-250.7, 2,048 342.2-343.5 /
  // 331.5-331.8, 4,096 459.7-463.0 / 452.5-452.8; one register per token
  // piece instead of two also removes the spills of the two-block down
  // shapes).  The padding rows' products are zeros and are dropped.
  // Otherwise 64-bit row pointers, a padding row reading row 0's bytes.
  constexpr bool kPadZero = OFF32;
  constexpr uint32_t kPadOff = 0x80000000u;
  const Rsrc ar = make_rsrc(A, kPadZero ? static_cast<uint32_t>(
                                              static_cast<uint64_t>(GATEUP ? ntok : kTopK * ntok) * kRowBytes)
                                        : 0u);
  const int r0 = tid / 8, c = tid % 8;
  uint32_t aoff[kPadZero ? T::kChunks : 1];
  const uint8_t* arow[kPadZero ? 1 : T::kChunks];
#pragma unroll
  for (int i = 0; i < T::kChunks; ++i) {
    const int r = r0 + T::kRowStep * i;
    const int slot = grp_rows[tile.row_begin + (r < tile.rows ? r : 0)];
    const size_t off = static_cast<size_t>(GATEUP ? slot / kTopK : slot) * kRowBytes + c * 16;
    if constexpr (kPadZero)
      aoff[i] = r < tile.rows ? static_cast<uint32_t>(off) : kPadOff;
    else
      arow[i] = static_cast<const uint8_t*>(A) + off;
  }
  constexpr bool kWholeBlocks = T::kRowStep % 32 == 0;
  static_assert(T::kRowStep % 16 == 0 && T::kChunks >= 1, "whole 16-row groups per pass");
  auto st_at = [&](int i) {
    const int r = r0 + T::kRowStep * i;
    return ((c / 4) * TB * kKS + (c / 2) % 2) * kWave + (c % 2) * 32 + ((r % 32) ^ swz(c)) +
           (r / 32) * kKS * kWave;
  };
  int st_pos[kWholeBlocks ? 1 : T::kChunks];
#pragma unroll
  for (int i = 0; i < (kWholeBlocks ? 1 : T::kChunks); ++i) st_pos[i] = st_at(i);
  // MFMA operand position of this lane for stage sp of a pair, K step (bf16)
  // or K half (FP8) j.
  int rd_pos[2][kKS];
#pragma unroll
  for (int sp = 0; sp < 2; ++sp)
#pragma unroll
    for (int j = 0; j < kKS; ++j)
      rd_pos[sp][j] = (sp * TB * kKS + j) * kWave + (lane & 32) + ((lane & 31) ^ swz(sp * 4 + j * 2 + lane / 32));

  // This wavefront's FB packed row blocks, the fragments of a block
  // contiguous (two per stage), read as buffer loads: the expert's packed
  // matrix (12 MB at most) is the buffer, the wavefront's first block a
  // scalar offset, the lane's 16 bytes of a fragment the only per-lane offset.
  constexpr uint32_t kBlockBytes = static_cast<uint32_t>(kStages * kKS) * kFragBytes;
  const Rsrc wr = make_rsrc(static_cast<const uint8_t*>(Wp) +
                                static_cast<size_t>(uniform(tile.expert)) * T::kBlocks * kBlockBytes,
                            T::kBlocks * kBlockBytes);
  const uint32_t wbase = uniform(static_cast<uint32_t>((nb * T::kBlocksPerTile + wave * FB) * kBlockBytes));
  const uint32_t wlane = lane * 16;

  // FP8 scales, loaded first (stored to LDS with the first token pieces):
  // thread tid takes entries tid + kThreads * i of [group][tile row] (one
  // tile row: padding rows take row 0's scales, and their results are
  // dropped), lane l < kWsPerWave entry l of its wavefront's weight scales.
  constexpr int kXsPer = FP8 ? kG * T::kBM / T::kThreads : 1;
  float xs_st[kXsPer];
  float ws_st = 0.f;
  if constexpr (FP8) {
    const int r = tid % T::kBM;
    const int slot = grp_rows[tile.row_begin + (r < tile.rows ? r : 0)];
    const float* src = As + static_cast<size_t>(GATEUP ? slot / kTopK : slot) * kG;
#pragma unroll
    for (int i = 0; i < kXsPer; ++i) xs_st[i] = src[(tid + T::kThreads * i) / T::kBM];
    if (lane < kWsPerWave) {
      const int f = lane / (kH * kG), h = lane / kG % kH, g = lane % kG;
      const int blk = nb * T::kBlocksPerTile + wave * FB + f;
      const int e = uniform(tile.expert);
      // gate/up: [expert][gate | up][128-row block][group]; down: [expert][128-row block][group]
      ws_st = GATEUP ? Ws[((e * 2 + h) * (kFF / 128) + blk / 8) * kG + g]
                     : Ws[(e * (kHidden / 128) + blk / 4) * kG + g];
    }
  }

  uint4 wring[kWSlots][FB][kKS];
  // Stages past the end reload the last stage (in bounds, never used).
  auto load_w = [&](int s, uint4 (&wv)[FB][kKS]) {
    const uint32_t sc = s < kStages ? s : kStages - 1;
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
      for (int j = 0; j < kKS; ++j)
        wv[f][j] = buf_ld<NTW>(wr, wlane, wbase + f * kBlockBytes + (sc * kKS + j) * kFragBytes);
  };
  constexpr int kPairs = kStages / 2;
  uint4 stg[T::kChunks];
  auto load_x = [&](int pair) {
    const int pc = pair < kPairs ? pair : kPairs - 1;
#pragma unroll
    for (int i = 0; i < T::kChunks; ++i) {
      if constexpr (kPadZero)
        stg[i] = buf_ld<false>(ar, aoff[i], pc * kPairBytes);
      else
        stg[i] = ld16(arow[i] + pc * kPairBytes);
    }
  };
  auto store_x = [&](int pb) {
#pragma unroll
    for (int i = 0; i < T::kChunks; ++i)
      tok[pb][kWholeBlocks ? st_pos[0] + i * (T::kRowStep / 32) * kKS * kWave : st_pos[i]] = stg[i];
  };

  f32x16 acc[TB][FB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tb][f][r] = 0.f;

#pragma unroll
  for (int s = 0; s < kWSlots - 1; ++s) load_w(s, wring[s]);
  load_x(0);
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < kXsPer; ++i) xs_lds[tid + T::kThreads * i] = xs_st[i];
    if (lane < kWsPerWave) ws_lds[wave * kWsPerWave + lane] = ws_st;
  }
  store_x(0);
  load_x(1);
  __syncthreads();

  // The fences keep the issue order written here, which the wait counts
  // below rely on: weight loads, then the next LDS operands, then MFMAs.
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  if constexpr (!FP8) {
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
    auto mma = [&](const uint4 (&wj)[FB][kKS], int j, const uint4 (&d)[TB]) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        if (!GATEUP || tb == 0 || tb * 32 < live_rows)
#pragma unroll
          for (int f = 0; f < FB; ++f) acc[tb][f] = mfma32(wj[f][j], d[tb], acc[tb][f]);
    };
    read_tk(0, 0, 0, tk[0]);

    // Stage s of pair p (LDS buffer pb = p % 2) multiplies with ring slot
    // s % 4 and loads the weights of stage s + 3 into the free slot; the LDS
    // operands of each K step are read one step ahead.  The first stage of a
    // pair stores the next pair's tokens (loaded one pair ago) into the other
    // buffer, whose last readers passed the previous barrier, and loads the
    // pair after that.  The second stage's barrier comes once its own LDS
    // reads are done, before its last MFMAs: it publishes the stored tokens
    // and frees buffer pb for the next store.
    auto stage = [&](int s, int sp, int pb, uint4 (&wc)[FB][kKS], uint4 (&wn)[FB][kKS]) {
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
    for (int s = 0; s < kStages; s += kWSlots) {
#pragma unroll
      for (int q = 0; q < kWSlots; ++q)
        stage(s + q, q % 2, q / 2, wring[q], wring[(q + kWSlots - 1) % kWSlots]);
    }
  } else {
    // Token operands of one token block (both K halves), double-buffered by
    // token block: the operands of block tb + 1 (or of the next stage's
    // block 0) are read while block tb multiplies.
    uint4 tk[2][kKS];
    auto read_tk = [&](int pb, int sp, int tb, uint4 (&d)[kKS]) {
#pragma unroll
      for (int j = 0; j < kKS; ++j) d[j] = tok[pb][rd_pos[sp][j] + tb * kKS * kWave];
    };
    // Scales of group g: the lane's token rows, the wavefront's blocks (the
    // same in every lane: kept in scalar registers).
    float xn[TB], wn[FB][kH];
    auto read_scales = [&](int g) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) xn[tb] = xs_lds[g * T::kBM + tb * 32 + lane % 32];
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int h = 0; h < kH; ++h)
          wn[f][h] = __int_as_float(__builtin_amdgcn_readfirstlane(
              __float_as_int(ws_lds[wave * kWsPerWave + (f * kH + h) * kG + g])));
    };
    // Units: where a scale is 0 the unit stays (that group adds nothing).
    constexpr float kFltMin = 1.17549435e-38f;  // smallest normal fp32
    auto ratio = [](float& u, float s) {
      float k = 1.f;
      if (s != 0.f) {
        k = u * __builtin_amdgcn_rcpf(s);
        // A subnormal scale would overflow the reciprocal: there (rarely,
        // per lane) the ratio is an IEEE division.
        if (!(s >= kFltMin)) k = u / s;
        u = s;
      }
      return k;
    };
    float ux[TB], uw[FB][kH];
    read_scales(0);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) ux[tb] = xn[tb] != 0.f ? xn[tb] : 1.f;
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
      for (int h = 0; h < kH; ++h) uw[f][h] = wn[f][h] != 0.f ? wn[f][h] : 1.f;
    read_tk(0, 0, 0, tk[0]);

    // Stage s of pair p (LDS buffer pb = p % 2; pair p is scale group p)
    // multiplies with ring slot s % 4 and loads the weights of stage s + 3
    // into the free slot.  The first stage of a pair reads the group's
    // scales and re-expresses the sums in its units (each token block just
    // before its MFMAs), stores the next pair's tokens (loaded one pair ago)
    // into the other buffer, whose last readers passed the previous barrier,
    // and loads the pair after that.  The second stage's barrier, before its
    // first read of the next pair's buffer, publishes the stored tokens and
    // frees buffer pb for the next store.
    auto stage = [&](int s, int sp, int pb, uint4 (&wc)[FB][kKS], uint4 (&wnext)[FB][kKS]) {
      load_w(s + kWSlots - 1, wnext);
      float kx[TB], kw[FB][kH];
      if (sp == 0) {
        read_scales(s / 2);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) kx[tb] = ratio(ux[tb], xn[tb]);
#pragma unroll
        for (int f = 0; f < FB; ++f)
#pragma unroll
          for (int h = 0; h < kH; ++h) kw[f][h] = ratio(uw[f][h], wn[f][h]);
      }
      fence();
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        if (tb + 1 < TB) {
          read_tk(pb, sp, tb + 1, tk[(tb + 1) % 2]);
        } else {
          if (sp == 1) __syncthreads();
          read_tk(sp == 0 ? pb : pb ^ 1, sp ^ 1, 0, tk[0]);
        }
        fence();
        if (!GATEUP || tb == 0 || tb * 32 < live_rows) {
#pragma unroll
          for (int f = 0; f < FB; ++f) {
            if (sp == 0) {
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[tb][f][r] *= kx[tb] * kw[f][GATEUP && r >= 8 ? 1 : 0];
            }
            acc[tb][f] = mfma32_fp8(wc[f][0], wc[f][1], tk[tb % 2][0], tk[tb % 2][1], acc[tb][f]);
          }
        }
        fence();
      }
      if (sp == 0) {
        store_x(pb ^ 1);
        load_x(s / 2 + 2);
        fence();
      }
    };
    for (int s = 0; s < kStages; s += kWSlots) {
#pragma unroll
      for (int q = 0; q < kWSlots; ++q)
        stage(s + q, q % 2, q / 2, wring[q], wring[(q + kWSlots - 1) % kWSlots]);
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tb][f][r] *= ux[tb] * uw[f][GATEUP && r >= 8 ? 1 : 0];
  }

  // acc[tb][f]: token row tb*32 + lane % 32 of the tile; rows
  // mfma32_row(r, lane) of packed block nb * kBlocksPerTile + wave * FB + f.
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int row = tb * 32 + lane % 32;
    if (row >= tile.rows) continue;
    const int slot = grp_rows[tile.row_begin + row];
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

// Tile shapes by batch size.  With few tokens per expert the kernels are
// bound by the weight stream, each expert has one or two m-tiles, and the
// tile count barely exceeds what the device holds, so the last round of
// tiles runs on a fraction of the CUs; narrower tiles make that tail
// shorter, and token tiles no taller than the experts' token counts keep
// the registers, LDS and MFMAs of all-padding rows out of the weight
// stream (more workgroups per CU, more weight loads in flight).
//  * Up to 256 tokens (bf16: from 5; FP8: from 5): 128 weight rows (4
//    wavefronts x one block), token tiles of 32 rows up to 96 tokens (bf16)
//    and of 64 rows otherwise (the FP8 mode needs an even number of token
//    blocks).  Up to 96 tokens down, and bf16 gate/up, take 64 weight rows
//    (2 wavefronts x one block), which doubles their tile counts.  Down us,
//    128 / 64 weight rows: N = 64 bf16 46.1 / 44.5, FP8 31.3 / 30.7-30.9;
//    N = 256: 55.4 / 59.5.  bf16 gate/up: N = 16 58.2 / 55.6, 32 62.5 /
//    63.6, 64 85.6-85.9 / 84.6, 96 80.8 / 76.1; FP8 gate/up at N = 64 46.6 /
//    48.1 (kept at 128 rows).  Measured, layer us at N = 64 (the 64-token decode workload;
//    the streaming kernels / 128 token rows / 64 / 32): bf16 143.4-146.5 /
//    140.3-141.5 / 137.5-137.7 / 136.6-136.9; FP8 102.0-102.5 (streaming) /
//    90.6-95.9 / 84.0-84.4.  First N tokens of the 4,096-token workload
//    (streaming / 64 rows / 32 rows): bf16 N = 8: 68.5 / 65.4 / 64.7-65.3;
//    48: 112.6-113.4 / 103.3 / 102.5-102.9; 96: 135.3-135.8 / 132.8 / 131.0;
//    192: 184.1 (512 weight rows) / 150.6-150.9 / 176.5; FP8 (streaming /
//    64 rows / 128 rows) N = 8: 52.3 / 47.7 / 51.7; 32: 79.3 / 65.8 / 73.7;
//    128: 111.9 / 87.5 / 92.8; 256: 157.6 / 102.4 / 109.8; 512: 129.4 /
//    129.3 / 129.7.
//  * bf16, 257-512 tokens: 128 weight rows, 128 token rows; 513-2048: 256
//    rows (8 wavefronts x one block); above, gate/up 512 rows (8 x two).
//    Down: 128 rows up to 512 tokens, 256 rows (8 x one) for 513-2048, 256
//    rows (4 x two) for 2049-6144, 512 rows (8 x two) above.  Measured
//    (layer of seed 4, first N tokens; gate/up 512 / 128 / 256 rows, us):
//    N = 256: 132 / 112 / -; 320: - / 112 / 117; 512: - / 119 / 121; 640: -
//    / 130 / 126; 1024: - / 140 / 133; earlier, 4096: 245 / - / 261.  Down
//    by N (us, same box, mean of two runs for the 256-row form; 256 rows as
//    4 x two / 256 rows as 8 x one / 512 rows as 8 x two): N = 1024: 83.1 /
//    78.6 / 83.8; 2048: 112.3 / 104.5 / 115.8; 4096: 157.3 / 160.3 / 165.7;
//    6144: 210.6 / 217.6 / 209.9; 8192: 277.6 / 299.0 / 264.8; 16384: 497.2
//    / 541.0 / 470.8.  With eight wavefronts a workgroup has a CU to itself
//    and its token tile feeds twice the weight rows.
//  * FP8, 257-2048 tokens: 128 weight rows and 128 token rows for both
//    kernels; above, gate/up 512 rows (8 x two), down 256 rows (4 x two) up
//    to 6144 tokens and 512 (8 x two) above.  Measured (us, gate/up 128 /
//    256 / 512 rows; down 128 / 256 (8 x one) / 512 / 256 (4 x two) rows):
//    N = 512: 66.9 / 72.3 / 87.7, 49.2 / 48.7 / 49.9 / 54.8; 2048: 115.2 /
//    117.6-118.8 / 120.5, 80.5 / 88.3 / 83.5 / 82.7; 4096: 180.5-181.1 /
//    182.0 / 165.5, 129.2-129.7 / 128.1-128.9 / 125.1-125.4 / 122.0-122.4.
// Weight loads: up to kOneTouchTokens tokens most experts have a single
// m-tile, so each weight byte is read once and the loads are non-temporal
// (layer us, same box, plain / non-temporal: N = 160: 149.5-152.9 /
// 141.8-144.3; 320: 174.1-177.9 / 164.5-168.5; 640: 219-220 both); above,
// the m-tiles of an expert share its weight tiles through the L2 and
// non-temporal loads cost (N = 2048: 333 / 362-368; 4096: 465-476 / 532-535).
// The FP8 kernels follow the same rule (FP8 layer us: N = 300: 141.1-141.6 /
// 138.0-138.9; 400: 156.1-156.3 / 152.3-152.4; 512: 166.4-167.0 /
// 165.5-165.9).
constexpr int64_t kOneTouchTokens = 512;
constexpr int64_t kShortTileTokens = 256;  // 128 weight rows, short token tiles
constexpr int64_t kBf16TB1Tokens = 96;     // bf16: 32-row token tiles up to here; 64 weight rows (down: FP8 too)
constexpr int64_t kFp8NarrowTokens = 2048; // FP8: 128 x 128 tiles up to here

template <bool GATEUP, int FB, int WAVES = (GATEUP ? 8 : 4), int TB = 4, bool FP8 = false,
          bool NTW = false, bool SELF = false, typename Out>
hipError_t launch_tiled(const void* A, const void* W, const int32_t* idx, int32_t* offsets,
                        int32_t* row2slot, Out* out, int64_t N, hipStream_t stream,
                        const float* Ws = nullptr, const float* As = nullptr) {
  uint16_t* H = nullptr;
  float* Y = nullptr;
  if constexpr (GATEUP) H = out; else Y = out;
  // Token matrices below 2 GB are addressed with 32-bit offsets, padding
  // rows with offset 2^31 (see the kernel); the one-block shapes serve at
  // most 2,048 tokens, whose token matrices always are.
  constexpr int kRowBytes = (GATEUP ? kHidden : kFF) * (FP8 ? 1 : 2);
  const bool off32 = (GATEUP ? N : kTopK * N) * kRowBytes < (int64_t{1} << 31);
  const dim3 grid(static_cast<unsigned>(tiled_grid<GATEUP, FB, WAVES, TB>(N)));
  const dim3 block(TileShape<GATEUP, FB, WAVES, TB>::kThreads);
  if constexpr (FB == 1) {
    if (!off32) return hipErrorInvalidValue;
    hipLaunchKernelGGL((expert_tiled_kernel<GATEUP, FB, WAVES, TB, FP8, NTW, SELF, true>), grid, block, 0,
                       stream, A, W, idx, static_cast<int>(N), offsets, row2slot, H, Y, Ws, As);
  } else if (off32) {
    hipLaunchKernelGGL((expert_tiled_kernel<GATEUP, FB, WAVES, TB, FP8, NTW, SELF, true>), grid, block, 0,
                       stream, A, W, idx, static_cast<int>(N), offsets, row2slot, H, Y, Ws, As);
  } else {
    hipLaunchKernelGGL((expert_tiled_kernel<GATEUP, FB, WAVES, TB, FP8, NTW, SELF, false>), grid, block, 0,
                       stream, A, W, idx, static_cast<int>(N), offsets, row2slot, H, Y, Ws, As);
  }
  return hipGetLastError();
}

}  // namespace

// bf16: up to 512 tokens (N = 320 / 512, layer us, dispatch step / grouping
// in the gate/up kernel: 192.5-196.2 / 188.6-189.6, 215.5-216.7 /
// 211.6-212.0; with the grouping up to 1,024 tokens N = 1,024 took
// 250.4-253.1 / 251.2-254.2).  FP8: up to 256 tokens (at N = 320 the FP8
// layer took 136.8-137.3 with the dispatch step, 143.1-143.6 without).
bool gateup_groups_slots(int64_t N, bool fp8) { return N <= (fp8 ? kShortTileTokens : kSelfTokens); }
static_assert(kShortTileTokens <= kSelfShortTokens && kOneTouchTokens == kSelfTokens,
              "the grouping fits the tiles that take it");

hipError_t launch_gateup_tiled(const uint16_t* X, const uint16_t* Wgu, const int32_t* idx,
                               int32_t* offsets, int32_t* row2slot, uint16_t* H, int64_t N,
                               hipStream_t stream) {
  if (N <= kBf16TB1Tokens)
    return launch_tiled<true, 1, 2, 1, false, true, true>(X, Wgu, idx, offsets, row2slot, H, N, stream);
  if (N <= kShortTileTokens)
    return launch_tiled<true, 1, 4, 2, false, true, true>(X, Wgu, idx, offsets, row2slot, H, N, stream);
  if (N <= kOneTouchTokens)
    return launch_tiled<true, 1, 4, 4, false, true, true>(X, Wgu, idx, offsets, row2slot, H, N, stream);
  if (N <= 2048) return launch_tiled<true, 1>(X, Wgu, idx, offsets, row2slot, H, N, stream);
  return launch_tiled<true, 2>(X, Wgu, idx, offsets, row2slot, H, N, stream);
}

// The down kernels only read the grouping (their SELF mode is off).
hipError_t launch_down_tiled(const uint16_t* H, const uint16_t* Wd, const int32_t* offsets,
                             const int32_t* row2slot, float* Y, int64_t N, hipStream_t stream) {
  int32_t* off = const_cast<int32_t*>(offsets);
  int32_t* r2s = const_cast<int32_t*>(row2slot);
  if (N <= kBf16TB1Tokens)
    return launch_tiled<false, 1, 2, 1, false, true>(H, Wd, nullptr, off, r2s, Y, N, stream);
  if (N <= kShortTileTokens)
    return launch_tiled<false, 1, 4, 2, false, true>(H, Wd, nullptr, off, r2s, Y, N, stream);
  if (N <= kOneTouchTokens)
    return launch_tiled<false, 1, 4, 4, false, true>(H, Wd, nullptr, off, r2s, Y, N, stream);
  if (N <= 2048) return launch_tiled<false, 1, 8>(H, Wd, nullptr, off, r2s, Y, N, stream);
  if (N <= 6144) return launch_tiled<false, 2>(H, Wd, nullptr, off, r2s, Y, N, stream);
  return launch_tiled<false, 2, 8>(H, Wd, nullptr, off, r2s, Y, N, stream);
}

hipError_t launch_gateup_tiled_fp8(const uint8_t* Xq, const uint8_t* Wq, const float* Ws,
                                   const float* Xs, const int32_t* idx, int32_t* offsets,
                                   int32_t* row2slot, uint16_t* H, int64_t N, hipStream_t stream) {
  if (N <= kShortTileTokens)
    return launch_tiled<true, 1, 4, 2, true, true, true>(Xq, Wq, idx, offsets, row2slot, H, N, stream, Ws, Xs);
  if (N <= kOneTouchTokens)
    return launch_tiled<true, 1, 4, 4, true, true>(Xq, Wq, idx, offsets, row2slot, H, N, stream, Ws, Xs);
  if (N <= kFp8NarrowTokens)
    return launch_tiled<true, 1, 4, 4, true>(Xq, Wq, idx, offsets, row2slot, H, N, stream, Ws, Xs);
  return launch_tiled<true, 2, 8, 4, true>(Xq, Wq, idx, offsets, row2slot, H, N, stream, Ws, Xs);
}

hipError_t launch_down_tiled_fp8(const uint8_t* Hq, const uint8_t* Wq, const float* Ws,
                                 const float* Hs, const int32_t* offsets, const int32_t* row2slot,
                                 float* Y, int64_t N, hipStream_t stream) {
  int32_t* off = const_cast<int32_t*>(offsets);
  int32_t* r2s = const_cast<int32_t*>(row2slot);
  if (N <= kBf16TB1Tokens)
    return launch_tiled<false, 1, 2, 2, true, true>(Hq, Wq, nullptr, off, r2s, Y, N, stream, Ws, Hs);
  if (N <= kShortTileTokens)
    return launch_tiled<false, 1, 4, 2, true, true>(Hq, Wq, nullptr, off, r2s, Y, N, stream, Ws, Hs);
  if (N <= kOneTouchTokens)
    return launch_tiled<false, 1, 4, 4, true, true>(Hq, Wq, nullptr, off, r2s, Y, N, stream, Ws, Hs);
  if (N <= kFp8NarrowTokens)
    return launch_tiled<false, 1, 4, 4, true>(Hq, Wq, nullptr, off, r2s, Y, N, stream, Ws, Hs);
  // The two-block shapes spill a few registers (outside the stage loop)
  // only with 64-bit row pointers (token matrices of 2 GB or more).
  if (N <= 6144)
    return launch_tiled<false, 2, 4, 4, true>(Hq, Wq, nullptr, off, r2s, Y, N, stream, Ws, Hs);
  return launch_tiled<false, 2, 8, 4, true>(Hq, Wq, nullptr, off, r2s, Y, N, stream, Ws, Hs);
}

}  // namespace lfm

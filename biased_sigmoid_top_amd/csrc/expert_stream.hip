// Expert GEMMs that stream the weights straight into MFMA registers: the
// path of the smallest batches (up to kDecodeMaxTokens tokens).
//
// Method: each selected expert is a gated SiLU MLP with three matrices
// (flozi.net guide "LFM2.5-24B-A2B: Biased Routing, Short Convolutions and
// Ten KV Caches", section "The router has two different scores"):
//   H = silu(X_e W_gate_e^T) * (X_e W_up_e^T)    (bf16 out, fp32 accumulate)
//   Y = H_e W_down_e^T                           (fp32 out)
// and the expert path groups tokens by expert (section "What to verify in a
// deployment").
//
// With a handful of tokens per expert the work is bound by reading each
// active expert's weights from HBM once.  Weights are in the packed
// fragment layout (pack.hip), so each wavefront load of a weight operand is
// one contiguous 1 KB non-temporal read that lands directly in the A
// registers of a 32x32x16 MFMA, and every weight fragment is read once.  Up
// to 32 tokens of an expert form the B operand of one pass.
//
// Work split: the work is cut into units -- one expert's 16 H columns (128
// KB of gate/up weights) or 32 output features (96 KB of down weights) --
// and the grid is one workgroup per CU, each taking a contiguous range of
// units cut at equal numbers of (unit, 32-token pass) sub-units (measured:
// handing units out from a device counter is slower, because same-address
// atomics serialise).  The wavefronts of a workgroup stream a unit
// together, each over its slice of K, and add their partial tiles in LDS in
// wavefront order (so the result does not depend on the grid).  While a
// unit is computed the next units' weights are already in flight.  A
// wavefront keeps its slice of the token rows (the B operand) in registers
// across the units of one expert and pass, and loads them ahead of the
// weight prefetch when they change.  Every workgroup first groups the batch's slots by expert in
// LDS (a stable counting sort with per-expert token bitmasks); no dispatch
// step and no host readback are needed.
//
// H and Y rows are stored in slot order (row t*4 + j holds token t's j-th
// selected expert), which the combine step reads back contiguously.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kPassRows = 32;                      // tokens per pass (one 32x32 MFMA tile)
constexpr int kStreamWaves = 16;                   // most wavefronts of a streaming workgroup
constexpr int kMaskWords = kStreamMaxTokens / 32;

// Byte offset of the first K-step fragment of row block b of expert e.
template <bool GATEUP>
__device__ __forceinline__ uint32_t block_bytes(int e, int b) {
  return static_cast<uint32_t>(GATEUP ? (e * kGateupBlocks + b) * kGateupSteps
                                      : (e * kDownBlocks + b) * kDownSteps) * kFragBytes;
}

// Grouping of the batch's slots by expert, in LDS.
struct Grouping {
  int cnt[kExperts];
  int off[kExperts + 1];
  int active[kExperts];
  int n_active;
  uint32_t mask[kExperts][kMaskWords];  // bit t: token t chose the expert
  int list[kStreamMaxTokens * kTopK];   // slots grouped by expert, token order
};

// Workgroup state: the grouping and the wavefronts' partial tiles.
struct StreamShared {
  Grouping G;
  float red[kStreamWaves][16][kWave];  // value r of lane l of each wavefront
};

// Groups the slots t*4 + j of N <= kStreamMaxTokens tokens by expert.
__device__ void group_slots(const int32_t* __restrict__ idx, int N, Grouping& G) {
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  for (int i = tid; i < kExperts * kMaskWords; i += nthreads) (&G.mask[0][0])[i] = 0u;
  if (tid < kExperts) G.cnt[tid] = 0;
  __syncthreads();
  for (int t = tid; t < N; t += nthreads) {
    const int4 v = *reinterpret_cast<const int4*>(idx + static_cast<size_t>(t) * kTopK);
    const int es[kTopK] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
      atomicOr(&G.mask[es[j]][t / 32], 1u << (t % 32));
      atomicAdd(&G.cnt[es[j]], 1);
    }
  }
  __syncthreads();
  if (tid < kWave) {
    const int c = G.cnt[tid];
    const int incl = wave_inclusive_scan(c, tid);
    G.off[tid] = incl - c;
    if (tid == kExperts - 1) G.off[kExperts] = incl;
    const unsigned long long act = __ballot(c > 0);
    if (c > 0) G.active[__popcll(act & ((1ull << tid) - 1ull))] = tid;
    if (tid == 0) G.n_active = __popcll(act);
  }
  __syncthreads();
  for (int t = tid; t < N; t += nthreads) {
    const int4 v = *reinterpret_cast<const int4*>(idx + static_cast<size_t>(t) * kTopK);
    const int es[kTopK] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
      const int e = es[j];
      int rank = __popc(G.mask[e][t / 32] & ((1u << (t % 32)) - 1u));
      for (int w = 0; w < t / 32; ++w) rank += __popc(G.mask[e][w]);
      G.list[G.off[e] + rank] = t * kTopK + j;
    }
  }
  __syncthreads();
}

// Contiguous share [begin, end) of the units of all active experts (in
// active-expert order, kUnitsPerExpert per expert) for this workgroup.  A
// unit is streamed once per pass of 32 tokens of its expert, so the shares
// are cut at equal numbers of (unit, pass) sub-units; with one pass per
// expert this is an equal split of the units.
template <int kUnitsPerExpert>
__device__ __forceinline__ void my_share(const Grouping& G, int& begin, int& end) {
  const int n = uniform(G.n_active);
  auto passes = [&](int i) { return (G.cnt[G.active[i]] + kPassRows - 1) / kPassRows; };
  int64_t total = 0;
  for (int i = 0; i < n; ++i) total += static_cast<int64_t>(kUnitsPerExpert) * passes(i);
  // First unit whose first sub-unit is at or after sub-unit t.
  auto unit_at = [&](int64_t t) {
    int64_t P = 0;
    for (int i = 0; i < n; ++i) {
      const int w = passes(i);
      const int64_t next = P + static_cast<int64_t>(kUnitsPerExpert) * w;
      if (t < next) return i * kUnitsPerExpert + static_cast<int>((t - P + w - 1) / w);
      P = next;
    }
    return n * kUnitsPerExpert;
  };
  begin = uniform(unit_at(total * blockIdx.x / gridDim.x));
  end = uniform(unit_at(total * (blockIdx.x + 1) / gridDim.x));
}

// This lane's token of a pass: slot of row lane % 32 (rows past `rows`
// repeat the first row; their results are discarded).
__device__ __forceinline__ int pass_slot(const int* slots, int rows, int lane) {
  const int r = lane % 32;
  return slots[r < rows ? r : 0];
}

// Position in a workgroup's sequence of sub-units: unit u, pass `pass` over
// the expert's rows (kPassRows at a time), half p of the unit's K range.
// All values are uniform.
struct Cursor {
  int u, pass, p;
};

// The per-wavefront pipeline shared by the two kernels.
//   GATEUP: unit = row block b of the packed gate/up weights of one expert
//           (16 H columns: 16 gate rows and 16 up rows); B operand = rows
//           of X; K = 2048 (128 K steps of 16).
//   down:   unit = row block b of W_down (32 output features); B operand =
//           rows of H; K = 1536 (96 K steps).
// Each wavefront covers kS = K steps / 16 consecutive K steps of every
// unit, in two halves of kF = kS / 2.  The weights of a half (kF fragments
// per wavefront, 64 KB (gate/up) or 48 KB (down) per workgroup) go through
// a ring of three register buffers, so two halves are in flight while one
// is multiplied.  The 16 partial 32x32 tiles of a unit are added in LDS in
// wavefront order.
template <bool GATEUP, int WAVES>
__device__ __forceinline__ void stream_units(const uint16_t* __restrict__ B,
                                             const uint16_t* __restrict__ Wp,
                                             uint16_t* __restrict__ H, float* __restrict__ Y,
                                             int N, StreamShared& S) {
  constexpr int K = GATEUP ? kHidden : kFF;
  constexpr int kS = (GATEUP ? kGateupSteps : kDownSteps) / WAVES;  // K steps per wavefront
  constexpr int kF = kS / 2;
  constexpr int kUnitsPerExpert = GATEUP ? kGateupBlocks : kDownBlocks;
  int begin, end;
  my_share<kUnitsPerExpert>(S.G, begin, end);
  if (begin >= end) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint32_t lane_bytes = lane * 16;
  const uint32_t kcol_bytes = (wave * kS * 16 + (lane / 32) * 8) * 2;  // this lane's first K column
  const Rsrc wr = make_rsrc(Wp, static_cast<uint32_t>(kExperts) * 2 * kFF * kHidden * (GATEUP ? 2 : 1));
  const Rsrc br = make_rsrc(B, static_cast<uint32_t>(N) * (GATEUP ? 1 : kTopK) * K * 2);

  auto expert_of = [&](int u) { return uniform(S.G.active[u / kUnitsPerExpert]); };
  auto count_of = [&](int e) { return uniform(S.G.off[e + 1] - S.G.off[e]); };
  // Next (unit, pass) after c: the next unit of the expert's run in the
  // share, else the run's first unit for the next pass, else the next
  // expert's first unit.
  auto next_unit = [&](Cursor& c) {
    const int run = c.u / kUnitsPerExpert;
    if (++c.u < min(end, (run + 1) * kUnitsPerExpert)) return;
    if (++c.pass * kPassRows < count_of(expert_of(c.u - 1))) {
      c.u = max(begin, run * kUnitsPerExpert);
      return;
    }
    c.pass = 0;
  };
  // Order of the sub-units: within the share's units of one expert, all
  // units for one pass of 32 tokens, then all again for the next pass, so
  // the token rows change once per pass (an expert's weights are streamed
  // once per pass either way).  Past the end of the share a cursor stays
  // put (its loads are dummies), so no expert past the last active one is
  // looked up.
  auto advance = [&](Cursor& c) {
    if (c.u >= end) return;
    c.p ^= 1;
    if (c.p == 0) next_unit(c);
  };
  // Issues the weight loads of sub-unit c.  Past the end of the share the
  // loads are still issued, with an offset outside the buffer (they return
  // zeros without touching memory), so that every path through the loop
  // has the same number of loads in flight and the waits stay exact.
  auto issue = [&](const Cursor& c, uint4 (&w)[kF]) {
    const bool live = c.u < end;
    const int u = live ? c.u : begin;
    const uint32_t base = uniform(block_bytes<GATEUP>(expert_of(u), u % kUnitsPerExpert) +
                                  (wave * kS + c.p * kF) * kFragBytes);
    const uint32_t voff = live ? lane_bytes : 0x80000000u + lane_bytes;
#pragma unroll
    for (int f = 0; f < kF; ++f) w[f] = buf_ld<true>(wr, voff, base + f * kFragBytes);
  };

  uint4 w0[kF], w1[kF], w2[kF], xb[kS];
  f32x16 acc;
  int xe = -1, xpass = -1;  // expert and pass whose rows are in xb
  // Loads this lane's token row for the pass of cursor c (unless present).
  auto load_rows = [&](const Cursor& c) {
    if (c.u >= end) return;
    const int e = expert_of(c.u);
    if (e == xe && c.pass == xpass) return;
    const int r0 = c.pass * kPassRows;
    const int rows = min(kPassRows, count_of(e) - r0);
    const int slot = pass_slot(S.G.list + S.G.off[e] + r0, rows, lane);
    const uint32_t bo = (GATEUP ? slot / kTopK : slot) * (K * 2) + kcol_bytes;
#pragma unroll
    for (int f = 0; f < kS; ++f) xb[f] = buf_ld<false>(br, bo, f * 32);
    xe = e;
    xpass = c.pass;
  };

  Cursor cp{begin, 0, 0}, ld{begin, 0, 0};
  load_rows(cp);
  issue(ld, w0);
  advance(ld);
  issue(ld, w1);
  advance(ld);

  // One sub-unit: wc holds its weights; the loads two sub-units ahead go
  // to wi.  Order: multiply, then (at the end of a unit) the next unit's
  // token rows, then the weight loads, then the cross-wavefront reduction,
  // so a multiply only ever waits for its own operands.
  auto step = [&](auto half, uint4 (&wc)[kF], uint4 (&wi)[kF]) -> bool {
    constexpr int P = decltype(half)::value;
    if (cp.u >= end) return false;
    if (P == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    }
#pragma unroll
    for (int f = 0; f < kF; ++f) acc = mfma32(wc[f], xb[P * kF + f], acc);
    const Cursor cur = cp;
    advance(cp);
    if (P == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S.red[wave][r][lane] = acc[r];
      load_rows(cp);
    }
    issue(ld, wi);
    advance(ld);
    if (P == 1) {
      __syncthreads();
      const int e = expert_of(cur.u);
      const int r0 = cur.pass * kPassRows;
      const int rows = min(kPassRows, count_of(e) - r0);
      const int* slots = S.G.list + S.G.off[e] + r0;
      const int b = cur.u % kUnitsPerExpert;
      // Thread (r, ln) adds value r of lane ln over the wavefronts (token
      // ln % 32, row mfma32_row(r, ln) of the unit's 32-row tile), for r =
      // its wavefront index and, with fewer than 16 wavefronts, r + WAVES.
      const int ln = threadIdx.x % kWave;
      if (ln % 32 < rows) {
        const int slot = slots[ln % 32];
        for (int r = threadIdx.x / kWave; r < 16; r += WAVES) {
          if (GATEUP) {
            if (r < 8) {  // rows r (gate) and r + 8 (up) hold H column mfma32_row(r, ln)
              float gs = 0.f, us = 0.f;
#pragma unroll
              for (int w = 0; w < WAVES; ++w) {
                gs += S.red[w][r][ln];
                us += S.red[w][r + 8][ln];
              }
              H[static_cast<size_t>(slot) * kFF + b * 16 + mfma32_row(r, ln)] =
                  f32_to_bf16(silu(gs) * us);
            }
          } else {
            float ys = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) ys += S.red[w][r][ln];
            Y[static_cast<size_t>(slot) * kHidden + b * 32 + mfma32_row(r, ln)] = ys;
          }
        }
      }
      __syncthreads();
    }
    return true;
  };
  // Both halves of one pass: a and b hold their weights, c is free.
  auto pass = [&](uint4 (&a)[kF], uint4 (&b)[kF], uint4 (&c)[kF]) -> bool {
    if (!step(std::integral_constant<int, 0>{}, a, c)) return false;
    return step(std::integral_constant<int, 1>{}, b, a);
  };
  // Sub-unit s uses buffer s % 3: unrolled by three passes.
  for (;;) {
    if (!pass(w0, w1, w2)) break;
    if (!pass(w2, w0, w1)) break;
    if (!pass(w1, w2, w0)) break;
  }
}

// FP8 experts (pack_fp8.hip): 1 KB fragments of 32 rows x 32 K, one
// 16-byte load per lane holding its operands of two 16-wide K steps; a fp32
// scale per 128 x 128 weight block.  Each wavefront covers GPW 128-wide K
// groups of a unit (gate/up: 2 groups, 8 wavefronts; down: 1 group, 12
// wavefronts).  A group is both a weight block's columns and an activation
// group: the wavefront loads its slice of the bf16 token rows, quantises it
// per token and group (largest magnitude of the token's 128 values, codes
// E4M3(x * (448 / amax)), scale amax / 448 -- the activation quantisation
// of the inferencekey.com page's FP8_BLOCK entry), multiplies each group
// into its own accumulator, and adds the groups' products times weight scale
// x token scale into its partial tile before the cross-wavefront sum.  Two
// groups per wavefront halve the partial tiles a unit reduces through LDS
// (measured gate/up: 62.1 -> 58.9 us at N = 64, 40 experts; no gain for
// down).  One unit per step (4 GPW fragments per wavefront), three units in
// the register ring.
//
// The products run on the bf16 MFMA: both operands' codes are widened to
// bf16 in registers (E4M3 values are bf16 values, and their products are
// exact in fp32), so the sums are fp32 sums of exact products.  The FP8
// MFMA is not used: measured on gfx950, it adds each group of 8 products
// after aligning them to the group's largest exponent and truncating to 13
// fraction bits, an error of up to 2^-10 of the largest product, where the
// bf16 MFMA returns the correctly rounded fp32 sum.  The loop is bound by
// the weight stream, so the widening costs no time.
constexpr uint32_t kFp8FragBytes = 1024;

template <bool GATEUP>
__device__ __forceinline__ uint32_t fp8_block_bytes(int e, int b) {
  constexpr int kPairs = (GATEUP ? kHidden : kFF) / 32;
  constexpr int kBlocks = GATEUP ? kGateupBlocks : kDownBlocks;
  return static_cast<uint32_t>((e * kBlocks + b) * kPairs) * kFp8FragBytes;
}

template <bool GATEUP, int GPW, int RING>
__device__ __forceinline__ void stream_units_fp8(const uint16_t* __restrict__ B,
                                                 const uint8_t* __restrict__ Wq,
                                                 const float* __restrict__ Ws,
                                                 uint16_t* __restrict__ H, float* __restrict__ Y,
                                                 int N, StreamShared& S) {
  constexpr int K = GATEUP ? kHidden : kFF;
  constexpr int kWaves = K / (128 * GPW);  // GPW 128-wide groups per wavefront
  constexpr int kFrags = 4 * GPW;          // 128 K = 4 fragments of 32 K
  constexpr int kSteps = 8 * GPW;          // 16-wide K steps per wavefront
  constexpr int kUnitsPerExpert = GATEUP ? kGateupBlocks : kDownBlocks;
  int begin, end;
  my_share<kUnitsPerExpert>(S.G, begin, end);
  if (begin >= end) return;
  const int lane = threadIdx.x & (kWave - 1);
  // Uniform, so that the per-group scale reads are scalar loads: a vector
  // load here would make the wait for it drain the weight ring at every unit.
  const int wave = uniform(static_cast<int>(threadIdx.x / kWave));
  const uint32_t lane_bytes = lane * 16;
  const uint32_t kcol_bytes = (wave * 128 * GPW + (lane / 32) * 8) * 2;  // this lane's first bf16 K column
  const Rsrc wr = make_rsrc(Wq, static_cast<uint32_t>(kExperts) * kHidden * kFF * (GATEUP ? 2 : 1));
  const Rsrc br = make_rsrc(B, static_cast<uint32_t>(N) * (GATEUP ? 1 : kTopK) * K * 2);

  auto expert_of = [&](int u) { return uniform(S.G.active[u / kUnitsPerExpert]); };
  auto count_of = [&](int e) { return uniform(S.G.off[e + 1] - S.G.off[e]); };
  // Next (unit, pass) after c: the next unit of the expert's run in the
  // share, else the run's first unit for the next pass, else the next
  // expert's first unit.
  auto next_unit = [&](Cursor& c) {
    const int run = c.u / kUnitsPerExpert;
    if (++c.u < min(end, (run + 1) * kUnitsPerExpert)) return;
    if (++c.pass * kPassRows < count_of(expert_of(c.u - 1))) {
      c.u = max(begin, run * kUnitsPerExpert);
      return;
    }
    c.pass = 0;
  };
  // Sub-unit order as in stream_units: pass-major within the share's units
  // of one expert.
  auto advance = [&](Cursor& c) {
    if (c.u >= end) return;
    next_unit(c);
  };
  // Weight loads of unit c (past the end of the share: an offset outside the
  // buffer, which returns zeros, so every path keeps the same loads in flight).
  auto issue = [&](const Cursor& c, uint4 (&w)[kFrags]) {
    const bool live = c.u < end;
    const int u = live ? c.u : begin;
    const uint32_t base = uniform(fp8_block_bytes<GATEUP>(expert_of(u), u % kUnitsPerExpert) +
                                  wave * kFrags * kFp8FragBytes);
    const uint32_t voff = live ? lane_bytes : 0x80000000u + lane_bytes;
#pragma unroll
    for (int f = 0; f < kFrags; ++f) w[f] = buf_ld<true>(wr, voff, base + f * kFp8FragBytes);
  };

  // Token rows: 8 bf16 K steps per group and lane as loaded; quantised in
  // place to the bf16 values of their E4M3 codes (K step k stays in xb[k]).
  uint4 w[RING][kFrags], xb[kSteps];
  float xscale[GPW] = {};
  bool fresh = false;
  int xe = -1, xpass = -1;
  auto load_rows = [&](const Cursor& c) {
    if (c.u >= end) return;
    const int e = expert_of(c.u);
    if (e == xe && c.pass == xpass) return;
    const int r0 = c.pass * kPassRows;
    const int rows = min(kPassRows, count_of(e) - r0);
    const int slot = pass_slot(S.G.list + S.G.off[e] + r0, rows, lane);
    const uint32_t bo = (GATEUP ? slot / kTopK : slot) * (K * 2) + kcol_bytes;
#pragma unroll
    for (int f = 0; f < kSteps; ++f) xb[f] = buf_ld<false>(br, bo, f * 32);
    xe = e;
    xpass = c.pass;
    fresh = true;
  };
  auto quantize_rows = [&] {
#pragma unroll
    for (int g = 0; g < GPW; ++g) {
      // Largest magnitude of the group: on the bf16 bit patterns (the order
      // of finite non-negative floats is that of their bits).
      uint32_t m = 0;
#pragma unroll
      for (int f = 8 * g; f < 8 * g + 8; ++f) {
        const uint32_t w4[4] = {xb[f].x, xb[f].y, xb[f].z, xb[f].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) m = max(m, max(w4[k] & 0x7fffu, (w4[k] >> 16) & 0x7fffu));
      }
      float amax = __uint_as_float(m << 16);
      // Lanes l and l ^ 32 hold the two halves of the same token's group.
      amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
      const float inv = amax > 0.f ? 448.f / amax : 0.f;
      xscale[g] = amax / 448.f;
      auto q4 = [&](uint32_t lo, uint32_t hi) {
        return e4m3x4(__uint_as_float(lo << 16) * inv, __uint_as_float(lo & 0xffff0000u) * inv,
                      __uint_as_float(hi << 16) * inv, __uint_as_float(hi & 0xffff0000u) * inv);
      };
#pragma unroll
      for (int k = 8 * g; k < 8 * g + 8; ++k)
        xb[k] = e4m3x8_to_bf16(q4(xb[k].x, xb[k].y), q4(xb[k].z, xb[k].w));
    }
  };

  Cursor cp{begin, 0, 0}, ld{begin, 0, 0};
  load_rows(cp);
#pragma unroll
  for (int r = 0; r + 1 < RING; ++r) {
    issue(ld, w[r]);
    advance(ld);
  }

  // One unit: multiply the weights in wc, issue the loads RING - 1 units ahead
  // into wi, add the partial tiles.  Past the end of the share (the last
  // round of the loop) the arithmetic and the stores are skipped while the
  // loads and barriers still run: the loop then has a single exit, and the
  // compiler's counts of loads in flight stay exact around it (with an exit
  // after every unit they merge into a full drain of the ring each unit).
  auto step = [&](uint4 (&wc)[kFrags], uint4 (&wi)[kFrags]) {
    const bool live = cp.u < end;
    const Cursor cur = cp;
    if (live) {
      if (fresh) {
        quantize_rows();
        fresh = false;
      }
      // One accumulator per K group: the groups have their own scales.
      f32x16 acc[GPW];
#pragma unroll
      for (int g = 0; g < GPW; ++g) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[g][r] = 0.f;
#pragma unroll
        for (int f = 4 * g; f < 4 * g + 4; ++f) {
          acc[g] = mfma32(e4m3x8_to_bf16(wc[f].x, wc[f].y), xb[2 * f], acc[g]);
          acc[g] = mfma32(e4m3x8_to_bf16(wc[f].z, wc[f].w), xb[2 * f + 1], acc[g]);
        }
      }
      const int e = expert_of(cur.u);
      const int b = cur.u % kUnitsPerExpert;
      // Each group's products times weight scale x token scale, the groups
      // added in order: this wavefront's partial tile.
      if (GATEUP) {
        float sg[GPW], su[GPW];
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
          const int kg = wave * GPW + g;
          sg[g] = Ws[((e * 2 + 0) * (kFF / 128) + b / 8) * (kHidden / 128) + kg] * xscale[g];
          su[g] = Ws[((e * 2 + 1) * (kFF / 128) + b / 8) * (kHidden / 128) + kg] * xscale[g];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = acc[0][r] * (r < 8 ? sg[0] : su[0]);
#pragma unroll
          for (int g = 1; g < GPW; ++g) v += acc[g][r] * (r < 8 ? sg[g] : su[g]);
          S.red[wave][r][lane] = v;
        }
      } else {
        float sd[GPW];
#pragma unroll
        for (int g = 0; g < GPW; ++g)
          sd[g] = Ws[(e * (kHidden / 128) + b / 4) * (kFF / 128) + wave * GPW + g] * xscale[g];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = acc[0][r] * sd[0];
#pragma unroll
          for (int g = 1; g < GPW; ++g) v += acc[g][r] * sd[g];
          S.red[wave][r][lane] = v;
        }
      }
    }
    advance(cp);
    load_rows(cp);
    issue(ld, wi);
    advance(ld);
    __syncthreads();
    if (live) {
      const int e = expert_of(cur.u);
      const int b = cur.u % kUnitsPerExpert;
      const int r0 = cur.pass * kPassRows;
      const int rows = min(kPassRows, count_of(e) - r0);
      const int* slots = S.G.list + S.G.off[e] + r0;
      // Thread (r, ln) adds value r of lane ln over the wavefronts (token
      // ln % 32, row mfma32_row(r, ln) of the unit's 32-row tile), for r =
      // its wavefront index and, with fewer than 16 wavefronts, r + kWaves.
      const int ln = threadIdx.x % kWave;
      if (ln % 32 < rows) {
        const int slot = slots[ln % 32];
        for (int r = threadIdx.x / kWave; r < 16; r += kWaves) {
          if (GATEUP) {
            if (r < 8) {  // rows r (gate) and r + 8 (up) hold H column mfma32_row(r, ln)
              float gs = 0.f, us = 0.f;
#pragma unroll
              for (int w = 0; w < kWaves; ++w) {
                gs += S.red[w][r][ln];
                us += S.red[w][r + 8][ln];
              }
              H[static_cast<size_t>(slot) * kFF + b * 16 + mfma32_row(r, ln)] = f32_to_bf16(silu(gs) * us);
            }
          } else {
            float ys = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) ys += S.red[w][r][ln];
            Y[static_cast<size_t>(slot) * kHidden + b * 32 + mfma32_row(r, ln)] = ys;
          }
        }
      }
    }
    __syncthreads();
  };
  // Unit s uses buffer s % RING.
  do {
#pragma unroll
    for (int r = 0; r < RING; ++r) step(w[r], w[(r + RING - 1) % RING]);
  } while (cp.u < end);
}

// K groups of 128 per wavefront: gate/up 2 (8 wavefronts), down 1 (12).
constexpr int kFp8GateupGroups = 2;
constexpr int kFp8DownGroups = 1;
constexpr int kFp8Ring = 3;  // units of weights in the register ring (two in flight)
constexpr int kFp8GateupThreads = kHidden / (128 * kFp8GateupGroups) * kWave;
constexpr int kFp8DownThreads = kFF / (128 * kFp8DownGroups) * kWave;

__global__ __launch_bounds__(kFp8GateupThreads) void gateup_decode_fp8_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wq, const float* __restrict__ Ws,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ H, int N) {
  __shared__ StreamShared S;
  group_slots(idx, N, S.G);
  stream_units_fp8<true, kFp8GateupGroups, kFp8Ring>(X, Wq, Ws, H, nullptr, N, S);
}

__global__ __launch_bounds__(kFp8DownThreads) void down_decode_fp8_kernel(
    const uint16_t* __restrict__ H, const uint8_t* __restrict__ Wq, const float* __restrict__ Ws,
    const int32_t* __restrict__ idx, float* __restrict__ Y, int N) {
  __shared__ StreamShared S;
  group_slots(idx, N, S.G);
  stream_units_fp8<false, kFp8DownGroups, kFp8Ring>(H, Wq, Ws, nullptr, Y, N, S);
}

// Wavefronts splitting K: gate/up 16 (8 K steps each), down 16 (6 each).
// Eight wavefronts with twice the K each (half the partial tiles per unit)
// measured the same at N = 64 (gate/up 89.5-91.7 us, down 53.2-53.7 us
// either way, one box): unlike the FP8 kernels, a bf16 unit carries enough
// bytes for its reduction to stay a small share of its time.
constexpr int kGateupWaves = 16;
constexpr int kDownWaves = 16;

__global__ __launch_bounds__(kGateupWaves * kWave) void gateup_decode_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wgu,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ H, int N) {
  __shared__ StreamShared S;
  group_slots(idx, N, S.G);
  stream_units<true, kGateupWaves>(X, Wgu, H, nullptr, N, S);
}

__global__ __launch_bounds__(kDownWaves * kWave) void down_decode_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,
    const int32_t* __restrict__ idx, float* __restrict__ Y, int N) {
  __shared__ StreamShared S;
  group_slots(idx, N, S.G);
  stream_units<false, kDownWaves>(H, Wd, nullptr, Y, N, S);
}

int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

int64_t max_mtiles(int64_t N, int tile_rows) {
  const int64_t rows = N * kTopK;
  const int64_t a = (rows + static_cast<int64_t>(kExperts) * (tile_rows - 1)) / tile_rows;
  const int64_t b = static_cast<int64_t>(kExperts) * ((N + tile_rows - 1) / tile_rows);
  return a < b ? a : b;
}

hipError_t launch_gateup_decode(const uint16_t* X, const uint16_t* Wgu, const int32_t* idx,
                                uint16_t* H, int N, hipStream_t stream) {
  hipLaunchKernelGGL(gateup_decode_kernel, dim3(cu_count()), dim3(kGateupWaves * kWave), 0, stream, X,
                     Wgu, idx, H, N);
  return hipGetLastError();
}

hipError_t launch_down_decode(const uint16_t* H, const uint16_t* Wd, const int32_t* idx,
                              float* Y, int N, hipStream_t stream) {
  hipLaunchKernelGGL(down_decode_kernel, dim3(cu_count()), dim3(kDownWaves * kWave), 0, stream, H, Wd,
                     idx, Y, N);
  return hipGetLastError();
}

hipError_t launch_gateup_decode_fp8(const uint16_t* X, const uint8_t* Wq, const float* scales,
                                    const int32_t* idx, uint16_t* H, int N, hipStream_t stream) {
  hipLaunchKernelGGL(gateup_decode_fp8_kernel, dim3(cu_count()), dim3(kFp8GateupThreads), 0, stream,
                     X, Wq, scales, idx, H, N);
  return hipGetLastError();
}

hipError_t launch_down_decode_fp8(const uint16_t* H, const uint8_t* Wq, const float* scales,
                                  const int32_t* idx, float* Y, int N, hipStream_t stream) {
  hipLaunchKernelGGL(down_decode_fp8_kernel, dim3(cu_count()), dim3(kFp8DownThreads), 0, stream, H,
                     Wq, scales, idx, Y, N);
  return hipGetLastError();
}

}  // namespace lfm

// Expert GEMMs that stream the weights straight into MFMA registers: the
// decode-shaped path (few tokens per expert).
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
// one contiguous 1 KB non-temporal read that lands directly in the MFMA A
// registers, and every weight fragment is read once.
//
// Work split: the work is cut into units -- one expert's 16 H columns (128
// KB of gate/up weights) or 32 output features (96 KB of down weights) --
// and the grid is one 16-wavefront workgroup per CU, each taking an equal
// contiguous range of units (measured: handing units out from a device
// counter is slower, because same-address atomics serialise).  The 16
// wavefronts of a workgroup stream a unit together, each over one
// sixteenth of K, and add their partial tiles in LDS in wavefront order
// (so the result does not depend on the grid).  While a unit is computed
// the next unit's weights are already in flight.  A wavefront keeps its
// slice of the token rows (the B operand) in registers across the units of
// one expert, and loads them ahead of the weight prefetch when the expert
// changes.  Every workgroup first groups the batch's slots by expert in
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

constexpr int kFrag = 512;                         // bf16 elements per 16x32 fragment
constexpr int kDecodeTT = 2;                       // token tiles of 16 per pass
constexpr int kPassRows = 16 * kDecodeTT;
constexpr int kStreamThreads = 1024;               // 16 wavefronts: one workgroup per CU
constexpr int kStreamWaves = kStreamThreads / kWave;
constexpr int kMaskWords = kDecodeMaxTokens / 32;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer loads: a uniform base (SGPRs) plus a 32-bit per-lane byte offset,
// so that a wavefront's many loads share one address register.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16 bytes at byte offset voff + soff.  NT: read once, non-temporal.
template <bool NT>
__device__ __forceinline__ uint4 buf_ld(Rsrc r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT ? 2 : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr uint32_t kFragBytes = kFrag * 2;

// A value that is the same in every lane, made known to be so (kept in a
// scalar register).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

// Byte offset of the gate fragment (first K step) of 16-column block hb of
// expert e; the up fragment follows it, and K steps are 8 fragments apart
// (64-column groups of 4 blocks x gate/up).
__device__ __forceinline__ uint32_t gateup_frag_bytes(int e, int hb) {
  return static_cast<uint32_t>(((e * (kFF / 64) + hb / 4) * (kHidden / 32) * 8 + (hb % 4) * 2)) *
         kFragBytes;
}

// Byte offset of down-weight row tile rt (first K fragment) of expert e; the
// K fragments of a tile are 8 fragments apart, and the 8 tiles of a 128-row
// block are adjacent.
__device__ __forceinline__ uint32_t down_frag_bytes(int e, int rt) {
  return static_cast<uint32_t>(((e * (kHidden / 128) + rt / 8) * (kFF / 32) * 8 + rt % 8)) *
         kFragBytes;
}

// Grouping of the batch's slots by expert, in LDS.
struct Grouping {
  int cnt[kExperts];
  int off[kExperts + 1];
  int active[kExperts];
  int n_active;
  uint32_t mask[kExperts][kMaskWords];  // bit t: token t chose the expert
  int list[kDecodeMaxTokens * kTopK];   // slots grouped by expert, token order
};

// Workgroup state: the grouping and the wavefronts' partial tiles.
struct StreamShared {
  Grouping G;
  f32x4 red[kStreamWaves][2][kDecodeTT][kWave];
};

// Groups the slots t*4 + j of N <= kDecodeMaxTokens tokens by expert.
__device__ void group_slots(const int32_t* __restrict__ idx, int N, Grouping& G) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kExperts * kMaskWords; i += kStreamThreads) (&G.mask[0][0])[i] = 0u;
  if (tid < kExperts) G.cnt[tid] = 0;
  __syncthreads();
  for (int t = tid; t < N; t += kStreamThreads) {
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
  for (int t = tid; t < N; t += kStreamThreads) {
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

// Contiguous share [begin, end) of `units` work units for this workgroup.
__device__ __forceinline__ void my_share(int units, int& begin, int& end) {
  begin = static_cast<int>(static_cast<int64_t>(units) * blockIdx.x / gridDim.x);
  end = static_cast<int>(static_cast<int64_t>(units) * (blockIdx.x + 1) / gridDim.x);
}

// Once the wavefronts' partial tiles are in LDS, thread (tt, ln, q) of the
// first 512 adds up accumulator value q of lane ln of token tile tt: token
// row 16 tt + ln % 16, column 4 (ln / 16) + q of the 16-wide tile.
struct Owner {
  bool on;
  int tt, ln, q, row;
};
__device__ __forceinline__ Owner owner() {
  Owner o;
  o.on = threadIdx.x < kDecodeTT * kWave * 4;
  o.tt = (threadIdx.x / 256) % kDecodeTT;
  o.ln = (threadIdx.x / 4) % kWave;
  o.q = threadIdx.x % 4;
  o.row = o.tt * 16 + (o.ln & 15);
  return o;
}

// This lane's rows of a pass: slot of row tt*16 + r16 (rows past `rows`
// repeat the first row; their results are discarded).
__device__ __forceinline__ int pass_slot(const int* slots, int rows, int tt, int r16) {
  const int r = tt * 16 + r16;
  return slots[r < rows ? r : 0];
}

// Position in a workgroup's sequence of sub-units: unit u, pass `pass` over
// the expert's rows (kPassRows at a time), half p (gate / up fragments, or
// the first / second output tile of the unit).  All values are uniform.
struct Cursor {
  int u, pass, p;
};

// The per-wavefront pipeline shared by the two kernels.
//   GATEUP: unit = 16 H columns of one expert; half p streams the gate (0)
//           or up (1) weights; B operand = rows of X; K = 2048.
//   down:   unit = 32 output features of one expert; half p streams row
//           tile 2 (u % 64) + p; B operand = rows of H; K = 1536.
// Each wavefront covers kF = K / 32 / 16 K fragments of every half.  The
// weights of a half (kF fragments per wavefront, 64 KB (gate/up) or 48 KB
// (down) per workgroup) go through a ring of three register buffers, so two
// halves are in flight while one is multiplied.
template <bool GATEUP>
__device__ __forceinline__ void stream_units(const uint16_t* __restrict__ B,
                                             const uint16_t* __restrict__ Wp,
                                             uint16_t* __restrict__ H, float* __restrict__ Y,
                                             int N, StreamShared& S) {
  constexpr int K = GATEUP ? kHidden : kFF;
  constexpr int kF = (K / 32) / kStreamWaves;
  constexpr int kUnitsPerExpert = GATEUP ? kFF / 16 : kHidden / 32;
  int begin, end;
  my_share(uniform(S.G.n_active) * kUnitsPerExpert, begin, end);
  if (begin >= end) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r16 = lane & 15;
  const uint32_t lane_bytes = lane * 16;
  const uint32_t kcol_bytes = (wave * kF * 32 + (lane >> 4) * 8) * 2;  // this lane's first K column
  const Rsrc wr = make_rsrc(Wp, static_cast<uint32_t>(kExperts) * 2 * kFF * kHidden * (GATEUP ? 2 : 1));
  const Rsrc br = make_rsrc(B, static_cast<uint32_t>(N) * (GATEUP ? 1 : kTopK) * K * 2);

  auto expert_of = [&](int u) { return uniform(S.G.active[u / kUnitsPerExpert]); };
  auto count_of = [&](int e) { return uniform(S.G.off[e + 1] - S.G.off[e]); };
  auto advance = [&](Cursor& c) {
    c.p ^= 1;
    if (c.p == 0 && ++c.pass * kPassRows >= count_of(expert_of(c.u))) {
      c.pass = 0;
      ++c.u;
    }
  };
  // Issues the weight loads of sub-unit c.  Past the end of the share the
  // loads are still issued, with an offset outside the buffer (they return
  // zeros without touching memory), so that every path through the loop
  // has the same number of loads in flight and the waits stay exact.
  auto issue = [&](const Cursor& c, uint4 (&w)[kF]) {
    const bool live = c.u < end;
    const int u = live ? c.u : begin;
    const int e = expert_of(u);
    const int j = u % kUnitsPerExpert;
    const uint32_t base =
        uniform((GATEUP ? gateup_frag_bytes(e, j) : down_frag_bytes(e, 2 * j)) +
                (c.p + wave * kF * 8) * kFragBytes);
    const uint32_t voff = live ? lane_bytes : 0x80000000u + lane_bytes;
#pragma unroll
    for (int f = 0; f < kF; ++f) w[f] = buf_ld<true>(wr, voff, base + f * 8 * kFragBytes);
  };

  uint4 w0[kF], w1[kF], w2[kF], xb[kDecodeTT][kF];
  f32x4 acc[2][kDecodeTT];
  int xe = -1, xpass = -1;  // expert and pass whose rows are in xb
  // Loads this lane's token rows for the pass of cursor c (unless present).
  auto load_rows = [&](const Cursor& c) {
    if (c.u >= end) return;
    const int e = expert_of(c.u);
    if (e == xe && c.pass == xpass) return;
    const int r0 = c.pass * kPassRows;
    const int rows = min(kPassRows, count_of(e) - r0);
    const int* slots = S.G.list + S.G.off[e] + r0;
#pragma unroll
    for (int tt = 0; tt < kDecodeTT; ++tt) {
      const int slot = pass_slot(slots, rows, tt, r16);
      const uint32_t bo = (GATEUP ? slot / kTopK : slot) * (K * 2) + kcol_bytes;
#pragma unroll
      for (int f = 0; f < kF; ++f) xb[tt][f] = buf_ld<false>(br, bo, f * 64);
    }
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
  auto step = [&](auto half, uint4 (&wc)[kF], uint4 (&wi)[kF]) {
    constexpr int P = decltype(half)::value;
    if (P == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int tt = 0; tt < kDecodeTT; ++tt) acc[h][tt] = f32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int f = 0; f < kF; ++f)
#pragma unroll
      for (int tt = 0; tt < kDecodeTT; ++tt) acc[P][tt] = mfma16(wc[f], xb[tt][f], acc[P][tt]);
    const Cursor cur = cp;
    advance(cp);
    if (P == 1) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int tt = 0; tt < kDecodeTT; ++tt) S.red[wave][h][tt][lane] = acc[h][tt];
      load_rows(cp);
    }
    issue(ld, wi);
    advance(ld);
    if (P == 1) {
      __syncthreads();
      const int e = expert_of(cur.u);
      const int r0 = cur.pass * kPassRows;
      const int rows = min(kPassRows, count_of(e) - r0);
      const Owner own = owner();
      if (own.on && own.row < rows) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int w = 0; w < kStreamWaves; ++w) {
          s0 += S.red[w][0][own.tt][own.ln][own.q];
          s1 += S.red[w][1][own.tt][own.ln][own.q];
        }
        const int slot = S.G.list[S.G.off[e] + r0 + own.row];
        const int col = (cur.u % kUnitsPerExpert) * (GATEUP ? 16 : 32) + 4 * (own.ln >> 4) + own.q;
        if (GATEUP) {
          H[static_cast<size_t>(slot) * kFF + col] = f32_to_bf16(silu(s0) * s1);
        } else {
          float* dst = Y + static_cast<size_t>(slot) * kHidden + col;
          dst[0] = s0;
          dst[16] = s1;
        }
      }
      __syncthreads();
    }
  };
  // Both halves of one pass: a and b hold their weights, c is free.
  auto pass = [&](uint4 (&a)[kF], uint4 (&b)[kF], uint4 (&c)[kF]) -> bool {
    if (cp.u >= end) return false;
    step(std::integral_constant<int, 0>{}, a, c);
    step(std::integral_constant<int, 1>{}, b, a);
    return true;
  };
  // Sub-unit s uses buffer s % 3: unrolled by three passes.
  for (;;) {
    if (!pass(w0, w1, w2)) break;
    if (!pass(w2, w0, w1)) break;
    if (!pass(w1, w2, w0)) break;
  }
}

__global__ __launch_bounds__(kStreamThreads) void gateup_decode_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wgu,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ H, int N) {
  __shared__ StreamShared S;
  group_slots(idx, N, S.G);
  stream_units<true>(X, Wgu, H, nullptr, N, S);
}

__global__ __launch_bounds__(kStreamThreads) void down_decode_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,
    const int32_t* __restrict__ idx, float* __restrict__ Y, int N) {
  __shared__ StreamShared S;
  group_slots(idx, N, S.G);
  stream_units<false>(H, Wd, nullptr, Y, N, S);
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
  hipLaunchKernelGGL(gateup_decode_kernel, dim3(cu_count()), dim3(kStreamThreads), 0, stream, X,
                     Wgu, idx, H, N);
  return hipGetLastError();
}

hipError_t launch_down_decode(const uint16_t* H, const uint16_t* Wd, const int32_t* idx,
                              float* Y, int N, hipStream_t stream) {
  hipLaunchKernelGGL(down_decode_kernel, dim3(cu_count()), dim3(kStreamThreads), 0, stream, H, Wd,
                     idx, Y, N);
  return hipGetLastError();
}

}  // namespace lfm

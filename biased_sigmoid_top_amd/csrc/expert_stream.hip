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
// registers, and every weight fragment is read by exactly one wavefront.
// The token rows (B operand; few, shared by all workgroups of an expert)
// come through the caches.  Loads for the next K step are issued before the
// MFMAs of the current one.
//
// Grid: one workgroup per (expert, column block) for all 64 experts.  A
// workgroup groups its own tokens: it scans the router's selections and
// lists, in token order, the slots t*4 + j routed to its expert (ballot and
// popcount, so the order is the token order on every run).  Experts without
// tokens exit at once.  No separate dispatch step, no host readback.
//
// H and Y rows are stored in slot order (row t*4 + j holds token t's j-th
// selected expert), which the combine step reads back contiguously.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kFrag = 512;                         // bf16 elements per 16x32 fragment
constexpr int kGateUpBlocks = kFF / 64;            // 24: 4 waves x 16 H columns
constexpr int kDownTiles = 2;                      // 16-row output tiles per wave
constexpr int kDownBlocks = kHidden / (64 * kDownTiles);  // 4 waves x 16 kDownTiles features
constexpr int kStepFrags = 2;                      // K fragments (of 32) per pipeline step
constexpr int kDecodeTT = 2;                       // token tiles of 16 per pass

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming read: used once, so marked non-temporal.
__device__ __forceinline__ uint4 ld_stream(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Lists, in token order, the slots t*4 + j whose selection is `expert`.
// Returns the count (same value in every thread).  list holds >= N entries.
__device__ int gather_expert_slots(const int32_t* __restrict__ idx, int N, int expert,
                                   int* list, int* wave_tot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  constexpr int kWaves = kStreamThreads / kWave;
  int base = 0;
  for (int t0 = 0; t0 < N; t0 += kStreamThreads) {
    const int t = t0 + threadIdx.x;
    int j_e = -1;
    if (t < N) {
      const int4 v = *reinterpret_cast<const int4*>(idx + static_cast<size_t>(t) * kTopK);
      j_e = v.x == expert ? 0 : v.y == expert ? 1 : v.z == expert ? 2 : v.w == expert ? 3 : -1;
    }
    const unsigned long long m = __ballot(j_e >= 0);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wave] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wave_tot[w];
    if (j_e >= 0) list[off + before] = t * kTopK + j_e;
    for (int w = 0; w < kWaves; ++w) base += wave_tot[w];
    __syncthreads();
  }
  return base;
}

// One wavefront: H columns hb*16 .. hb*16+15 for `rows` (<= 16 TT) token
// rows whose slots are slots[0 .. rows).
template <int TT>
__device__ __forceinline__ void gateup_wave(const uint16_t* __restrict__ X,
                                            const uint16_t* __restrict__ wg,
                                            const uint16_t* __restrict__ wu, const int* slots,
                                            int rows, int hb, uint16_t* __restrict__ H) {
  constexpr int kSteps = (kHidden / 32) / kStepFrags;
  const int lane = threadIdx.x & (kWave - 1);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int ntt = __builtin_amdgcn_readfirstlane((rows + 15) / 16);
  const uint16_t* xr[TT];
  int my_slot[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int r = tt * 16 + r16;
    my_slot[tt] = slots[r < rows ? r : 0];
    xr[tt] = X + static_cast<size_t>(my_slot[tt] / kTopK) * kHidden + g * 8;
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
      ag[f] = ld_stream(wg + kf * 8 * kFrag);
      au[f] = ld_stream(wu + kf * 8 * kFrag);
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

  // Lane holds token row (tt*16 + r16) and H columns hb*16 + 4g + r.
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    if (tt * 16 + r16 < rows) {
      uint32_t p[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float h0 = silu(accg[tt][2 * q]) * accu[tt][2 * q];
        const float h1 = silu(accg[tt][2 * q + 1]) * accu[tt][2 * q + 1];
        p[q] = static_cast<uint32_t>(f32_to_bf16(h0)) | (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
      }
      uint16_t* dst = H + static_cast<size_t>(my_slot[tt]) * kFF + hb * 16 + 4 * g;
      *reinterpret_cast<uint2*>(dst) = make_uint2(p[0], p[1]);
    }
  }
}

// This lane's piece of down-weight row tile rt (first K fragment) of expert
// e; the K fragments of a tile are 8 fragments apart, and the 8 tiles of a
// 128-row block are adjacent.
__device__ __forceinline__ const uint16_t* down_weights(const uint16_t* Wd, int e, int rt) {
  return Wd + ((static_cast<size_t>(e) * (kHidden / 128) + rt / 8) * (kFF / 32) * 8 + rt % 8) *
                  kFrag + (threadIdx.x & (kWave - 1)) * 8;
}

// One wavefront: output features rt0*16 .. (rt0 + kDownTiles)*16 - 1 for
// `rows` token rows.  w0 points at the wavefront's first weight tile; the
// tiles follow each other in the packed layout.
template <int TT>
__device__ __forceinline__ void down_wave(const uint16_t* __restrict__ H,
                                          const uint16_t* __restrict__ w0, const int* slots,
                                          int rows, int rt0, float* __restrict__ Y) {
  constexpr int kSteps = (kFF / 32) / kStepFrags;
  constexpr int FT = kDownTiles;
  const int lane = threadIdx.x & (kWave - 1);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int ntt = __builtin_amdgcn_readfirstlane((rows + 15) / 16);
  const uint16_t* hr[TT];
  int my_slot[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int r = tt * 16 + r16;
    my_slot[tt] = slots[r < rows ? r : 0];
    hr[tt] = H + static_cast<size_t>(my_slot[tt]) * kFF + g * 8;
  }
  f32x4 acc[FT][TT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[ft][tt] = f32x4{0, 0, 0, 0};

  uint4 cw[FT][kStepFrags], ch[TT][kStepFrags];
  auto load = [&](int s, uint4 (&aw)[FT][kStepFrags], uint4 (&bh)[TT][kStepFrags]) {
#pragma unroll
    for (int f = 0; f < kStepFrags; ++f) {
      const int kf = s * kStepFrags + f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) aw[ft][f] = ld_stream(w0 + (kf * 8 + ft) * kFrag);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        bh[tt][f] = (tt == 0 || tt < ntt) ? ld16(hr[tt] + kf * 32) : make_uint4(0, 0, 0, 0);
    }
  };
  auto compute = [&](const uint4 (&aw)[FT][kStepFrags], const uint4 (&bh)[TT][kStepFrags]) {
#pragma unroll
    for (int f = 0; f < kStepFrags; ++f)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          if (tt == 0 || tt < ntt) acc[ft][tt] = mfma16(aw[ft][f], bh[tt][f], acc[ft][tt]);
  };

  load(0, cw, ch);
  for (int s = 0; s < kSteps - 1; ++s) {
    uint4 nw[FT][kStepFrags], nh[TT][kStepFrags];
    load(s + 1, nw, nh);
    compute(cw, ch);
#pragma unroll
    for (int f = 0; f < kStepFrags; ++f) {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) cw[ft][f] = nw[ft][f];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) ch[tt][f] = nh[tt][f];
    }
  }
  compute(cw, ch);

  // Lane holds token row (tt*16 + r16) and features (rt0 + ft)*16 + 4g + r.
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    if (tt * 16 + r16 < rows) {
      float* dst = Y + static_cast<size_t>(my_slot[tt]) * kHidden + rt0 * 16 + 4 * g;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
        *reinterpret_cast<float4*>(dst + ft * 16) =
            make_float4(acc[ft][tt][0], acc[ft][tt][1], acc[ft][tt][2], acc[ft][tt][3]);
    }
  }
}

__global__ __launch_bounds__(kStreamThreads) void gateup_decode_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wgu,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ H, int N) {
  __shared__ int list[kDecodeMaxTokens];
  __shared__ int wave_tot[kStreamThreads / kWave];
  const int e = blockIdx.x / kGateUpBlocks;
  const int nb = blockIdx.x % kGateUpBlocks;
  const int count = gather_expert_slots(idx, N, e, list, wave_tot);
  if (count == 0) return;
  const int cb = threadIdx.x / kWave;
  const int hb = nb * 4 + cb;
  const uint16_t* wg = Wgu + ((static_cast<size_t>(e) * kGateUpBlocks + nb) * (kHidden / 32) * 8 +
                              cb * 2) * kFrag + (threadIdx.x & (kWave - 1)) * 8;
  const uint16_t* wu = wg + kFrag;
  for (int r0 = 0; r0 < count; r0 += 16 * kDecodeTT)
    gateup_wave<kDecodeTT>(X, wg, wu, list + r0, min(16 * kDecodeTT, count - r0), hb, H);
}

__global__ __launch_bounds__(kStreamThreads) void down_decode_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,
    const int32_t* __restrict__ idx, float* __restrict__ Y, int N) {
  __shared__ int list[kDecodeMaxTokens];
  __shared__ int wave_tot[kStreamThreads / kWave];
  const int e = blockIdx.x / kDownBlocks;
  const int nb = blockIdx.x % kDownBlocks;
  const int count = gather_expert_slots(idx, N, e, list, wave_tot);
  if (count == 0) return;
  const int rt0 = (nb * 4 + threadIdx.x / kWave) * kDownTiles;
  const uint16_t* w0 = down_weights(Wd, e, rt0);
  for (int r0 = 0; r0 < count; r0 += 16 * kDecodeTT)
    down_wave<kDecodeTT>(H, w0, list + r0, min(16 * kDecodeTT, count - r0), rt0, Y);
}

// Grouped variants: workgroups walk (m-tile, column block) over the
// expert-grouped rows that the dispatch step produced (row -> slot map).
template <int TT>
__global__ __launch_bounds__(kStreamThreads) void gateup_grouped_stream_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wgu,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row2slot,
    uint16_t* __restrict__ H) {
  MTile tile;
  if (!map_mtile(offsets, blockIdx.x / kGateUpBlocks, 16 * TT, tile)) return;
  const int nb = blockIdx.x % kGateUpBlocks;
  const int cb = threadIdx.x / kWave;
  const int hb = nb * 4 + cb;
  const uint16_t* wg =
      Wgu + ((static_cast<size_t>(tile.expert) * kGateUpBlocks + nb) * (kHidden / 32) * 8 + cb * 2) *
                kFrag + (threadIdx.x & (kWave - 1)) * 8;
  const uint16_t* wu = wg + kFrag;
  gateup_wave<TT>(X, wg, wu, row2slot + tile.row_begin, tile.rows, hb, H);
}

template <int TT>
__global__ __launch_bounds__(kStreamThreads) void down_grouped_stream_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row2slot,
    float* __restrict__ Y) {
  MTile tile;
  if (!map_mtile(offsets, blockIdx.x / kDownBlocks, 16 * TT, tile)) return;
  const int rt0 = ((blockIdx.x % kDownBlocks) * 4 + threadIdx.x / kWave) * kDownTiles;
  const uint16_t* w0 = down_weights(Wd, tile.expert, rt0);
  down_wave<TT>(H, w0, row2slot + tile.row_begin, tile.rows, rt0, Y);
}

}  // namespace

int64_t max_mtiles(int64_t N, int tile_rows) {
  const int64_t rows = N * kTopK;
  const int64_t a = (rows + static_cast<int64_t>(kExperts) * (tile_rows - 1)) / tile_rows;
  const int64_t b = static_cast<int64_t>(kExperts) * ((N + tile_rows - 1) / tile_rows);
  return a < b ? a : b;
}

hipError_t launch_gateup_grouped_stream(const uint16_t* X, const uint16_t* Wgu,
                                        const int32_t* offsets, const int32_t* row2slot,
                                        uint16_t* H, int64_t N, hipStream_t stream) {
  const int64_t grid = max_mtiles(N, 16 * kDecodeTT) * kGateUpBlocks;
  hipLaunchKernelGGL(gateup_grouped_stream_kernel<kDecodeTT>, dim3(grid), dim3(kStreamThreads), 0,
                     stream, X, Wgu, offsets, row2slot, H);
  return hipGetLastError();
}

hipError_t launch_down_grouped_stream(const uint16_t* H, const uint16_t* Wd,
                                      const int32_t* offsets, const int32_t* row2slot, float* Y,
                                      int64_t N, hipStream_t stream) {
  const int64_t grid = max_mtiles(N, 16 * kDecodeTT) * kDownBlocks;
  hipLaunchKernelGGL(down_grouped_stream_kernel<kDecodeTT>, dim3(grid), dim3(kStreamThreads), 0,
                     stream, H, Wd, offsets, row2slot, Y);
  return hipGetLastError();
}

hipError_t launch_gateup_decode(const uint16_t* X, const uint16_t* Wgu, const int32_t* idx,
                                uint16_t* H, int N, hipStream_t stream) {
  hipLaunchKernelGGL(gateup_decode_kernel, dim3(kExperts * kGateUpBlocks), dim3(kStreamThreads),
                     0, stream, X, Wgu, idx, H, N);
  return hipGetLastError();
}

hipError_t launch_down_decode(const uint16_t* H, const uint16_t* Wd, const int32_t* idx,
                              float* Y, int N, hipStream_t stream) {
  hipLaunchKernelGGL(down_decode_kernel, dim3(kExperts * kDownBlocks), dim3(kStreamThreads), 0,
                     stream, H, Wd, idx, Y, N);
  return hipGetLastError();
}

}  // namespace lfm

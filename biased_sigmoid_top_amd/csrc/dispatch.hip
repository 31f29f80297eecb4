// Token dispatch: per-expert totals from the router's per-block histogram, a
// wavefront prefix scan into expert row offsets, and a deterministic stable
// permutation of the (token, slot) pairs into expert-grouped order.
//
// Method: flozi.net guide "LFM2.5-24B-A2B: Biased Routing, Short
// Convolutions and Ten KV Caches", sections "The router has two different
// scores" (dispatch and token regrouping, uneven expert loads) and "What to
// verify in a deployment" (the expert path groups tokens by expert).
//
// Row of slot (t, j) routed to expert e:
//   offsets[e] + (slots of e in earlier dispatch blocks)
//              + (tokens t' < t of this block that also chose e).
// Everything is integer arithmetic, so the result does not depend on
// scheduling.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kDispatchTokens = 256;  // tokens per workgroup (one per thread)
constexpr int kMaskWords = kDispatchTokens / 32;

__global__ __launch_bounds__(kDispatchTokens) void dispatch_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ blockcounts, int route_tokens,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row2tok, int32_t* __restrict__ slot2row,
    int N) {
  __shared__ int part_tot[4][kExperts];
  __shared__ int part_base[4][kExperts];
  __shared__ int s_excl[kExperts];
  __shared__ int s_base[kExperts];
  __shared__ uint32_t mask[kExperts][kMaskWords];

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kDispatchTokens;

  // Per-expert totals over all router blocks, and over the router blocks
  // that precede this dispatch block.
  {
    const int q = tid / kExperts;
    const int e = tid % kExperts;
    const int nrb = (N + route_tokens - 1) / route_tokens;
    const int first_rb = t0 / route_tokens;
    int tot = 0, base = 0;
    for (int rb = q; rb < nrb; rb += 4) {
      const int v = blockcounts[static_cast<size_t>(rb) * kExperts + e];
      tot += v;
      base += rb < first_rb ? v : 0;
    }
    part_tot[q][e] = tot;
    part_base[q][e] = base;
  }
  for (int i = tid; i < kExperts * kMaskWords; i += kDispatchTokens) (&mask[0][0])[i] = 0u;
  __syncthreads();

  if (tid < kWave) {
    const int e = tid;
    const int tot = part_tot[0][e] + part_tot[1][e] + part_tot[2][e] + part_tot[3][e];
    const int base = part_base[0][e] + part_base[1][e] + part_base[2][e] + part_base[3][e];
    const int incl = wave_inclusive_scan(tot, e);
    s_excl[e] = incl - tot;
    s_base[e] = base;
    if (blockIdx.x == 0) {
      offsets[e] = incl - tot;
      if (e == kExperts - 1) offsets[kExperts] = incl;
    }
  }

  // Bit t of mask[e] is set when token t of this block chose expert e.
  const int t = t0 + tid;
  int my_e[kTopK];
  if (t < N) {
    const int4 v = *reinterpret_cast<const int4*>(idx + static_cast<size_t>(t) * kTopK);
    my_e[0] = v.x; my_e[1] = v.y; my_e[2] = v.z; my_e[3] = v.w;
#pragma unroll
    for (int j = 0; j < kTopK; ++j) atomicOr(&mask[my_e[j]][tid / 32], 1u << (tid % 32));
  }
  __syncthreads();

  if (t < N) {
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
      const int e = my_e[j];
      int rank = __popc(mask[e][tid / 32] & ((1u << (tid % 32)) - 1u));
      for (int wd = 0; wd < tid / 32; ++wd) rank += __popc(mask[e][wd]);
      const int row = s_excl[e] + s_base[e] + rank;
      slot2row[static_cast<size_t>(t) * kTopK + j] = row;
      row2tok[row] = t;
    }
  }
}

}  // namespace

hipError_t launch_dispatch(const int32_t* idx, const int32_t* blockcounts, int route_tokens,
                           int32_t* offsets, int32_t* row2tok, int32_t* slot2row, int N,
                           hipStream_t stream) {
  const int grid = (N + kDispatchTokens - 1) / kDispatchTokens;
  hipLaunchKernelGGL(dispatch_kernel, dim3(grid), dim3(kDispatchTokens), 0, stream, idx,
                     blockcounts, route_tokens, offsets, row2tok, slot2row, N);
  return hipGetLastError();
}

}  // namespace lfm

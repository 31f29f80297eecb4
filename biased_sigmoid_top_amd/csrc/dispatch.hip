// Token dispatch for the grouped path: per-expert totals from the router's
// per-block histogram, a wavefront prefix scan into expert row offsets, and
// a deterministic stable permutation of the (token, slot) pairs into
// expert-grouped order.
//
// Method: flozi.net guide "LFM2.5-24B-A2B: Biased Routing, Short
// Convolutions and Ten KV Caches", sections "The router has two different
// scores" (dispatch and token regrouping, uneven expert loads) and "What to
// verify in a deployment" (the expert path groups tokens by expert).
//
// Grouped row of slot (t, j) routed to expert e:
//   offsets[e] + (slots of e in earlier dispatch blocks)
//              + (tokens t' < t of this block that also chose e).
// Everything is integer arithmetic, so the result does not depend on
// scheduling.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kDispatchThreads = 1024;             // one token per thread
constexpr int kMaskWords = kDispatchThreads / 32;  // token bitmask per expert
constexpr int kRowGroups = kDispatchThreads / 16;  // 64 groups x 16 lanes of 4 experts
static_assert(kMaskWords == 32 && kDispatchThreads / kWave * 4 == kExperts,
              "the word prefix scan gives each wavefront four experts of 32 words");

__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ blockcounts, int route_tokens,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row2slot, int N) {
  __shared__ int4 part_tot[kRowGroups][kExperts / 4];
  __shared__ int4 part_base[kRowGroups][kExperts / 4];
  __shared__ int s_excl[kExperts];
  __shared__ int s_base[kExperts];
  __shared__ uint32_t mask[kExperts][kMaskWords];
  __shared__ int word_base[kExperts][kMaskWords];  // tokens of e in earlier mask words

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kDispatchThreads;

  // Per-expert totals over all router blocks, and over the router blocks
  // before this dispatch block: group q adds router blocks q, q + 64, ...
  // four experts at a time.
  {
    const int q = tid / 16;
    const int e4 = tid % 16;
    const int nrb = (N + route_tokens - 1) / route_tokens;
    const int first_rb = t0 / route_tokens;
    int4 tot = make_int4(0, 0, 0, 0), base = make_int4(0, 0, 0, 0);
#pragma unroll 4
    for (int rb = q; rb < nrb; rb += kRowGroups) {
      const int4 v = *reinterpret_cast<const int4*>(blockcounts + static_cast<size_t>(rb) * kExperts + 4 * e4);
      tot.x += v.x; tot.y += v.y; tot.z += v.z; tot.w += v.w;
      if (rb < first_rb) { base.x += v.x; base.y += v.y; base.z += v.z; base.w += v.w; }
    }
    part_tot[q][e4] = tot;
    part_base[q][e4] = base;
  }
  for (int i = tid; i < kExperts * kMaskWords; i += kDispatchThreads) (&mask[0][0])[i] = 0u;
  __syncthreads();

  if (tid < kWave) {
    const int e = tid;
    const int* pt = reinterpret_cast<const int*>(&part_tot[0][0]);
    const int* pb = reinterpret_cast<const int*>(&part_base[0][0]);
    int tot = 0, base = 0;
    for (int q = 0; q < kRowGroups; ++q) {
      tot += pt[q * kExperts + e];
      base += pb[q * kExperts + e];
    }
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

  // Exclusive prefix of the mask words' popcounts, per expert: wavefront w
  // scans experts 4w .. 4w + 3, two at a time, one 32-lane half each.
  {
    const int lane = tid & (kWave - 1);
    const int word = lane & 31;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int e = 4 * (tid / kWave) + 2 * it + lane / 32;
      const int c = __popc(mask[e][word]);
      int incl = c;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        const int o = __shfl_up(incl, off, 32);
        if (word >= off) incl += o;
      }
      word_base[e][word] = incl - c;
    }
  }
  __syncthreads();

  if (t < N) {
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
      const int e = my_e[j];
      const int rank = word_base[e][tid / 32] + __popc(mask[e][tid / 32] & ((1u << (tid % 32)) - 1u));
      row2slot[s_excl[e] + s_base[e] + rank] = t * kTopK + j;
    }
  }
}

}  // namespace

hipError_t launch_dispatch(const int32_t* idx, const int32_t* blockcounts, int32_t* offsets,
                           int32_t* row2slot, int N, hipStream_t stream) {
  const int grid = (N + kDispatchThreads - 1) / kDispatchThreads;
  hipLaunchKernelGGL(dispatch_kernel, dim3(grid), dim3(kDispatchThreads), 0, stream, idx,
                     blockcounts, route_block_tokens(N), offsets, row2slot, N);
  return hipGetLastError();
}

}  // namespace lfm

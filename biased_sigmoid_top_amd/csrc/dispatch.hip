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

// Caller-given routing (the expert path without the router): copies the
// selections and weights of 16 tokens per wavefront into the workspace and
// writes the same per-16-token histogram the router writes.  The
// selections become memory-safe on the way: an id is taken modulo 64, and
// an id that repeats an earlier one of the same token is replaced by the
// lowest id that is neither among the token's earlier (final) ids nor
// among its later given ones, so every token ends with four distinct ids
// in [0, 64) and valid input passes through unchanged.  Lane i holds entry
// i % 4 of token 16 * block + i / 4.
__global__ __launch_bounds__(kWave) void ingest_routing_kernel(
    const int32_t* __restrict__ idx_in, const float* __restrict__ w_in, int32_t* __restrict__ idx,
    float* __restrict__ w, int32_t* __restrict__ blockcounts, int route_tokens, int N) {
  __shared__ int counts[kExperts];
  const int lane = threadIdx.x;
  const int j = lane % kTopK;
  const int t = blockIdx.x * route_tokens + lane / kTopK;
  const bool live = lane / kTopK < route_tokens && t < N;
  const size_t at = static_cast<size_t>(t) * kTopK + j;
  const int given = live ? (idx_in[at] & (kExperts - 1)) : 0;
  // The four given ids of this lane's token, from the lanes of its quad.
  int v[kTopK];
#pragma unroll
  for (int q = 0; q < kTopK; ++q) v[q] = __shfl(given, (lane & ~(kTopK - 1)) + q, kWave);
#pragma unroll
  for (int q = 1; q < kTopK; ++q) {
    bool repeat = false;
    for (int p = 0; p < q; ++p) repeat = repeat || v[p] == v[q];
    if (!repeat) continue;
    for (int e = 0; e < kExperts; ++e) {  // at most 6 ids are excluded
      bool used = false;
      for (int p = 0; p < kTopK; ++p) used = used || (p != q && v[p] == e);
      if (!used) { v[q] = e; break; }
    }
  }
  counts[lane] = 0;
  __syncthreads();
  if (live) {
    idx[at] = v[j];
    w[at] = w_in[at];
    atomicAdd(&counts[v[j]], 1);
  }
  __syncthreads();
  if (blockcounts != nullptr) blockcounts[static_cast<size_t>(blockIdx.x) * kExperts + lane] = counts[lane];
}

}  // namespace

hipError_t launch_ingest_routing(const int32_t* idx_in, const float* w_in, int32_t* idx, float* w,
                                 int32_t* blockcounts, int N, hipStream_t stream) {
  const int rt = route_block_tokens(N);
  if (rt != kWave / kTopK) return hipErrorInvalidValue;  // one wavefront holds a block's entries
  const int grid = (N + rt - 1) / rt;
  hipLaunchKernelGGL(ingest_routing_kernel, dim3(grid), dim3(kWave), 0, stream, idx_in, w_in, idx,
                     w, blockcounts, rt, N);
  return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* idx, const int32_t* blockcounts, int32_t* offsets,
                           int32_t* row2slot, int N, hipStream_t stream) {
  const int grid = (N + kDispatchThreads - 1) / kDispatchThreads;
  hipLaunchKernelGGL(dispatch_kernel, dim3(grid), dim3(kDispatchThreads), 0, stream, idx,
                     blockcounts, route_block_tokens(N), offsets, row2slot, N);
  return hipGetLastError();
}

}  // namespace lfm

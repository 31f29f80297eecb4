// Expert weight packing into the MFMA operand-fragment layout.
//
// The guide ("LFM2.5-24B-A2B: Biased Routing, Short Convolutions and Ten KV
// Caches", section "The router has two different scores") notes that the
// runtime representation may pack an expert's two input matrices together
// without changing the function.  This library packs every expert matrix
// into fragments of 32 rows x 16 columns (1 KB), each stored in the order in
// which the 64 lanes of a wavefront hold a 32x32x16 MFMA operand: bytes
// [16 l, 16 l + 16) of a fragment are row (l % 32), columns
// 8 (l / 32) .. 8 (l / 32) + 7.  A wavefront then loads one operand with a
// single contiguous 1 KB read.
//
// Fragments are ordered (expert, 32-row block, 16-column K step), so the K
// steps of one row block are contiguous:
//   gate/up: fragment (e * 96 + b) * 128 + ks holds rows 16 b .. 16 b + 15
//            of W_gate (fragment rows 0..15) and the same rows of W_up
//            (fragment rows 16..31) of expert e, columns ks*16 .. ks*16+15.
//            An MFMA on it yields the gate and the up value of an H column
//            in the same lane.
//   down:    fragment (e * 64 + b) * 96 + ks holds rows 32 b .. 32 b + 31 of
//            W_down of expert e, columns ks*16 .. ks*16+15.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kPackThreads = 256;

// One thread moves one 16-byte piece (8 consecutive columns of one row).
// Expert e's gate and up matrices start at Wg + e * estride and
// Wu + e * estride (estride = 1536 * 2048 for two [64, 1536, 2048] tensors,
// 2 * 1536 * 2048 for one [64, 3072, 2048] tensor of gate rows then up rows).
__global__ __launch_bounds__(kPackThreads) void pack_gateup_kernel(
    const uint16_t* __restrict__ Wg, const uint16_t* __restrict__ Wu, size_t estride,
    uint16_t* __restrict__ out) {
  const size_t piece = static_cast<size_t>(blockIdx.x) * kPackThreads + threadIdx.x;
  const int lane = static_cast<int>(piece % kWave);
  const size_t frag = piece / kWave;
  const int ks = static_cast<int>(frag % kGateupSteps);
  const size_t eb = frag / kGateupSteps;  // e * 96 + b
  const size_t e = eb / kGateupBlocks;
  const int b = static_cast<int>(eb % kGateupBlocks);
  const int i = lane % 32;
  const int row = b * 16 + (i % 16);
  const int col = ks * 16 + (lane / 32) * 8;
  const uint16_t* src = (i < 16 ? Wg : Wu) + e * estride + row * static_cast<size_t>(kHidden) + col;
  *reinterpret_cast<uint4*>(out + piece * 8) = ld16(src);
}

__global__ __launch_bounds__(kPackThreads) void pack_down_kernel(const uint16_t* __restrict__ Wd,
                                                                 uint16_t* __restrict__ out) {
  const size_t piece = static_cast<size_t>(blockIdx.x) * kPackThreads + threadIdx.x;
  const int lane = static_cast<int>(piece % kWave);
  const size_t frag = piece / kWave;
  const int ks = static_cast<int>(frag % kDownSteps);
  const size_t eb = frag / kDownSteps;  // e * 64 + b
  const size_t e = eb / kDownBlocks;
  const int b = static_cast<int>(eb % kDownBlocks);
  const int row = b * 32 + lane % 32;
  const int col = ks * 16 + (lane / 32) * 8;
  const uint16_t* src = Wd + (e * kHidden + row) * static_cast<size_t>(kFF) + col;
  *reinterpret_cast<uint4*>(out + piece * 8) = ld16(src);
}

}  // namespace

hipError_t launch_pack_gateup(const uint16_t* Wg, const uint16_t* Wu, size_t estride, uint16_t* out,
                              hipStream_t stream) {
  const size_t pieces = static_cast<size_t>(kExperts) * 2 * kFF * kHidden / 8;
  hipLaunchKernelGGL(pack_gateup_kernel, dim3(pieces / kPackThreads), dim3(kPackThreads), 0,
                     stream, Wg, Wu, estride, out);
  return hipGetLastError();
}

hipError_t launch_pack_down(const uint16_t* Wd, uint16_t* out, hipStream_t stream) {
  const size_t pieces = static_cast<size_t>(kExperts) * kHidden * kFF / 8;
  hipLaunchKernelGGL(pack_down_kernel, dim3(pieces / kPackThreads), dim3(kPackThreads), 0, stream,
                     Wd, out);
  return hipGetLastError();
}

}  // namespace lfm

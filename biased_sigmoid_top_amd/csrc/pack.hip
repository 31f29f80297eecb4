// Expert weight packing into the MFMA operand-fragment layout.
//
// The guide ("LFM2.5-24B-A2B: Biased Routing, Short Convolutions and Ten KV
// Caches", section "The router has two different scores") notes that the
// runtime representation may pack an expert's two input matrices together
// without changing the function.  This library packs every expert matrix
// into 16-row x 32-column fragments of 1 KB, each stored in the order in
// which the 64 lanes of a wavefront hold a 16x16x32 MFMA operand: bytes
// [16 l, 16 l + 16) of a fragment are row (l % 16), columns
// 8 (l / 16) .. 8 (l / 16) + 7.  A wavefront then loads one operand with a
// single contiguous 1 KB read.
//
//   gate/up: fragment ((e * 96 + hb) * 2 + p) * 64 + kf holds rows
//            hb*16 .. hb*16+15 of W_gate (p = 0) or W_up (p = 1) of expert
//            e, columns kf*32 .. kf*32+31.
//   down:    fragment (e * 128 + rt) * 48 + kf holds rows rt*16 .. rt*16+15
//            of W_down of expert e, columns kf*32 .. kf*32+31.
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kPackThreads = 256;

// One thread moves one 16-byte piece (8 consecutive columns of one row).
__global__ __launch_bounds__(kPackThreads) void pack_gateup_kernel(
    const uint16_t* __restrict__ Wg, const uint16_t* __restrict__ Wu, uint16_t* __restrict__ out) {
  const size_t piece = static_cast<size_t>(blockIdx.x) * kPackThreads + threadIdx.x;
  const int lane = static_cast<int>(piece % kWave);
  const size_t frag = piece / kWave;
  const int kf = static_cast<int>(frag % (kHidden / 32));
  const size_t t = frag / (kHidden / 32);
  const int p = static_cast<int>(t % 2);
  const size_t ehb = t / 2;  // e * 96 + hb
  const size_t e = ehb / (kFF / 16);
  const int hb = static_cast<int>(ehb % (kFF / 16));
  const int row = hb * 16 + (lane % 16);
  const int col = kf * 32 + (lane / 16) * 8;
  const uint16_t* src = (p == 0 ? Wg : Wu) + (e * kFF + row) * static_cast<size_t>(kHidden) + col;
  *reinterpret_cast<uint4*>(out + piece * 8) = ld16(src);
}

__global__ __launch_bounds__(kPackThreads) void pack_down_kernel(const uint16_t* __restrict__ Wd,
                                                                 uint16_t* __restrict__ out) {
  const size_t piece = static_cast<size_t>(blockIdx.x) * kPackThreads + threadIdx.x;
  const int lane = static_cast<int>(piece % kWave);
  const size_t frag = piece / kWave;
  const int kf = static_cast<int>(frag % (kFF / 32));
  const size_t ert = frag / (kFF / 32);  // e * 128 + rt
  const size_t e = ert / (kHidden / 16);
  const int rt = static_cast<int>(ert % (kHidden / 16));
  const int row = rt * 16 + (lane % 16);
  const int col = kf * 32 + (lane / 16) * 8;
  const uint16_t* src = Wd + (e * kHidden + row) * static_cast<size_t>(kFF) + col;
  *reinterpret_cast<uint4*>(out + piece * 8) = ld16(src);
}

}  // namespace

hipError_t launch_pack_gateup(const uint16_t* Wg, const uint16_t* Wu, uint16_t* out,
                              hipStream_t stream) {
  const size_t pieces = static_cast<size_t>(kExperts) * 2 * kFF * kHidden / 8;
  hipLaunchKernelGGL(pack_gateup_kernel, dim3(pieces / kPackThreads), dim3(kPackThreads), 0,
                     stream, Wg, Wu, out);
  return hipGetLastError();
}

hipError_t launch_pack_down(const uint16_t* Wd, uint16_t* out, hipStream_t stream) {
  const size_t pieces = static_cast<size_t>(kExperts) * kHidden * kFF / 8;
  hipLaunchKernelGGL(pack_down_kernel, dim3(pieces / kPackThreads), dim3(kPackThreads), 0, stream,
                     Wd, out);
  return hipGetLastError();
}

}  // namespace lfm

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
// Fragments are ordered so that, for one 32-wide K step, everything a
// workgroup of the expert kernels needs is one contiguous 8 KB run:
//   gate/up: fragment ((e * 24 + nb) * 64 + kf) * 8 + cb * 2 + p holds rows
//            nb*64 + cb*16 .. +15 of W_gate (p = 0) or W_up (p = 1) of
//            expert e, columns kf*32 .. kf*32+31   (nb < 24, cb < 4).
//   down:    fragment ((e * 16 + rb) * 48 + kf) * 8 + rt holds rows
//            rb*128 + rt*16 .. +15 of W_down of expert e, columns
//            kf*32 .. kf*32+31                     (rb < 16, rt < 8).
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
  const int q = static_cast<int>(frag % 8);  // cb * 2 + p
  const size_t t = frag / 8;
  const int kf = static_cast<int>(t % (kHidden / 32));
  const size_t enb = t / (kHidden / 32);     // e * 24 + nb
  const size_t e = enb / (kFF / 64);
  const int nb = static_cast<int>(enb % (kFF / 64));
  const int cb = q / 2, p = q % 2;
  const int row = nb * 64 + cb * 16 + (lane % 16);
  const int col = kf * 32 + (lane / 16) * 8;
  const uint16_t* src = (p == 0 ? Wg : Wu) + (e * kFF + row) * static_cast<size_t>(kHidden) + col;
  *reinterpret_cast<uint4*>(out + piece * 8) = ld16(src);
}

__global__ __launch_bounds__(kPackThreads) void pack_down_kernel(const uint16_t* __restrict__ Wd,
                                                                 uint16_t* __restrict__ out) {
  const size_t piece = static_cast<size_t>(blockIdx.x) * kPackThreads + threadIdx.x;
  const int lane = static_cast<int>(piece % kWave);
  const size_t frag = piece / kWave;
  const int rt = static_cast<int>(frag % 8);
  const size_t t = frag / 8;
  const int kf = static_cast<int>(t % (kFF / 32));
  const size_t erb = t / (kFF / 32);         // e * 16 + rb
  const size_t e = erb / (kHidden / 128);
  const int rb = static_cast<int>(erb % (kHidden / 128));
  const int row = rb * 128 + rt * 16 + (lane % 16);
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

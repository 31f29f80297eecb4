// FP8 (E4M3) block quantisation of the expert weights, packed into the
// operand-fragment layout of the 32x32x16 MFMAs (each lane's 8 codes of a
// 16-wide K step are its operand, widened to bf16 in registers by the
// weight-streaming kernels); two consecutive fragments give a lane its 32
// codes of a 32x32x64 FP8 MFMA (the grouped kernels).
//
// Method: the inferencekey.com page on the 24B reasoning MoE (German
// edition, "Für Engineers" part, the quantisation entry) describes the
// model's FP8 checkpoint as compressed-tensors FP8_BLOCK: weights in FP8
// (F8_E4M3) statically, in blocks of 128 x 128; activations dynamically per
// group of 128; the router not quantised.  Each 128 x 128 block of W_gate,
// W_up ([1536, 2048]) and W_down ([2048, 1536]) with largest magnitude
// amax is stored as codes E4M3(x * (448 / amax)) -- fp32 arithmetic, round
// to nearest even (the gfx950 conversion instruction, which also keeps the
// sign of zero) -- with the dequantisation scale amax / 448; an all-zero
// block has scale 0.
//
// Layout: fragments of 32 rows x 32 columns (1 KB).  Bytes [16 l, 16 l + 16)
// of a fragment are row l % 32: bytes 0..7 columns 8 h .. 8 h + 7 and bytes
// 8..15 columns 16 + 8 h .. 16 + 8 h + 7, with h = l / 32 -- the operands
// of lane l for the two 16-wide K steps of the fragment, so one 16-byte load
// per lane feeds two MFMAs.  Fragments are ordered (expert, 32-row block,
// 32-column K pair):
//   gate/up: fragment (e * 96 + b) * 64 + kp holds rows 16 b .. 16 b + 15 of
//            W_gate (fragment rows 0..15) and the same rows of W_up (rows
//            16..31), columns 32 kp .. 32 kp + 31;
//   down:    fragment (e * 64 + b) * 48 + kp holds rows 32 b .. 32 b + 31 of
//            W_down, columns 32 kp .. 32 kp + 31.
// Scales (fp32): gate/up [64][2][12][16] (expert, gate or up, 128-row block,
// 128-column block); down [64][16][12].
#include "common.hpp"
#include "launch.hpp"

namespace lfm {

namespace {

constexpr int kQBlock = 128;                  // rows and columns of a weight block
constexpr int kQThreads = 256;
constexpr int kQChunks = kQBlock * kQBlock / 8 / kQThreads;  // 8-column runs per thread

// One workgroup per 128 x 128 block.  W: the matrix's first element of the
// block's row 0, column 0 (row pitch `cols`); dst(r, c) gives the packed byte
// offset of row r, column c (c a multiple of 8) of the block.
template <typename Dst>
__device__ __forceinline__ void quantize_block(const uint16_t* __restrict__ W, int cols,
                                               uint8_t* __restrict__ out, float* __restrict__ scale,
                                               Dst dst) {
  __shared__ float wave_max[kQThreads / kWave];
  const int tid = threadIdx.x;
  float v[kQChunks][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kQChunks; ++i) {
    const int q = tid + kQThreads * i;
    const int r = q / (kQBlock / 8), c = (q % (kQBlock / 8)) * 8;
    const uint4 x = ld16(W + static_cast<size_t>(r) * cols + c);
    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[i][2 * k] = __uint_as_float(w4[k] << 16);
      v[i][2 * k + 1] = __uint_as_float(w4[k] & 0xffff0000u);
      amax = fmaxf(amax, fmaxf(fabsf(v[i][2 * k]), fabsf(v[i][2 * k + 1])));
    }
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  if ((tid & (kWave - 1)) == 0) wave_max[tid / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const float inv = amax > 0.f ? 448.f / amax : 0.f;
  if (tid == 0) *scale = amax / 448.f;
#pragma unroll
  for (int i = 0; i < kQChunks; ++i) {
    const int q = tid + kQThreads * i;
    const int r = q / (kQBlock / 8), c = (q % (kQBlock / 8)) * 8;
    const uint32_t lo = e4m3x4(v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv);
    const uint32_t hi = e4m3x4(v[i][4] * inv, v[i][5] * inv, v[i][6] * inv, v[i][7] * inv);
    *reinterpret_cast<uint2*>(out + dst(r, c)) = make_uint2(lo, hi);
  }
}

// Byte offset, inside a 1 KB fragment, of fragment row i, column c (c % 32 a
// multiple of 8).
__device__ __forceinline__ uint32_t frag_byte(int i, int c) {
  const int cc = c % 32;
  const int lane = i + 32 * ((cc % 16) / 8);
  return lane * 16 + (cc / 16) * 8;
}

// Block (e, m, rb, kb): m = 0 gate, 1 up; rb < 12 row blocks, kb < 16 column blocks.
// Expert e's matrices start at Wg + e * estride and Wu + e * estride.
__global__ __launch_bounds__(kQThreads) void pack_fp8_gateup_kernel(
    const uint16_t* __restrict__ Wg, const uint16_t* __restrict__ Wu, size_t estride,
    uint8_t* __restrict__ out, float* __restrict__ scales) {
  constexpr int kRB = kFF / kQBlock, kKB = kHidden / kQBlock;
  const int kb = blockIdx.x % kKB;
  const int rb = (blockIdx.x / kKB) % kRB;
  const int m = (blockIdx.x / (kKB * kRB)) % 2;
  const int e = blockIdx.x / (kKB * kRB * 2);
  const uint16_t* W = (m == 0 ? Wg : Wu) + static_cast<size_t>(e) * estride +
                      static_cast<size_t>(rb * kQBlock) * kHidden + kb * kQBlock;
  quantize_block(W, kHidden, out, scales + blockIdx.x, [=](int r, int c) {
    const int R = rb * kQBlock + r, C = kb * kQBlock + c;
    const size_t frag = (static_cast<size_t>(e) * kGateupBlocks + R / 16) * (kHidden / 32) + C / 32;
    return frag * 1024 + frag_byte(R % 16 + 16 * m, C);
  });
}

// Block (e, rb, kb): rb < 16 row blocks, kb < 12 column blocks.
__global__ __launch_bounds__(kQThreads) void pack_fp8_down_kernel(
    const uint16_t* __restrict__ Wd, uint8_t* __restrict__ out, float* __restrict__ scales) {
  constexpr int kRB = kHidden / kQBlock, kKB = kFF / kQBlock;
  const int kb = blockIdx.x % kKB;
  const int rb = (blockIdx.x / kKB) % kRB;
  const int e = blockIdx.x / (kKB * kRB);
  const uint16_t* W = Wd + (static_cast<size_t>(e) * kHidden + rb * kQBlock) * kFF + kb * kQBlock;
  quantize_block(W, kFF, out, scales + blockIdx.x, [=](int r, int c) {
    const int R = rb * kQBlock + r, C = kb * kQBlock + c;
    const size_t frag = (static_cast<size_t>(e) * kDownBlocks + R / 32) * (kFF / 32) + C / 32;
    return frag * 1024 + frag_byte(R % 32, C);
  });
}

}  // namespace

hipError_t launch_pack_fp8_gateup(const uint16_t* Wg, const uint16_t* Wu, size_t estride, uint8_t* out,
                                  float* scales, hipStream_t stream) {
  const int blocks = kExperts * 2 * (kFF / kQBlock) * (kHidden / kQBlock);
  hipLaunchKernelGGL(pack_fp8_gateup_kernel, dim3(blocks), dim3(kQThreads), 0, stream, Wg, Wu, estride,
                     out, scales);
  return hipGetLastError();
}

hipError_t launch_pack_fp8_down(const uint16_t* Wd, uint8_t* out, float* scales,
                                hipStream_t stream) {
  const int blocks = kExperts * (kHidden / kQBlock) * (kFF / kQBlock);
  hipLaunchKernelGGL(pack_fp8_down_kernel, dim3(blocks), dim3(kQThreads), 0, stream, Wd, out,
                     scales);
  return hipGetLastError();
}

}  // namespace lfm

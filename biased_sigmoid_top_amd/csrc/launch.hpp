// Host-side launchers of the device kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lfm {

// Tokens per router workgroup for N tokens (16 or 64); the per-block
// histogram has ceil(N / route_block_tokens(N)) rows.
int route_block_tokens(int64_t N);

// Upper bound of the number of m-tiles of tile_rows rows over all experts.
int64_t max_mtiles(int64_t N, int tile_rows);

// Expert e's gate and up matrices start at Wg + e * estride, Wu + e * estride.
hipError_t launch_pack_gateup(const uint16_t* Wg, const uint16_t* Wu, size_t estride, uint16_t* out,
                              hipStream_t stream);
hipError_t launch_pack_down(const uint16_t* Wd, uint16_t* out, hipStream_t stream);

// FP8 (E4M3) block quantisation + packing of the expert weights.
hipError_t launch_pack_fp8_gateup(const uint16_t* Wg, const uint16_t* Wu, size_t estride, uint8_t* out,
                                  float* scales, hipStream_t stream);
hipError_t launch_pack_fp8_down(const uint16_t* Wd, uint8_t* out, float* scales,
                                hipStream_t stream);

hipError_t launch_rmsnorm(const float* x, uint16_t* X, int64_t N, hipStream_t stream);

// Scratch bytes of the router's partial logits for N tokens.
size_t route_partial_bytes(int64_t N);
// With Xq and Xs (the FP8 layer's grouped path) the router also writes X's
// E4M3 codes and group scales, as launch_quantize_groups(X, N, 2048, Xq, Xs).
hipError_t launch_route(const uint16_t* X, const uint16_t* Wr, const float* bias, int32_t* idx,
                        float* w, int32_t* blockcounts, float* part, int N, hipStream_t stream,
                        uint8_t* Xq = nullptr, float* Xs = nullptr);

// Caller-given selections and weights -> workspace copies (ids made
// memory-safe) and the per-block histogram (when blockcounts is not null).
hipError_t launch_ingest_routing(const int32_t* idx_in, const float* w_in, int32_t* idx, float* w,
                                 int32_t* blockcounts, int N, hipStream_t stream);
hipError_t launch_dispatch(const int32_t* idx, const int32_t* blockcounts, int32_t* offsets,
                           int32_t* row2slot, int N, hipStream_t stream);

// Weight-streaming path: persistent kernels (one workgroup per CU) that
// group their own tokens (bf16 experts: N <= kDecodeMaxTokens; FP8 experts:
// N <= kStreamMaxTokens).
hipError_t launch_gateup_decode(const uint16_t* X, const uint16_t* Wgu, const int32_t* idx,
                                uint16_t* H, int N, hipStream_t stream);
hipError_t launch_down_decode(const uint16_t* H, const uint16_t* Wd, const int32_t* idx,
                              float* Y, int N, hipStream_t stream);
// The same with FP8 expert weights; the bf16 token rows are quantised per
// group of 128 as they are loaded.
hipError_t launch_gateup_decode_fp8(const uint16_t* X, const uint8_t* Wq, const float* scales,
                                    const int32_t* idx, uint16_t* H, int N, hipStream_t stream);
hipError_t launch_down_decode_fp8(const uint16_t* H, const uint8_t* Wq, const float* scales,
                                  const int32_t* idx, float* Y, int N, hipStream_t stream);

// FP8 grouped path: rows quantised per 128-wide group (E4M3 codes, one byte
// each, in the run order of quant.hip; fp32 scales [rows][K / 128]), then
// the tiled kernels in FP8 mode (the FP8 matrix cores).
hipError_t launch_quantize_groups(const uint16_t* A, int64_t rows, int K, uint8_t* Q, float* S,
                                  hipStream_t stream);
hipError_t launch_gateup_tiled_fp8(const uint8_t* Xq, const uint8_t* Wq, const float* Ws,
                                   const float* Xs, const int32_t* idx, int32_t* offsets,
                                   int32_t* row2slot, uint16_t* H, int64_t N, hipStream_t stream);
hipError_t launch_down_tiled_fp8(const uint8_t* Hq, const uint8_t* Wq, const float* Ws,
                                 const float* Hs, const int32_t* offsets, const int32_t* row2slot,
                                 float* Y, int64_t N, hipStream_t stream);

// Grouped path, LDS-tiled MFMA kernels.  Where gateup_groups_slots(N, fp8)
// the gate/up kernels (bf16 or FP8 mode) group the slots themselves from idx
// (no dispatch step) and write offsets and row2slot for the down kernels;
// otherwise they read the dispatch step's.
bool gateup_groups_slots(int64_t N, bool fp8);
hipError_t launch_gateup_tiled(const uint16_t* X, const uint16_t* Wgu, const int32_t* idx,
                               int32_t* offsets, int32_t* row2slot, uint16_t* H, int64_t N,
                               hipStream_t stream);
hipError_t launch_down_tiled(const uint16_t* H, const uint16_t* Wd, const int32_t* offsets,
                             const int32_t* row2slot, float* Y, int64_t N, hipStream_t stream);

hipError_t launch_combine(const float* Y, const float* w, const float* resid, float* out,
                          int64_t N, hipStream_t stream);
// x <- x + sum_j w Y (as launch_combine with resid = out = x), then
// Xn = bf16(RMSNorm(x)) of the new rows, bit for bit launch_rmsnorm's.
hipError_t launch_combine_norm(const float* Y, const float* w, float* x, uint16_t* Xn, int64_t N,
                               hipStream_t stream);

}  // namespace lfm

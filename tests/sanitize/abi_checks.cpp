// Host-side checks of the C ABI, built with AddressSanitizer and UBSan (host
// code only) by tests/test_abi_sanitized.py.  Every call here fails or
// returns before the library makes any HIP call, so no GPU is needed: null,
// negative, oversized and misaligned arguments, overlapping outputs, small or
// misaligned workspaces, N = 0, and the workspace size arithmetic up to the
// largest N.  Exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "lfm_moe.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "check failed (line %d): %s\n", line, what);
    ++failures;
  }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

// Fake device addresses: 16-byte aligned, far apart, never dereferenced.
template <typename T>
T* fake(int i, uintptr_t offset = 0) {
  return reinterpret_cast<T*>(static_cast<uintptr_t>(0x7f0000000000ull) + (static_cast<uintptr_t>(i) << 36) +
                              offset);
}

bool has_message() { return std::strlen(lfm_moe_last_error()) > 0; }

}  // namespace

int main() {
  EXPECT(lfm_moe_abi_version() == LFM_MOE_ABI_VERSION);
  const int64_t N = 64;
  const auto X = fake<const uint16_t>(0);
  const auto Wr = fake<const uint16_t>(1);
  const auto b = fake<const float>(2);
  const auto Wgu = fake<const uint16_t>(3);
  const auto Wd = fake<const uint16_t>(4);
  float* out = fake<float>(5);

  // Layer: N == 0 is a no-op; bad N; nulls; misalignment; overlaps.
  EXPECT(lfm_moe_forward(X, Wr, b, Wgu, Wd, out, 0, nullptr) == LFM_MOE_OK);
  EXPECT(lfm_moe_forward(X, Wr, b, Wgu, Wd, out, -1, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT && has_message());
  EXPECT(lfm_moe_forward(X, Wr, b, Wgu, Wd, out, LFM_MOE_MAX_TOKENS + 1, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_forward(nullptr, Wr, b, Wgu, Wd, out, N, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_forward(X, Wr, b, Wgu, Wd, nullptr, N, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_forward(fake<const uint16_t>(0, 2), Wr, b, Wgu, Wd, out, N, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_forward(X, Wr, b, Wgu, Wd, fake<float>(3, 4096), N, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_forward(X, Wr, b, Wgu, Wd, fake<float>(0, 256), N, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);

  // Caller workspace: null, misaligned, too small, overlapping the output.
  const size_t need = lfm_moe_workspace_bytes(N);
  void* ws = fake<void>(6);
  EXPECT(lfm_moe_forward_ws(X, Wr, b, Wgu, Wd, out, N, nullptr, need, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_forward_ws(X, Wr, b, Wgu, Wd, out, N, fake<void>(6, 16), need, nullptr) ==
         LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_forward_ws(X, Wr, b, Wgu, Wd, out, N, ws, need - 1, nullptr) == LFM_MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(lfm_moe_forward_ws(X, Wr, b, Wgu, Wd, out, N, fake<void>(5, 0) , need, nullptr) ==
         LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_forward_ws(X, Wr, b, Wgu, Wd, out, 0, nullptr, 0, nullptr) == LFM_MOE_OK);

  // Block forward (x in place), router, RMSNorm, packing.
  float* x = fake<float>(7);
  EXPECT(lfm_moe_block_forward(x, Wr, b, Wgu, Wd, 0, nullptr) == LFM_MOE_OK);
  EXPECT(lfm_moe_block_forward(nullptr, Wr, b, Wgu, Wd, N, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_block_forward_ws(x, Wr, b, Wgu, Wd, N, ws, 0, nullptr) == LFM_MOE_ERR_WORKSPACE_TOO_SMALL);
  {
    const lfm_moe_block_weights blocks[2] = {{Wr, b, Wgu, Wd}, {Wr, b, Wgu, nullptr}};
    EXPECT(lfm_moe_stack_forward_ws(x, blocks, 2, N, ws, need, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
    EXPECT(lfm_moe_stack_forward_ws(x, blocks, -1, N, ws, need, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
    EXPECT(lfm_moe_stack_forward_ws(x, nullptr, 1, N, ws, need, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
    EXPECT(lfm_moe_stack_forward_ws(x, blocks, 1, N, ws, 0, nullptr) == LFM_MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(lfm_moe_stack_forward_ws(x, blocks, 2, 0, nullptr, 0, nullptr) == LFM_MOE_OK);
    EXPECT(lfm_moe_stack_forward_ws(x, blocks, 0, N, ws, need, nullptr) == LFM_MOE_OK);
  }
  EXPECT(lfm_moe_route(X, Wr, b, fake<int32_t>(8), fake<float>(8, 64), N, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_route(X, Wr, b, nullptr, fake<float>(9), N, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_route(X, Wr, b, fake<int32_t>(8), fake<float>(9), 0, nullptr) == LFM_MOE_OK);
  const size_t rneed = lfm_moe_route_workspace_bytes(N);
  EXPECT(rneed == 4u * 16 * 16 * 64 * 4 && lfm_moe_route_workspace_bytes(4096) == 0);
  EXPECT(lfm_moe_route_ws(X, Wr, b, fake<int32_t>(8), fake<float>(9), N, nullptr, rneed, nullptr) ==
         LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_route_ws(X, Wr, b, fake<int32_t>(8), fake<float>(9), N, ws, rneed - 4, nullptr) ==
         LFM_MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(lfm_moe_route_ws(X, Wr, b, fake<int32_t>(8), fake<float>(9), N, fake<void>(0, 256), rneed, nullptr) ==
         LFM_MOE_ERR_INVALID_ARGUMENT && has_message());
  EXPECT(lfm_moe_route_ws(X, Wr, b, fake<int32_t>(8), fake<float>(9), 0, nullptr, 0, nullptr) == LFM_MOE_OK);
  EXPECT(lfm_moe_pack_gateup_stacked(Wgu, fake<uint16_t>(3, 1024), nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_pack_fp8_gateup_stacked(Wgu, fake<uint8_t>(10), nullptr, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_rmsnorm(nullptr, fake<uint16_t>(9), N, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_rmsnorm(x, fake<uint16_t>(9), -5, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_pack_gateup(Wgu, nullptr, fake<uint16_t>(10), nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_pack_down(Wd, fake<uint16_t>(4, 512), nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);

  // FP8 entry points.
  const auto q8 = fake<const uint8_t>(11);
  const auto s8 = fake<const float>(12);
  const auto d8 = fake<const uint8_t>(13);
  const auto t8 = fake<const float>(14);
  EXPECT(lfm_moe_forward_fp8(X, Wr, b, q8, s8, d8, t8, out, 0, nullptr) == LFM_MOE_OK);
  EXPECT(lfm_moe_forward_fp8(X, Wr, b, q8, s8, d8, t8, out, LFM_MOE_FP8_MAX_TOKENS + 1, nullptr) ==
         LFM_MOE_ERR_INVALID_ARGUMENT && has_message());
  EXPECT(lfm_moe_forward_fp8(X, Wr, b, q8, nullptr, d8, t8, out, N, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_forward_fp8(X, Wr, b, q8, s8, d8, t8, fake<float>(11, 1024), N, nullptr) ==
         LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_forward_fp8_ws(X, Wr, b, q8, s8, d8, t8, out, N, ws, need - 16, nullptr) ==
         LFM_MOE_ERR_WORKSPACE_TOO_SMALL);

  // Expert path on given routing: nulls, workspace, routing overlapping out or the workspace.
  const auto ri = fake<const int32_t>(16);
  const auto rw = fake<const float>(17);
  EXPECT(lfm_moe_experts_ws(X, ri, rw, Wgu, Wd, out, 0, nullptr, 0, nullptr) == LFM_MOE_OK);
  EXPECT(lfm_moe_experts_ws(X, nullptr, rw, Wgu, Wd, out, N, ws, need, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_experts_ws(X, ri, rw, Wgu, Wd, out, N, ws, need - 1, nullptr) == LFM_MOE_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(lfm_moe_experts_ws(X, ri, fake<const float>(6, 512), Wgu, Wd, out, N, ws, need, nullptr) ==
         LFM_MOE_ERR_INVALID_ARGUMENT && has_message());
  EXPECT(lfm_moe_experts_ws(X, ri, rw, Wgu, Wd, fake<float>(16, 0), N, ws, need, nullptr) ==
         LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_experts_fp8_ws(X, ri, rw, q8, s8, d8, nullptr, out, N, ws, need, nullptr) ==
         LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_experts_fp8_ws(X, ri, rw, q8, s8, d8, t8, out, LFM_MOE_FP8_MAX_TOKENS + 1, ws, need, nullptr) ==
         LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_pack_fp8_gateup(Wgu, Wgu, fake<uint8_t>(3, 512), fake<float>(15), nullptr) ==
         LFM_MOE_ERR_INVALID_ARGUMENT);
  EXPECT(lfm_moe_pack_fp8_down(Wd, fake<uint8_t>(16), nullptr, nullptr) == LFM_MOE_ERR_INVALID_ARGUMENT);

  // Workspace arithmetic up to the largest N: every region 256-byte aligned and inside the total.
  const int64_t sizes[] = {0, 1, 17, 96, 97, 256, 2048, 2049, 4096, 16384, LFM_MOE_MAX_TOKENS};
  for (int64_t n : sizes) {
    const size_t total = lfm_moe_workspace_bytes(n);
    // H (bf16) and Y (fp32) rows of all 4n slots fit (the router partials
    // region empties above 2,048 tokens, so the total is not monotone in n).
    EXPECT(total >= static_cast<size_t>(4 * n) * (1536 * 2 + 2048 * 4));
    for (int r = 0; r < LFM_MOE_WS_REGIONS; ++r) {
      const size_t off = lfm_moe_workspace_offset(n, r);
      EXPECT(off % 256 == 0);
      EXPECT(off <= total);
    }
  }
  EXPECT(lfm_moe_workspace_offset(64, LFM_MOE_WS_REGIONS) == SIZE_MAX);
  EXPECT(lfm_moe_workspace_offset(-1, 0) == SIZE_MAX);
  lfm_moe_release();  // nothing allocated: no HIP call

  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("abi checks ok\n");
  return 0;
}

// C ABI of the MoE layer: argument checks, workspace layout and the launch
// sequence route -> dispatch -> gate/up -> down -> combine on one stream.
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "lfm_moe.h"
#include "common.hpp"
#include "launch.hpp"

using namespace lfm;

namespace {

thread_local std::string g_last_error;

lfm_moe_status fail(lfm_moe_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

lfm_moe_status hip_fail(hipError_t e, const char* what) {
  return fail(LFM_MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                                   hipGetErrorString(e) + ")");
}

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Sizes of the workspace regions, in lfm_moe_ws_region order.
void region_sizes(int64_t N, size_t (&sz)[LFM_MOE_WS_REGIONS]) {
  const size_t n = static_cast<size_t>(N);
  const size_t rows = n * kTopK;
  const size_t nrb = (n + route_block_tokens(N) - 1) / route_block_tokens(N);
  sz[LFM_MOE_WS_IDX] = rows * sizeof(int32_t);
  sz[LFM_MOE_WS_W] = rows * sizeof(float);
  sz[LFM_MOE_WS_BLOCKCOUNTS] = nrb * kExperts * sizeof(int32_t);
  sz[LFM_MOE_WS_OFFSETS] = (kExperts + 1) * sizeof(int32_t);
  sz[LFM_MOE_WS_ROW2SLOT] = rows * sizeof(int32_t);
  sz[LFM_MOE_WS_H] = rows * kFF * sizeof(uint16_t);
  sz[LFM_MOE_WS_Y] = rows * kHidden * sizeof(float);
  sz[LFM_MOE_WS_X] = n * kHidden * sizeof(uint16_t);
  sz[LFM_MOE_WS_ROUTER_PARTIAL] = route_partial_bytes(N);
  // FP8 grouped path only: quantised rows and their per-128 group scales.
  const bool fp8_grouped = N > LFM_MOE_FP8_STREAM_TOKENS;
  sz[LFM_MOE_WS_XQ] = fp8_grouped ? n * kHidden : 0;  // one byte per code
  sz[LFM_MOE_WS_XS] = fp8_grouped ? n * (kHidden / 128) * sizeof(float) : 0;
  sz[LFM_MOE_WS_HQ] = fp8_grouped ? rows * kFF : 0;
  sz[LFM_MOE_WS_HS] = fp8_grouped ? rows * (kFF / 128) * sizeof(float) : 0;
}

size_t region_offset(int64_t N, int region) {
  size_t sz[LFM_MOE_WS_REGIONS];
  region_sizes(N, sz);
  size_t off = 0;
  for (int r = 0; r < region; ++r) off += align_up(sz[r]);
  return off;
}

size_t workspace_bytes(int64_t N) { return region_offset(N, LFM_MOE_WS_REGIONS); }

bool misaligned(const void* p, size_t a = 16) {
  return (reinterpret_cast<uintptr_t>(p) % a) != 0;
}

struct Span {
  const void* p;
  size_t bytes;
};

bool overlap(Span a, Span b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Checks shared by every layer entry point.  Returns OK, or the error.
// With_router false (the expert path on caller-given routing): W_r and
// bias are not used and not checked.
lfm_moe_status check_layer_args(const void* x, size_t x_bytes, const uint16_t* W_r,
                                const float* bias, const uint16_t* W_gateup,
                                const uint16_t* W_down, const void* out, size_t out_bytes,
                                int64_t N, bool out_is_input, bool with_router = true) {
  if (N < 0) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "N must be >= 0");
  if (N > LFM_MOE_MAX_TOKENS) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "N exceeds LFM_MOE_MAX_TOKENS");
  if (N == 0) return LFM_MOE_OK;
  if (!x || (with_router && (!W_r || !bias)) || !W_gateup || !W_down || !out)
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (misaligned(x) || (with_router && (misaligned(W_r) || misaligned(bias))) || misaligned(W_gateup) ||
      misaligned(W_down) || misaligned(out))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  const Span o{out, out_bytes};
  const Span ins[] = {{W_r, with_router ? sizeof(uint16_t) * kExperts * kHidden : 0},
                      {bias, with_router ? sizeof(float) * kExperts : 0},
                      {W_gateup, sizeof(uint16_t) * kExperts * 2 * kFF * kHidden},
                      {W_down, sizeof(uint16_t) * kExperts * kHidden * kFF}};
  for (const Span& s : ins)
    if (overlap(o, s)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps a weight tensor");
  if (!out_is_input && overlap(o, Span{x, x_bytes}))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps the input");
  return LFM_MOE_OK;
}

// The caller workspace: present, aligned, large enough, and apart from the
// output and from every input tensor (its regions are written while the
// inputs are still being read).
lfm_moe_status check_ws(void* ws, size_t ws_bytes, int64_t N, Span out,
                        std::initializer_list<Span> inputs) {
  if (!ws) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null workspace");
  if (misaligned(ws, kAlign)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (ws_bytes < workspace_bytes(N))
    return fail(LFM_MOE_ERR_WORKSPACE_TOO_SMALL,
                "workspace of " + std::to_string(ws_bytes) + " bytes, need " +
                    std::to_string(workspace_bytes(N)));
  const Span w{ws, ws_bytes};
  if (overlap(w, out)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "workspace overlaps the output");
  for (const Span& s : inputs)
    if (overlap(w, s)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "workspace overlaps an input");
  return LFM_MOE_OK;
}

// Spans of the bf16 layer's weights and of the FP8 experts.
Span gateup_span(const void* p) { return {p, sizeof(uint16_t) * kExperts * 2 * kFF * kHidden}; }
Span down_span(const void* p) { return {p, sizeof(uint16_t) * kExperts * kHidden * kFF}; }
Span router_span(const void* p) { return {p, p ? sizeof(uint16_t) * kExperts * kHidden : 0}; }
Span bias_span(const void* p) { return {p, p ? sizeof(float) * kExperts : 0}; }

// Checks of the caller-given routing of the expert-path entry points: the
// selections and weights are read once (at the start of the call) and may
// overlap each other, but neither the output nor the workspace.
lfm_moe_status check_routing_args(const int32_t* idx, const float* w, int64_t N, Span out, void* ws,
                                  size_t ws_bytes) {
  if (!idx || !w) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (misaligned(idx) || misaligned(w))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  const size_t sel = static_cast<size_t>(N) * kTopK * 4;
  const Span ins[] = {{idx, sel}, {w, sel}};
  for (const Span& s : ins) {
    if (overlap(out, s)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps the routing");
    if (overlap(Span{ws, ws_bytes}, s))
      return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "workspace overlaps the routing");
  }
  return LFM_MOE_OK;
}

// Checks of the stage entry points: tensors present and aligned, the
// workspace as for the layer and apart from them.
lfm_moe_status check_stage(int64_t N, void* ws, size_t ws_bytes, Span out, std::initializer_list<Span> ins) {
  if (N < 0) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "N must be >= 0");
  if (N > LFM_MOE_MAX_TOKENS) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "N exceeds LFM_MOE_MAX_TOKENS");
  if (N == 0) return LFM_MOE_OK;
  for (const Span& s : ins)
    if (!s.p) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
    else if (misaligned(s.p)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  if (out.bytes != 0) {
    if (!out.p) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
    if (misaligned(out.p)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  }
  return check_ws(ws, ws_bytes, N, out, ins);
}

// Library-owned workspaces, one per device and purpose (the layer's, and
// the router's partial logits for lfm_moe_route), grown on demand.
constexpr int kMaxDevices = 64;
enum WsKind { kLayerWs = 0, kRouteWs = 1, kWsKinds = 2 };
std::mutex g_ws_mu;
void* g_ws[kWsKinds][kMaxDevices] = {};
size_t g_ws_bytes[kWsKinds][kMaxDevices] = {};

lfm_moe_status internal_ws(WsKind kind, size_t need, void** ws, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_ws_mu);
  void*& buf = g_ws[kind][dev];
  size_t& have = g_ws_bytes[kind][dev];
  if (have < need) {
    if (buf) {
      e = hipFree(buf);  // hipFree waits for work that may still use it
      buf = nullptr;
      have = 0;
      if (e != hipSuccess) return hip_fail(e, "hipFree(workspace)");
    }
    e = hipMalloc(&buf, need);
    if (e != hipSuccess) {
      buf = nullptr;
      (void)hipGetLastError();
      return fail(LFM_MOE_ERR_OUT_OF_MEMORY, "hipMalloc of " + std::to_string(need) + " workspace bytes failed");
    }
    have = need;
  }
  *ws = buf;
  *bytes = have;
  return LFM_MOE_OK;
}

lfm_moe_status internal_ws(int64_t N, void** ws, size_t* bytes) {
  return internal_ws(kLayerWs, workspace_bytes(N), ws, bytes);
}

// Workspace of lfm_moe_forward_noalloc: a static device array, one per GPU,
// held until the process ends.  In host code its name is only a stand-in
// for the symbol; the kernels get its device address, looked up once per
// device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[LFM_MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

lfm_moe_status scratch_address(void** p) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(LFM_MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave no address");
    g_scratch[dev] = ptr;
  }
  *p = g_scratch[dev];
  return LFM_MOE_OK;
}

// Per-kernel timing for measurements (lfm_moe_timing_*).
constexpr int kStages = LFM_MOE_STAGES;
constexpr int kMaxMarks = kStages + 1;
constexpr size_t kMaxPending = 4096;

struct TimedCall {
  hipEvent_t ev[kMaxMarks];
  int stage[kStages];
  int n = 0;  // kernels recorded
};

struct TimingState {
  std::mutex mu;
  bool on = false;
  std::vector<TimedCall> pending;
  double total_ms[kStages] = {};
  int64_t launches[kStages] = {};
} g_timing;

// Waits for and folds the pending records into the totals (mu held).
hipError_t drain_pending() {
  hipError_t first = hipSuccess;
  for (TimedCall& c : g_timing.pending) {
    hipError_t e = hipEventSynchronize(c.ev[c.n]);
    for (int i = 0; i < c.n && e == hipSuccess; ++i) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, c.ev[i], c.ev[i + 1]);
      if (e == hipSuccess) {
        g_timing.total_ms[c.stage[i]] += ms;
        g_timing.launches[c.stage[i]] += 1;
      }
    }
    if (e != hipSuccess && first == hipSuccess) first = e;
    for (int i = 0; i <= c.n; ++i) (void)hipEventDestroy(c.ev[i]);
  }
  g_timing.pending.clear();
  return first;
}

// Records an event before the first kernel of a call and after each kernel.
class StageTimer {
 public:
  explicit StageTimer(hipStream_t s) : stream_(s) {
    std::lock_guard<std::mutex> lock(g_timing.mu);
    on_ = g_timing.on;
    if (on_) on_ = record(0);
  }
  void after(int stage) {
    if (!on_) return;
    call_.stage[call_.n] = stage;
    if (record(call_.n + 1)) ++call_.n;
    else on_ = false;
  }
  // Hands a complete record to the pending list; otherwise (timing off
  // mid-call after a failed event call, or no kernel recorded) destroys the
  // events it created.
  ~StageTimer() {
    if (on_ && call_.n > 0) {
      std::lock_guard<std::mutex> lock(g_timing.mu);
      if (g_timing.pending.size() >= kMaxPending) (void)drain_pending();
      g_timing.pending.push_back(call_);
      return;
    }
    for (int i = 0; i < created_; ++i) (void)hipEventDestroy(call_.ev[i]);
  }

 private:
  bool record(int i) {
    if (hipEventCreate(&call_.ev[i]) != hipSuccess) return false;
    created_ = i + 1;
    return hipEventRecord(call_.ev[i], stream_) == hipSuccess;
  }
  hipStream_t stream_;
  bool on_ = false;
  int created_ = 0;  // events created so far (ev[0 .. created_ - 1])
  TimedCall call_;
};

template <typename T>
T* region(void* ws, int64_t N, lfm_moe_ws_region r) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + region_offset(N, r));
}

// Decode-shaped batches take the expert-major streaming kernels, which
// group their own tokens; larger batches go through the dispatch step.
bool use_decode_path(int64_t N) { return N <= kDecodeMaxTokens; }
static_assert(kDecodeMaxTokens == LFM_MOE_FP8_STREAM_TOKENS && kDecodeMaxTokens <= kStreamMaxTokens,
              "both layers stream the same batches, which the streaming kernels can group");

// The router's outputs in the workspace: from the router, or copied from
// caller-given selections and weights (idx_in, w_in not null), with the
// per-block histogram when the grouped path needs it.  With Xq (FP8 layer)
// the router also quantises X into Xq / Xs; the copy does not.
hipError_t route_or_ingest(const uint16_t* X, const uint16_t* W_r, const float* bias,
                           const int32_t* idx_in, const float* w_in, int32_t* idx, float* w,
                           int32_t* blockcounts, float* part, int n, hipStream_t stream,
                           uint8_t* Xq = nullptr, float* Xs = nullptr) {
  if (idx_in != nullptr) return launch_ingest_routing(idx_in, w_in, idx, w, blockcounts, n, stream);
  return launch_route(X, W_r, bias, idx, w, blockcounts, part, n, stream, Xq, Xs);
}

// route -> [dispatch] -> gate/up -> down -> combine.  Arguments already
// checked.  With idx_in and w_in the router is replaced by a copy of them.
// With X_next (then resid == out) the combine also stores the next block's
// input bf16(RMSNorm(out)) there.
lfm_moe_status run_layer(const uint16_t* X, const uint16_t* W_r, const float* bias,
                         const int32_t* idx_in, const float* w_in,
                         const uint16_t* W_gateup, const uint16_t* W_down, const float* resid,
                         float* out, int64_t N, void* ws, hipStream_t stream, StageTimer& timer,
                         uint16_t* X_next = nullptr) {
  int32_t* idx = region<int32_t>(ws, N, LFM_MOE_WS_IDX);
  float* w = region<float>(ws, N, LFM_MOE_WS_W);
  int32_t* blockcounts = region<int32_t>(ws, N, LFM_MOE_WS_BLOCKCOUNTS);
  int32_t* offsets = region<int32_t>(ws, N, LFM_MOE_WS_OFFSETS);
  int32_t* row2slot = region<int32_t>(ws, N, LFM_MOE_WS_ROW2SLOT);
  uint16_t* H = region<uint16_t>(ws, N, LFM_MOE_WS_H);
  float* Y = region<float>(ws, N, LFM_MOE_WS_Y);
  float* part = region<float>(ws, N, LFM_MOE_WS_ROUTER_PARTIAL);
  const int n = static_cast<int>(N);
  const bool decode = use_decode_path(N);
  const bool dispatch = !decode && !gateup_groups_slots(N, false);
  hipError_t e;
  if ((e = route_or_ingest(X, W_r, bias, idx_in, w_in, idx, w, dispatch ? blockcounts : nullptr, part, n,
                           stream)) != hipSuccess)
    return hip_fail(e, idx_in ? "routing copy kernel launch" : "route kernel launch");
  timer.after(1);
  if (decode) {
    if ((e = launch_gateup_decode(X, W_gateup, idx, H, n, stream)) != hipSuccess)
      return hip_fail(e, "gate/up kernel launch");
    timer.after(3);
    if ((e = launch_down_decode(H, W_down, idx, Y, n, stream)) != hipSuccess)
      return hip_fail(e, "down kernel launch");
    timer.after(4);
  } else {
    if (dispatch) {
      if ((e = launch_dispatch(idx, blockcounts, offsets, row2slot, n, stream)) != hipSuccess)
        return hip_fail(e, "dispatch kernel launch");
      timer.after(2);
    }
    if ((e = launch_gateup_tiled(X, W_gateup, idx, offsets, row2slot, H, N, stream)) != hipSuccess)
      return hip_fail(e, "gate/up kernel launch");
    timer.after(3);
    if ((e = launch_down_tiled(H, W_down, offsets, row2slot, Y, N, stream)) != hipSuccess)
      return hip_fail(e, "down kernel launch");
    timer.after(4);
  }
  e = X_next != nullptr ? launch_combine_norm(Y, w, out, X_next, N, stream)
                       : launch_combine(Y, w, resid, out, N, stream);
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  timer.after(5);
  return LFM_MOE_OK;
}

size_t act_bytes(int64_t N, size_t elem) {
  return static_cast<size_t>(N < 0 ? 0 : N) * kHidden * elem;
}

// FP8 experts: one byte per weight, a fp32 scale per 128 x 128 block.
constexpr size_t kFp8GateupBytes = static_cast<size_t>(kExperts) * 2 * kFF * kHidden;
constexpr size_t kFp8DownBytes = static_cast<size_t>(kExperts) * kHidden * kFF;
constexpr size_t kFp8GateupScaleBytes = sizeof(float) * kExperts * 2 * (kFF / 128) * (kHidden / 128);
constexpr size_t kFp8DownScaleBytes = sizeof(float) * kExperts * (kHidden / 128) * (kFF / 128);

// Checks of the FP8 layer entry points (with_router as for check_layer_args).
lfm_moe_status check_fp8_args(const uint16_t* X, const uint16_t* W_r, const float* bias,
                              const uint8_t* W_gateup_fp8, const float* scales_gateup,
                              const uint8_t* W_down_fp8, const float* scales_down, const float* out,
                              int64_t N, bool with_router = true) {
  if (N < 0) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "N must be >= 0");
  if (N > LFM_MOE_FP8_MAX_TOKENS) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "N exceeds LFM_MOE_FP8_MAX_TOKENS");
  if (N == 0) return LFM_MOE_OK;
  if (!X || (with_router && (!W_r || !bias)) || !W_gateup_fp8 || !scales_gateup || !W_down_fp8 ||
      !scales_down || !out)
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (misaligned(X) || (with_router && (misaligned(W_r) || misaligned(bias))) || misaligned(W_gateup_fp8) ||
      misaligned(scales_gateup) || misaligned(W_down_fp8) || misaligned(scales_down) || misaligned(out))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  const Span o{out, act_bytes(N, 4)};
  const Span ins[] = {{X, act_bytes(N, 2)},
                      {W_r, with_router ? sizeof(uint16_t) * kExperts * kHidden : 0},
                      {bias, with_router ? sizeof(float) * kExperts : 0},
                      {W_gateup_fp8, kFp8GateupBytes},
                      {scales_gateup, kFp8GateupScaleBytes},
                      {W_down_fp8, kFp8DownBytes},
                      {scales_down, kFp8DownScaleBytes}};
  for (const Span& s : ins)
    if (overlap(o, s)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps an input");
  return LFM_MOE_OK;
}

// The FP8 layer on checked arguments: route (or the caller's routing),
// FP8 gate/up and down (weight streaming, each workgroup groups the slots
// itself, or the grouped kernels in FP8 mode), combine.
lfm_moe_status run_fp8(const uint16_t* X, const uint16_t* W_r, const float* bias,
                       const int32_t* idx_in, const float* w_in, const uint8_t* W_gateup_fp8, const float* scales_gateup,
                       const uint8_t* W_down_fp8, const float* scales_down, float* out, int64_t N,
                       void* ws, hipStream_t stream) {
  StageTimer timer(stream);
  int32_t* idx = region<int32_t>(ws, N, LFM_MOE_WS_IDX);
  float* w = region<float>(ws, N, LFM_MOE_WS_W);
  uint16_t* H = region<uint16_t>(ws, N, LFM_MOE_WS_H);
  float* Y = region<float>(ws, N, LFM_MOE_WS_Y);
  float* part = region<float>(ws, N, LFM_MOE_WS_ROUTER_PARTIAL);
  const int n = static_cast<int>(N);
  const bool streaming = N <= LFM_MOE_FP8_STREAM_TOKENS;
  const bool dispatch = !streaming && !gateup_groups_slots(N, true);
  int32_t* blockcounts = region<int32_t>(ws, N, LFM_MOE_WS_BLOCKCOUNTS);
  uint8_t* Xq = region<uint8_t>(ws, N, LFM_MOE_WS_XQ);
  float* Xs = region<float>(ws, N, LFM_MOE_WS_XS);
  // The grouped path's router quantises X as it reads it (one launch fewer);
  // caller-given routing leaves that to quantize_groups.
  const bool route_quantises = !streaming && idx_in == nullptr;
  hipError_t e;
  if ((e = route_or_ingest(X, W_r, bias, idx_in, w_in, idx, w, dispatch ? blockcounts : nullptr, part,
                           n, stream, route_quantises ? Xq : nullptr, route_quantises ? Xs : nullptr)) !=
      hipSuccess)
    return hip_fail(e, idx_in ? "routing copy kernel launch" : "route kernel launch");
  timer.after(1);
  if (streaming) {
    if ((e = launch_gateup_decode_fp8(X, W_gateup_fp8, scales_gateup, idx, H, n, stream)) != hipSuccess)
      return hip_fail(e, "fp8 gate/up kernel launch");
    timer.after(3);
    if ((e = launch_down_decode_fp8(H, W_down_fp8, scales_down, idx, Y, n, stream)) != hipSuccess)
      return hip_fail(e, "fp8 down kernel launch");
    timer.after(4);
  } else {
    // Grouped: dispatch (unless the gate/up kernel groups the slots), X
    // quantised per group (by the router; with caller-given routing by
    // quantize_groups, timed as the dispatch stage), gate/up, H quantised
    // per group (timed with down), down.
    int32_t* offsets = region<int32_t>(ws, N, LFM_MOE_WS_OFFSETS);
    int32_t* row2slot = region<int32_t>(ws, N, LFM_MOE_WS_ROW2SLOT);
    uint8_t* Hq = region<uint8_t>(ws, N, LFM_MOE_WS_HQ);
    float* Hs = region<float>(ws, N, LFM_MOE_WS_HS);
    if (dispatch && (e = launch_dispatch(idx, blockcounts, offsets, row2slot, n, stream)) != hipSuccess)
      return hip_fail(e, "dispatch kernel launch");
    if (!route_quantises && (e = launch_quantize_groups(X, N, kHidden, Xq, Xs, stream)) != hipSuccess)
      return hip_fail(e, "quantize kernel launch");
    if (dispatch || !route_quantises) timer.after(2);
    if ((e = launch_gateup_tiled_fp8(Xq, W_gateup_fp8, scales_gateup, Xs, idx, offsets, row2slot, H,
                                     N, stream)) != hipSuccess)
      return hip_fail(e, "fp8 gate/up kernel launch");
    timer.after(3);
    if ((e = launch_quantize_groups(H, N * kTopK, kFF, Hq, Hs, stream)) != hipSuccess)
      return hip_fail(e, "quantize kernel launch");
    if ((e = launch_down_tiled_fp8(Hq, W_down_fp8, scales_down, Hs, offsets, row2slot, Y, N,
                                   stream)) != hipSuccess)
      return hip_fail(e, "fp8 down kernel launch");
    timer.after(4);
  }
  if ((e = launch_combine(Y, w, nullptr, out, N, stream)) != hipSuccess)
    return hip_fail(e, "combine kernel launch");
  timer.after(5);
  return LFM_MOE_OK;
}

}  // namespace

extern "C" {

int lfm_moe_abi_version(void) { return LFM_MOE_ABI_VERSION; }

const char* lfm_moe_last_error(void) { return g_last_error.c_str(); }

size_t lfm_moe_workspace_bytes(int64_t N) {
  if (N < 0 || N > LFM_MOE_MAX_TOKENS) return 0;
  return workspace_bytes(N);
}

size_t lfm_moe_workspace_offset(int64_t N, int region) {
  if (N < 0 || N > LFM_MOE_MAX_TOKENS || region < 0 || region >= LFM_MOE_WS_REGIONS)
    return static_cast<size_t>(-1);
  return region_offset(N, region);
}

lfm_moe_status lfm_moe_rmsnorm(const float* x, uint16_t* X, int64_t N, hipStream_t stream) {
  g_last_error.clear();
  if (N < 0 || N > LFM_MOE_MAX_TOKENS) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "N out of range");
  if (N == 0) return LFM_MOE_OK;
  if (!x || !X) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (misaligned(x) || misaligned(X)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  if (overlap(Span{x, act_bytes(N, 4)}, Span{X, act_bytes(N, 2)}))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps the input");
  hipError_t e = launch_rmsnorm(x, X, N, stream);
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "rmsnorm kernel launch");
}

lfm_moe_status lfm_moe_pack_gateup(const uint16_t* W_gate, const uint16_t* W_up,
                                   uint16_t* W_gateup, hipStream_t stream) {
  g_last_error.clear();
  if (!W_gate || !W_up || !W_gateup) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (misaligned(W_gate) || misaligned(W_up) || misaligned(W_gateup))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  const size_t half = sizeof(uint16_t) * kExperts * kFF * kHidden;
  const Span o{W_gateup, 2 * half};
  if (overlap(o, Span{W_gate, half}) || overlap(o, Span{W_up, half}))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps an input");
  hipError_t e = launch_pack_gateup(W_gate, W_up, static_cast<size_t>(kFF) * kHidden, W_gateup, stream);
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "pack kernel launch");
}

lfm_moe_status lfm_moe_pack_gateup_stacked(const uint16_t* W_gateup, uint16_t* W_gateup_packed,
                                           hipStream_t stream) {
  g_last_error.clear();
  if (!W_gateup || !W_gateup_packed) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (misaligned(W_gateup) || misaligned(W_gateup_packed))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  const size_t bytes = sizeof(uint16_t) * kExperts * 2 * kFF * kHidden;
  if (overlap(Span{W_gateup, bytes}, Span{W_gateup_packed, bytes}))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps the input");
  const size_t half = static_cast<size_t>(kFF) * kHidden;
  hipError_t e = launch_pack_gateup(W_gateup, W_gateup + half, 2 * half, W_gateup_packed, stream);
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "pack kernel launch");
}

lfm_moe_status lfm_moe_pack_down(const uint16_t* W_down, uint16_t* W_down_packed,
                                 hipStream_t stream) {
  g_last_error.clear();
  if (!W_down || !W_down_packed) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (misaligned(W_down) || misaligned(W_down_packed))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  const size_t bytes = sizeof(uint16_t) * kExperts * kHidden * kFF;
  if (overlap(Span{W_down, bytes}, Span{W_down_packed, bytes}))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps the input");
  hipError_t e = launch_pack_down(W_down, W_down_packed, stream);
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "pack kernel launch");
}

lfm_moe_status lfm_moe_pack_fp8_gateup(const uint16_t* W_gate, const uint16_t* W_up,
                                       uint8_t* W_gateup_fp8, float* scales_gateup,
                                       hipStream_t stream) {
  g_last_error.clear();
  if (!W_gate || !W_up || !W_gateup_fp8 || !scales_gateup)
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (misaligned(W_gate) || misaligned(W_up) || misaligned(W_gateup_fp8) || misaligned(scales_gateup))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  const size_t half = sizeof(uint16_t) * kExperts * kFF * kHidden;
  const Span outs[] = {{W_gateup_fp8, kFp8GateupBytes}, {scales_gateup, kFp8GateupScaleBytes}};
  for (const Span& o : outs)
    if (overlap(o, Span{W_gate, half}) || overlap(o, Span{W_up, half}))
      return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps an input");
  if (overlap(outs[0], outs[1])) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "codes overlap scales");
  hipError_t e = launch_pack_fp8_gateup(W_gate, W_up, static_cast<size_t>(kFF) * kHidden, W_gateup_fp8,
                                        scales_gateup, stream);
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "fp8 pack kernel launch");
}

lfm_moe_status lfm_moe_pack_fp8_gateup_stacked(const uint16_t* W_gateup, uint8_t* W_gateup_fp8,
                                               float* scales_gateup, hipStream_t stream) {
  g_last_error.clear();
  if (!W_gateup || !W_gateup_fp8 || !scales_gateup)
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (misaligned(W_gateup) || misaligned(W_gateup_fp8) || misaligned(scales_gateup))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  const Span in{W_gateup, sizeof(uint16_t) * kExperts * 2 * kFF * kHidden};
  const Span outs[] = {{W_gateup_fp8, kFp8GateupBytes}, {scales_gateup, kFp8GateupScaleBytes}};
  for (const Span& o : outs)
    if (overlap(o, in)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps the input");
  if (overlap(outs[0], outs[1])) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "codes overlap scales");
  const size_t half = static_cast<size_t>(kFF) * kHidden;
  hipError_t e = launch_pack_fp8_gateup(W_gateup, W_gateup + half, 2 * half, W_gateup_fp8, scales_gateup, stream);
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "fp8 pack kernel launch");
}

lfm_moe_status lfm_moe_pack_fp8_down(const uint16_t* W_down, uint8_t* W_down_fp8,
                                     float* scales_down, hipStream_t stream) {
  g_last_error.clear();
  if (!W_down || !W_down_fp8 || !scales_down)
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (misaligned(W_down) || misaligned(W_down_fp8) || misaligned(scales_down))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  const Span in{W_down, sizeof(uint16_t) * kExperts * kHidden * kFF};
  const Span outs[] = {{W_down_fp8, kFp8DownBytes}, {scales_down, kFp8DownScaleBytes}};
  for (const Span& o : outs)
    if (overlap(o, in)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps the input");
  if (overlap(outs[0], outs[1])) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "codes overlap scales");
  hipError_t e = launch_pack_fp8_down(W_down, W_down_fp8, scales_down, stream);
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "fp8 pack kernel launch");
}

lfm_moe_status lfm_moe_forward_fp8_ws(const uint16_t* X, const uint16_t* W_r, const float* bias,
                                      const uint8_t* W_gateup_fp8, const float* scales_gateup,
                                      const uint8_t* W_down_fp8, const float* scales_down, float* out,
                                      int64_t N, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_fp8_args(X, W_r, bias, W_gateup_fp8, scales_gateup, W_down_fp8,
                                     scales_down, out, N);
  if (st != LFM_MOE_OK || N == 0) return st;
  if ((st = check_ws(ws, ws_bytes, N, Span{out, act_bytes(N, 4)},
                     {{X, act_bytes(N, 2)}, router_span(W_r), bias_span(bias), {W_gateup_fp8, kFp8GateupBytes},
                      {scales_gateup, kFp8GateupScaleBytes}, {W_down_fp8, kFp8DownBytes},
                      {scales_down, kFp8DownScaleBytes}})) != LFM_MOE_OK)
    return st;
  return run_fp8(X, W_r, bias, nullptr, nullptr, W_gateup_fp8, scales_gateup, W_down_fp8, scales_down,
                 out, N, ws, stream);
}

lfm_moe_status lfm_moe_experts_fp8_ws(const uint16_t* X, const int32_t* idx, const float* w,
                                      const uint8_t* W_gateup_fp8, const float* scales_gateup,
                                      const uint8_t* W_down_fp8, const float* scales_down, float* out,
                                      int64_t N, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_fp8_args(X, nullptr, nullptr, W_gateup_fp8, scales_gateup, W_down_fp8,
                                     scales_down, out, N, false);
  if (st != LFM_MOE_OK || N == 0) return st;
  const Span o{out, act_bytes(N, 4)};
  if ((st = check_ws(ws, ws_bytes, N, o,
                     {{X, act_bytes(N, 2)}, {W_gateup_fp8, kFp8GateupBytes}, {scales_gateup, kFp8GateupScaleBytes},
                      {W_down_fp8, kFp8DownBytes}, {scales_down, kFp8DownScaleBytes}})) != LFM_MOE_OK)
    return st;
  if ((st = check_routing_args(idx, w, N, o, ws, ws_bytes)) != LFM_MOE_OK) return st;
  return run_fp8(X, nullptr, nullptr, idx, w, W_gateup_fp8, scales_gateup, W_down_fp8, scales_down,
                 out, N, ws, stream);
}

lfm_moe_status lfm_moe_forward_fp8(const uint16_t* X, const uint16_t* W_r, const float* bias,
                                   const uint8_t* W_gateup_fp8, const float* scales_gateup,
                                   const uint8_t* W_down_fp8, const float* scales_down, float* out,
                                   int64_t N, hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_fp8_args(X, W_r, bias, W_gateup_fp8, scales_gateup, W_down_fp8,
                                     scales_down, out, N);
  if (st != LFM_MOE_OK || N == 0) return st;
  void* ws = nullptr;
  size_t bytes = 0;
  if ((st = internal_ws(N, &ws, &bytes)) != LFM_MOE_OK) return st;
  return run_fp8(X, W_r, bias, nullptr, nullptr, W_gateup_fp8, scales_gateup, W_down_fp8, scales_down,
                 out, N, ws, stream);
}

}  // extern "C"

namespace {

// Checks of the router entry points' tensors.
lfm_moe_status check_route_args(const uint16_t* X, const uint16_t* W_r, const float* bias,
                                const int32_t* idx, const float* w, int64_t N) {
  if (N < 0 || N > LFM_MOE_MAX_TOKENS) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "N out of range");
  if (N == 0) return LFM_MOE_OK;
  if (!X || !W_r || !bias || !idx || !w) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if (misaligned(X) || misaligned(W_r) || misaligned(bias) || misaligned(idx) || misaligned(w))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  const size_t sel = static_cast<size_t>(N) * kTopK * 4;
  const Span outs[] = {{idx, sel}, {w, sel}};
  if (overlap(outs[0], outs[1])) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "idx overlaps w");
  const Span ins[] = {{X, act_bytes(N, 2)}, router_span(W_r), bias_span(bias)};
  for (const Span& o : outs)
    for (const Span& i : ins)
      if (overlap(o, i)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "output overlaps an input");
  return LFM_MOE_OK;
}

lfm_moe_status run_route(const uint16_t* X, const uint16_t* W_r, const float* bias, int32_t* idx,
                         float* w, int64_t N, void* ws, hipStream_t stream) {
  hipError_t e = launch_route(X, W_r, bias, idx, w, nullptr, static_cast<float*>(ws), static_cast<int>(N),
                              stream);
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "route kernel launch");
}

}  // namespace

extern "C" {

size_t lfm_moe_route_workspace_bytes(int64_t N) {
  if (N < 0 || N > LFM_MOE_MAX_TOKENS) return 0;
  return route_partial_bytes(N);
}

lfm_moe_status lfm_moe_route_ws(const uint16_t* X, const uint16_t* W_r, const float* bias,
                                int32_t* idx, float* w, int64_t N, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_route_args(X, W_r, bias, idx, w, N);
  if (st != LFM_MOE_OK || N == 0) return st;
  const size_t need = route_partial_bytes(N);
  if (need > 0) {
    if (!ws) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null workspace");
    if (misaligned(ws, kAlign)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
      return fail(LFM_MOE_ERR_WORKSPACE_TOO_SMALL,
                  "workspace of " + std::to_string(ws_bytes) + " bytes, need " + std::to_string(need));
    const Span wsp{ws, ws_bytes};
    const size_t sel = static_cast<size_t>(N) * kTopK * 4;
    const Span others[] = {{X, act_bytes(N, 2)}, router_span(W_r), bias_span(bias), {idx, sel}, {w, sel}};
    for (const Span& o : others)
      if (overlap(wsp, o)) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "workspace overlaps a tensor argument");
  }
  return run_route(X, W_r, bias, idx, w, N, ws, stream);
}

lfm_moe_status lfm_moe_route(const uint16_t* X, const uint16_t* W_r, const float* bias,
                             int32_t* idx, float* w, int64_t N, hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_route_args(X, W_r, bias, idx, w, N);
  if (st != LFM_MOE_OK || N == 0) return st;
  void* ws = nullptr;
  size_t bytes = 0;
  const size_t need = route_partial_bytes(N);
  if (need > 0 && (st = internal_ws(kRouteWs, need, &ws, &bytes)) != LFM_MOE_OK) return st;
  return run_route(X, W_r, bias, idx, w, N, ws, stream);
}

lfm_moe_status lfm_moe_forward_ws(const uint16_t* X, const uint16_t* W_r, const float* bias,
                                  const uint16_t* W_gateup, const uint16_t* W_down, float* out,
                                  int64_t N, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_layer_args(X, act_bytes(N, 2), W_r, bias, W_gateup, W_down, out,
                                       act_bytes(N, 4), N, false);
  if (st != LFM_MOE_OK || N == 0) return st;
  if ((st = check_ws(ws, ws_bytes, N, Span{out, act_bytes(N, 4)},
                     {{X, act_bytes(N, 2)}, router_span(W_r), bias_span(bias), gateup_span(W_gateup),
                      down_span(W_down)})) != LFM_MOE_OK)
    return st;
  StageTimer timer(stream);
  return run_layer(X, W_r, bias, nullptr, nullptr, W_gateup, W_down, nullptr, out, N, ws, stream, timer);
}

lfm_moe_status lfm_moe_forward(const uint16_t* X, const uint16_t* W_r, const float* bias,
                               const uint16_t* W_gateup, const uint16_t* W_down, float* out,
                               int64_t N, hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_layer_args(X, act_bytes(N, 2), W_r, bias, W_gateup, W_down, out,
                                       act_bytes(N, 4), N, false);
  if (st != LFM_MOE_OK || N == 0) return st;
  void* ws = nullptr;
  size_t bytes = 0;
  if ((st = internal_ws(N, &ws, &bytes)) != LFM_MOE_OK) return st;
  StageTimer timer(stream);
  return run_layer(X, W_r, bias, nullptr, nullptr, W_gateup, W_down, nullptr, out, N, ws, stream, timer);
}

lfm_moe_status lfm_moe_forward_noalloc(const uint16_t* X, const uint16_t* W_r, const float* bias,
                                       const uint16_t* W_gateup, const uint16_t* W_down, float* out,
                                       int64_t N, hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_layer_args(X, act_bytes(N, 2), W_r, bias, W_gateup, W_down, out,
                                       act_bytes(N, 4), N, false);
  if (st != LFM_MOE_OK || N == 0) return st;
  if (N > LFM_MOE_NOALLOC_MAX_TOKENS)
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT,
                "N = " + std::to_string(N) + " exceeds LFM_MOE_NOALLOC_MAX_TOKENS (" +
                    std::to_string(LFM_MOE_NOALLOC_MAX_TOKENS) + "); use lfm_moe_forward_ws");
  if (workspace_bytes(N) > sizeof(scratch))
    return fail(LFM_MOE_ERR_WORKSPACE_TOO_SMALL,
                "the static workspace holds " + std::to_string(sizeof(scratch)) + " bytes, N = " +
                    std::to_string(N) + " needs " + std::to_string(workspace_bytes(N)));
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != LFM_MOE_OK) return st;
  StageTimer timer(stream);
  return run_layer(X, W_r, bias, nullptr, nullptr, W_gateup, W_down, nullptr, out, N, ws, stream, timer);
}

lfm_moe_status lfm_moe_experts_ws(const uint16_t* X, const int32_t* idx, const float* w,
                                  const uint16_t* W_gateup, const uint16_t* W_down, float* out,
                                  int64_t N, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_layer_args(X, act_bytes(N, 2), nullptr, nullptr, W_gateup, W_down, out,
                                       act_bytes(N, 4), N, false, false);
  if (st != LFM_MOE_OK || N == 0) return st;
  const Span o{out, act_bytes(N, 4)};
  if ((st = check_ws(ws, ws_bytes, N, o, {{X, act_bytes(N, 2)}, gateup_span(W_gateup), down_span(W_down)})) !=
      LFM_MOE_OK)
    return st;
  if ((st = check_routing_args(idx, w, N, o, ws, ws_bytes)) != LFM_MOE_OK) return st;
  StageTimer timer(stream);
  return run_layer(X, nullptr, nullptr, idx, w, W_gateup, W_down, nullptr, out, N, ws, stream, timer);
}

lfm_moe_status lfm_moe_block_forward_ws(float* x_inout, const uint16_t* W_r, const float* bias,
                                        const uint16_t* W_gateup, const uint16_t* W_down,
                                        int64_t N, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_layer_args(x_inout, act_bytes(N, 4), W_r, bias, W_gateup, W_down,
                                       x_inout, act_bytes(N, 4), N, true);
  if (st != LFM_MOE_OK || N == 0) return st;
  if ((st = check_ws(ws, ws_bytes, N, Span{x_inout, act_bytes(N, 4)},
                     {router_span(W_r), bias_span(bias), gateup_span(W_gateup), down_span(W_down)})) != LFM_MOE_OK)
    return st;
  uint16_t* X = region<uint16_t>(ws, N, LFM_MOE_WS_X);
  StageTimer timer(stream);
  hipError_t e = launch_rmsnorm(x_inout, X, N, stream);
  if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel launch");
  timer.after(0);
  return run_layer(X, W_r, bias, nullptr, nullptr, W_gateup, W_down, x_inout, x_inout, N, ws, stream, timer);
}

// Stage entry points: the layer's own kernels one stage at a time on the
// regions of a caller workspace.
lfm_moe_status lfm_moe_stage_dispatch(const int32_t* idx, const float* w, int64_t N, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  g_last_error.clear();
  const size_t sel = static_cast<size_t>(N < 0 ? 0 : N) * kTopK * 4;
  lfm_moe_status st = check_stage(N, ws, ws_bytes, Span{nullptr, 0}, {{idx, sel}, {w, sel}});
  if (st != LFM_MOE_OK || N == 0) return st;
  const int n = static_cast<int>(N);
  int32_t* idx_ws = region<int32_t>(ws, N, LFM_MOE_WS_IDX);
  int32_t* blockcounts = region<int32_t>(ws, N, LFM_MOE_WS_BLOCKCOUNTS);
  hipError_t e = launch_ingest_routing(idx, w, idx_ws, region<float>(ws, N, LFM_MOE_WS_W), blockcounts, n, stream);
  if (e != hipSuccess) return hip_fail(e, "routing copy kernel launch");
  e = launch_dispatch(idx_ws, blockcounts, region<int32_t>(ws, N, LFM_MOE_WS_OFFSETS),
                      region<int32_t>(ws, N, LFM_MOE_WS_ROW2SLOT), n, stream);
  if (e != hipSuccess) return hip_fail(e, "dispatch kernel launch");
  return LFM_MOE_OK;
}

lfm_moe_status lfm_moe_stage_gateup(const uint16_t* X, const uint16_t* W_gateup, int64_t N, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_stage(N, ws, ws_bytes, Span{nullptr, 0}, {{X, act_bytes(N, 2)}, gateup_span(W_gateup)});
  if (st != LFM_MOE_OK || N == 0) return st;
  uint16_t* H = region<uint16_t>(ws, N, LFM_MOE_WS_H);
  const hipError_t e =
      use_decode_path(N)
          ? launch_gateup_decode(X, W_gateup, region<int32_t>(ws, N, LFM_MOE_WS_IDX), H, static_cast<int>(N), stream)
          : launch_gateup_tiled(X, W_gateup, region<int32_t>(ws, N, LFM_MOE_WS_IDX),
                                region<int32_t>(ws, N, LFM_MOE_WS_OFFSETS),
                                region<int32_t>(ws, N, LFM_MOE_WS_ROW2SLOT), H, N, stream);
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "gate/up kernel launch");
}

lfm_moe_status lfm_moe_stage_down(const uint16_t* W_down, int64_t N, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_stage(N, ws, ws_bytes, Span{nullptr, 0}, {down_span(W_down)});
  if (st != LFM_MOE_OK || N == 0) return st;
  const uint16_t* H = region<uint16_t>(ws, N, LFM_MOE_WS_H);
  float* Y = region<float>(ws, N, LFM_MOE_WS_Y);
  const hipError_t e =
      use_decode_path(N)
          ? launch_down_decode(H, W_down, region<int32_t>(ws, N, LFM_MOE_WS_IDX), Y, static_cast<int>(N), stream)
          : launch_down_tiled(H, W_down, region<int32_t>(ws, N, LFM_MOE_WS_OFFSETS),
                              region<int32_t>(ws, N, LFM_MOE_WS_ROW2SLOT), Y, N, stream);
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "down kernel launch");
}

lfm_moe_status lfm_moe_stage_combine(const float* resid, float* out, int64_t N, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  g_last_error.clear();
  const size_t ob = act_bytes(N, 4);
  lfm_moe_status st = resid != nullptr
                          ? check_stage(N, ws, ws_bytes, Span{out, ob}, {{resid, ob}})
                          : check_stage(N, ws, ws_bytes, Span{out, ob}, {});
  if (st != LFM_MOE_OK || N == 0) return st;
  if (resid != nullptr && resid != out && overlap(Span{resid, ob}, Span{out, ob}))
    return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "resid overlaps out without being it");
  const hipError_t e = launch_combine(region<float>(ws, N, LFM_MOE_WS_Y), region<float>(ws, N, LFM_MOE_WS_W),
                                      resid, out, N, stream);
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "combine kernel launch");
}

lfm_moe_status lfm_moe_stack_forward_ws(float* x_inout, const lfm_moe_block_weights* blocks, int n_blocks,
                                        int64_t N, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (n_blocks < 0) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "n_blocks must be >= 0");
  if (n_blocks > 0 && blocks == nullptr) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null block array");
  // Every block's arguments are checked before anything is launched.
  lfm_moe_status st = LFM_MOE_OK;
  for (int l = 0; l < n_blocks && st == LFM_MOE_OK; ++l) {
    const lfm_moe_block_weights& b = blocks[l];
    st = check_layer_args(x_inout, act_bytes(N, 4), b.W_r, b.bias, b.W_gateup, b.W_down, x_inout,
                          act_bytes(N, 4), N, true);
    if (st == LFM_MOE_OK && N > 0)
      st = check_ws(ws, ws_bytes, N, Span{x_inout, act_bytes(N, 4)},
                    {router_span(b.W_r), bias_span(b.bias), gateup_span(b.W_gateup), down_span(b.W_down)});
  }
  if (st != LFM_MOE_OK || N == 0 || n_blocks == 0) return st;
  uint16_t* X = region<uint16_t>(ws, N, LFM_MOE_WS_X);
  hipError_t e;
  for (int l = 0; l < n_blocks; ++l) {
    StageTimer timer(stream);
    if (l == 0) {
      if ((e = launch_rmsnorm(x_inout, X, N, stream)) != hipSuccess) return hip_fail(e, "rmsnorm kernel launch");
      timer.after(0);
    }
    const lfm_moe_block_weights& b = blocks[l];
    if ((st = run_layer(X, b.W_r, b.bias, nullptr, nullptr, b.W_gateup, b.W_down, x_inout, x_inout, N, ws,
                        stream, timer, l + 1 < n_blocks ? X : nullptr)) != LFM_MOE_OK)
      return st;
  }
  return LFM_MOE_OK;
}

lfm_moe_status lfm_moe_block_forward(float* x_inout, const uint16_t* W_r, const float* bias,
                                     const uint16_t* W_gateup, const uint16_t* W_down, int64_t N,
                                     hipStream_t stream) {
  g_last_error.clear();
  lfm_moe_status st = check_layer_args(x_inout, act_bytes(N, 4), W_r, bias, W_gateup, W_down,
                                       x_inout, act_bytes(N, 4), N, true);
  if (st != LFM_MOE_OK || N == 0) return st;
  void* ws = nullptr;
  size_t bytes = 0;
  if ((st = internal_ws(N, &ws, &bytes)) != LFM_MOE_OK) return st;
  return lfm_moe_block_forward_ws(x_inout, W_r, bias, W_gateup, W_down, N, ws, bytes, stream);
}

void lfm_moe_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  bool any = false;
  for (int k = 0; k < kWsKinds; ++k)
    for (int d = 0; d < kMaxDevices; ++d) any = any || g_ws[k][d] != nullptr;
  if (!any) return;  // nothing to free: no HIP call at all
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return;
  for (int k = 0; k < kWsKinds; ++k)
    for (int d = 0; d < kMaxDevices; ++d) {
      if (!g_ws[k][d]) continue;
      if (hipSetDevice(d) == hipSuccess) (void)hipFree(g_ws[k][d]);
      g_ws[k][d] = nullptr;
      g_ws_bytes[k][d] = 0;
    }
  (void)hipSetDevice(cur);
}

lfm_moe_status lfm_moe_timing_enable(int on) {
  g_last_error.clear();
  std::lock_guard<std::mutex> lock(g_timing.mu);
  hipError_t e = drain_pending();
  g_timing.on = on != 0;
  for (int i = 0; i < kStages; ++i) {
    g_timing.total_ms[i] = 0.0;
    g_timing.launches[i] = 0;
  }
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "timing events");
}

lfm_moe_status lfm_moe_timing_read(double* total_ms, int64_t* launches) {
  g_last_error.clear();
  if (!total_ms || !launches) return fail(LFM_MOE_ERR_INVALID_ARGUMENT, "null output pointer");
  std::lock_guard<std::mutex> lock(g_timing.mu);
  hipError_t e = drain_pending();
  for (int i = 0; i < kStages; ++i) {
    total_ms[i] = g_timing.total_ms[i];
    launches[i] = g_timing.launches[i];
  }
  return e == hipSuccess ? LFM_MOE_OK : hip_fail(e, "timing events");
}

}  // extern "C"

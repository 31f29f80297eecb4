/*
 * lfm_moe.h -- C ABI of the biased-sigmoid top-4 sparse feed-forward (MoE)
 * layer of LFM2.5-24B-A2B on AMD Instinct MI355X (gfx950).
 *
 * The operation is the one defined in the flozi.net guide "LFM2.5-24B-A2B:
 * Biased Routing, Short Convolutions and Ten KV Caches" (English edition),
 * section "The router has two different scores":
 *
 *   l_t   = W_r x_t                        64 router logits per token
 *   s_t   = sigmoid(l_t)                   applied to each logit on its own
 *   c_t   = s_t + bias                     stored bias, selection only
 *   S_t   = the 4 experts with largest c_t (ties: lower expert id first)
 *   w_tj  = s_t[S_tj] / (sum_j' s_t[S_tj'] + 1e-6) * 1.0   (routed scale 1)
 *   y_e(x)= W_down_e (silu(W_gate_e x) * (W_up_e x))       2048->1536->2048
 *   out_t = sum_j w_tj y_{S_tj}(x_t)       tokens grouped by expert, weighted
 *                                          outputs accumulated (section
 *                                          "What to verify in a deployment")
 *
 * Fixed shapes: d = 2048, E = 64 experts, top-k = 4, ff = 1536.
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers to contiguous row-major arrays,
 *    16-byte aligned.  bf16 arguments are raw bfloat16 bit patterns
 *    (uint16_t).  Weights are stored [out_features, in_features].
 *  - Ownership: the caller owns every tensor argument; the library never
 *    frees or keeps them.  Work is enqueued asynchronously on `stream`, so
 *    the caller keeps them alive until the stream has passed this call.
 *  - Synchrony: no host synchronisation and no device-to-host copy happens
 *    inside a call.  LFM_MOE_OK means "enqueued"; a fault inside a kernel
 *    surfaces at the caller's next synchronisation.
 *  - Errors: return codes only, nothing aborts.  Argument checks run before
 *    any HIP call.  N == 0 returns LFM_MOE_OK and launches nothing.
 *    lfm_moe_last_error() gives a thread-local message for the last failure.
 *  - Determinism: bitwise reproducible for fixed inputs, N and build (no
 *    floating-point atomics; fixed reduction and combine orders).
 */
#ifndef LFM_MOE_H
#define LFM_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LFM_MOE_ABI_VERSION 7
#define LFM_MOE_HIDDEN 2048
#define LFM_MOE_EXPERTS 64
#define LFM_MOE_TOPK 4
#define LFM_MOE_FF 1536
/* Largest N accepted: grouped rows (4N) and their element offsets stay in range. */
#define LFM_MOE_MAX_TOKENS (1LL << 24)
/* Largest N of lfm_moe_forward_fp8, and the largest N it runs on the
 * weight-streaming kernels (the smallest batches; larger ones take the
 * grouped kernels in FP8 mode).  lfm_moe_forward takes the same split. */
#define LFM_MOE_FP8_MAX_TOKENS LFM_MOE_MAX_TOKENS
#define LFM_MOE_FP8_STREAM_TOKENS 4

typedef enum {
  LFM_MOE_OK = 0,
  LFM_MOE_ERR_INVALID_ARGUMENT = 1, /* NULL with N > 0, N < 0, N too large, misaligned */
  LFM_MOE_ERR_WORKSPACE_TOO_SMALL = 2,
  LFM_MOE_ERR_OUT_OF_MEMORY = 3,    /* the internal workspace could not grow */
  LFM_MOE_ERR_HIP = 4               /* a HIP runtime or launch error */
} lfm_moe_status;

/* Returns LFM_MOE_ABI_VERSION of the built library. */
int lfm_moe_abi_version(void);

/* Message of the last failed call on this thread ("" if none).  Valid until
 * the next call on the same thread. */
const char* lfm_moe_last_error(void);

/*
 * RMS normalisation of the residual stream, the step before the
 * feed-forward network (guide, section "The exact checkpoint"):
 *   X[t, :] = bf16( x[t, :] / sqrt(mean(x[t, :]^2) + 1e-6) )   (unit weight)
 * x: [N, 2048] fp32 (read).  X: [N, 2048] bf16 (written).  Sums in fp32,
 * in a fixed order; rounding to bf16 is round-to-nearest-even.
 */
lfm_moe_status lfm_moe_rmsnorm(const float* x, uint16_t* X, int64_t N, hipStream_t stream);

/*
 * Router (guide, section "The router has two different scores"): logits
 * X W_r^T in fp32 (bf16 inputs, fp32 accumulation), sigmoid per logit in
 * fp32, biased top-4 selection, unbiased weights normalised by sum + 1e-6.
 *   X:    [N, 2048] bf16, the normalised hidden states (read)
 *   W_r:  [64, 2048] bf16 router matrix (read)
 *   bias: [64] fp32 stored expert bias (read; used for selection only)
 *   idx:  [N, 4] int32 (written): selected experts by descending selection
 *         score s + bias, equal scores ordered by lower expert id
 *   w:    [N, 4] fp32 (written): w[t, j] = s[idx[t, j]] / (sum_j s + 1e-6)
 * The logits are summed from 16 partial products over 128-wide K slices,
 * in a fixed order.  Up to 2048 tokens the partials pass through a
 * workspace of lfm_moe_route_workspace_bytes(N) bytes (none above): the
 * library-owned one of the current device (grown on demand, kept until
 * lfm_moe_release(); separate from the layer's), so calls to lfm_moe_route
 * that overlap in time on one device race on it -- use lfm_moe_route_ws
 * with distinct workspaces for those.
 */
lfm_moe_status lfm_moe_route(const uint16_t* X, const uint16_t* W_r, const float* bias,
                             int32_t* idx, float* w, int64_t N, hipStream_t stream);

/* Bytes of workspace lfm_moe_route_ws needs for N tokens (0 above 2048 tokens). */
size_t lfm_moe_route_workspace_bytes(int64_t N);

/*
 * lfm_moe_route with a caller-owned workspace `ws` of `ws_bytes` bytes
 * (device memory, 256-byte aligned, at least lfm_moe_route_workspace_bytes(N),
 * overlapping no tensor argument; may be NULL when that size is 0).  The
 * same selections and weights as lfm_moe_route, bit for bit.  Concurrent
 * calls need distinct workspaces.
 */
lfm_moe_status lfm_moe_route_ws(const uint16_t* X, const uint16_t* W_r, const float* bias,
                                int32_t* idx, float* w, int64_t N, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * Expert weight packing (guide, section "The router has two different
 * scores": the runtime representation may pack the two input matrices of
 * an expert together; packing does not change the function).
 *
 * The packed layout is made of 1 KB fragments of 32 rows x 16 columns;
 * bytes [16 l, 16 l + 16) of a fragment hold row (l % 32), columns
 * 8 (l / 32) .. 8 (l / 32) + 7 -- the order in which the 64 lanes of a
 * wavefront hold a 32x32x16 MFMA operand.  Fragments are ordered (expert,
 * 32-row block, 16-column step), the steps of one block contiguous.
 *
 * lfm_moe_pack_gateup: W_gate, W_up [64, 1536, 2048] bf16 row-major (read)
 *   -> W_gateup [64 * 3072 * 2048] bf16 (written): fragment
 *   (e * 96 + b) * 128 + ks holds, of expert e and columns ks*16 .. +15,
 *   rows 16 b .. 16 b + 15 of W_gate as its rows 0..15 and the same rows
 *   of W_up as its rows 16..31 (b < 96, ks < 128).
 * lfm_moe_pack_down: W_down [64, 2048, 1536] bf16 row-major (read)
 *   -> W_down_packed [64 * 2048 * 1536] bf16 (written): fragment
 *   (e * 64 + b) * 96 + ks holds rows 32 b .. 32 b + 31 of W_down of
 *   expert e, columns ks*16 .. ks*16+15 (b < 64, ks < 96).
 * lfm_moe_pack_gateup_stacked: the same packed output from one
 *   W_gateup [64, 3072, 2048] bf16 tensor (read) whose rows 0..1535 of
 *   expert e are W_gate[e] and rows 1536..3071 are W_up[e] -- the stacked
 *   gate/up layout of the layer's definition; bit-identical to
 *   lfm_moe_pack_gateup on the two halves.
 * Outputs must not overlap the inputs.  A pure permutation: bit exact.
 */
lfm_moe_status lfm_moe_pack_gateup(const uint16_t* W_gate, const uint16_t* W_up,
                                   uint16_t* W_gateup, hipStream_t stream);
lfm_moe_status lfm_moe_pack_gateup_stacked(const uint16_t* W_gateup, uint16_t* W_gateup_packed,
                                           hipStream_t stream);
lfm_moe_status lfm_moe_pack_down(const uint16_t* W_down, uint16_t* W_down_packed,
                                 hipStream_t stream);

/*
 * The whole layer: out[N, 2048] fp32 = sum_j w[t, j] * y_{idx[t, j]}(X[t]).
 *   X:        [N, 2048] bf16 normalised hidden states (read)
 *   W_r:      [64, 2048] bf16, bias: [64] fp32 (read), as for lfm_moe_route
 *   W_gateup: packed gate/up weights of all 64 experts, as written by
 *             lfm_moe_pack_gateup or lfm_moe_pack_gateup_stacked (read).
 *             The layer takes its expert weights only in this packed form:
 *             a [64, 3072, 2048] stacked gate/up tensor (or separate
 *             [64, 1536, 2048] gate and up tensors) is packed once, and
 *             packing changes no value.
 *   W_down:   packed down weights, as written by lfm_moe_pack_down from the
 *             [64, 2048, 1536] tensor (read)
 *   out:      [N, 2048] fp32 (written; must not overlap any input)
 * Expert hidden activations are rounded to bf16 before the down
 * projection; every accumulation is fp32.  Uses a workspace that the
 * library owns (one per device, grown on demand with hipMalloc and kept
 * until lfm_moe_release()); calls that overlap in time on one device must
 * use lfm_moe_forward_ws with separate workspaces instead.
 */
lfm_moe_status lfm_moe_forward(const uint16_t* X, const uint16_t* W_r, const float* bias,
                               const uint16_t* W_gateup, const uint16_t* W_down,
                               float* out, int64_t N, hipStream_t stream);

/* Bytes of workspace lfm_moe_forward_ws / lfm_moe_block_forward_ws need for N tokens. */
size_t lfm_moe_workspace_bytes(int64_t N);

/* Regions of the workspace, for inspection of the intermediate steps. */
typedef enum {
  LFM_MOE_WS_IDX = 0,       /* [N, 4] int32 selected experts */
  LFM_MOE_WS_W = 1,         /* [N, 4] fp32 mixture weights */
  LFM_MOE_WS_BLOCKCOUNTS = 2, /* [ceil(N / 16), 64] int32 per-16-token histogram (dispatch step) */
  LFM_MOE_WS_OFFSETS = 3,   /* [65] int32: offsets[e] = first grouped row of expert e, offsets[64] = 4N */
  LFM_MOE_WS_ROW2SLOT = 4,  /* [4N] int32 grouped row -> slot t*4 + j (stable: token order inside an expert) */
  LFM_MOE_WS_H = 5,         /* [4N, 1536] bf16 expert hidden rows, slot order (row t*4 + j) */
  LFM_MOE_WS_Y = 6,         /* [4N, 2048] fp32 expert output rows, slot order (row t*4 + j) */
  LFM_MOE_WS_X = 7,         /* [N, 2048] bf16 normalised input (block forward only) */
  LFM_MOE_WS_ROUTER_PARTIAL = 8, /* [ceil(N/16), 16, 16, 64] fp32 router partial logits per K slice;
                                    empty above 2048 tokens, where the router keeps them in LDS */
  LFM_MOE_WS_XQ = 9,        /* [N, 2048] uint8: X's E4M3 codes per 128-wide group (FP8 layer above
                               LFM_MOE_FP8_STREAM_TOKENS only); in each 32-wide piece of a row the
                               8-code runs are stored in the order 0, 2, 1, 3 */
  LFM_MOE_WS_XS = 10,       /* [N, 16] fp32: their scales */
  LFM_MOE_WS_HQ = 11,       /* [4N, 1536] uint8: H's E4M3 codes, slot order (same layout and condition) */
  LFM_MOE_WS_HS = 12,       /* [4N, 12] fp32: their scales */
  LFM_MOE_WS_REGIONS = 13
} lfm_moe_ws_region;

/* Byte offset of `region` inside a workspace sized for N tokens; (size_t)-1 if invalid. */
size_t lfm_moe_workspace_offset(int64_t N, int region);

/*
 * lfm_moe_forward with a caller-owned workspace `ws` of `ws_bytes` bytes
 * (device memory, 256-byte aligned, at least lfm_moe_workspace_bytes(N),
 * overlapping neither the output nor any input tensor: every _ws entry
 * point returns LFM_MOE_ERR_INVALID_ARGUMENT otherwise).
 * The workspace holds the intermediate results listed in lfm_moe_ws_region
 * after the call completes.  Batches of up to 4 tokens take the
 * weight-streaming kernels, which group their own tokens and leave
 * BLOCKCOUNTS, OFFSETS and ROW2SLOT unwritten; batches of 5 to 512 tokens
 * are grouped by the gate/up kernel, which writes OFFSETS and ROW2SLOT
 * (BLOCKCOUNTS stays unwritten); larger batches write all three.  (The FP8
 * layer groups 5 to 256 tokens in its gate/up kernel.)
 * Concurrent calls need distinct workspaces.
 */
lfm_moe_status lfm_moe_forward_ws(const uint16_t* X, const uint16_t* W_r, const float* bias,
                                  const uint16_t* W_gateup, const uint16_t* W_down,
                                  float* out, int64_t N, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * The expert path alone, on routing the caller supplies (steps after the
 * router: grouping by expert, the gated SiLU experts and the weighted
 * combine of the guide's sections "The router has two different scores"
 * and "What to verify in a deployment"):
 *   out[t] = sum_j w[t, j] * y_{idx[t, j]}(X[t]),  j = 0..3 in that order.
 *   X:   [N, 2048] bf16 (read)
 *   idx: [N, 4] int32 expert ids, w: [N, 4] fp32 mixture weights (read once,
 *        copied into the IDX and W workspace regions; they may overlap each
 *        other but neither out nor the workspace)
 *   W_gateup, W_down, out, ws, ws_bytes, stream: as for lfm_moe_forward_ws.
 * Ids are taken modulo 64, and an id that repeats an earlier id of the
 * same token is replaced by the lowest id that is neither among the
 * token's earlier ids (as replaced) nor among its later given ones; the
 * IDX region shows the ids used.  Valid routing (four distinct ids in
 * [0, 64) per token) is used as given, and then the result equals that of
 * lfm_moe_forward_ws for a router that selected idx and w, bit for bit.
 * For tests that hold the routing fixed (the oracle's) and for callers that
 * route elsewhere.  0 <= N <= LFM_MOE_MAX_TOKENS; N == 0 is a no-op.
 */
lfm_moe_status lfm_moe_experts_ws(const uint16_t* X, const int32_t* idx, const float* w,
                                  const uint16_t* W_gateup, const uint16_t* W_down,
                                  float* out, int64_t N, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * Stage entry points (for tests that check one stage at a time): the
 * layer's own kernels for one stage, on the regions of a caller workspace
 * of at least lfm_moe_workspace_bytes(N) bytes (guide, section "What to
 * verify in a deployment": route, group the tokens by expert, run each
 * expert on its group, combine the weighted outputs; section "The router
 * has two different scores" for what the router hands over).  Called in
 * the order dispatch, gate/up, down, combine on one workspace, they give
 * lfm_moe_experts_ws's result bit for bit (the same kernels on the same
 * regions).  Between calls a test may overwrite the H region (bf16
 * [4N, 1536], slot order) or the Y region (fp32 [4N, 2048], slot order)
 * with values of its own, to check the next stage alone; the IDX, W,
 * OFFSETS and ROW2SLOT regions must hold what lfm_moe_stage_dispatch (or a
 * layer call with the same N) stored there (for 5 to 256 tokens the gate/up
 * stage recomputes OFFSETS and ROW2SLOT from IDX, with the same result).
 * Asynchronous on stream; arguments checked before any HIP call; N == 0 is
 * a no-op; 0 <= N <= LFM_MOE_MAX_TOKENS.
 *
 * lfm_moe_stage_dispatch: idx [N, 4] int32, w [N, 4] fp32 (read; replaced
 *   by the rule of lfm_moe_experts_ws where invalid) -> IDX and W regions
 *   (the routing used), BLOCKCOUNTS, OFFSETS [65] (expert e's grouped rows
 *   are OFFSETS[e] .. OFFSETS[e+1]-1) and ROW2SLOT [4N] (grouped row ->
 *   slot t*4 + j; within an expert, slots in token order).
 * lfm_moe_stage_gateup: X [N, 2048] bf16, W_gateup (pack output) -> H
 *   region: H[t*4 + j] = bf16(silu(X_t Wg_e^T) * (X_t Wu_e^T)), e = IDX[t, j].
 * lfm_moe_stage_down: W_down (pack output), H region -> Y region:
 *   Y[t*4 + j] = H[t*4 + j] Wd_e^T (fp32).
 * lfm_moe_stage_combine: Y and W regions -> out [N, 2048] fp32:
 *   out[t] = (resid[t] +) sum_j W[t, j] Y[t*4 + j] in the order j = 0..3.
 *   resid may be NULL, or equal to out (in place); it may not otherwise
 *   overlap out.
 * Tensors may not overlap the workspace.
 */
lfm_moe_status lfm_moe_stage_dispatch(const int32_t* idx, const float* w, int64_t N, void* ws, size_t ws_bytes,
                                      hipStream_t stream);
lfm_moe_status lfm_moe_stage_gateup(const uint16_t* X, const uint16_t* W_gateup, int64_t N, void* ws,
                                    size_t ws_bytes, hipStream_t stream);
lfm_moe_status lfm_moe_stage_down(const uint16_t* W_down, int64_t N, void* ws, size_t ws_bytes,
                                  hipStream_t stream);
lfm_moe_status lfm_moe_stage_combine(const float* resid, float* out, int64_t N, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/*
 * One block's feed-forward half (guide, section "The exact checkpoint":
 * normalise, feed-forward network, residual):
 *   x_inout[t] <- x_inout[t] + MoE(bf16(RMSNorm(x_inout[t])))
 * x_inout: [N, 2048] fp32 residual stream (read and written in place);
 * other arguments as for lfm_moe_forward.  The _ws form takes a caller
 * workspace of lfm_moe_workspace_bytes(N) bytes.
 */
lfm_moe_status lfm_moe_block_forward(float* x_inout, const uint16_t* W_r, const float* bias,
                                     const uint16_t* W_gateup, const uint16_t* W_down,
                                     int64_t N, hipStream_t stream);
lfm_moe_status lfm_moe_block_forward_ws(float* x_inout, const uint16_t* W_r, const float* bias,
                                        const uint16_t* W_gateup, const uint16_t* W_down,
                                        int64_t N, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * A stack of MoE blocks (guide, section "The exact checkpoint": every block
 * normalises, applies its feed-forward network and adds the residual):
 *   for l = 0 .. n_blocks - 1:
 *     x_inout[t] <- x_inout[t] + MoE_l(bf16(RMSNorm(x_inout[t])))
 * blocks: host array of n_blocks entries, block l's device weights (each as
 * for lfm_moe_block_forward; blocks may share weights); read during the
 * call only.  x_inout, N, ws, ws_bytes, stream as for
 * lfm_moe_block_forward_ws.  The result equals n_blocks calls of
 * lfm_moe_block_forward_ws bit for bit, with one launch fewer per block
 * after the first: the combine of block l stores block l + 1's normalised
 * input itself.  Every block's arguments are checked before anything is
 * launched.  n_blocks == 0 or N == 0 is a no-op.
 */
typedef struct lfm_moe_block_weights {
  const uint16_t* W_r;       /* [64, 2048] bf16 */
  const float* bias;         /* [64] fp32 */
  const uint16_t* W_gateup;  /* lfm_moe_pack_gateup / _stacked output */
  const uint16_t* W_down;    /* lfm_moe_pack_down output */
} lfm_moe_block_weights;

lfm_moe_status lfm_moe_stack_forward_ws(float* x_inout, const lfm_moe_block_weights* blocks, int n_blocks,
                                        int64_t N, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * FP8 experts (inferencekey.com page on the 24B reasoning MoE, German
 * edition, "Für Engineers" part, the quantisation entry: the FP8 checkpoint
 * is compressed-tensors FP8_BLOCK -- weights FP8 (E4M3) statically in
 * 128 x 128 blocks, activations FP8 dynamically per group of 128, router
 * not quantised).
 *
 * Quantisation of a block or group with largest magnitude amax > 0: codes
 * E4M3(x * (448 / amax)) (OCP E4M3FN; fp32 arithmetic; round to nearest
 * even; a value rounding to zero keeps its sign), dequantisation scale
 * amax / 448 (fp32); amax = 0 gives zero codes and scale 0.
 *
 * lfm_moe_pack_fp8_gateup: W_gate, W_up [64, 1536, 2048] bf16 (read) ->
 *   W_gateup_fp8 [64 * 3072 * 2048] bytes and scales_gateup
 *   [64][2][12][16] fp32 (written): scale (e, m, rb, kb) of the 128 x 128
 *   block rows 128 rb.., columns 128 kb.. of W_gate (m = 0) or W_up (m = 1).
 *   Codes in 1 KB fragments of 32 rows x 32 columns: bytes [16 l, 16 l + 16)
 *   of a fragment are row l % 32, bytes 0..7 its columns 8 h .. 8 h + 7 and
 *   bytes 8..15 columns 16 + 8 h .. 16 + 8 h + 7 (h = l / 32); fragment
 *   (e * 96 + b) * 64 + kp holds rows 16 b .. 16 b + 15 of W_gate as its
 *   rows 0..15 and the same rows of W_up as its rows 16..31, columns
 *   32 kp .. 32 kp + 31.
 * lfm_moe_pack_fp8_gateup_stacked: the same codes and scales from one
 *   stacked W_gateup [64, 3072, 2048] bf16 tensor (rows 0..1535 gate,
 *   1536..3071 up of each expert).
 * lfm_moe_pack_fp8_down: W_down [64, 2048, 1536] bf16 (read) ->
 *   W_down_fp8 [64 * 2048 * 1536] bytes, scales_down [64][16][12] fp32
 *   (written); fragment (e * 64 + b) * 48 + kp holds rows 32 b .. 32 b + 31,
 *   columns 32 kp .. 32 kp + 31, in the same lane order.
 * lfm_moe_forward_fp8: the layer with these experts, 0 <= N <=
 *   LFM_MOE_FP8_MAX_TOKENS.  Router and mixture weights as in
 *   lfm_moe_forward; each expert's input rows (X, then the bf16 hidden rows)
 *   are quantised per group of 128 features as above; the products of
 *   codes are summed per 128-wide K group, then scaled by weight scale x
 *   activation scale; out [N, 2048] fp32.  Up to LFM_MOE_FP8_STREAM_TOKENS
 *   tokens the expert kernels stream the weights and quantise the rows in
 *   registers (exact products, fp32 sums); above, the rows are grouped by
 *   expert (by the gate/up kernel up to 256 tokens, by the dispatch step
 *   beyond), X and H are quantised into the XQ/XS and HQ/HS workspace
 *   regions and the grouped kernels multiply on the FP8 matrix core, whose
 *   sums are not fp32 sums: it aligns each step's 64 products and drops the
 *   bits below the alignment (measured: within 2^-11.6 of the sum of their
 *   magnitudes).  Library-owned workspace, as lfm_moe_forward.
 * lfm_moe_forward_fp8_ws: the same with a caller workspace, as
 *   lfm_moe_forward_ws (same size and regions: the routing, the bf16 hidden
 *   rows H and the fp32 expert rows Y, both in slot order t * 4 + j; up to
 *   LFM_MOE_FP8_STREAM_TOKENS tokens the regions of the grouped path are not
 *   written).
 * lfm_moe_experts_fp8_ws: the FP8 expert path on caller-given routing
 *   idx [N, 4] int32 and w [N, 4] fp32, with the same rules as
 *   lfm_moe_experts_ws; on valid routing bit-identical to
 *   lfm_moe_forward_fp8_ws for a router that selected idx and w.
 * Pointers 16-byte aligned; outputs must not overlap inputs; asynchronous on
 * `stream`.
 */
lfm_moe_status lfm_moe_pack_fp8_gateup(const uint16_t* W_gate, const uint16_t* W_up,
                                       uint8_t* W_gateup_fp8, float* scales_gateup,
                                       hipStream_t stream);
lfm_moe_status lfm_moe_pack_fp8_gateup_stacked(const uint16_t* W_gateup, uint8_t* W_gateup_fp8,
                                               float* scales_gateup, hipStream_t stream);
lfm_moe_status lfm_moe_pack_fp8_down(const uint16_t* W_down, uint8_t* W_down_fp8,
                                     float* scales_down, hipStream_t stream);
lfm_moe_status lfm_moe_forward_fp8(const uint16_t* X, const uint16_t* W_r, const float* bias,
                                   const uint8_t* W_gateup_fp8, const float* scales_gateup,
                                   const uint8_t* W_down_fp8, const float* scales_down, float* out,
                                   int64_t N, hipStream_t stream);
lfm_moe_status lfm_moe_forward_fp8_ws(const uint16_t* X, const uint16_t* W_r, const float* bias,
                                      const uint8_t* W_gateup_fp8, const float* scales_gateup,
                                      const uint8_t* W_down_fp8, const float* scales_down, float* out,
                                      int64_t N, void* ws, size_t ws_bytes, hipStream_t stream);
lfm_moe_status lfm_moe_experts_fp8_ws(const uint16_t* X, const int32_t* idx, const float* w,
                                      const uint8_t* W_gateup_fp8, const float* scales_gateup,
                                      const uint8_t* W_down_fp8, const float* scales_down, float* out,
                                      int64_t N, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * lfm_moe_forward that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  Same arguments, kernels and result (bit
 * for bit) as lfm_moe_forward, for 0 <= N <= LFM_MOE_NOALLOC_MAX_TOKENS; a
 * larger N returns LFM_MOE_ERR_INVALID_ARGUMENT before any HIP call.  Its
 * workspace is a static device array of LFM_MOE_NOALLOC_SCRATCH_BYTES bytes
 * that every GPU the library runs on holds until the process ends; no call
 * makes hipMalloc, hipFree or any other allocation (the array's device
 * address is looked up once per device, at the first call on it).  Every
 * call on one GPU uses that GPU's one array and leaves the last call's
 * intermediates in it, so calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and give wrong
 * results: serialise them, or use lfm_moe_forward_ws.
 */
#define LFM_MOE_NOALLOC_MAX_TOKENS 256
#define LFM_MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
lfm_moe_status lfm_moe_forward_noalloc(const uint16_t* X, const uint16_t* W_r, const float* bias,
                                       const uint16_t* W_gateup, const uint16_t* W_down,
                                       float* out, int64_t N, hipStream_t stream);

/* Frees the library-owned workspaces, the layer's and the router's (call with no work of
 * this library in flight). */
void lfm_moe_release(void);

/*
 * Measurement support: device time per kernel of the layer.  While timing
 * is on, every layer call records a hipEvent on its stream before its first
 * kernel and after each kernel; lfm_moe_timing_read() waits for those
 * events and returns, per stage, the summed milliseconds between
 * consecutive events and the number of launches.  Stages: 0 rmsnorm,
 * 1 route, 2 dispatch, 3 gate/up, 4 down, 5 combine.  Turning timing on
 * clears the totals.  The events cost a little host time per call; leave
 * timing off outside measurements.  Not meant for concurrent use from
 * several threads.
 */
#define LFM_MOE_STAGES 6
lfm_moe_status lfm_moe_timing_enable(int on);
lfm_moe_status lfm_moe_timing_read(double* total_ms /* [LFM_MOE_STAGES] */,
                                   int64_t* launches /* [LFM_MOE_STAGES] */);

#ifdef __cplusplus
}
#endif

#endif /* LFM_MOE_H */

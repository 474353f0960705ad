/*
 * prox.h - C ABI of the Prox two-stage sparse SwiGLU FFN decode library
 * (MI355X / gfx950, HIP).
 *
 * The method (sources cited by page and section):
 *   [blog]  "Prox 完全拆解：先用便宜代理找通道，再用精确计算守住 SwiGLU 的质量"
 *           (deep-dive blog post on Prox)
 *   [paper] "Prox: 通过近似中间通道显著性实现 LLM 中免训练的 FFN 激活稀疏化"
 *           (Chinese rendering of arXiv 2607.27591)
 *
 *   Stage 1 ([blog] "Stage 1"): keep the input coordinates with
 *     |x_i| >= tau_x, run an INT4 proxy of W_up and W_gate over those rows
 *     only, form the proxy state s~ = u~ * SiLU(g~) and keep the intermediate
 *     channels with |s~_j| >= tau_s (one mask shared by all three projections).
 *   Stage 2 ([blog] "Stage 2"): with the dense x and the original weights,
 *     compute u_j, g_j for the kept channels only, s_j = u_j * SiLU(g_j), and
 *     y = sum over kept j of s_j * W_down[j, :].
 *   Pi^in / Pi^out and I(m) are as defined in [paper] section 2.2.
 *
 * Conventions for every entry point
 *   - Pointers marked "device" are HIP device memory; "host" are host memory.
 *     The caller owns every buffer; the library never allocates or frees
 *     device memory on the decode path and keeps no pointer after returning.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it unless a function says it blocks.
 *   - Arguments are validated before anything is enqueued.  On a validation
 *     failure nothing is enqueued and PROX_ERR_INVALID_ARG or
 *     PROX_ERR_UNSUPPORTED is returned.  A failed kernel launch returns
 *     PROX_ERR_HIP.  The message of the last failure on the calling thread is
 *     available from prox_last_error().  No C++ exception crosses the ABI and
 *     the library never aborts the process.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Shapes: d_model % 64 == 0, d_ff % 128 == 0, 64 <= d_model <= 12288,
 *     128 <= d_ff <= 65536 (bounds that keep every block within 64 KB of LDS).  Device pointers to weights, x and y must be
 *     16-byte aligned; workspaces 256-byte aligned.
 *   - Weight dtype: PROX_F32 or PROX_BF16 (bf16 bit patterns, RNE).  x uses
 *     the weight dtype; y and all accumulation are fp32.
 *   - Thresholds: tau >= 0 or +inf; NaN or negative values are rejected.
 *     tau = 0 keeps everything; +inf keeps nothing.
 *   - Concurrent calls must use distinct workspaces.
 */
#ifndef PROX_H
#define PROX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PROX_ABI_VERSION 4

typedef enum {
  PROX_OK = 0,
  PROX_ERR_INVALID_ARG = -1,
  PROX_ERR_UNSUPPORTED = -2,
  PROX_ERR_HIP = -3,
  PROX_ERR_INTERNAL = -4
} prox_status;

typedef enum { PROX_F32 = 0, PROX_BF16 = 1 } prox_dtype;

/*
 * One packed FFN layer.  A plain descriptor of caller-owned device buffers;
 * sizes come from prox_layer_sizes().
 *
 * proxy_q     [d_model][qstride] bytes, qstride = d_ff when d_ff/128 is odd,
 *             else d_ff + 128 (the last 128 bytes of a row are zero padding;
 *             an odd multiple of 128 spreads one column slice of many rows
 *             over the HBM channels).  Row i holds the INT4 proxy codes of
 *             input coordinate i for both W_up and W_gate, so a kept input
 *             coordinate selects one contiguous d_ff-byte run.  Within a row,
 *             each group of 16 output columns c0..c0+15 takes 16 bytes:
 *             8 bytes of up codes, then 8 bytes of gate codes.  In each 8-byte
 *             half, byte b holds column c0+2b in its low nibble and column
 *             c0+2b+1 in its high nibble.  A nibble stores code + 8 (offset
 *             binary), codes are in [-7, 7]; nibble value 0 is never written.
 * proxy_scale [2][d_model] fp32: per-row scales of the up (0) and gate (1)
 *             proxies.  Proxy weight = scale[row] * code.
 * w_upgate_t  [d_ff][2][d_model] in wdtype: for channel j, W_up[:, j] then
 *             W_gate[:, j], each a contiguous d_model-long run.
 * w_down      [d_ff][d_model] in wdtype, row-major (row j = W_down[j, :]).
 * activation  the gate non-linearity of the FFN, used in the proxy state and
 *             in Stage 2 alike: PROX_ACT_SILU (SwiGLU, SiLU(z) = z/(1+e^-z)) or
 *             PROX_ACT_GELU_TANH (GeGLU, Gemma-3 style: GELU in its tanh form
 *             0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))).  The pages
 *             evaluate the method on SwiGLU models and on GeGLU-style Gemma-3
 *             ([blog] evidence section).
 * proxy_kind  which proxy Stage 1 reads: PROX_PROXY_INT4 (proxy_q and
 *             proxy_scale, the method's proxy) or PROX_PROXY_W16, the 16-bit
 *             proxy of the pages' precision ablation ([blog] evidence section,
 *             ablation A1: a 16-bit proxy in place of INT4 at the same budget),
 *             here the layer's own bf16 weights (bf16 layers only).  Stage 2
 *             is the same for both.  A grouped batch (batch >= 2) runs the
 *             grouped kernels for INT4 and the per-token kernels for W16.
 * reserved    must be 0.
 * proxy_w16   PROX_PROXY_W16 only (may be NULL otherwise): [d_model][wstride]
 *             bytes, wstride = 4 d_ff rounded to an odd multiple of 128 (zero
 *             padding).  Row i holds W_up[i, :] and W_gate[i, :] as bf16 in the
 *             column groups of proxy_q: each group of 16 output columns takes
 *             64 bytes, the 16 up values then the 16 gate values.
 * With PROX_PROXY_W16, proxy_q and proxy_scale may be NULL.
 * proxy_qt    optional (NULL = absent): a channel-major copy of proxy_q for
 *             groups of tokens (prox_pack_proxy_qt; PROX_PROXY_INT4 only).
 *             When present, Stage 1 of every group that runs the grouped
 *             kernels (3..8 tokens, or 2 when they are forced) of a decode,
 *             and of every group of 3..8 tokens of prox_proxy_state, reads it
 *             instead of the union of the tokens' proxy rows: every proxy row
 *             once, as contiguous 1 KB runs, with no partial sums between
 *             blocks.  A group whose x (d_model values per token) and proxy
 *             scales (8 bytes per input row) do not fit in one CU's LDS
 *             beside the kernel's operand buffers (16 to 64 KB) runs the
 *             union-of-rows Stage 1 instead.
 *             Results are those of the method either way; the two Stage-1
 *             kernels round the proxy state differently (well within the
 *             decode's documented tolerance).  Layout, for 16-channel group g
 *             (channels 16g .. 16g+15, g < d_ff / 16) and 128-row chunk k of
 *             the inputs (rows 128k .. 128k+127; rows past d_model hold code
 *             0): 2048 bytes at offset (k * (d_ff / 16) + g) * 2048 (chunk-
 *             major), the up codes then the gate codes, 1024 bytes each.  In each 1024-byte
 *             half, the 16 bytes at 16 * l (l = 0..63) hold channel 16g + l % 16
 *             and rows 128k + 32 (l / 16) + 8s + e for s = 0..3 (the 4-byte
 *             word s) and e = 0..7, row e of word s in nibble
 *             {0, 4, 1, 5, 2, 6, 3, 7}[e] (nibble 0 = bits 0..3), each nibble
 *             code + 8 as in proxy_q.  Bytes: prox_proxy_qt_size().
 */
typedef enum { PROX_ACT_SILU = 0, PROX_ACT_GELU_TANH = 1 } prox_activation;
typedef enum { PROX_PROXY_INT4 = 0, PROX_PROXY_W16 = 1 } prox_proxy_kind;

typedef struct {
  int32_t d_model;
  int32_t d_ff;
  int32_t wdtype;     /* prox_dtype */
  int32_t activation; /* prox_activation */
  void* proxy_q;
  float* proxy_scale;
  void* w_upgate_t;
  void* w_down;
  int32_t proxy_kind; /* prox_proxy_kind */
  int32_t reserved;
  void* proxy_w16;
  void* proxy_qt;
} prox_layer;

/* Version of this ABI (PROX_ABI_VERSION). */
int32_t prox_abi_version(void);

/* Message of the last failure on the calling thread ("" if none).  The
 * returned pointer stays valid until the next library call on that thread. */
const char* prox_last_error(void);

/* Byte sizes of the four layer buffers, in prox_layer order:
 * bytes_out[0] = proxy_q, [1] = proxy_scale, [2] = w_upgate_t, [3] = w_down.
 * bytes_out is host memory of 4 size_t. */
prox_status prox_layer_sizes(int32_t d_model, int32_t d_ff, int32_t wdtype, size_t* bytes_out);

/* Workspace bytes needed by prox_ffn_decode / prox_ffn_stage2 /
 * prox_proxy_state for `batch` tokens (1 <= batch <= 256). */
prox_status prox_workspace_size(int32_t d_model, int32_t d_ff, int32_t batch, size_t* bytes);

/* Workspace bytes needed by prox_calibrate for n_tokens calibration tokens. */
prox_status prox_calibrate_workspace_size(int32_t d_model, int32_t d_ff, int32_t n_tokens,
                                          size_t* bytes);

/*
 * Computation-budget allocator ([blog] computation-budget section).  With the
 * dense FFN counted as 3 units (up, gate, down), Stage 1 costs
 * 2 * alpha * (1 - s1) units and Stage 2 costs 3 * (1 - s2), where s1 is the
 * input sparsity (1 - keep_x), s2 the channel sparsity and alpha the time of
 * the INT4 proxy pass over every input (both proxies) divided by the time of
 * one dense projection, measured on the target GPU.  The effective sparsity
 * is e = 1 - cost / 3 = s2 - 2 * alpha * (1 - s1) / 3.  Host arithmetic in
 * double; no GPU work; outputs are host floats.
 *   prox_budget_effective: e for (s1, s2, alpha).
 *   prox_budget_s2: the s2 that reaches e_target at s1:
 *     s2 = e_target + 2 * alpha * (1 - s1) / 3; PROX_ERR_UNSUPPORTED (and
 *     *s2_out untouched) when that exceeds 1, i.e. the target is out of reach
 *     at this s1.
 * Arguments: s1, s2, e_target in [0, 1]; alpha finite and > 0; else
 * PROX_ERR_INVALID_ARG.
 */
prox_status prox_budget_effective(float s1, float s2, float alpha, float* e_out);
prox_status prox_budget_s2(float e_target, float s1, float alpha, float* s2_out);

/* Zero a workspace (device, ws_bytes) on `stream`.  A decode workspace must be
 * zeroed once before its first use (this call or any zero fill); every
 * completed call leaves it ready for the next one. */
prox_status prox_workspace_init(void* ws, size_t ws_bytes, void* stream);

/*
 * Offline packing ([blog] "Stage 1": symmetric per-row INT4 proxies of W_up
 * and W_gate, resident on the GPU; W_down has no proxy).
 *   W_up, W_gate  device [d_model][d_ff] in wdtype (paper orientation, y = x W)
 *   W_down        device [d_ff][d_model] in wdtype
 *   out           host descriptor whose device buffers receive the layout above
 * Per row r of each proxy matrix: a = max_j |W[r, j]|; scale = fp32(a / 7)
 * (IEEE division); code = clamp(rint_half_even(fp32(W[r, j] / scale)), -7, 7);
 * a zero row has scale 0 and codes 0.  W_down is copied unless out->w_down
 * already equals W_down.  Asynchronous.  Inputs and outputs must not overlap
 * (except the W_down identity case).
 */
prox_status prox_pack_proxy(const void* W_up, const void* W_gate, const void* W_down,
                            const prox_layer* out, void* stream);

/*
 * Bytes of the channel-major proxy copy (proxy_qt, layout at prox_layer):
 * d_ff * 128 * ceil(d_model / 128), i.e. d_model * d_ff when d_model is a
 * multiple of 128.
 */
prox_status prox_proxy_qt_size(int32_t d_model, int32_t d_ff, size_t* bytes);

/*
 * Fills layer->proxy_qt (device, 16-byte aligned, prox_proxy_qt_size bytes)
 * from layer->proxy_q, which must already hold the packed proxy on `stream`
 * (prox_pack_proxy): a pure re-layout of the same codes, no arithmetic on
 * weights ([blog] "Stage 1": the INT4 proxy, here stored a second way for
 * groups of tokens).  PROX_PROXY_INT4 layers only (PROX_ERR_UNSUPPORTED
 * otherwise).  Asynchronous.
 */
prox_status prox_pack_proxy_qt(const prox_layer* layer, void* stream);

/*
 * Bytes of the 16-bit proxy (proxy_w16) of a bf16 layer: d_model * wstride.
 * f32 layers give PROX_ERR_UNSUPPORTED.
 */
prox_status prox_proxy16_size(int32_t d_model, int32_t d_ff, int32_t wdtype, size_t* bytes);

/*
 * Offline packing of the 16-bit proxy ([blog] evidence section, ablation A1):
 * copies W_up and W_gate (device [d_model][d_ff] bf16, paper orientation)
 * into out->proxy_w16 in the layout documented at prox_layer, padding zeroed.
 * bf16 layers only (PROX_ERR_UNSUPPORTED otherwise); out->proxy_w16 must be
 * non-NULL and 16-byte aligned.  Asynchronous.
 */
prox_status prox_pack_proxy16(const void* W_up, const void* W_gate, const prox_layer* out, void* stream);

/*
 * Offline calibration of the two per-layer scalar thresholds ([blog] evidence
 * section, calibration paragraph: fixed per-layer thresholds from activation
 * samples).
 *   X_cal       device [n_tokens][d_model] in wdtype, 1 <= n_tokens <= 65536
 *   keep_x      fraction of pooled |x| values kept, in [0, 1]
 *   sparsity_s  fraction of pooled proxy-state magnitudes dropped, in [0, 1]
 *   tau_x,tau_s HOST outputs
 *   ws          device, >= prox_calibrate_workspace_size bytes (no zeroing needed)
 * tau_x is the n-th largest |x| with n = ceil(keep_x * N), N = n_tokens*d_model
 * (evaluated in double); tau_s is the n-th largest |s~| over all tokens with
 * n = ceil((1 - (double)sparsity_s) * n_tokens * d_ff), s~ being the Stage-1
 * proxy state under tau_x.  n = 0 gives +inf.  BLOCKS until done (the call
 * synchronises `stream`).
 */
prox_status prox_calibrate(const prox_layer* layer, const void* X_cal, int32_t n_tokens,
                           float keep_x, float sparsity_s, float* tau_x, float* tau_s,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Calibration the way the pages describe it ([blog] end-to-end decoding
 * section, calibration paragraph: at most 200,000 activation samples per
 * layer and a 4,096-bin histogram).  The pages leave the sampling and the
 * binning open; this call takes, for each threshold, the values at positions
 * floor(i N / M), i < M = min(N, max_samples), of the N pooled magnitudes
 * (|X_cal| for tau_x; |s~| under this tau_x for tau_s), bins them linearly
 * with width w = fp32(max / n_bins) (bin = min(n_bins - 1, floor(fp32(v /
 * w)))), and returns the lower edge fp32(b * w) of the bin where the count
 * from the top first reaches ceil(keep * M) (keep = keep_x, or 1 - sparsity_s
 * in double); keep 0 gives +inf, an all-zero sample 0.  The threshold keeps
 * at least the requested fraction of the sample (the whole bin is kept).
 *   max_samples in [1, 2^24], n_bins in [2, 8192] (the pages: 200000, 4096)
 *   ws          device, >= prox_calibrate_hist_workspace_size bytes
 * Non-finite calibration values give PROX_ERR_INVALID_ARG.  Other arguments
 * as prox_calibrate; BLOCKS until done.
 */
prox_status prox_calibrate_hist_workspace_size(int32_t d_model, int32_t d_ff, int32_t n_tokens,
                                               int32_t max_samples, int32_t n_bins, size_t* bytes);
prox_status prox_calibrate_hist(const prox_layer* layer, const void* X_cal, int32_t n_tokens,
                                float keep_x, float sparsity_s, int32_t max_samples, int32_t n_bins,
                                float* tau_x, float* tau_s, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step through one FFN layer for `batch` independent tokens
 * (each token gets its own masks).
 *   x           device [batch][d_model] in wdtype
 *   tau_x,tau_s the layer's thresholds
 *   y           device [batch][d_model] fp32 (overwritten)
 *   mask_idx    device [batch][d_ff] int32: ascending kept channel indices,
 *               the first mask_count[b] entries of row b are valid
 *   mask_count  device [batch] int32 (k_s per token)
 *   in_count    device [batch] int32 (k_x per token) or NULL
 *   ws          device, >= prox_workspace_size(batch) bytes, zeroed once
 * Asynchronous: kernels on `stream`, no host synchronisation.  batch 1 runs
 * three kernels (Stage 1, the Stage-2 up/gate gather, the down projection;
 * prox_ffn_decode_stages can fuse the last two, see PROX_STAGE_FUSED_STAGE2).
 * batch >= 2 runs groups of up to 8 tokens; a group of 3 or
 * more tokens runs the grouped kernels, a smaller one the per-token kernels
 * (prox_ffn_decode_stages can force either).  Grouped (the pages study
 * batch 1 and leave larger batches open, [blog] limitations section): Stage 1
 * reads each proxy row of the union of the group's kept input rows once and
 * gives a token a zero weight on the rows it rejects (with layer->proxy_qt:
 * every proxy row, from the channel-major copy); for bf16 weights Stage 2
 * reads each channel of the union of the group's channel lists once (s = 0
 * for a token that drops the channel) and adds the down projection's partial
 * sums in fixed order, so y is reproducible bit for bit; fp32 layers run
 * Stage 2 per token.  Every token's masks, k_x, k_s and y follow the batch-1
 * definition.
 */
prox_status prox_ffn_decode(const prox_layer* layer, const void* x, int32_t batch,
                            float tau_x, float tau_s, float* y, int32_t* mask_idx,
                            int32_t* mask_count, int32_t* in_count, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory or
 * pass a workspace: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  Same arguments, results and kernels as
 * prox_ffn_decode, without `ws` / `ws_bytes`: the workspace is a file-scope
 * device array of PROX_NOALLOC_SCRATCH_BYTES bytes inside the library, one
 * copy per GPU, held until the process ends.  The call allocates and frees
 * nothing (no hipMalloc, no allocating library routine).
 *   - prox_workspace_size(d_model, d_ff, batch) must not exceed
 *     PROX_NOALLOC_SCRATCH_BYTES, else PROX_ERR_UNSUPPORTED and nothing is
 *     enqueued (32 MiB holds, e.g., 18 tokens of the Qwen3-8B-shaped layer
 *     and 12 of the Qwen3-32B-shaped one).
 *   - The first call on a GPU, and a call whose shape differs from the
 *     previous call's on that GPU or whose batch exceeds every earlier one,
 *     also enqueues a fill kernel that clears the used part of the array.
 *   - Every call on one GPU uses that GPU's array: calls that overlap in time
 *     on one GPU (other streams, other host threads) race and give wrong
 *     results; serialise them, e.g. on one stream.  The array keeps the last
 *     call's contents.
 * Asynchronous (kernels on `stream`).
 */
#define PROX_NOALLOC_SCRATCH_BYTES (32u << 20)
prox_status prox_ffn_decode_noalloc(const prox_layer* layer, const void* x, int32_t batch,
                                    float tau_x, float tau_s, float* y, int32_t* mask_idx,
                                    int32_t* mask_count, int32_t* in_count, void* stream);

/*
 * prox_ffn_decode that also records four hipEvent_t (host array `events`,
 * passed as void*): [0] before Stage 1, [1] after Stage 1, [2] after the
 * Stage-2 up/gate kernel, [3] after the down kernel.  For timing only.
 */
prox_status prox_ffn_decode_events(const prox_layer* layer, const void* x, int32_t batch,
                                   float tau_x, float tau_s, float* y, int32_t* mask_idx,
                                   int32_t* mask_count, int32_t* in_count, void* ws,
                                   size_t ws_bytes, void* stream, void* const* events);

/*
 * Runs a subset of the three decode kernels, for profiling one kernel alone.
 *   stages      bit mask: PROX_STAGE_PROXY (Stage 1: input mask, INT4 proxy,
 *               channel bitmap in ws, in_count), PROX_STAGE_UPGATE (channel
 *               list from the bitmap -> mask_idx, mask_count; s_j in ws; zeroes
 *               y), PROX_STAGE_DOWN (accumulates y from mask_idx, mask_count and
 *               the s_j in ws; the grouped bf16 path at batch >= 2 instead
 *               writes y from its partial sums).  7 is prox_ffn_decode.
 * A stage run without its predecessors reads what an earlier call with the
 * same layer, x, thresholds, outputs and workspace left there.  Other
 * arguments as prox_ffn_decode.  Asynchronous.
 */
#define PROX_STAGE_PROXY 1
#define PROX_STAGE_UPGATE 2
#define PROX_STAGE_DOWN 4
/* with batch >= 2: run the per-token kernels (each token reads its own rows
 * and channels) for every group; same results up to fp32 summation order */
#define PROX_STAGE_PER_TOKEN 8
/* with batch >= 2: run the grouped kernels for every group (by default a group
 * of fewer than 3 tokens runs the per-token kernels, which are faster there);
 * not together with PROX_STAGE_PER_TOKEN */
#define PROX_STAGE_GROUPED 16
/* with batch 1 and both Stage-2 bits: run Stage 2 as one launch, the up/gate
 * gather and the down projection joined by an in-kernel grid barrier (one
 * block per CU; each block issues its first W_down rows, known from the
 * Stage-1 mask, before it waits).  Same results up to the fp32 order of the
 * atomic additions into y.  Measured slower than the two launches on MI355X
 * (device-coherent stores and polls are slow while the weight stream holds the
 * memory system); kept for comparison.  It is a cooperative launch (the
 * runtime starts it with every block resident at once); where the device has
 * no cooperative launches or cannot hold the grid, the two kernels run
 * instead.  The barrier's wait is also bounded (prox_set_wait_limit): a call
 * whose blocks did not all arrive in time sets mask_count[0] = -1 and the
 * workspace error word (prox_workspace_check) and leaves y undefined. */
#define PROX_STAGE_FUSED_STAGE2 32
prox_status prox_ffn_decode_stages(const prox_layer* layer, const void* x, int32_t batch,
                                   float tau_x, float tau_s, float* y, int32_t* mask_idx,
                                   int32_t* mask_count, int32_t* in_count, void* ws,
                                   size_t ws_bytes, void* stream, int32_t stages);

/*
 * Error word of a decode workspace: PROX_ERR_INTERNAL (and the word cleared)
 * when a call on it gave up a bounded wait (the fused Stage-2 grid barrier,
 * see PROX_STAGE_FUSED_STAGE2), else PROX_OK.  ws device, ws_bytes >= 4.  BLOCKS
 * (synchronises `stream`).
 */
prox_status prox_workspace_check(const void* ws, size_t ws_bytes, void* stream);

/*
 * Bound of the library's in-kernel waits, in ticks of the GPU's 100 MHz
 * real-time clock, for calls enqueued after this one (process-wide; default
 * 4,000,000 = 40 ms).  0 gives up at the first unsatisfied check; tests use it
 * to exercise the give-up path without any wait.  *previous (host, nullable)
 * receives the old bound.
 */
prox_status prox_set_wait_limit(uint32_t ticks, uint32_t* previous);

/*
 * Stage 2 alone ([blog] "Stage 2") from a caller-given channel list.
 *   mask_idx    device [batch][d_ff] int32, ascending indices in [0, d_ff);
 *               entries outside that range are skipped
 *   mask_count  device [batch] int32, clamped to [0, d_ff]
 *   y           device [batch][d_model] fp32 (overwritten)
 * Asynchronous.
 */
prox_status prox_ffn_stage2(const prox_layer* layer, const void* x, int32_t batch,
                            const int32_t* mask_idx, const int32_t* mask_count, float* y,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Stage 1 alone: the proxy state s~ ([blog] "Stage 1", equations for u~, h~,
 * s~) for every channel.  Groups of tokens run the Stage-1 kernel that
 * prox_ffn_decode runs for them, so s~ is what the decode thresholds.
 *   s_tilde     device [batch][d_ff] fp32
 *   in_count    device [batch] int32 or NULL
 * Asynchronous.
 */
prox_status prox_proxy_state(const prox_layer* layer, const void* x, int32_t batch,
                             float tau_x, float* s_tilde, int32_t* in_count, void* ws,
                             size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PROX_H */

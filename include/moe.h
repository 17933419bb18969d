/* moe.h -- C ABI of the MI355X (gfx950) low-bit MoE expert layer.
 *
 * One GPU's share of a mixture-of-experts FFN layer, for decode (1-256
 * tokens) and prefill: top-k routing result -> local token permute ->
 * per-token FP8 activation quantisation -> grouped GEMM1 (gate|up) over FP8
 * e4m3 or MXFP4 block-scaled expert weights with fused SwiGLU and
 * requantisation -> grouped GEMM2 -> top-k weighted combine back to token
 * order.  This is the local compute of the FP8/FP4 MoE operator of the
 * GC-MoE abstract (its grouped GEMMs with SwiGLU and requantisation fused
 * in, its combine step, and shared experts as an option) and the GMM1 ->
 * SwiGLU -> GMM2 -> combine chain of the FusedDeepMoE family analysis
 * (unified execution flow figure); the cross-GPU dispatch / all-to-all is
 * not part of it.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns
 *     every buffer; the library never allocates, frees or synchronises.
 *     Scratch comes from the caller's workspace `ws` of `ws_bytes` bytes
 *     (size from moe_workspace_size; the workspace may hold any bytes on
 *     entry).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work; results are ready when the stream is.
 *     Calls on different streams need distinct workspaces.
 *   - Outputs are fully overwritten; nothing accumulates into caller memory.
 *   - Return value: MOE_OK or an error code below.  Every error except
 *     MOE_ERR_HIP is detected on the host before anything is enqueued.
 *     NULL pointers are rejected first, before any shape, size or layout
 *     check (the onnxruntime QMoE PR's expert store likewise rejects null or
 *     zero-byte buffers before range validation); a pointer may be NULL only
 *     where its buffer has zero bytes (T = 0) or the call documents it as
 *     optional.  Device faults surface at the caller's next synchronisation.
 *   - Pointers must be 16-byte aligned (MOE_ERR_MISALIGNED otherwise).
 *
 * Number formats
 *   e4m3 = OCP FP8 E4M3FN (bias 7, max 448, no infinities); e2m1 = OCP FP4
 *   (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6); e8m0 = 2^(c-127).  bf16 values
 *   are uint16 bit patterns.
 *
 * Activation quantisation rule (per token, per group of G = act_group
 * consecutive channels; the FusedDeepMoE analysis's QuantToken / BlockQuant
 * with 448 in place of 127): a = max |x| in fp32, m = 448 / max(a, 2^-64)
 * (fp32, correctly rounded), code = e4m3(x * m) round-to-nearest-even with
 * saturation and the sign kept, scale = 1 / m (fp32).  Value = dec(code) *
 * scale.  The same rule requantises the SwiGLU output per row.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_NULL_ARG = 1,    /* a required pointer is NULL */
  MOE_ERR_BAD_SHAPE = 2,   /* T < 0; H, I, E or topk < 1; topk > E; sizes not multiples of the blocks */
  MOE_ERR_UNSUPPORTED = 3, /* a format / block / group combination that is not built */
  MOE_ERR_WORKSPACE = 4,   /* ws_bytes smaller than moe_workspace_size() */
  MOE_ERR_MISALIGNED = 5,  /* a pointer is not 16-byte aligned */
  MOE_ERR_HIP = 6          /* the HIP runtime reported an error at launch */
};

enum { MOE_WFMT_FP8_BLOCK = 0, MOE_WFMT_MXFP4 = 1, MOE_WFMT_NVFP4 = 2 };
enum { MOE_AFMT_FP8 = 0, MOE_AFMT_MXFP4 = 1 };

/* Layer shape (host struct).
 *   T tokens on this GPU, H hidden size, I expert FFN width, E local experts,
 *   topk slots per token.
 *   wfmt = MOE_WFMT_FP8_BLOCK: e4m3 weights, one fp32 scale per
 *          wblk x wblk block (wblk 32 or 128), act_group must equal wblk.
 *   wfmt = MOE_WFMT_MXFP4: e2m1 weights packed two per byte (even K index in
 *          the low nibble) with one e8m0 scale per 32 along K (wblk = 32);
 *          act_group must be 128.
 *   wfmt = MOE_WFMT_NVFP4: e2m1 weights packed the same way, one e4m3 scale
 *          per 16 along K (wblk = 16) and one fp32 scale per expert matrix
 *          (moe_weights' w1g..sw2g): weight = code * block scale * matrix
 *          scale (the pages name NVFP4 beside MXFP4 in the onnxruntime QMoE
 *          PR's shared 4-bit expert layouts; this is its published
 *          two-level definition).  act_group must be 128 and act_fmt FP8;
 *          both operands are multiplied as fp16 (exact).
 *   has_shared = 1 adds one always-on shared expert (same format and I) to
 *   every token with weight 1 (GC-MoE abstract: shared experts as an
 *   option; FusedDeepMoE shared-expert path: all tokens in one group).
 *   act_fmt = MOE_AFMT_FP8: activations and the requantised SwiGLU output
 *          are e4m3 with one fp32 scale per act_group channels (the rule
 *          below).
 *   act_fmt = MOE_AFMT_MXFP4: the 4-bit-activation variant (the W4A8 family
 *          member of the FusedDeepMoE analysis, with Microscaling FP4 in
 *          place of int4): e2m1 codes packed two per byte (even channel in
 *          the low nibble) with one e8m0 scale per 32 channels, X =
 *          2^(floor(log2 amax) - 2) clamped to the e8m0 range, code =
 *          e2m1(x / X) round-to-nearest-even saturating at +-6.  Needs
 *          wfmt = MOE_WFMT_MXFP4 (MOE_ERR_UNSUPPORTED otherwise),
 *          act_group = 32, H a multiple of 256 and H, I <= 8192
 *          (MOE_ERR_UNSUPPORTED otherwise).  The scale arrays the stage calls
 *          take as float* (xs, hs) then hold e8m0 bytes: [T][H/32] and
 *          [rows][I/32]; the code arrays xq, hq hold H/2 and I/2 bytes per row.
 * Limits: 1 <= E <= 1024, topk <= 32, H and I multiples of 128,
 *   T * topk < 2^24, T * H < 2^31 and (T * topk + T * has_shared) * I < 2^31. */
typedef struct moe_cfg {
  int32_t T, H, I, E, topk;
  int32_t wfmt;
  int32_t wblk;
  int32_t act_group;
  int32_t has_shared;
  int32_t act_fmt;
} moe_cfg;

/* Expert weights (host struct of device pointers).
 *   prepacked = 0: the CANONICAL row-major tensors -- FP8: w1 uint8
 *     [E][2I][H] (rows 0..I-1 gate, I..2I-1 up, K contiguous), w1s float
 *     [E][2I/wblk][H/wblk]; w2 uint8 [E][H][I], w2s float [E][H/wblk][I/wblk].
 *     MXFP4: w1 uint8 [E][2I][H/2], w1s uint8 [E][2I][H/32]; w2 uint8
 *     [E][H][I/2], w2s uint8 [E][H][I/32].  NVFP4: w1 uint8 [E][2I][H/2],
 *     w1s uint8 e4m3 [E][2I][H/16], w1g float [E]; w2 uint8 [E][H][I/2],
 *     w2s uint8 e4m3 [E][H][I/16], w2g float [E] (sw1g, sw2g: [1]).
 *   prepacked = 1: the same tensors in the TILED layout written by
 *     moe_prepack_weights (codes and MXFP4 scales re-laid out, e4m3 block
 *     scales unchanged; same sizes).
 * The GEMM entry points and moe_layer read only the tiled layout and return
 * MOE_ERR_UNSUPPORTED for prepacked == 0, the way the FusedDeepMoE family
 * analysis's framework kernel entry takes GMM1 weights already permuted
 * (its gmm1_permuted_weight argument) and the onnxruntime QMoE PR marks
 * pre-arranged weights with a weights_prepacked flag.
 * sw1..sw2s: the shared expert with a leading dimension of 1 (may be NULL
 * when has_shared == 0).  w1g..sw2g: NVFP4's fp32 matrix scales, 4-byte
 * aligned (NULL for the other formats; the tiled layout keeps them as they
 * are). */
typedef struct moe_weights {
  const void *w1, *w1s, *w2, *w2s;
  const void *sw1, *sw1s, *sw2, *sw2s;
  int32_t prepacked;
  const float *w1g, *w2g, *sw1g, *sw2g;
} moe_weights;

/* Bytes of workspace moe_layer and the stage calls need for this shape
 * (host only; no device work).  *bytes is written on MOE_OK.  The caller
 * allocates it once per shape and passes it to every call, as the
 * FusedDeepMoE family analysis sizes its operator workspace on the host
 * from the tiling (W4A8 workspace computation: a fixed reserve plus the
 * stage buffers).  Layer intermediates, split-K partial sums and arrival
 * counters live there; contents on entry do not matter. */
int moe_workspace_size(const moe_cfg* cfg, size_t* bytes);

/* Steps 1-4: expert histogram, exclusive prefix-scan offsets (the group
 * list), stable expand index, and per-token FP8 activation quantisation
 * (FusedDeepMoE analysis: CalAndSendTokenCount, gmGroupList, gmExpandIdx and
 * QuantToken).
 *   x          bf16 [T][H]
 *   topk_ids   int32 [T][topk]; ids outside [0, E) are masked slots (not
 *              counted, expand_idx = -1, no contribution)
 *   counts     int32 [E + has_shared] rows per expert (counts[E] = T for the
 *              shared expert)
 *   offsets    int32 [E + 1 + has_shared] exclusive scan of counts
 *   expand_idx int32 [T*topk]: row of slot i = t*topk + j; rows of one
 *              expert hold its slots in ascending i (stable)
 *   row_token  int32 [T*topk + T*has_shared]: token of each row, -1 after
 *              the last row; shared rows are offsets[E] + t
 *   xq, xs     e4m3 codes uint8 [T][H] and fp32 scales [T][H/act_group]
 * ws / ws_bytes: needed only when T*topk > 4096 (the slots are then placed
 * in chunks whose counts live in the workspace): at least
 * moe_workspace_size(cfg) bytes, else MOE_ERR_WORKSPACE / MOE_ERR_NULL_ARG;
 * otherwise unused (may be NULL / 0). */
int moe_permute(const moe_cfg* cfg, const uint16_t* x, const int32_t* topk_ids, int32_t* counts,
                int32_t* offsets, int32_t* expand_idx, int32_t* row_token, uint8_t* xq, float* xs,
                void* ws, size_t ws_bytes, void* stream);

/* Step 5 (+ shared rows): for every row r of group e (e = E is the shared
 * expert), G[r][n] = sum_k xq_deq[row_token[r]][k] * w1_deq[e][n][k] for
 * n < 2I with fp32 accumulation, h = silu(G[:, :I]) * G[:, I:], then h
 * requantised per row and act_group with the activation rule (FusedDeepMoE
 * analysis: GmmDeqSwigluQuant, OpDequant, OpSwiglu, OpBlockQuant).
 *   xq, xs      as produced by moe_permute
 *   row_token   int32 [rows]; offsets int32 [E + 1 + has_shared]
 *   hq, hs      outputs: uint8 [rows][I] and fp32 [rows][I/act_group],
 *               rows = offsets[E + has_shared] (rows past that untouched) */
int moe_grouped_gemm1_swiglu(const moe_cfg* cfg, const uint8_t* xq, const float* xs,
                             const int32_t* row_token, const int32_t* offsets, const moe_weights* w,
                             uint8_t* hq, float* hs, void* ws, size_t ws_bytes, void* stream);

/* Step 6: y[r][n] = sum_k hq_deq[r][k] * w2_deq[e][n][k], n < H, fp32
 * accumulation (FusedDeepMoE analysis: GmmDeq).
 *   hq, hs   uint8 [rows][I], fp32 [rows][I/act_group]
 *   offsets  int32 [E + 1 + has_shared]
 *   y        fp32 [rows][H] output */
int moe_grouped_gemm2(const moe_cfg* cfg, const uint8_t* hq, const float* hs, const int32_t* offsets,
                      const moe_weights* w, float* y, void* ws, size_t ws_bytes, void* stream);

/* Step 8: out[t][:] = sum over j ascending of valid slots
 * topk_weights[t][j] * y[expand_idx[t*topk + j]][:] (+ y[offsets[E] + t][:]
 * with weight 1 when has_shared), fp32 accumulation, bf16 round-to-nearest-
 * even (FusedDeepMoE analysis: ReducePermute; GC-MoE abstract's combine).
 *   y fp32 [rows][H]; expand_idx int32 [T*topk]; offsets int32 [E+1+has_shared];
 *   topk_weights fp32 [T][topk]; out bf16 [T][H] */
int moe_combine(const moe_cfg* cfg, const float* y, const int32_t* expand_idx, const int32_t* offsets,
                const float* topk_weights, uint16_t* out, void* stream);

/* Steps 1-8 in one call (internally fused where it pays):
 *   x bf16 [T][H], topk_ids int32 [T][topk], topk_weights fp32 [T][topk],
 *   out bf16 [T][H]; ws of at least moe_workspace_size(cfg) bytes.
 * Between GEMM2 and the combine the rows y are kept as bf16 (round to
 * nearest even) instead of fp32, halving that round trip through memory;
 * every sum is still accumulated in fp32.  The result equals the stage
 * calls chained with y rounded to bf16 before moe_combine. */
int moe_layer(const moe_cfg* cfg, const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
              const moe_weights* w, uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/* Steps 1-8 with GEMM1, GEMM2 and the combine in ONE persistent launch
 * (after the routing and quantisation launch), for decode shapes: the
 * layer's chain of launches collapsed into one kernel whose dependent steps
 * run on device-side counters (the GC-MoE abstract runs its decode layer as
 * a CUDA graph of three nodes; the FusedDeepMoE family analysis keeps the
 * GMM1 -> SwiGLU -> GMM2 -> combine chain inside one operator, unified
 * execution flow figure).  A grid of about as many workgroups as fit on the
 * GPU takes GEMM1's, GEMM2's and the combine's units in that order from one
 * ticket counter; a unit waits only for units of earlier tickets (a GEMM2
 * unit for its work item's GEMM1 slices, the combine for GEMM2), so the
 * launch always finishes.  The h and y rows pass between workgroups through
 * device-coherent loads and stores.  Same arithmetic as moe_layer: the
 * output is bit-identical to moe_layer's for the same inputs.
 * Arguments as moe_layer (ws of at least moe_workspace_size(cfg) bytes; its
 * counters are zeroed by the routing launch), plus
 *   status  int32 device pointer or NULL: set to the number of waits that
 *           expired (each wait gives up after about a second, its unit is
 *           skipped and every later wait gives up at once; 0 in every
 *           correct run -- a nonzero value means the output is not valid).
 * Shapes: those moe_layer runs on its decode kernels (few rows per expert)
 * with FP8 activations; others return MOE_ERR_UNSUPPORTED (host check,
 * before any launch).  T == 0 returns MOE_OK without a launch.  Like
 * moe_layer, calls on one workspace must not overlap; the call allocates
 * nothing and enqueues only kernels (it can be captured in a graph). */
int moe_layer_persistent(const moe_cfg* cfg, const uint16_t* x, const int32_t* topk_ids,
                         const float* topk_weights, const moe_weights* w, uint16_t* out, void* ws,
                         size_t ws_bytes, int32_t* status, void* stream);

/* Polls each wait of moe_layer_persistent makes before it expires (default
 * 2^20, about a second; process-wide, read when a call is enqueued).  A
 * diagnostic: 0 makes every wait that finds its producer unfinished expire
 * at once, which exercises the expiry path (status > 0, the launch still
 * ends) without a slow run.  MOE_ERR_BAD_SHAPE for polls < 0. */
int moe_layer_persistent_spin_limit(int polls);

/* The router in front of the layer: the routing GEMM and the routing
 * selection, which the DeepGEMM 26/09 news page fuses into one kernel for its
 * Mega Gate (here two launches, the GEMM's fp32 partial logits meeting in
 * ws): for every token t,
 *   logit[e] = sum_h x[t][h] * gate_w[e][h]    (bf16 products, fp32 sums)
 *   topk_ids[t][0..topk) = the topk experts with the largest logits, in
 *     descending order, equal logits going to the lower expert id
 *   topk_weights[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the
 *     topk selected logits (the softmax renormalised over the top-k)
 * The outputs are exactly moe_layer's topk_ids / topk_weights inputs.
 *   x       bf16 [T][H]; gate_w bf16 [E][H] (one gate row per expert)
 *   topk_ids int32 [T][topk]; topk_weights fp32 [T][topk]
 * Uses cfg's T, H, E and topk (the rest must still be valid); E <= 256
 * (MOE_ERR_UNSUPPORTED otherwise).  Logits are summed in fp32, so two
 * experts whose exact logits differ by less than that rounding may come
 * out in either order.
 *   ws: device scratch of at least moe_route_workspace_size(cfg) bytes
 *   (contents on entry ignored; may be NULL when that size is 0, i.e. T = 0).
 *   The gate GEMM is split along K over enough workgroups to fill the GPU;
 *   the splits' fp32 partial logits meet in ws, sized on the host as the
 *   layer's workspace is (FusedDeepMoE W4A8 workspace computation):
 *   splits x T (rounded up to 16, or to 64 above 512 tokens) x E x 4 bytes.
 * Errors as for every entry point (MOE_ERR_WORKSPACE: ws_bytes too small). */
int moe_route_workspace_size(const moe_cfg* cfg, size_t* bytes);
int moe_route(const moe_cfg* cfg, const uint16_t* x, const uint16_t* gate_w, int32_t* topk_ids, float* topk_weights,
              void* ws, size_t ws_bytes, void* stream);

/* moe_layer for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and kernels as moe_layer, bit-identical results, but
 * no workspace argument.  Scratch is a static device array of
 * MOE_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on every GPU it
 * runs on until the process ends; shapes whose moe_workspace_size exceeds
 * it return MOE_ERR_WORKSPACE (host check; e.g. the H=4096 E=64 top-8
 * I=1536 layer fits up to T = 453, the H=7168 E=256 top-8 I=2048 layer
 * with a shared expert up to T = 235).  The call allocates and frees
 * nothing.  The device is the current one (the stream's); the first call on
 * a device looks up the array's address (hipGetSymbolAddress), so make it
 * once outside any graph capture; later calls only enqueue kernels.
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents (the kernels clear what must start at zero): calls that
 * overlap on one GPU -- on different streams, or from different threads --
 * race and must be serialised by the caller.
 * Arguments and errors as moe_layer, plus MOE_ERR_HIP if the array's
 * address cannot be resolved and MOE_ERR_UNSUPPORTED for device ids >= 64. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
int moe_layer_static(const moe_cfg* cfg, const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                     const moe_weights* w, uint16_t* out, void* stream);

/* One-time re-layout of a layer's expert weights (canonical row-major, as
 * above) into the tiled layout the GEMM entry points read -- the step a
 * caller runs when weights are loaded, as the FusedDeepMoE family analysis
 * keeps its GMM weights in the matrix unit's blocked (zN) layout and hands
 * the framework entry permuted GMM1 weights (GMM type definitions; FWK
 * kernel entry).  Every tensor of `canonical` is read and the matching one
 * of `packed` written (w1, w1s, w2, w2s, and sw1..sw2s when has_shared);
 * `packed` holds buffers of the canonical sizes, distinct from the
 * canonical ones (MOE_ERR_UNSUPPORTED otherwise).  canonical->prepacked
 * must be 0 (MOE_ERR_UNSUPPORTED otherwise: the tensors are already
 * tiled); on MOE_OK packed->prepacked is set to 1 (the struct itself is
 * host memory written by the call).  Only cfg's E, H, I, wfmt, wblk and
 * has_shared matter (the rest must still be valid).
 *
 * Tiled layout of a [mats][N][K] tensor: tile (k step ks, row tile rt) =
 * rows 16 rt..16 rt+15 x K 128 ks..128 ks+127, stored at
 * ((m * K/128 + ks) * N/16 + rt) * B with B = 2048 (e4m3) or 1024 (e2m1)
 * bytes, in the lane order of the gfx950 scaled-MFMA operand: byte l*16+i
 * (l < 64, i < 16) is row-major byte 16 (l/16) + i of row 16 rt + l%16 in
 * the step's K chunk (128 bytes for e4m3, 64 for e2m1), and for e4m3 byte
 * 1024 + l*16 + i is row-major byte 64 + 16 (l/16) + i of that chunk.
 * MXFP4 scales: 64 bytes per tile in the same order, byte l = scale of row
 * 16 rt + l%16 and 32-block 4 ks + l/16.  NVFP4 codes tile as MXFP4's;
 * NVFP4 scales: 128 bytes per tile, byte 8 m + j = scale of row 16 rt + m
 * and 16-block 8 ks + j.  e4m3 block scales of the FP8 format and NVFP4's
 * matrix scales keep their row-major layout (copied when the packed pointer
 * differs).  Work is
 * enqueued on `stream` like every other call. */
int moe_prepack_weights(const moe_cfg* cfg, const moe_weights* canonical, moe_weights* packed, void* stream);

/* Diagnostic: read `bytes` (a multiple of 16) of device memory at `buf`
 * once -- a plain HBM read stream, the achievable-bandwidth reference for
 * the weight-streaming GEMMs.  Four workgroups of four waves per CU; each
 * wave reads one contiguous region with 16-byte non-temporal loads.  `sink`
 * (device, at least 16 * CU-count bytes; 4 KiB covers an MI355X) receives
 * the XOR of the 32-bit words each workgroup read, one word per workgroup,
 * so the XOR over the first 4 * CU-count sink words equals the XOR over the
 * buffer.
 * MOE_ERR_NULL_ARG, MOE_ERR_MISALIGNED, MOE_ERR_BAD_SHAPE (bytes % 16) and
 * MOE_ERR_WORKSPACE (sink too small) are host checks. */
int moe_stream_read(const void* buf, size_t bytes, void* sink, size_t sink_bytes, void* stream);

/* Diagnostic: the issued rate of the scaled 16x16x128 MFMA the GEMMs use,
 * for the operand formats of `wfmt` (MOE_WFMT_FP8_BLOCK: e4m3 x e4m3;
 * MOE_WFMT_MXFP4: e2m1 weights x e4m3 activations; MOE_RATE_E2M1_E2M1:
 * e2m1 x e2m1, the 4-bit-activation layer's GEMMs).  Four workgroups of four
 * waves per CU each run `iters` (1 .. 65536) rounds of eight independent
 * MFMAs on operands that are all 1.0 with unit scales; `sink` (device, at
 * least 16 * CU-count bytes; 4 KiB covers an MI355X) receives one fp32 per
 * workgroup, exactly 4096 * iters.  `*flops` (host, may be NULL) is set to the
 * FLOP count enqueued (2 * 16 * 16 * 128 per MFMA), so FLOP/s = *flops / the
 * call's duration on `stream`.  MOE_ERR_NULL_ARG (sink), MOE_ERR_MISALIGNED,
 * MOE_ERR_UNSUPPORTED (other wfmt), MOE_ERR_BAD_SHAPE (iters) and
 * MOE_ERR_WORKSPACE (sink too small) are host checks. */
enum { MOE_RATE_E2M1_E2M1 = 16 };  /* not a weight format: the probe's third operand pair */
int moe_mfma_rate(int wfmt, int iters, void* sink, size_t sink_bytes, double* flops, void* stream);

/* Diagnostic: the fp32 -> e4m3 conversion every quantiser of the layer
 * uses (activation codes in moe_permute, requantised h in GEMM1), applied
 * to n values: saturation at +-448, round to nearest even, the sign kept
 * (values that round to zero give 0x00 or 0x80) -- the activation rule's
 * "code = e4m3(x * m)" step.  v (device, n fp32; NaN is outside the
 * contract) -> codes (device, n bytes).  Exposed so the conversion can be
 * checked against an independent encoder on every finite fp32 pattern.
 * MOE_ERR_NULL_ARG (v or codes NULL with n > 0), MOE_ERR_MISALIGNED and
 * MOE_ERR_BAD_SHAPE (n >= 2^40) are host checks. */
int moe_encode_e4m3(const float* v, size_t n, uint8_t* codes, void* stream);

/* Static description of an error code (host only). */
const char* moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */

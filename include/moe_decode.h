/*
 * moe_decode.h — C ABI of the MI355X (gfx950) Flint-style MoE layer.
 *
 * The layer ("Day-0 Support for Flint on vLLM", Model architecture): a
 * sigmoid router over 256 experts picks the top 6 for each token, and one
 * shared expert that every token uses is added.  Each expert is a SiLU-gated
 * FFN, y_e = D_e (SiLU(G_e x) * (U_e x)), with G_e, U_e [512 x 2048] and
 * D_e [2048 x 512].  The layer output is
 *     y = sum_j w_j y_{e_j} + y_shared,     w_j = s_j / sum_sel s,  s = sigmoid(W_r x).
 * Weights are NVFP4, run weight-only with BF16 activations (W4A16), or BF16
 * (Model architecture section); only the selected experts' weights are read
 * (Optimization section, Fig. 2 list, small-batch MoE kernels); routing and
 * the expert combine are fused into the neighbouring GEMV kernels on the
 * low-latency path for up to 8 requests (Optimization section).
 *
 * Conventions for every entry point
 *  - Every data pointer is a DEVICE pointer owned by the caller, 16-byte
 *    aligned (workspace: 256-byte aligned).  The library allocates nothing,
 *    keeps no state between calls, never synchronises and never reads
 *    routing back to the host, so a call can be captured in a HIP graph.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it; device-side faults surface at the caller's
 *    next synchronisation.
 *  - Arguments are checked before anything is launched; on error nothing is
 *    launched and the status says why.  MOE_ERR_UNSUPPORTED means a valid
 *    request this library does not serve (another shape, B > 8, ...): the
 *    caller should fall back to a generic implementation, the convention the
 *    Flint pages describe for configurations outside their kernels
 *    (Usage notes section).
 *  - Calls sharing a workspace must be ordered (same stream, or events).
 *    The single-launch decode entry points (moe_decode_forward and
 *    moe_decode_forward_timed on Flint's shape, moe_decode_forward_ex,
 *    moe_decode_stack_forward, moe_decode_chain_forward) run 256
 *    workgroups that hand data to each other inside the launch, so all 256
 *    must be resident at once: such a call needs the device to itself, with
 *    no other kernel (another such call included, on any workspace) running
 *    beside it.  If compute units are taken by other work, workgroups wait
 *    for data that does not come; every wait is bounded, so the kernel still
 *    ends, but the output is invalid and the workspace's wait-status word
 *    records it (moe_workspace_status).  The other entry points have no
 *    such requirement and calls on distinct workspaces may overlap.
 *  - No C++ exception crosses this boundary.
 *
 * Tensor layouts (E experts in a set; H = hidden, I = inter: 2048 and 512
 * for Flint)
 *  x, out         bf16 [T][H], token-major.
 *  router_w       bf16 [E_routed][H] (row e gives logit e).
 *  NVFP4 expert set (16-element blocks along the input dimension):
 *    w13          u8  [E][2][I][H/2]   codes of gate (index 0) and up (1);
 *                                      byte j of a row holds element 2j in
 *                                      bits 0-3 and element 2j+1 in bits 4-7;
 *                                      a code is E2M1 (sign, 2-bit exponent
 *                                      with bias 1, 1-bit mantissa).
 *    w13_scale    u8  [E][2][I][H/16]  E4M3FN block scales.
 *    w2           u8  [E][H][I/2]      codes of down.
 *    w2_scale     u8  [E][H][I/16]     E4M3FN block scales.
 *    global       f32 [E][3]           per-tensor scales (gate, up, down).
 *    weight value = e2m1(code) * e4m3(block scale) * global.
 *  BF16 expert set: w13 bf16 [E][2][I][H], w2 bf16 [E][H][I]; the scale and
 *    global pointers must be NULL.
 *  MXFP8 expert set (OCP Microscaling: 32-element blocks along the input
 *  dimension; the expert format of the last 8 layers of Inkling-2-Small in
 *  the AREX article on vLLM's Day-0 support for it, 48-layer MoE section):
 *    w13          u8  [E][2][I][H]     E4M3FN elements of gate and up.
 *    w13_scale    u8  [E][2][I][H/32]  E8M0 block scales (2^(b - 127)).
 *    w2           u8  [E][H][I]        E4M3FN elements of down.
 *    w2_scale     u8  [E][H][I/32]     E8M0 block scales.
 *    global       NULL (the MX formats have no tensor scale).
 *    weight value = e4m3(element) * 2^(scale - 127).
 *  The shared experts are one expert set of E = n_shared experts in the same
 *  format (NULL when n_shared is 0); each is added with weight 1.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, aliasing output      */
  MOE_ERR_UNSUPPORTED = -2, /* valid request outside what this library runs */
  MOE_ERR_MISALIGNED = -3,  /* a pointer breaks the alignment rule above     */
  MOE_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required    */
  MOE_ERR_HIP = -5          /* a HIP launch failed                           */
} moe_status;

/* MOE_W_NVFP4_A4: NVFP4 weights and NVFP4 activations (W4A4).  The experts'
 * inputs x and h are quantised on the fly with the Four Over Six block
 * scale (the AREX article on vLLM's Day-0 support for Inkling-2-Small,
 * 48-layer MoE section): per vector (a token's x; one (expert, token) h of
 * I values) a global amax / 2688, and per 16-block the E4M3 scale mapping
 * the block maximum to 6 or to 4, whichever reconstructs with the smaller
 * mean absolute error (a tie keeps 6), every step an fp32 operation in a
 * stated order.  The router uses x itself.  Decode entry points only;
 * weights as MOE_W_NVFP4.  Flint's shape at B <= 8 runs on the
 * single-launch kernel, every workgroup quantising all of x and of h itself
 * with the same decisions (its roundings by gfx950's converts, checked by
 * moe_a4_convert_check); other shapes run on the general path, which
 * quantises each vector once.  Setting the environment variable
 * MOE_DECODE_SPLIT=1 sends every decode call to the multi-launch paths
 * (a test switch: both compute the same layer). */
typedef enum {
  MOE_W_NVFP4 = 0,
  MOE_W_BF16 = 1,
  MOE_W_MXFP8 = 2,
  MOE_W_NVFP4_A4 = 3
} moe_wformat;

/* Layer shape.  Every entry point serves the Flint layer {2048, 512, 256, 6,
 * 1, NVFP4 | BF16} (Model architecture section: hidden 2048, 256 experts,
 * sigmoid top-6, one shared expert) on its fast paths.  The decode entry
 * points (moe_decode_route, moe_decode_forward, moe_decode_forward_timed)
 * also serve the other MoE shapes the pages name, and more, on a general
 * path: Inkling's 256 experts with top-6 and 2 shared experts,
 * Inkling-2-Small's 384 experts with top-8 and none (the AREX article,
 * 48-layer MoE section), in NVFP4, BF16, MXFP8 or NVFP4 with NVFP4
 * activations (MOE_W_NVFP4_A4, also for Flint's shape); its limits are
 * 32 <= H <= 8192 and 32 <= I <= 4096, both multiples of 32;
 * 1 <= top_k <= 8; top_k <= n_experts <= 512; 0 <= n_shared <= 2.  The
 * prefill and fused-neighbour entry points and the dequant probe return
 * MOE_ERR_UNSUPPORTED for any shape but Flint's, and so does any entry point
 * for a shape outside these limits. */
typedef struct {
  int32_t hidden;    /* H */
  int32_t inter;     /* I, per expert */
  int32_t n_experts; /* routed experts */
  int32_t top_k;
  int32_t n_shared;
  int32_t wfmt;      /* moe_wformat */
} moe_shape;

typedef struct {
  const void* w13;
  const void* w13_scale;
  const void* w2;
  const void* w2_scale;
  const float* global;
} moe_experts;

/* Version of this ABI (incremented on any incompatible change). */
int32_t moe_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status status);

/* Workspace bytes needed for `tokens` tokens: prefill = 0 for the decode
 * entry points (tokens 1..8), 1 for moe_prefill_forward.  Returns 0 when the
 * shape or token count is not served.  The workspace must be zero-filled
 * once before its first use (e.g. allocated with torch.zeros).  After that
 * it carries state from call to call that the caller must leave alone: the
 * single-launch decode kernels keep per-workgroup call counters (epochs) and
 * epoch-tagged hand-over slots in its first region, and every call advances
 * them consistently.  One workspace may serve every entry point (decode,
 * stacks, prefill, the general shapes), as long as it is large enough for
 * each: the other paths write only past that first region.  After a call
 * whose wait status is nonzero (moe_workspace_status), zero-fill the
 * workspace again before using it. */
size_t moe_workspace_bytes(const moe_shape* shape, int32_t tokens, int32_t prefill);

/* Router GEMV + sigmoid + top-k + renormalisation for B = 1..8 tokens
 * (Model architecture: sigmoid top-6; Optimization: routing fused into the
 * router GEMV).  logits_e = sum_k W_r[e][k] x[k] in fp32, s_e = sigmoid;
 * the k largest are chosen (ties go to the lower expert index), returned in
 * descending score order, with w_j = s_j / sum of the chosen s.
 *   x        bf16 [B][H]          ids  int32 [B][top_k]   (written)
 *   router_w bf16 [E][H]          w    f32   [B][top_k]   (written)
 * B > 8 returns MOE_ERR_UNSUPPORTED. */
moe_status moe_decode_route(const moe_shape* shape, const void* x, int32_t B,
                            const void* router_w, int32_t* ids, float* w, void* ws,
                            size_t ws_bytes, void* stream);

/* The whole layer for B = 1..8 tokens (the low-latency decode path):
 * route, then the SiLU-gated GEMVs of only the selected experts and of the
 * shared expert, then the weighted combine.  Products and sums are fp32;
 * h = SiLU(gate x) * (up x) is handed to the down GEMV as bf16 (the
 * activation type of W4A16) and the output is rounded once to bf16.  At
 * B > 1 each expert chosen by several tokens has its weights read once for
 * all of them.
 *   out      bf16 [B][H]   (written; must not overlap x)
 *   ids_out  int32 [B][top_k], w_out f32 [B][top_k]: the routing used
 *            (each nullable). */
moe_status moe_decode_forward(const moe_shape* shape, const void* x, int32_t B,
                              const void* router_w, const moe_experts* routed,
                              const moe_experts* shared, void* out, int32_t* ids_out,
                              float* w_out, void* ws, size_t ws_bytes, void* stream);

/* moe_decode_forward that also records the layer's kernel execution on two
 * caller-created HIP events (hipEvent_t, timing enabled): ev_start at the
 * kernel's start and ev_stop at its end (through hipExtLaunchKernel), so
 * hipEventElapsedTime gives the kernel's own duration without launch gaps.
 * For measurement; when the single-launch path is not available the events
 * bracket the three launches instead.  NULL events: MOE_ERR_INVALID_ARG. */
moe_status moe_decode_forward_timed(const moe_shape* shape, const void* x, int32_t B,
                                    const void* router_w, const moe_experts* routed,
                                    const moe_experts* shared, void* out, int32_t* ids_out,
                                    float* w_out, void* ws, size_t ws_bytes, void* stream,
                                    void* ev_start, void* ev_stop);

/* moe_decode_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Flint's shape (NVFP4 or BF16), B =
 * 1..8; other shapes and B > 8 return MOE_ERR_UNSUPPORTED (they need more
 * than the library's own workspace holds).  The library keeps that
 * workspace in a static device array of the decode workspace's size (about
 * 1.36 MB; moe_workspace_bytes of Flint's decode shape), one per GPU, held
 * until the process ends; the first call on a GPU looks its address up and
 * zero-fills it with a kernel on `stream`.  The call allocates nothing.
 * Every call on one GPU shares that array, which keeps the state of the last
 * call: calls on one GPU must not overlap (same stream, or ordered by
 * events); overlapping calls race and give wrong results.  Output, arguments
 * and errors otherwise as moe_decode_forward, bit for bit. */
moe_status moe_decode_forward_noalloc(const moe_shape* shape, const void* x, int32_t B,
                                      const void* router_w, const moe_experts* routed,
                                      const moe_experts* shared, void* out, int32_t* ids_out,
                                      float* w_out, void* stream);

/* Small-batch dense GEMV on packed NVFP4 weights, for the non-expert
 * projections and the dense MLP of the first two layers (Optimization
 * section, Fig. 2 change list: a dense GEMV on the packed weights; Model
 * architecture section: layers 0 and 1 use a dense MLP):
 *   y[t][n] = global * sum_k e2m1(codes[n][k]) * e4m3(scales[n][k / 16]) * x[t][k]
 * with fp32 accumulation and y rounded once to bf16.  The weight uses the
 * expert tensors' packing (element 2j in the low nibble of byte j, one E4M3
 * scale per 16 consecutive k, one fp32 tensor scale).
 *   x       bf16 [B][K], 16-byte aligned      codes  u8 [N][K/2], 16-byte aligned
 *   scales  u8 [N][K/16], 2-byte aligned      global f32 [1] (device)
 *   y       bf16 [B][N] (written; must not overlap x)
 * B = 1..8, K a multiple of 32, N >= 1; K > 8192 or B * K > 32768 returns
 * MOE_ERR_UNSUPPORTED.  Needs no workspace; stream-ordered, no sync. */
moe_status moe_nvfp4_gemv(const void* x, int32_t B, int32_t K, int32_t N, const void* codes,
                          const void* scales, const float* global, void* y, void* stream);

/* The same layer for T >= 1 tokens at prefill sizes (Optimization section:
 * the MoE kernels were also the largest prefill gain, measured on an
 * 8,192-token prefill): tokens are grouped by expert and each expert runs as
 * a dense bf16 matrix-core GEMM over its tokens.  Arguments as
 * moe_decode_forward, with T tokens; the workspace comes from
 * moe_workspace_bytes(shape, T, 1). */
moe_status moe_prefill_forward(const moe_shape* shape, const void* x, int32_t T,
                               const void* router_w, const moe_experts* routed,
                               const moe_experts* shared, void* out, int32_t* ids_out,
                               float* w_out, void* ws, size_t ws_bytes, void* stream);

/* One layer of a stack for moe_decode_stack_forward: its router and expert
 * sets, with the same meaning and rules as moe_decode_forward's arguments.
 * The layout (11 pointers, 88 bytes) is part of the ABI. */
typedef struct {
  const void* router_w;
  moe_experts routed;
  moe_experts shared;
} moe_layer;

/* A stack of n_layers independent Flint layers that all read the same x
 * (B = 1..8 tokens), in ONE launch: out[l] = layer_l(x).  Every workgroup
 * runs layer l + 1 as soon as its part of layer l is done, so there is no
 * launch gap between layers (the pages hide that gap with programmatic
 * dependent launch: Optimization section, low-latency path and Fig. 3).
 * Each layer computes exactly what moe_decode_forward computes (the same
 * arithmetic, bit for bit).  At B = 1 the stacked launches (this one and
 * moe_decode_chain_forward) exchange the router logits inside each XCD,
 * which relies on the hardware dealing a launch's workgroups out to the 8
 * XCDs in turn; were the deal different, the logit wait gives up and the
 * workspace status reports it (bit 0).
 *   layers   DEVICE array of n_layers moe_layer, 8-byte aligned; its
 *            contents cannot be checked on the host: every pointer in it
 *            must follow moe_decode_forward's rules for the shape.
 *   out      bf16 [n_layers][B][H] (written; must not overlap x or ws)
 *   ids_out  int32 [n_layers][B][top_k] or NULL: the routing of each layer.
 * Flint's shape only (NVFP4 or BF16); the workspace is moe_decode_forward's.
 * Where the single-launch kernel cannot run: MOE_ERR_UNSUPPORTED. */
moe_status moe_decode_stack_forward(const moe_shape* shape, int32_t n_layers,
                                    const moe_layer* layers, const void* x, int32_t B, void* out,
                                    int32_t* ids_out, void* ws, size_t ws_bytes, void* stream);

/* A chained residual stack of n_layers Flint layers in ONE launch: the
 * residual stream of a pre-norm decoder ("Day-0 Support for Flint on vLLM",
 * Model architecture: 49 layers, 47 of them MoE), MoE layers only:
 *   x_0 = x,   x_{l+1} = bf16(x_l + layer_l(norm_l(x_l))),   out[l] = x_{l+1},
 * where norm_l is the pre-MoE RMSNorm of moe_fuse with weight norm_w[l] (or
 * the identity when norm_w is NULL).  Layer l equals
 * moe_decode_forward_ex(x_l, {norm_w[l], norm_eps, residual = x_l}) bit for
 * bit.  Layer l + 1 starts from all of x_{l+1}: only its weight loads that
 * depend on neither its input nor its routing (router row, shared expert)
 * are issued early, during layer l (the pages load the next kernel's
 * weights early under programmatic dependent launch: Optimization section,
 * low-latency path and Fig. 3).
 *   layers   DEVICE array of n_layers moe_layer (as moe_decode_stack_forward)
 *   x        bf16 [B][H], B = 1..8 (B > 8: MOE_ERR_UNSUPPORTED)
 *   norm_w   bf16 [n_layers][H] or NULL; norm_eps > 0 and finite when set
 *   out      bf16 [n_layers][B][H] (written; must not overlap x, norm_w, the
 *            layer table or ws)
 *   ids_out  int32 [n_layers][B][top_k] or NULL: the routing of each layer.
 * Flint's shape only (NVFP4 or BF16); the workspace is moe_decode_forward's.
 * Where the single-launch kernel cannot run: MOE_ERR_UNSUPPORTED. */
moe_status moe_decode_chain_forward(const moe_shape* shape, int32_t n_layers,
                                    const moe_layer* layers, const void* x, int32_t B,
                                    const void* norm_w, float norm_eps, void* out,
                                    int32_t* ids_out, void* ws, size_t ws_bytes, void* stream);

/* Wait status of a workspace: copies its status word to *status (DEVICE
 * int32, 4-byte aligned) and clears the word, in one kernel on `stream`, so
 * it can be captured in a HIP graph with the calls it checks.  The word
 * collects, since the last status call, the waits of the single-launch
 * decode kernels that gave up because their data never arrived (see the
 * concurrency rule above): bit 0 the router-logit exchange, bit 1 the h
 * hand-over between the GEMVs, bit 2 the residual-stream hand-over of a
 * chained stack.  Zero: every call since the last status call completed
 * its hand-overs; nonzero: those calls' outputs are invalid and the
 * workspace must be zero-filled before its next use (a caller can then fall
 * back, the convention of the Usage notes section).
 *   ws     the workspace (256-byte aligned, ws_bytes >= 256)
 *   status int32 [1] (device; must not overlap ws) */
moe_status moe_workspace_status(void* ws, size_t ws_bytes, int32_t* status, void* stream);

/* The layer's neighbours, fused into it (Optimization section, low-latency
 * path: the norm and the combine fused into the adjacent GEMV kernels; the
 * norm kernels are one of the Fig. 2 steps).  Each part is optional.
 *   norm_w    bf16 [H] or NULL.  When set, the layer runs on
 *             xn[t][k] = bf16(x[t][k] * norm_w[k] / sqrt(mean_j x[t][j]^2 + norm_eps)),
 *             the pre-MoE RMSNorm, computed in fp32 and rounded once to
 *             bf16 (router and experts take bf16 activations, W4A16).
 *   norm_eps  > 0 and finite when norm_w is set (ignored otherwise).
 *   residual  bf16 [T][H] or NULL.  When set, out = bf16(residual + y), the
 *             residual add done in fp32 before the single rounding of the
 *             output.  It may be x itself, or out itself (an in-place
 *             update of the residual stream); it must not partly overlap
 *             out.
 *   xn_out    bf16 [T][H] or NULL: receives the normalised input exactly as
 *             the layer used it (needs norm_w; must not overlap x, out or
 *             residual).  For checking routing decisions against a
 *             reference on the same bf16 input. */
typedef struct {
  const void* norm_w;
  float norm_eps;
  const void* residual;
  void* xn_out;
} moe_fuse;

/* moe_decode_forward with the neighbours of moe_fuse fused in (fuse may be
 * NULL: then the result equals moe_decode_forward's bit for bit).  Runs only
 * as the single-launch decode kernel: where that cannot run (a GPU with
 * fewer than 256 compute units) it returns MOE_ERR_UNSUPPORTED. */
moe_status moe_decode_forward_ex(const moe_shape* shape, const void* x, int32_t B,
                                 const moe_fuse* fuse, const void* router_w,
                                 const moe_experts* routed, const moe_experts* shared, void* out,
                                 int32_t* ids_out, float* w_out, void* ws, size_t ws_bytes,
                                 void* stream);

/* moe_prefill_forward with the neighbours of moe_fuse fused in (fuse may be
 * NULL).  The norm runs as one pass over x ahead of the routing GEMM (each
 * token's mean square is needed before its first product); the residual add
 * is done in the combine.  Same workspace as moe_prefill_forward. */
moe_status moe_prefill_forward_ex(const moe_shape* shape, const void* x, int32_t T,
                                  const moe_fuse* fuse, const void* router_w,
                                  const moe_experts* routed, const moe_experts* shared, void* out,
                                  int32_t* ids_out, float* w_out, void* ws, size_t ws_bytes,
                                  void* stream);

/* Diagnostics for tests of the general decode path: byte offsets, in its
 * workspace for `shape`, of
 *   [0] the entry count (int32);   [1] the entries (int32 [66]: a routed
 *   expert id, or n_experts + s for shared expert s), routed ones in
 *   ascending id first;   [2] their token masks (uint32 [66]);
 *   [3] h before any quantisation (bf16 [66][8][inter], entry-major);
 *   W4A4 only: [4] the quantised x as e2m1 * e4m3 (bf16 [8][hidden]),
 *   [5] the x globals (f32 [8]), [6] the quantised h as e2m1 * e4m3 (bf16
 *   [66][8][inter]), [7] the h globals (f32 [66][8]).
 * Valid after a decode call that took the general path on that workspace
 * (for Flint's shape in W4A4 that needs MOE_DECODE_SPLIT=1);
 * MOE_ERR_UNSUPPORTED for shapes the general path does not serve. */
moe_status moe_general_workspace_layout(const moe_shape* shape, size_t offsets[8]);

/* Parity probe of the in-register NVFP4 decode: writes tensor `tensor`
 * (0 gate, 1 up, 2 down) of expert `expert` of an NVFP4 set as fp32,
 * out[r][c] = fp32(e2m1 * e4m3) * global (the first product is exact, so this
 * is one rounding of the exact weight).  out: f32 [I][H] for gate/up,
 * [H][I] for down.  The set must hold more than `expert` experts (not
 * checked: the caller knows its set size). */
moe_status moe_nvfp4_dequant(const moe_shape* shape, const moe_experts* set, int32_t expert,
                             int32_t tensor, float* out, void* stream);

/* Check of the hardware converts behind the W4A4 quantiser's roundings
 * (Inkling-2-Small article, 48-layer MoE section: NVFP4 activations with
 * the Four Over Six block scale).  The single-launch W4A4 kernel rounds
 * block scales to E4M3 (nearest-even, saturating at 448) and scaled values
 * to E2M1 (nearest-even, saturating at 6) with gfx950's fp32 -> FP8 / FP4
 * converts; this runs them over every fp32 bit pattern against the
 * roundings written out as arithmetic and writes the mismatch counts:
 *   counts  device pointer to 2 uint64, overwritten: [0] E2M1 mismatches
 *           over all finite fp32 values, [1] E4M3 mismatches over all
 *           non-negative finite ones (both 0 on a conforming device).
 * Asynchronous on `stream`; about 2^33 conversions.  MOE_ERR_INVALID_ARG for
 * a null pointer, MOE_ERR_MISALIGNED for one not 8-byte aligned. */
moe_status moe_a4_convert_check(uint64_t* counts, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */

/*
 * pblock.h -- C ABI of the MI355X (gfx950) forward pass of one parallel
 * transformer block with sliding-window causal attention:
 *
 *     y = [x +] Attn_SWA(LN(x)) + MLP(LN(x))
 *
 * Source of the method: the MegaScale guided reading on the
 * ai-training-network-primer site.  Section 2 ("Changing the model to help the
 * system") defines the parallel block (attention and feed-forward fed from the
 * same input, outputs summed) and sliding-window attention (each token attends
 * to a fixed window of nearby tokens).  Section 3 (tensor and sequence
 * parallelism) places a layer-norm before the parallel linear layers and a
 * reduce-scatter of partial sums after them.  Section 4 ("Operators") names
 * the operators: exact attention, LayerNorm, GeLU.
 *
 * Readings of what the pages leave open (fixed here for every entry point):
 *   - one LayerNorm output u = LN(x) feeds both branches; biased variance,
 *     eps from the cfg (1e-5 by default), affine gamma/beta;
 *   - GeLU is the exact erf form z/2 * (1 + erf(z / sqrt 2));
 *   - query i attends to keys j with max(0, i-W+1) <= j <= i (W keys, itself
 *     included); windows never cross sequences; W >= S is full causal;
 *   - scores are q.k / sqrt(hd); no positional encoding, no biases, no dropout.
 *
 * Layouts (all row-major, contiguous, caller-owned DEVICE memory):
 *   x, out   [B, S, d]                       (token-major)
 *   ln_gamma, ln_beta  [d]
 *   w_in     [3*H*hd + ffn, d]   rows = [Q heads; K heads; V heads; FC1],
 *                                 each head's hd rows contiguous, head-major
 *   w_out    [d, H*hd + ffn]     columns = [attention heads (head-major); FC2]
 * Element type: PBLOCK_BF16 (all of x, gamma, beta, w_in, w_out, out are
 * bf16) or PBLOCK_F32 (all fp32: the debug path).  Accumulation is fp32 in
 * both; bf16 intermediates are rounded to nearest even.
 *
 * Errors: every function returns PBLOCK_OK (0) or a negative pblock_status.
 * All argument checks run before anything is enqueued; on error nothing is
 * launched and `out` is untouched.  Faults inside kernels are asynchronous and
 * surface at the caller's next synchronisation of the stream.  No C++
 * exception crosses this boundary.  pblock_last_error() gives the detail of
 * the most recent failure on the calling thread.
 */
#ifndef PBLOCK_H
#define PBLOCK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PBLOCK_OK = 0,
  PBLOCK_ERR_NULL = -1,          /* a required pointer is NULL */
  PBLOCK_ERR_SHAPE = -2,         /* a dimension is out of the supported range */
  PBLOCK_ERR_DTYPE = -3,         /* dtype is neither PBLOCK_F32 nor PBLOCK_BF16 */
  PBLOCK_ERR_ALIGN = -4,         /* a tensor pointer is not 16-byte aligned */
  PBLOCK_ERR_ALIAS = -5,         /* out overlaps x or a weight */
  PBLOCK_ERR_CFG_MISMATCH = -6,  /* forward cfg incompatible with the handle's */
  PBLOCK_ERR_DEVICE = -7,        /* no gfx950 device current */
  PBLOCK_ERR_NOMEM = -8,         /* workspace allocation failed */
  PBLOCK_ERR_HIP = -9,           /* a HIP runtime call or launch failed */
  PBLOCK_ERR_ARG = -10           /* any other invalid argument */
} pblock_status;

typedef enum { PBLOCK_F32 = 0, PBLOCK_BF16 = 1 } pblock_dtype;

/* Block shape.  Supported ranges (else PBLOCK_ERR_SHAPE):
 *   B >= 1, S >= 1, B*S <= 2^24;  W >= 1 (W >= S means full causal);
 *   hd in {64, 128};  1 <= H <= 4096;  d, H*hd, ffn positive multiples of 64;
 *   d <= 32768, H*hd <= 2^20, ffn <= 2^20.
 * add_residual: 1 -> y = x + branches; 0 -> y = branches only (the partial
 * sum one tensor-parallel shard contributes to the reduce-scatter).
 * ln_eps > 0. */
typedef struct {
  int32_t B, S, d, H, hd, ffn, W;
  int32_t dtype;
  int32_t add_residual;
  float ln_eps;
} pblock_cfg;

typedef struct {
  const void* ln_gamma; /* [d] */
  const void* ln_beta;  /* [d] */
  const void* w_in;     /* [3*H*hd + ffn, d] */
  const void* w_out;    /* [d, H*hd + ffn] */
} pblock_weights;

typedef struct pblock_s* pblock_t;

/* Validates cfg (host only, touches no device).  Returns 0 or an error. */
int pblock_validate_cfg(const pblock_cfg* cfg);

/* Bytes of device workspace a handle for cfg allocates, or a negative status.
 * Host only.  The workspace holds the intermediates u [Mt, d], QKV [M, 3*H*hd],
 * AG [Mt, H*hd + ffn] (M = B*S; the GEMM row operands u and AG get M rounded
 * up to 256 plus 256 more rows, Mt, since the GEMM reads its row operand to
 * the end of a 256-row tile from any starting row), for bf16 the GEMM
 * scratch for the split-K tail wave (one fp32 256x256 partial tile per
 * compute unit; this estimate assumes 256), and the rotary-embedding table of
 * pblock_forward_variant (fp32 cos and sin for hd/2 pairs at M positions). */
int64_t pblock_workspace_bytes(const pblock_cfg* cfg);

/* Algorithmic FLOPs of one forward for cfg: 2*M*d*(3*H*hd+ffn) +
 * 2*M*(H*hd+ffn)*d + 4*B*H*hd*sum_i min(i+1, W), M = B*S.  Host only;
 * returns a negative value for an invalid cfg. */
double pblock_flops(const pblock_cfg* cfg);

/* Creates a handle on the current HIP device: validates cfg, checks the device
 * is gfx950, and allocates the workspace (hipMalloc) sized for cfg's B*S.  The
 * handle owns the workspace until pblock_destroy.  *out_handle is set only on
 * success. */
int pblock_create(const pblock_cfg* cfg, pblock_t* out_handle);

/* Enqueues the block forward on `stream` (a hipStream_t; NULL = the null
 * stream) and returns without synchronising.  It enqueues kernels only (no
 * allocation, no host synchronisation, no memset), so a caller may capture
 * it in a HIP graph and replay it.  x, the weights and out are
 * device pointers owned by the caller; they must stay valid until the stream
 * passes this work.  cfg must equal the create cfg except that B and S may
 * differ as long as B*S does not exceed the create cfg's B*S.  A handle's
 * workspace is shared by its calls: do not run one handle on two streams at
 * once.  out must not overlap x or any weight. */
int pblock_forward(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg,
                   void* out, void* stream);

/* pblock_forward without a handle and without allocating, for callers that cannot call
 * hipMalloc: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The intermediates (u, QKV, AG and the GEMM tail partials, laid out as in a
 * handle's workspace) live in a static device array of 256 MiB that the library holds on every
 * GPU it runs on until the process ends; its address is looked up once per device on the first
 * call there.  A cfg whose intermediates need more than 256 MiB gives PBLOCK_ERR_SHAPE (the
 * 175B shard and the small workload fit; the 8192-token workloads do not).  The same kernels
 * and launches as pblock_forward, so the results are the same bits.  Calls on one GPU share its
 * array: calls that overlap in time on one GPU (two streams, two threads) race and give wrong
 * results; calls on one stream, one after another, are safe.  Nothing in the array needs to
 * start at zero, so it is never cleared.  Per-kernel timing does not cover this entry point.
 * x, weights, out and cfg rules as pblock_forward (any B*S up to the 256 MiB limit). */
int pblock_forward_static(const void* x, const pblock_weights* w, const pblock_cfg* cfg, void* out,
                          void* stream);

/* The standard (serial) layer the parallel block replaces, built from the same
 * kernels for comparison (MegaScale guided reading, section 2: the usual layer
 * is sequential, its feed-forward part taking the attention part's result as
 * input; section 8, Table 3 prices the parallel form at +4.6 MFU points).
 * Pre-LayerNorm form:
 *   h = x + Attn(LN1(x)),   y = h + W2 GeLU(W1 LN2(h))
 * LN1 = (w->ln_gamma, w->ln_beta), LN2 = (ln2_gamma, ln2_beta), both [d].  The
 * attention sub-layer uses W_in rows [0, 3*H*hd) and W_out columns [0, H*hd),
 * the feed-forward sub-layer W_in rows [3*H*hd, 3*H*hd + ffn) and W_out columns
 * [H*hd, H*hd + ffn): the same packed matrices as pblock_forward, so the two
 * forms can be timed on identical parameters.  cfg->add_residual must be 1
 * (PBLOCK_ERR_ARG otherwise).  out [B*S, d] holds h between the sub-layers.
 * Stream, ownership, alignment, aliasing and cfg rules as pblock_forward; the
 * LN2 parameters must be 16-byte aligned and must not overlap out. */
int pblock_forward_serial(pblock_t h, const void* x, const pblock_weights* w, const void* ln2_gamma,
                          const void* ln2_beta, const pblock_cfg* cfg, void* out, void* stream);

/* The block forward in n_chunks chunks of sequence positions, in order, for
 * overlapping tensor/sequence-parallel communication with compute (MegaScale
 * guided reading, section 3: the GEMMs next to an all-gather or reduce-scatter
 * are split into chunks so that one chunk's communication overlaps the next
 * chunk's computation).  Chunk k covers positions [k*S/n, (k+1)*S/n) (integer
 * division) of every sequence.  With ready_events (an array of n_chunks
 * hipEvent_t, entries may be NULL), for each chunk, in order, on `stream`:
 *   wait for ready_events[k] if non-NULL (e.g. the arrival of chunk k's rows of
 *   x from an all-gather);
 *   LayerNorm, the fused QKV+FC1 GEMM, attention for the chunk's queries (their
 *   keys reach back W-1 positions into earlier chunks) and the output GEMM for
 *   the chunk's rows;
 *   record done_events[k] if done_events and done_events[k] are non-NULL:
 *   chunk k's rows of out are final (the piece a reduce-scatter would send).
 * With ready_events NULL the input is whole: LayerNorm, the QKV+FC1 GEMM and
 * attention run once over all rows, then the output GEMM runs chunk by chunk,
 * recording done_events[k] after each (only the reduce-scatter side is cut).
 * Events are created and owned by the caller.  The result equals
 * pblock_forward's up to floating-point summation order.  1 <= n_chunks <= S
 * (PBLOCK_ERR_ARG otherwise); other rules as pblock_forward.  Per-kernel timing
 * does not cover this entry point. */
int pblock_forward_chunked(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg,
                           void* out, int32_t n_chunks, void* const* ready_events, void* const* done_events,
                           void* stream);

/* The block forward with its output published chunk by chunk from inside one output-GEMM
 * launch, for overlapping the reduce-scatter of tensor/sequence parallelism with the rest of
 * the GEMM (MegaScale guided reading, section 3: the GEMM next to the collective is cut into
 * chunks so that one chunk's communication overlaps the next chunk's computation).  Chunk k
 * holds positions [floor(k*S/n), floor((k+1)*S/n)) of every sequence, n = n_chunks.
 * LayerNorm, the fused QKV+FC1 GEMM and attention run once over every row; the output GEMM
 * (+ residual) then runs its tiles in chunk order (rows of earlier chunks first) as whole
 * waves of 256x256 tiles plus, for a remainder of at most half a wave, 128x256 half-height
 * tiles, with no k-split.  When the last tile touching chunk k has stored its rows, they are
 * written back for the whole device and flags[k] is set to `epoch` (a release store at
 * device scope): a kernel on another stream that reads flags[k] == epoch with acquire
 * semantics (pblock_pack_chunks does) then reads the final rows of chunk k.
 *   flags    [n_chunks] uint32, caller-owned device memory, 4-byte aligned; the library only
 *            stores epoch into it.  Start it at 0 (or any value other than the first epoch).
 *   epoch    nonzero, and different from the previous call's so that a consumer cannot take
 *            an earlier call's flag for this one's (e.g. a step counter).
 * 1 <= n_chunks <= min(S, 64) (PBLOCK_ERR_ARG); bf16 only (PBLOCK_ERR_DTYPE); flags must not
 * overlap out, x or a weight (PBLOCK_ERR_ALIAS).  The handle keeps one tile counter per chunk
 * (zeroed at creation, reset by each chunk's last tile), so a handle must not run two of these
 * calls at once.  The result equals pblock_forward's up to floating-point summation order.
 * Other rules, and per-kernel timing, as pblock_forward. */
int pblock_forward_rowchunks(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg,
                             void* out, int32_t n_chunks, uint32_t* flags, uint32_t epoch, void* stream);

/* The consumer side of pblock_forward_rowchunks (the local half of a reduce-scatter): for each
 * chunk k, waits until flags[k] == epoch, then copies chunk k's rows of out (bf16 [B, S, d])
 * into piece k of send, the rows rank k of a reduce-scatter receives: piece k starts at
 * element B*floor(k*S/n)*d and holds the chunk's rows sequence by sequence.  stamps[k]
 * receives the device real-time clock (100 MHz) at the moment the flag was seen.  Each wait is
 * bounded: after 2 s without the flag, stamps[k] = UINT64_MAX and piece k is not written (the
 * kernel always ends).  Run it on a stream other than the producer's, enqueued before the
 * producer's work, so that it consumes chunks while the output GEMM still runs.
 *   out, send   bf16, B*S*d elements each, 16-byte aligned; flags [n_chunks] uint32, 4-byte
 *               aligned; stamps [n_chunks] uint64, 8-byte aligned; all device memory owned by
 *               the caller, none overlapping another.
 * cfg gives B, S, d (its other fields are validated as usual); bf16 only; n_chunks as
 * pblock_forward_rowchunks.  Enqueued on `stream`, no sync. */
int pblock_pack_chunks(const void* out, const pblock_cfg* cfg, int32_t n_chunks, const uint32_t* flags,
                       uint32_t epoch, void* send, uint64_t* stamps, void* stream);

/* Switches for the choices the pages leave open (MegaScale guided reading: section 2
 * names the block's shape but no positional encoding, bias or normalisation layout;
 * section 4 names GeLU without its form).  All zero = pblock_forward.
 *   gelu_tanh  0: exact erf GeLU;  1: the tanh approximation
 *              z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) (Hendrycks and Gimpel,
 *              "Gaussian Error Linear Units", section 2).
 *   rope       0: no positional encoding;  1: rotary position embedding of q and k
 *              (RoFormer, Su et al., section 3): in each head the pair of features
 *              (2i, 2i+1) of the token at sequence position p (0-based, p = row mod S)
 *              turns by the angle p * rope_base^(-2i/hd); v is not rotated.
 *   rope_base  > 0 and finite when rope = 1 (10000 in RoFormer).
 *   two_ln     0: one LayerNorm feeds both branches;  1: the MLP branch gets its own,
 *              LN2 = (ln2_gamma, ln2_beta) of pblock_variant_weights. */
typedef struct {
  int32_t gelu_tanh;
  int32_t rope;
  float rope_base;
  int32_t two_ln;
} pblock_variant;

/* Extra parameters of the variant forward, in the cfg's dtype, 16-byte aligned device
 * memory owned by the caller; any may be NULL when unused:
 *   b_in       [3*H*hd + ffn]  bias of the input projection, same row order as w_in
 *              (added before the rotary embedding and before GeLU);
 *   b_out      [d]             bias of the output projection (added once: the attention
 *              out-projection and FC2 share one output);
 *   ln2_gamma, ln2_beta  [d]   the MLP branch's LayerNorm (required when two_ln = 1). */
typedef struct {
  const void* b_in;
  const void* b_out;
  const void* ln2_gamma;
  const void* ln2_beta;
} pblock_variant_weights;

/* The parallel block with the switches of `var`:
 *   ua = LN(x),  um = ua or LN2(x)
 *   [q|k|v] = ua W_qkv^T + b_in[:3A];  q, k rotated when rope = 1
 *   f = um W_1^T + b_in[3A:]
 *   y = [Attn_SWA(q, k, v) | GeLU(f)] W_out^T + b_out [+ x]
 * vw may be NULL when no bias and no second LayerNorm is used; var must not be NULL
 * (PBLOCK_ERR_NULL).  Switch values other than 0/1, or a bad rope_base, give
 * PBLOCK_ERR_ARG.  With rope = 1 the cos/sin table for positions [0, B*S of the create
 * cfg) is built in the handle's workspace (fp64, rounded to fp32) on `stream` the first
 * time a base is used, and again whenever the base changes or the call comes on another
 * stream than the one the table was last built on (so a call never relies on work enqueued
 * on a different stream; calls on one handle must still not overlap).  With two_ln = 1 the input
 * GEMM runs as two launches around the second LayerNorm.  Stream, ownership, alignment,
 * aliasing (out must not overlap the extra parameters either) and cfg rules as
 * pblock_forward; per-kernel timing covers it like pblock_forward (a second LayerNorm
 * counts as layernorm, both input GEMMs as gemm_in). */
int pblock_forward_variant(pblock_t h, const void* x, const pblock_weights* w, const pblock_variant_weights* vw,
                           const pblock_cfg* cfg, const pblock_variant* var, void* out, void* stream);

/* ---- Training: forward with saved activations, and the backward pass ----
 * The pages' setting is training; the backward pass mirrors the forward (MegaScale guided
 * reading, section 3: the overlap of the forward pass carries over to the backward pass as
 * well).  Gradients of L = sum(dy * y) by the chain rule through
 * LayerNorm, the input projection, the sliding-window softmax attention (FlashAttention-2
 * style: softmax weights recomputed from the saved log-sum-exp), GeLU and the output
 * projection.  bf16 only (PBLOCK_ERR_DTYPE otherwise), d <= 16384 (PBLOCK_ERR_SHAPE).
 *
 * The training workspace is caller-owned device memory, 256-byte aligned, of at least
 * pblock_train_workspace_bytes(cfg) bytes.  It holds the activations the forward saves
 * (u, q|k|v, [attention | GeLU], the FC1 pre-activation, the per-query log-sum-exp, the
 * LayerNorm row statistics) and the backward's scratch (dy copied into whole 256-row tiles when
 * B*S is not a multiple of 256 -- otherwise dy is read in place --, dO, dz, du, LayerNorm
 * partial sums).  The gradient GEMMs read the weights and the saved activations in
 * place (K-major operands), so nothing is transposed.
 * pblock_forward_train and the pblock_backward that consumes it must get the same cfg, x and
 * weights, and the workspace must not be touched in between. */
typedef struct {
  void* dx;         /* [B, S, d]           dL/dx (includes dy when cfg->add_residual = 1) */
  void* dln_gamma;  /* [d] */
  void* dln_beta;   /* [d] */
  void* dw_in;      /* [3*H*hd + ffn, d]   same layout as w_in */
  void* dw_out;     /* [d, H*hd + ffn]     same layout as w_out */
} pblock_grads;

/* Bytes of training workspace for cfg (host only), or a negative status. */
int64_t pblock_train_workspace_bytes(const pblock_cfg* cfg);

/* pblock_forward's result in out, plus the saved activations in ws (ws_bytes long).  Rules as
 * pblock_forward; out must not overlap ws, and ws must not overlap x or a weight. */
int pblock_forward_train(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg, void* out,
                         void* ws, int64_t ws_bytes, void* stream);

/* Gradients for the output gradient dy [B, S, d] of the forward that pblock_forward_train saved
 * in ws: every pointer of *grads is written (fp32 accumulation, one bf16 rounding of each
 * result; dx, dgamma and dbeta see du in fp32).  The gradients must not overlap each other,
 * x, dy, a weight or ws, and dy must not overlap ws (PBLOCK_ERR_ALIAS); all 16-byte aligned.
 * Enqueued on `stream`. */
int pblock_backward(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg, const void* dy,
                    const pblock_grads* grads, void* ws, int64_t ws_bytes, void* stream);

/* Frees the workspace and the handle.  NULL is a no-op.  The caller must have
 * synchronised every stream the handle was used on. */
int pblock_destroy(pblock_t h);

/* Static description of a status code. */
const char* pblock_strerror(int code);

/* Detail of the most recent failure on the calling thread ("" if none). */
const char* pblock_last_error(void);

/* Device pointers of the handle's intermediates after a forward, for
 * stage-by-stage inspection (owned by the handle, valid until destroy):
 *   u   [B*S, d]            LayerNorm output
 *   qkv [B*S, 3*H*hd]       Q | K | V projections (head-major within each)
 *   ag  [B*S, H*hd + ffn]   attention output (head-major) | GeLU(FC1)
 * Any of the out-pointers may be NULL. */
int pblock_intermediates(pblock_t h, void** u, void** qkv, void** ag);

/* Copies the intermediates of the handle's most recent forward (its B*S rows)
 * into caller-owned device buffers laid out as above, enqueued on `stream`.
 * Any destination may be NULL (skipped).  Returns PBLOCK_ERR_ARG if no forward
 * has run on the handle. */
int pblock_copy_intermediates(pblock_t h, void* u, void* qkv, void* ag, void* stream);

/* Per-kernel timing.  When enabled, pblock_forward, pblock_forward_serial,
 * pblock_forward_variant, pblock_forward_train and pblock_backward record HIP
 * events around each of their launches (or launch groups) on the call's stream;
 * pblock_kernel_times then synchronises on the last recorded event and writes
 * the summed milliseconds per category since the last reset into ms[0 .. n-1]
 * (at most 9), in the order [layernorm, gemm_in, attention, gemm_out,
 * bwd_prep, bwd_gemm_dgrad, bwd_attention, bwd_gemm_wgrad, bwd_layernorm],
 * plus the number of timed calls (the serial form's two LayerNorms count as
 * layernorm, its QKV and FC1 GEMMs as gemm_in, its output-projection and FC2
 * GEMMs as gemm_out; in pblock_forward, when the input GEMM ends in a split-K
 * tail of FC1 columns only, its reduce runs in the attention launch and counts
 * as attention).  Enabling or disabling resets the sums.  n must be >= 4.
 * The events come from a pool of 256 calls per handle: when it is used up, the
 * next timed call first synchronises on the recorded events and folds them
 * into the sums, so with timing on, every 256th call waits for the earlier
 * ones to finish.  Timing off (the default) records nothing and never waits.
 * Not for calls under graph capture. */
int pblock_set_timing(pblock_t h, int enable);
int pblock_kernel_times(pblock_t h, float* ms, int n, int* n_forwards);

/* Sliding-window attention on its own (the same kernel pblock_forward runs).
 *   qkv  [B*S, ld_qkv]: Q at columns [0, H*hd), K at [H*hd, 2*H*hd),
 *        V at [2*H*hd, 3*H*hd); ld_qkv >= 3*H*hd, a multiple of 8.
 *   o    [B*S, ld_o]: head h written to columns [h*hd, (h+1)*hd); ld_o >= H*hd,
 *        a multiple of 8.
 * Both strides at most 2^24 elements (PBLOCK_ERR_SHAPE otherwise: the kernels address
 * a tile of 64 rows with 32-bit offsets).  W >= S is full causal attention.
 * dtype as above; hd in {64, 128}.  Enqueued on `stream`, no sync. */
int pblock_swa_attention(const void* qkv, int64_t ld_qkv, void* o, int64_t ld_o, int32_t B, int32_t S,
                         int32_t H, int32_t hd, int32_t W, int32_t dtype, void* stream);

/* The GeLU forms the kernels' epilogues evaluate, on their own (an inspection entry: the
 * block's GeLU is exact erf GeLU per the readings above, and these are the device
 * approximations of it that the tests hold to their published error bounds):
 *   PBLOCK_ACT_GELU_ERF_F32   fp32 path: z Phi(z) with erfc from Numerical Recipes' erfcc
 *                             (2nd ed., section 6.2; fractional error of erfc < 1.2e-7);
 *   PBLOCK_ACT_GELU_ERF_BF16  bf16 path: z Phi(z) with erfc from Abramowitz and Stegun 7.1.26
 *                             (absolute error of erf < 1.5e-7);
 *   PBLOCK_ACT_GELU_TANH      the tanh form of the variant switch (Hendrycks and Gimpel);
 *   PBLOCK_ACT_GELU_ERF_GRAD  the backward pass's Phi(z) + z phi(z), A&S 7.1.26 for Phi.
 * z and out: n fp32 values each, device memory owned by the caller; out may equal z (in
 * place) but must not overlap it otherwise (PBLOCK_ERR_ALIAS).  0 <= n <= 2^40
 * (PBLOCK_ERR_SHAPE); an unknown form gives PBLOCK_ERR_ARG.  Enqueued on `stream`, no
 * sync. */
enum {
  PBLOCK_ACT_GELU_ERF_F32 = 0,
  PBLOCK_ACT_GELU_ERF_BF16 = 1,
  PBLOCK_ACT_GELU_TANH = 2,
  PBLOCK_ACT_GELU_ERF_GRAD = 3
};
int pblock_activation(const float* z, float* out, int64_t n, int32_t form, void* stream);

/* Measurement aid, not part of the block: a register-only loop of bf16 MFMAs on
 * `workgroups` workgroups of 4 wavefronts, each wavefront issuing independent
 * MFMAs worth 16 * 32768 FLOP per iteration, `iterations` times; it performs
 * workgroups * 4 * iterations * 16 * 32768 FLOP and writes one float per thread
 * to sink (workgroups * 256 floats, caller owned, device memory).  form picks
 * the instruction: PBLOCK_MFMA_16X16X32 (v_mfma_f32_16x16x32_bf16, the GEMMs'
 * instruction; 32 per iteration) or PBLOCK_MFMA_32X32X16
 * (v_mfma_f32_32x32x16_bf16; 16 per iteration).  Timing it gives the MFMA rate
 * the chip sustains at its present clock and power state, the ceiling the GEMMs
 * are compared with.  workgroups >= 1, iterations >= 1, an unknown form is
 * PBLOCK_ERR_ARG.  Enqueued on `stream`, no sync. */
enum {
  PBLOCK_MFMA_16X16X32 = 0,
  PBLOCK_MFMA_32X32X16 = 1
};
int pblock_mfma_loop(int32_t workgroups, int32_t iterations, int32_t form, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PBLOCK_H */

/*
 * gsa.h — C ABI of libgsa: SDPA-output ("G1") gated attention on AMD MI355X (gfx950).
 *
 * The operation, as the "GatedAttention [2025]" page states it:
 *   Y  = softmax(Q·Kᵀ / √d_k + causal mask) · V            (§1.2.1 SDPA equation,
 *                                                            causal per §1.4.1 eq.)
 *   Y' = Y ⊙ σ(X·W_θ),  σ(x) = 1 / (1 + e^{-x})            (§1.2.2 gating equation and
 *                                                            default activation)
 * applied per query head before the heads are concatenated (G1 position:
 * "10 · 门控" page, §3.2 position table).  The gate is elementwise (one score per
 * head and head dimension, shape n×q×d_k) or headwise (one scalar per head and
 * token, shape n×q) ("GatedAttention [2025]" §1.2.2, granularity (2)).  Key/value
 * heads are shared by groups of query heads (GQA, "GatedAttention [2025]" §1.3.1):
 * query head h reads key/value head h / (Hq / Hkv).
 *
 * Conventions for every entry point:
 *  - Pointers X, W, G, Q, K, V, Y, workspace are DEVICE pointers owned by the
 *    caller, to contiguous row-major tensors, each 16-byte aligned.  The library
 *    allocates no device memory and keeps no per-call state (gsa_decode_noalloc
 *    keeps its split partials in a fixed device array inside the library;
 *    gsa_backward creates one side stream and two events per device on its
 *    first call there, kept until the process ends).
 *  - dtype (gsa_dtype) is the element type of X, W, Q, K, V and Y'.  G is always
 *    float32.  Arithmetic is float32 (bf16 inputs multiply exactly into float32
 *    accumulators on the matrix cores).
 *  - Calls only ENQUEUE work on `stream` (a hipStream_t; NULL = the default
 *    stream) and return; results are visible after the caller synchronises.
 *  - Errors are returned as gsa_status; nothing aborts and no exception crosses
 *    the ABI.  All argument checks run before any HIP call, so they also work on
 *    a host without a GPU (which then gets GSA_ERR_NO_DEVICE).  A per-thread
 *    message describing the last failure is available from
 *    gsa_last_error_message().
 *  - Calls are thread-safe; concurrent calls on different streams are allowed
 *    (except gsa_decode_noalloc, whose calls on one GPU share a device scratch).
 */
#ifndef GSA_H
#define GSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gsa_status {
  GSA_OK = 0,
  GSA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, Hq % Hkv != 0, mode/G mismatch */
  GSA_ERR_UNSUPPORTED = 2,   /* a head dim, dtype, mode or device the library does not handle */
  GSA_ERR_MISALIGNED = 3,    /* a pointer not 16-byte aligned */
  GSA_ERR_WORKSPACE = 4,     /* decode or backward workspace missing or smaller than required */
  GSA_ERR_NO_DEVICE = 5,     /* no HIP device visible to the calling thread */
  GSA_ERR_HIP = 6            /* a HIP runtime or kernel-launch error */
} gsa_status;

typedef enum gsa_dtype { GSA_FP32 = 0, GSA_BF16 = 1 } gsa_dtype;

typedef enum gsa_gate_mode {
  GSA_GATE_NONE = 0,         /* plain causal SDPA, no gate (G must be NULL) */
  GSA_GATE_ELEMENTWISE = 1,  /* G is [rows, Hq*D]; column h*D + d gates head h, dim d */
  GSA_GATE_HEADWISE = 2,     /* G is [rows, Hq];   column h gates all of head h       */
  GSA_GATE_SHARED = 3        /* G is [rows, D];    column d gates dim d of every head
                                (gsa_forward_variant and gsa_decode_variant only; the
                                head-shared score is gsa_gate_head_mean's output) */
} gsa_gate_mode;

/* Gate activation applied by gsa_gate_logits ("GatedAttention [2025]" §1.2.2
   item (5); NS-sigmoid from §1.4.2 (iv)). */
typedef enum gsa_activation {
  GSA_ACT_IDENTITY = 0,      /* the raw logits Z = X·W_θ */
  GSA_ACT_SIGMOID = 1,       /* σ(Z) = 1 / (1 + e^{-Z}) (the default) */
  GSA_ACT_NS_SIGMOID = 2,    /* 0.5 + 0.5·σ(Z), range [0.5, 1] */
  GSA_ACT_SILU = 3           /* Z·σ(Z) */
} gsa_activation;

/* How gsa_forward_variant and gsa_decode_variant apply the gate ("GatedAttention [2025]" §1.2.2 item (4)). */
typedef enum gsa_combine { GSA_COMBINE_MUL = 0, GSA_COMBINE_ADD = 1 } gsa_combine;

/* Optional per-head normalisation of the SDPA output before the gate
   ("GatedAttention [2025]" §1.4.1, Table 3 row 5). */
typedef enum gsa_norm { GSA_NORM_NONE = 0, GSA_NORM_RMS = 1 } gsa_norm;

/* Library version, encoded as major*10000 + minor*100 + patch. */
int gsa_version(void);

/* Static, human-readable name of a status code. */
const char* gsa_status_string(int status);

/* Detail of the most recent failure on the calling thread ("" if none). */
const char* gsa_last_error_message(void);

/*
 * Gate projection with fused activation: G = act(X·W_θ) ("GatedAttention [2025]"
 * §1.2.2 gating equation; no bias, as the §3.2 snippet on "10 · 门控" has
 * bias=False).
 *   X : [M, d_model] of dtype   (M = B*S token rows, the hidden states after pre-norm)
 *   W : [d_model, N] of dtype   (N = Hq*D elementwise, Hq headwise, D shared)
 *   G : [M, N] float32 output
 *   activation: a gsa_activation; GSA_ACT_SIGMOID (1) stores σ(Z), the G1
 *     gate; GSA_ACT_IDENTITY (0) stores the raw logits Z = X·W_θ.
 * Requires d_model % 8 == 0.  Sizes must be positive.
 */
gsa_status gsa_gate_logits(const void* X, const void* W, float* G,
                           int64_t M, int64_t d_model, int64_t N,
                           int dtype, int activation, void* stream);

/*
 * Workspace bytes gsa_gate_logits_ws needs for these sizes: nonzero for the
 * shapes it splits over K (bf16, at most 128 rows, N a multiple of 8 and at
 * least 64, fewer than 256 output tiles of 64 × 64: e.g. the gate of one
 * decode step, M = batch), 0 for every other shape.
 */
size_t gsa_gate_logits_workspace_bytes(int64_t M, int64_t d_model, int64_t N, int dtype);

/*
 * gsa_gate_logits with a workspace, for few token rows (decode).  The gate
 * scores are the same function ("GatedAttention [2025]" §1.2.2 gating
 * equation), computed by splitting d_model s ways: each part's partial logits
 * go to the workspace (float32 [s, M, N]) and are added in part order before the
 * activation, so the result is deterministic.  Arguments as gsa_gate_logits,
 * plus the workspace (device memory of at least
 * gsa_gate_logits_workspace_bytes(M, d_model, N, dtype) bytes, 16-byte
 * aligned, contents on entry irrelevant).  When that size is 0 this call is
 * gsa_gate_logits and the workspace may be NULL.  Errors: those of
 * gsa_gate_logits, and a missing or short workspace -> GSA_ERR_WORKSPACE.
 */
gsa_status gsa_gate_logits_ws(const void* X, const void* W, float* G, int64_t M, int64_t d_model, int64_t N,
                              int dtype, int activation, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal gated SDPA forward (prefill): for every batch b, query head h and
 * query row i,  Y'[b,i,h,:] = (Σ_{j<=i} P_ij V[b,j,h/(Hq/Hkv),:]) ⊙ gate,
 * P_i = softmax_j(Q[b,i,h,:]·K[b,j,c,:] / √D) over j <= i (self included).
 *   Q : [B, S, Hq, D]   K, V : [B, S, Hkv, D]   (dtype)
 *   G : [B*S, Hq*D] (ELEMENTWISE) or [B*S, Hq] (HEADWISE) float32 scores from
 *       gsa_gate_logits; must be NULL iff mode == GSA_GATE_NONE
 *   Y : [B, S, Hq, D] output (dtype); the ungated SDPA output is never stored.
 * Requires D in {64, 128} and Hq % Hkv == 0.
 */
gsa_status gsa_forward(const void* Q, const void* K, const void* V, const float* G, void* Y,
                       int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                       int mode, int dtype, void* stream);

/*
 * gsa_forward that also writes, for the backward, each row's log-sum-exp of
 * its scaled scores over the visible keys ("GatedAttention [2025]" §1.2.1
 * SDPA equation, causal per §1.4.1):
 *   LSE : [B, Hq, S] float32 output, LSE[b,h,i] = ln Σ_{j<=i} exp(Q[b,i,h,:]·K[b,j,c,:] / √D)
 *         (4-byte aligned).  The other arguments are gsa_forward's.
 */
gsa_status gsa_forward_lse(const void* Q, const void* K, const void* V, const float* G, void* Y,
                           float* LSE, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                           int mode, int dtype, void* stream);

/*
 * Split count gsa_decode will use for these sizes: num_splits itself if > 0,
 * otherwise the automatic choice (about one split workgroup per CU when 4
 * divides Hkv, about four otherwise; at least 256 keys per split), rounded so
 * that every split gets keys.  Returns 0 for invalid sizes.
 */
int64_t gsa_decode_num_splits(int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D,
                              int num_splits);

/* Workspace bytes gsa_decode needs for these sizes (0 for invalid sizes). */
size_t gsa_decode_workspace_bytes(int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D,
                                  int num_splits);

/*
 * One decode step: a single query token per batch against a contiguous KV
 * cache of length L that already holds that token, so the query attends to
 * all L keys (the KV cache of the "GatedAttention [2025]" §1.3.1 GQA
 * explainer).  Same definition as gsa_forward with one query row per batch
 * sitting at position L-1.
 *   Q  : [B, 1, Hq, D]    Kc, Vc : [B, L, Hkv, D]   (dtype)
 *   G  : [B, Hq*D] or [B, Hq] float32 (see gsa_forward), NULL iff mode NONE
 *   Y  : [B, 1, Hq, D] output (dtype)
 *   num_splits: 0 = automatic; otherwise the number of chunks the cache is cut
 *     into along L (each chunk's partial max, sum and weighted values are
 *     merged exactly at the end).
 *   workspace: device scratch of at least gsa_decode_workspace_bytes(...) bytes
 *     (may be NULL when that is 0).  Its contents on entry do not matter.
 * Requires D in {64, 128} and Hq % Hkv == 0.
 */
gsa_status gsa_decode(const void* Q, const void* Kc, const void* Vc, const float* G, void* Y,
                      int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D,
                      int mode, int dtype, int num_splits,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device scratch gsa_decode_noalloc uses for its split partials:
   8 MiB per GPU, enough for B·Hq·nsplit·(D+4) float32 values up to 2097152
   (e.g. 64 batches × 32 query heads × 7 splits at D = 128). */
#define GSA_NOALLOC_SCRATCH_BYTES (8u << 20)

/* GSA_NOALLOC_SCRATCH_BYTES, as the library was built with it. */
size_t gsa_noalloc_scratch_bytes(void);

/*
 * gsa_decode for callers that cannot allocate memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It takes no
 * workspace and allocates nothing (no hipMalloc, hipFree or allocating library
 * call).  The split partials go to a device array inside the library, one per
 * GPU, of GSA_NOALLOC_SCRATCH_BYTES; each GPU holds it until the process ends.
 * Same arguments, results and kernels as gsa_decode without the workspace
 * pair; the caller still allocates Q, Kc, Vc, G and Y.
 * Errors: as gsa_decode; sizes whose partials
 * (gsa_decode_workspace_bytes(B, L, Hq, Hkv, D, num_splits)) exceed
 * GSA_NOALLOC_SCRATCH_BYTES -> GSA_ERR_WORKSPACE (use fewer splits, or
 * gsa_decode).  float32 decode needs no scratch.
 * Concurrency: every call on one GPU shares that GPU's scratch and leaves its
 * partials there; two calls that overlap in time on one GPU (different
 * streams, or threads without ordering) race and may return wrong results.
 * Calls ordered on one stream are safe.
 */
gsa_status gsa_decode_noalloc(const void* Q, const void* Kc, const void* Vc, const float* G, void* Y,
                              int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D,
                              int mode, int dtype, int num_splits, void* stream);

/* Workspace bytes gsa_gated_decode needs for these sizes (0 for invalid sizes). */
size_t gsa_gated_decode_workspace_bytes(int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int64_t d_model,
                                        int mode, int dtype, int num_splits);

/*
 * The whole decode step in one call: the gate scores of the B new tokens,
 * σ(X·W_θ) ("GatedAttention [2025]" §1.2.2 gating equation), and the gated
 * decode of gsa_decode (the KV cache of §1.3.1), i.e. gsa_gate_logits then
 * gsa_decode.
 *   X : [B, d_model] (the new tokens' hidden states), W : [d_model, N] (dtype),
 *       N = Hq·D (ELEMENTWISE) or Hq (HEADWISE); both NULL for GSA_GATE_NONE.
 *   Q, Kc, Vc, Y, num_splits: as gsa_decode.
 *   workspace: at least gsa_gated_decode_workspace_bytes(...) bytes, 16-byte
 *     aligned, contents on entry irrelevant.
 * It computes what gsa_gate_logits_ws (σ, into the workspace; the split-K path
 * for few rows) followed by gsa_decode computes, bit for bit; with bf16, the
 * elementwise gate and the split-K path the decode merge adds the gate's
 * partial logits itself (in part order) and applies σ, one launch fewer.
 * Errors: those of gsa_gate_logits and gsa_decode; X and W given without a
 * gate (or missing with one) -> GSA_ERR_INVALID_ARG.
 */
gsa_status gsa_gated_decode(const void* X, const void* W, const void* Q, const void* Kc, const void* Vc, void* Y,
                            int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int64_t d_model, int mode,
                            int dtype, int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes gsa_backward needs for these sizes (0 for invalid sizes;
 * d_model is ignored for GSA_GATE_NONE).
 */
size_t gsa_backward_workspace_bytes(int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                                    int64_t d_model, int mode);

/*
 * Backward of the gated prefill path for an upstream gradient dY of Y'.  The
 * gradients are the chain rule on the forward: through the product
 * Y' = Y ⊙ g to the SDPA output and to the gate, through σ (σ' = σ(1 − σ)) to
 * the gate scores Z = X·W_θ and through the projection to X and W_θ (the
 * "Gated Attention如何用1%的参数量…" page, §2.2 gradient analysis), and
 * through the causal softmax attention ("GatedAttention [2025]" §1.2.1 SDPA
 * equation, causal per §1.4.1) to Q, K and V, with K and V gradients summed
 * over each GQA group (§1.3.1).
 *   X  : [B*S, d_model] bf16   W : [d_model, N] bf16   G : [B*S, N] float32,
 *        the σ(X·W_θ) the forward used (gsa_gate_logits output);
 *        N = Hq*D (ELEMENTWISE) or Hq (HEADWISE).  All three NULL iff mode is
 *        GSA_GATE_NONE.
 *   Q, K, V, Y, LSE : the forward's inputs and its outputs from gsa_forward_lse
 *        (Y is the gated output Y').
 *   dY : [B, S, Hq, D] bf16 upstream gradient.
 *   outputs (overwritten, never accumulated into):
 *        dQ [B, S, Hq, D], dK and dV [B, S, Hkv, D] (bf16);
 *        dX [B*S, d_model] bf16, the gate projection's contribution to the
 *        gradient of X (a caller that also projects Q, K, V from X adds its own);
 *        dW [d_model, N] float32.  dX and dW are NULL iff mode is GSA_GATE_NONE.
 *   workspace: device scratch of at least gsa_backward_workspace_bytes(...)
 *        bytes, 16-byte aligned; contents on entry do not matter.
 * Requires dtype GSA_BF16, D in {64, 128}, Hq % Hkv == 0, and with a gate
 * d_model % 8 == 0 and N % 8 == 0.  The results are deterministic (no atomics).
 * Stream order: the call's work starts after earlier work on `stream`, and
 * later work on `stream` starts after all of it.  Inside that, when the
 * key/value grid is not cut into GQA slices, the dQ and dX kernels run on a
 * library-owned side stream of the current device (created on its first such
 * call, default priority) beside the dK/dV and dW kernels, forked from and
 * joined back to `stream` with events; while `stream` is being captured into
 * a graph every kernel goes on `stream` in sequence instead.
 */
gsa_status gsa_backward(const void* X, const void* W, const float* G, const void* Q, const void* K,
                        const void* V, const void* Y, const float* LSE, const void* dY, void* dX,
                        float* dW, void* dQ, void* dK, void* dV, int64_t B, int64_t S, int64_t Hq,
                        int64_t Hkv, int64_t D, int64_t d_model, int mode, int dtype, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * gsa_forward for the other points of the gate design space ("GatedAttention
 * [2025]" §1.2.2 items (3)-(5) and §1.4.1):
 *   Y'[b,i,h,:] = combine(norm(Y[b,i,h,:]), gate)
 * with Y the causal SDPA output (gsa_forward's definition), norm the identity
 * or a per-head RMSNorm over the D values (unit weight, ε = 1e-6), and
 * combine Y ⊙ g (GSA_COMBINE_MUL) or Y + g (GSA_COMBINE_ADD).  The gate values
 * g are G as given (already activated by gsa_gate_logits):
 *   layout GSA_GATE_ELEMENTWISE: G [B*S, Hq*D], column h*D + d
 *          GSA_GATE_HEADWISE:    G [B*S, Hq],   column h
 *          GSA_GATE_SHARED:      G [B*S, D],    column d for every head
 *          GSA_GATE_NONE:        G NULL: Y' = norm(Y)
 *   LSE: optional ([B, Hq, S] float32, as gsa_forward_lse; NULL skips it).
 * Other arguments and rules as gsa_forward.
 */
gsa_status gsa_forward_variant(const void* Q, const void* K, const void* V, const float* G, void* Y,
                               float* LSE, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                               int layout, int combine, int norm, int dtype, void* stream);

/*
 * gsa_decode with the design-space epilogue of gsa_forward_variant ("GatedAttention
 * [2025]" §1.2.2 items (3)-(5) and §1.4.1, on the KV cache of §1.3.1), applied at
 * the merge of the split partial results:
 *   Y'[b,0,h,:] = combine(norm(Y[b,0,h,:]), gate)
 * with Y gsa_decode's ungated output (one query per batch against all L
 * cached keys).  layout, combine and norm as gsa_forward_variant, with the gate
 * rows being the B decode tokens: G [B, Hq*D], [B, Hq] or [B, D] (already
 * activated), NULL for GSA_GATE_NONE.  The workspace, num_splits and every
 * other argument and rule as gsa_decode (the float32 path needs no workspace).
 * Errors: an unknown layout, combine or norm, or G given with GSA_GATE_NONE (or
 * missing with a gate) -> GSA_ERR_INVALID_ARG; the rest as gsa_decode.
 */
gsa_status gsa_decode_variant(const void* Q, const void* Kc, const void* Vc, const float* G, void* Y, int64_t B,
                              int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int layout, int combine, int norm,
                              int dtype, int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Head-shared gate scores ("GatedAttention [2025]" §1.2.2 item (3)b; the §1.3.2
 * Table 1 discussion, observation (ii), averages the n×q×d_k gating scores
 * over the q query heads into one n×d_k score; "10 · 门控" §3.2 Table 1 row 12):
 *   Gs[m, d] = (1/Hq) · Σ_{h<Hq} G[m, h·D + d]     (heads summed in order, float32)
 *   G  : [M, Hq·D] float32, the activated scores gsa_gate_logits wrote for a
 *        q·d_k-wide W_θ (the mean is taken after the activation)
 *   Gs : [M, D] float32 output, the gate of layout GSA_GATE_SHARED for
 *        gsa_forward_variant and gsa_decode_variant.  G and Gs may not overlap.
 * Requires D % 4 == 0, Hq and D at most 4096; both pointers 16-byte aligned.
 */
gsa_status gsa_gate_head_mean(const float* G, float* Gs, int64_t M, int64_t Hq, int64_t D, void* stream);

/*
 * Causal SDPA with G2 value gating ("GatedAttention [2025]" §1.2.2, position
 * G2: the gate on the value map; §1.3.2 Table 1 rows 6 and 11):
 *   Y[b,i,h,:] = Σ_{j<=i} P_ij · V'[b,j,c,:],   V' = V ⊙ g,  c = h / (Hq/Hkv)
 * with P the causal softmax of gsa_forward and g = σ(X·W_v) per key/value head
 * and dim (GSA_GATE_ELEMENTWISE: Gv [B·S, Hkv·D], column c·D + d) or per
 * key/value head (GSA_GATE_HEADWISE: Gv [B·S, Hkv], column c), float32 from
 * gsa_gate_logits.  Each product V·g is rounded once to the value dtype,
 * inside the kernel as the value tiles are staged (V' never reaches HBM); there
 * is no output gate.
 *   Q, K, V, Y and the rules as gsa_forward; LSE optional (as gsa_forward_lse,
 *   NULL skips it).
 */
gsa_status gsa_forward_value_gated(const void* Q, const void* K, const void* V, const float* Gv, void* Y,
                                   float* LSE, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                                   int layout, int dtype, void* stream);

/*
 * G2 value gating as a separate pass ("GatedAttention [2025]" §1.2.2, position
 * G2): the gate scales the value map before attention,
 *   Vout[t, c, d] = V[t, c, d] · G[t, c*D + d]   (GSA_GATE_ELEMENTWISE)
 *   Vout[t, c, d] = V[t, c, d] · G[t, c]         (GSA_GATE_HEADWISE)
 * for token rows t < B*S and key/value heads c; gsa_forward with mode
 * GSA_GATE_NONE on Vout then gives the G2-gated attention
 * (gsa_forward_value_gated does both in one pass, without Vout).
 *   V, Vout : [B, S, Hkv, D] of dtype (may not overlap)   G : float32 from
 *   gsa_gate_logits (σ of X·W_v).  D in {64, 128}; pointers 16-byte aligned.
 */
gsa_status gsa_value_gate(const void* V, const float* G, void* Vout, int64_t B, int64_t S, int64_t Hkv,
                          int64_t D, int layout, int dtype, void* stream);

/*
 * Fused input projection: Q, K, V and the gate from one pass over X,
 *   [Q | K | V | Z] = X · [W_Q | W_K | W_V | W_θ],   G = σ(Z)
 * (the QKV projections of "GatedAttention [2025]" §1.2.1 and the gate scores of
 * §1.2.2, which read the same X).  Head h of Q is columns h·D .. h·D+D−1 (so Q
 * is [M, Hq·D] = [B, S, Hq, D]); likewise K and V with the Hkv key/value heads.
 *   X : [M, d_model] bf16
 *   W : [d_model, Hq·D + 2·Hkv·D + n_gate] bf16, the four weights side by side
 *   Q : [M, Hq·D], K and V : [M, Hkv·D] bf16 outputs (rounded once)
 *   G : [M, n_gate] float32 output σ(Z) (n_gate = Hq·D elementwise, Hq
 *       headwise); NULL exactly when n_gate is 0 (no gate).
 * Requires dtype GSA_BF16, d_model and every output width multiples of 8, and
 * X and W below 2 GiB.
 */
gsa_status gsa_project_qkvg(const void* X, const void* W, void* Q, void* K, void* V, float* G, int64_t M,
                            int64_t d_model, int64_t Hq, int64_t Hkv, int64_t D, int64_t n_gate, int dtype,
                            void* stream);

/*
 * First-token attention share ("GatedAttention [2025]" §1.4.3, the F-Attn
 * column of Table 4; "10 · 门控" §3.4): the causal softmax probability each
 * query row gives token 0,
 *   F[b,h,i] = exp(Q[b,i,h,:]·K[b,0,c,:] / √D − LSE[b,h,i]),  c = h / (Hq/Hkv),
 * from the LSE a gsa_forward_lse call on the same Q and K wrote.
 *   Q : [B, S, Hq, D], K : [B, S, Hkv, D] (dtype; only key row 0 is read)
 *   LSE : [B, Hq, S] float32 (input)    F : [B, Hq, S] float32 (output)
 *   head_mean : NULL, or Hq + 1 floats (output): the mean of F over batches and
 *     rows for each head, then the mean of those Hq values.
 * Same shape rules as gsa_forward; LSE, F and head_mean 4-byte aligned.
 * Deterministic (fixed-order sums).
 */
gsa_status gsa_first_token_attention(const void* Q, const void* K, const float* LSE, float* F,
                                     float* head_mean, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                     int64_t D, int dtype, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif /* GSA_H */

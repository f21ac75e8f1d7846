/*
 * libmhc -- the mHC (Manifold-Constrained Hyper-Connections) layer forward on
 * AMD Instinct MI355X (gfx950), as a plain C ABI.
 *
 * The layer widens the residual state of every token to n streams of d
 * values, X (n x d), and wraps a sublayer F:
 *     x_hat = RMSNorm(vec(X))                      (over all n*d values)
 *     logits = alpha_blk * (x_hat . phi) + bias    (phi: n*d x (n*n + 2n))
 *     H_pre = sigmoid(l_pre), H_post = 2 sigmoid(l_post),
 *     H_res = Sinkhorn-Knopp(exp(Mat(l_res)))      (t_max passes: columns, then rows)
 *     h = H_pre . X          -> F -> Y = F(h)
 *     X' = H_res X + H_post^T Y
 * Sources: V. Dubrov, "DeepSeek mHC: Manifold-Constrained Hyper-Connections"
 * (slavadubrov.com), sections "Kernmechanismen" (Eq. 3), "Sinkhorn-Knopp-
 * projectie", "Details van de parameterisatie"; "mHC" study notes on
 * DeepSeek-V4 (t6page.pages.dev), equations dsv4-mhc-rmsnorm,
 * dsv4-mhc-a-tilde/b-tilde/c-tilde, dsv4-mhc-sinkhorn-init, dsv4-mhc-sinkhorn,
 * dsv4-mhc-gate, dsv4-mhc-hc-update, table tbl-dsv4-mhc-kernels.
 *
 * Conventions shared by every entry point
 *  - Pointers to tensors are DEVICE pointers (hipMalloc / torch CUDA memory);
 *    the mhc_params pointer is a HOST pointer.  The caller owns every buffer;
 *    the library never allocates or frees device memory.
 *  - Layouts are dense row-major:
 *      X, X_out  [T, n, d]   stream i of token t at X + (t*n + i)*d
 *      h, Y      [T, d]
 *      phi       [n*d, m]    fp32, m = n*n + 2n, row k multiplies vec(X)[k]
 *                            (vec stacks the streams: k = i*d + j); columns
 *                            pre (n) | res (n*n, row-major, row = output
 *                            stream) | post (n)
 *      bias      [m]         fp32, same column order as phi
 *      H         [T, m]      fp32 maps, same column order: H_pre | H_res | H_post
 *    The state dtype (X, h, Y, X_out) is MHC_FP32 or MHC_BF16; phi, bias and
 *    H are always fp32, arithmetic is fp32 on the device.
 *  - stream is a hipStream_t passed as void*; NULL is the default stream.
 *    Work is enqueued asynchronously on it; calls return before it runs.
 *  - Errors: arguments are checked on the host before anything is enqueued
 *    and a non-zero mhc_status is returned without touching device memory.
 *    A failed launch returns MHC_ERR_HIP.  Faults during execution surface at
 *    the caller's next synchronisation.  NaN and Inf propagate; they are not
 *    checked.  No entry point throws or aborts.
 *  - Device support: n in {1, 2, 4, 8} (the backward: n in {1, 2, 4}); d a
 *    multiple of 8; tensor base pointers 16-byte aligned.  T = 0 is a valid
 *    no-op.
 *  - Results are bitwise reproducible for fixed inputs and shapes: every
 *    reduction runs in a fixed order and no floating-point atomics are used.
 *  - The library keeps no mutable state between calls apart from a cache of
 *    device attributes; calls from several host threads are safe.  What
 *    carries over from one call to the next lives in caller-owned memory:
 *    mhc_pre's workspace header (see mhc_pre_ex).
 *  - Scratch memory: entry points that need it take a workspace whose size
 *    mhc_workspace_size(p, op) returns (0: none needed).
 */
#ifndef MHC_H
#define MHC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MHC_ABI_VERSION 8

typedef enum mhc_status {
  MHC_OK = 0,
  MHC_ERR_NULL = 1,         /* a required pointer is NULL */
  MHC_ERR_SHAPE = 2,        /* T, n, d, L, t_max or eps out of range, or sizes overflow */
  MHC_ERR_DTYPE = 3,        /* unknown state dtype */
  MHC_ERR_ALIGN = 4,        /* a tensor base pointer is not 16-byte aligned */
  MHC_ERR_UNSUPPORTED = 5,  /* valid for the method but not built for the device (n = 3, d % 8 != 0) */
  MHC_ERR_ALIAS = 6,        /* an output overlaps an input other than the permitted exact alias */
  MHC_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than the entry point's size query */
  MHC_ERR_HIP = 8,          /* a HIP runtime call or a kernel launch failed */
  MHC_ERR_SCRATCH = 9       /* the call needs more scratch than mhc_pre_noalloc's static buffer holds */
} mhc_status;

typedef enum mhc_dtype { MHC_FP32 = 0, MHC_BF16 = 1 } mhc_dtype;

/* Shape and hyperparameters of one mHC layer.  t_max = 20 and alpha = 0.01 at
 * initialisation are the pages' values ("mHC" notes, key hyperparameters);
 * eps sits under the square root of the RMSNorm (the pages give 1e-20, the
 * workloads here use 1e-6). */
typedef struct mhc_params {
  int64_t T;          /* tokens, >= 0 */
  int32_t n;          /* streams: 1, 2, 4 or 8 (backward: 1, 2 or 4) */
  int32_t d;          /* values per stream, multiple of 8 */
  int32_t dtype;      /* mhc_dtype of X, h, Y, X_out */
  int32_t t_max;      /* Sinkhorn-Knopp passes, 0 .. 1000 */
  float eps;          /* RMSNorm epsilon, finite, >= 0 */
  float alpha_pre;    /* gate scalars of the three maps */
  float alpha_res;
  float alpha_post;
  int32_t maps;       /* MHC_MAPS_MHC (0): the mHC maps; MHC_MAPS_HC (1): the
                         unconstrained HC form, for contrast (see below) */
} mhc_params;

/* The form of the maps.  MHC_MAPS_MHC is the method: H_pre = sigmoid(l_pre),
 * H_post = 2 sigmoid(l_post), H_res = Sinkhorn(exp(Mat(l_res))) with
 * l = alpha_blk z + bias.  MHC_MAPS_HC is the form mHC constrains (Dubrov,
 * "Kernmechanismen": a static bias plus an input-dependent term through
 * tanh, any sign), read as H = bias + alpha_blk * tanh(z) for all three maps,
 * no Sinkhorn.  The same z = x_hat . phi feeds both.  mhc_pre, mhc_pre_ex
 * (either form) and mhc_post_pre accept both; mhc_pre_bwd takes the mHC form
 * only (MHC_ERR_UNSUPPORTED otherwise). */
#define MHC_MAPS_MHC 0
#define MHC_MAPS_HC 1

/* ---- mhc_pre: RMSNorm + projection + gates + Sinkhorn + aggregation --------
 * Computes, per token, the maps H (fp32 [T, m]) and the sublayer input
 * h = H_pre . X ([T, d], state dtype) from X ([T, n, d]).  Defined by the
 * "mHC" notes, eqs. dsv4-mhc-rmsnorm, a/b/c-tilde, sinkhorn-init, sinkhorn,
 * gate; aggregation by Dubrov, "Kernmechanismen", Eq. 3 (the F(H_pre x_l)
 * term).  The RMS division is applied after the projection,
 * (x . phi) / r, which is the same value in exact arithmetic (the pages'
 * "reorder RMSNorm" fusion).
 *   X         in   [T, n, d] state dtype
 *   phi       in   [n*d, m] fp32
 *   bias      in   [m] fp32
 *   h         out  [T, d] state dtype; must not overlap any input
 *   H         out  [T, m] fp32; must not overlap any input or h
 *   workspace in/out scratch of at least mhc_pre_workspace_size(p) bytes,
 *             16-byte aligned, overlapping nothing else.  Its first 256 bytes
 *             (the header) carry the single pass's sequence number and error
 *             word from one call to the next; any initial contents work
 *             (zeroed memory included), and the library never needs it
 *             cleared.  The rest is scratch, unspecified on return.  Calls
 *             that share a workspace must not overlap in time (one stream, or
 *             ordered streams).  May be NULL only if the size query returns 0.
 * Returns MHC_ERR_WORKSPACE when workspace_bytes is too small. */
mhc_status mhc_pre(const mhc_params* p, const void* X, const float* phi, const float* bias,
                   void* h, float* H, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device scratch mhc_pre needs for these parameters (0 if p is
 * invalid).  The amount depends only on T, n and d and covers both forms of
 * mhc_pre_ex. */
size_t mhc_pre_workspace_size(const mhc_params* p);

/* ---- mhc_pre_ex: mhc_pre with a choice of algorithm -------------------------
 * Same computation, arguments and results as mhc_pre, which is
 * mhc_pre_ex(..., MHC_PRE_AUTO, NULL, stream).  The two forms differ only in
 * how many times they read X from HBM:
 *   MHC_PRE_TWO_PASS  a split-K projection pass, then a maps + aggregation
 *                     pass that reads X again; any valid shape.
 *   MHC_PRE_ONE_PASS  bf16 state, n <= 4, 1793 <= d <= 4096 and at least one
 *                     16-token tile per team: teams of S = ceil(d / 256)
 *                     workgroups (one per compute unit, all on one XCD)
 *                     split d, exchange per-token sums through the XCD's L2
 *                     and keep their slice of X in registers until H_pre is
 *                     known, so X is read once.  The team's members wait for
 *                     each other (bounded waits), so they must be resident
 *                     together, which an idle device gives an ordinary
 *                     launch of one workgroup per compute unit.  A second
 *                     kernel always follows on the stream: it advances the
 *                     sequence number in the workspace header and, should a
 *                     wait have run out (members not resident together),
 *                     recomputes every output with the single pass's own
 *                     arithmetic and order but without the exchange, so the
 *                     results are the same bits either way.  The call's tag
 *                     comes from the workspace, not the host, so the form
 *                     may be captured into a HIP graph and replayed.
 *                     Returns MHC_ERR_UNSUPPORTED when it does not apply.
 *   MHC_PRE_AUTO      the one-pass form where it measures faster on MI355X:
 *                     n = 4 and enough 16-token tiles per team, from 6 for
 *                     teams of 8 or 16 (T >= 1536 at d = 4096, 3072 at
 *                     d = 2048) to 24 for teams of 11, which leave 10 of an
 *                     XCD's 32 compute units idle (T >= 3840 at d = 2560,
 *                     teams of 10); else the two-pass form.
 *   MHC_PRE_ONE_PASS_FALLBACK_TEST
 *                     testing aid: the one-pass form with every workgroup
 *                     starting as if a wait had run out, so the recomputing
 *                     kernel produces every output.
 * Both forms sum every partial in a fixed order (results are bitwise
 * reproducible for a given form); the two forms agree to rounding.
 * algo_used (nullable, host pointer) receives the form that ran.
 * Workspace header after a one-pass call (64-bit words): [0] the tag of the
 * last one-pass call whose wait ran out, XORed with 0x5555555555555555
 * (earlier contents if none did), [1] the next call's sequence number, [2]
 * the tag of the call just made (its sequence number with the top bit set);
 * [0] == [2] ^ 0x5555555555555555 therefore means this call was recomputed.
 * The other forms leave the header alone. */
#define MHC_PRE_AUTO 0
#define MHC_PRE_TWO_PASS 1
#define MHC_PRE_ONE_PASS 2
#define MHC_PRE_ONE_PASS_FALLBACK_TEST 3
mhc_status mhc_pre_ex(const mhc_params* p, const void* X, const float* phi, const float* bias, void* h,
                      float* H, void* workspace, size_t workspace_bytes, int32_t algo, int32_t* algo_used,
                      void* stream);

/* ---- mhc_pre_noalloc: mhc_pre without allocation or workspace ----------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * computation, arguments, form choice (MHC_PRE_AUTO) and results as mhc_pre,
 * but no workspace argument: the scratch is a static device array of
 * MHC_PRE_NOALLOC_SCRATCH_BYTES per GPU inside the library, allocated when
 * the library's code is loaded on that GPU and held until the process ends.
 * The call itself allocates and frees nothing.
 *   Returns MHC_ERR_SCRATCH (before anything is enqueued) when
 *   mhc_pre_workspace_size(p) exceeds MHC_PRE_NOALLOC_SCRATCH_BYTES: at
 *   n = 4, d = 4096, bf16, up to about T = 19,700 tokens.
 * Every call on a GPU uses that GPU's one array, which keeps the last call's
 * contents (the single pass's sequence number carries over; nothing needs
 * clearing).  Calls that overlap in time on one GPU race on it: issue them on
 * one stream, or order them. */
#define MHC_PRE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
mhc_status mhc_pre_noalloc(const mhc_params* p, const void* X, const float* phi, const float* bias, void* h,
                           float* H, void* stream);

/* ---- mhc_post: stream mixing + broadcast-add --------------------------------
 * X_out[t, i, :] = sum_j H_res[t, i, j] X[t, j, :] + H_post[t, i] Y[t, :]
 * (Dubrov, "Kernmechanismen", Eq. 3; "mHC" notes eq. dsv4-mhc-hc-update and
 * the fused Post-Res kernel of table tbl-dsv4-mhc-kernels).  One pass over
 * the state: reads X, Y and the maps once and writes X_out once.
 *   X      in   [T, n, d] state dtype
 *   Y      in   [T, d] state dtype (the sublayer output F(h))
 *   H      in   [T, m] fp32 maps as written by mhc_pre (H_pre is not read)
 *   X_out  out  [T, n, d] state dtype; may be exactly X (in place); any other
 *               overlap with X, Y or H is MHC_ERR_ALIAS. */
mhc_status mhc_post(const mhc_params* p, const void* X, const void* Y, const float* H,
                    void* X_out, void* stream);

/* ---- mhc_post_pre: mhc_post of layer l, then mhc_pre of layer l+1 -------------
 * In a stack the state a layer writes is the state the next layer reads.
 * This entry point does both with one pass over the new state: it forms
 *   X_out = H_res X + H_post^T Y            (layer l's maps H, as mhc_post)
 * and, from the stored X_out, layer l+1's maps H_next and its sublayer input
 * h (as mhc_pre with phi, bias and p's alphas / eps / t_max).  The pages fuse
 * the layer's kernels for the same reason: the post kernel reads (n+1) C
 * values per token instead of (3n+1) C ("mHC" notes on DeepSeek-V4, table
 * tbl-dsv4-mhc-kernels).  The results are bitwise those of mhc_post followed
 * by mhc_pre_ex in the form that ran (*algo_used of mhc_post_pre_ex).
 *   X       in   [T, n, d] layer l's input state
 *   Y       in   [T, d] layer l's sublayer output
 *   H       in   [T, m] layer l's maps
 *   X_out   out  [T, n, d] X_{l+1}; may be exactly X (then the two-pass
 *                form runs), other overlap refused
 *   phi, bias    layer l+1's parameters
 *   h       out  [T, d] layer l+1's sublayer input
 *   H_next  out  [T, m] layer l+1's maps
 *   workspace    at least mhc_pre_workspace_size(p) bytes, as mhc_pre's
 *                (header included)
 * Forms (mhc_post_pre is mhc_post_pre_ex(..., MHC_PRE_AUTO, NULL, stream)):
 *   MHC_PRE_TWO_PASS  the post inside the split-K projection pass, which
 *                     stores X_out; the maps + aggregation pass reads X_out
 *                     again (per token: X, Y read, X_out written, X_out read
 *                     again, h written).
 *   MHC_PRE_ONE_PASS  mhc_pre's single pass with the post in front: each
 *                     team member mixes its slice of X and Y into X_out in
 *                     registers, stores it, and uses the stored values for
 *                     the projection and, once H_pre is known, for h, so
 *                     X_out never comes back from HBM (per token: X, Y read,
 *                     X_out, h written).  Same conditions as mhc_pre_ex's
 *                     single pass, and X_out must not overlap X (the
 *                     fallback kernel recomputes from X): MHC_ERR_ALIAS
 *                     when X_out == X, MHC_ERR_UNSUPPORTED when the shape
 *                     does not apply.
 *   MHC_PRE_AUTO      the single pass when X_out is separate from X, n = 4
 *                     and each team gets enough tiles: 10 to 48 by team
 *                     size (T >= 4096 at d = 4096, 5120 at d = 2048, 3840
 *                     at d = 2560; on MI355X at T = 16384, d = 4096:
 *                     265-272 us against 326-329 us for the two-pass
 *                     form), else the two-pass form.
 *   MHC_PRE_ONE_PASS_FALLBACK_TEST   as for mhc_pre_ex.
 * n = 1 and n = 8 run mhc_post, then mhc_pre's two-pass form. */
mhc_status mhc_post_pre(const mhc_params* p, const void* X, const void* Y, const float* H, void* X_out,
                        const float* phi, const float* bias, void* h, float* H_next, void* workspace,
                        size_t workspace_bytes, void* stream);
mhc_status mhc_post_pre_ex(const mhc_params* p, const void* X, const void* Y, const float* H, void* X_out,
                           const float* phi, const float* bias, void* h, float* H_next, void* workspace,
                           size_t workspace_bytes, int32_t algo, int32_t* algo_used, void* stream);

/* ---- backward ----------------------------------------------------------------
 * The pages give no backward formulas; they state that the layer is trained
 * with a custom backward that recomputes the maps rather than storing them
 * ("mHC" notes, table tbl-dsv4-mhc-mixed-precision and the kernel notes).  The
 * two entry points below are the chain rule of mhc_post and mhc_pre, split
 * where the sublayer sits: a training step calls mhc_post_bwd, then the
 * sublayer's own backward (dY -> dh), then mhc_pre_bwd.  G = dL/dX_out and
 * D = dL/dh arrive in the state dtype; parameter gradients are fp32.
 *
 * mhc_post_bwd: for X_out = H_res X + H_post^T Y,
 *   dX[t, j, :] = sum_i H_res[t, i, j] G[t, i, :]   written, state dtype
 *   dY[t, :]    = sum_i H_post[t, i]   G[t, i, :]   written, state dtype
 *   dH[t, n + i*n + j] = <G[t, i, :], X[t, j, :]>   written, fp32
 *   dH[t, n + n*n + i] = <G[t, i, :], Y[t, :]>      written, fp32
 * dH[t, 0 .. n-1] (the read map's part) is left untouched.
 *   X, G in [T, n, d]; Y in [T, d]; H in [T, m] (as written by mhc_pre)
 *   dX out [T, n, d], or NULL: then dX is not written, for a caller that
 *          lets mhc_pre_bwd_ex form the whole dX from G (one write of dX
 *          instead of a write, a read and a second write);
 *   dY out [T, d]; dH out [T, m]
 * No output may overlap an input or another output. */
mhc_status mhc_post_bwd(const mhc_params* p, const void* X, const void* Y, const float* H, const void* G,
                        void* dX, void* dY, float* dH, void* stream);

/* mhc_post_bwd_ex: mhc_post_bwd with a workspace, which lets it run in a
 * faster tiled form when d is a multiple of 512: a workgroup then covers 4
 * tokens x 512 values of d, so each token's dot products are formed per
 * 512-value slice, kept in the workspace and added in slice order.
 *   workspace  NULL: the scratch-free form that mhc_post_bwd runs.  Else at
 *              least mhc_post_bwd_workspace_size(p) bytes (fewer is
 *              MHC_ERR_WORKSPACE), 16-byte aligned, overlapping no other
 *              argument; contents on entry ignored, on return unspecified.
 * mhc_post_bwd_workspace_size returns 0 where the tiled form does not apply
 * (then the workspace is not used).  Both forms sum in a fixed order (bitwise
 * reproducible) and agree to rounding. */
size_t mhc_post_bwd_workspace_size(const mhc_params* p);
mhc_status mhc_post_bwd_ex(const mhc_params* p, const void* X, const void* Y, const float* H, const void* G,
                           void* dX, void* dY, float* dH, void* workspace, size_t workspace_bytes, void* stream);

/* mhc_pre_bwd: for h = H_pre X and the maps of mhc_pre, recomputed from X:
 *   dX    += H_pre D + the RMSNorm / projection path      read-modify-write,
 *            (dX as left by mhc_post_bwd)                 state dtype
 *   dphi   = sum_t x_hat_t dz_t^T     [n*d, m] fp32, written
 *   dbias  = sum_t dlogits_t          [m] fp32, written
 *   dalpha = per block (pre, res, post) sum_t <dlogits_t, z_t>   [3] fp32, written
 * with dlogits from dH[:, n:] (res and post parts, as written by
 * mhc_post_bwd) and dH_pre = <D, X_i> (computed here), through the gates and
 * Sinkhorn's 2 t_max normalisations in reverse.  Sums over tokens run in a
 * fixed order.  t_max must be <= 128 (else MHC_ERR_UNSUPPORTED).
 *   X in [T, n, d]; phi, bias as for mhc_pre; D in [T, d]; dH in [T, m]
 *   workspace: at least mhc_pre_bwd_workspace_size(p) bytes, 16-byte aligned;
 *   contents on entry ignored, on return unspecified.
 * No output may overlap an input or another output.  T = 0 writes zero
 * parameter gradients. */
size_t mhc_pre_bwd_workspace_size(const mhc_params* p);
mhc_status mhc_pre_bwd(const mhc_params* p, const void* X, const float* phi, const float* bias, const void* D,
                       const float* dH, void* dX, float* dphi, float* dbias, float* dalpha, void* workspace,
                       size_t workspace_bytes, void* stream);

/* mhc_pre_bwd_ex: mhc_pre_bwd, and with G (= dL/dX_out, [T, n, d], state
 * dtype) not NULL the whole dX in one write:
 *   dX[t, i, :] = sum_j H_res[t, j, i] G[t, j, :] + H_pre D + the RMSNorm /
 *                 projection path                      written, not read
 * with H_res recomputed from X like the other maps.  Use it after
 * mhc_post_bwd(_ex) with dX NULL: the pair then moves 32 KiB less per token
 * at n = 4, d = 4096, bf16, and rounds dX to the state dtype once.  G NULL is
 * mhc_pre_bwd.  G must not overlap an output. */
mhc_status mhc_pre_bwd_ex(const mhc_params* p, const void* X, const float* phi, const float* bias, const void* D,
                          const float* dH, const void* G, void* dX, float* dphi, float* dbias, float* dalpha,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---- mhc_amax: composite-map Amax Gain Magnitude ---------------------------
 * For each token, P = H_res,L-1 ... H_res,0 (each layer multiplies the running
 * product from the left) and
 *     gain_fwd = max_i sum_j |P_ij|   (largest absolute row sum)
 *     gain_bwd = max_j sum_i |P_ij|   (largest absolute column sum)
 *     amax     = max(gain_fwd, gain_bwd)
 * (Dubrov, "Het probleem van de samengestelde map"; "mHC" notes, section on
 * HC's composite mapping).  L = 0 gives P = I.
 *   H_stack    in   [L, T, m] fp32 (each layer's H as written by mhc_pre)
 *   amax, gain_fwd, gain_bwd   out [T] fp32, each may be NULL
 *   composite  out  [T, n, n] fp32 row-major, may be NULL
 * Outputs must not overlap H_stack or one another. */
mhc_status mhc_amax(int64_t T, int32_t n, int32_t L, const float* H_stack, float* amax,
                    float* gain_fwd, float* gain_bwd, float* composite, void* stream);

/* ---- mhc_gelu_half: the synthetic sublayer of the layer-stack workload ------
 * Y = 0.5 * GELU(h) = 0.5 * h * Phi(h) elementwise (the erf form, with Phi
 * evaluated as erfc(-h / sqrt 2) / 2: within 2e-5 relative of the exact value
 * in fp32), in the state dtype.  Stands in for attention / MLP so that a
 * many-layer stack can run without a GEMM; it is not part of the mHC method.
 *   h in [count], Y out [count]; Y may be exactly h, other overlap is an error. */
mhc_status mhc_gelu_half(int64_t count, int32_t dtype, const void* h, void* Y, void* stream);

/* ---- mhc_workspace_size: scratch bytes of an entry point ---------------------
 * One query for every entry point (the interface's size query): bytes of
 * device scratch the entry point named by op needs for the parameters p, or
 * 0 when it needs none, p is invalid or op unknown.  The per-entry-point
 * queries above return the same numbers.
 *   MHC_OP_PRE       mhc_pre and mhc_pre_ex (both forms)
 *   MHC_OP_POST      mhc_post (0)
 *   MHC_OP_POST_PRE  mhc_post_pre (= MHC_OP_PRE)
 *   MHC_OP_AMAX      mhc_amax (0)
 *   MHC_OP_POST_BWD  mhc_post_bwd_ex's tiled form (0 where it does not apply)
 *   MHC_OP_PRE_BWD   mhc_pre_bwd */
#define MHC_OP_PRE 0
#define MHC_OP_POST 1
#define MHC_OP_POST_PRE 2
#define MHC_OP_AMAX 3
#define MHC_OP_POST_BWD 4
#define MHC_OP_PRE_BWD 5
size_t mhc_workspace_size(const mhc_params* p, int32_t op);

/* Static description of a status code (never NULL; "unknown status" for a
 * value that is no mhc_status).  Takes an int so that any value a caller
 * passes is well defined. */
const char* mhc_status_string(int status);

/* MHC_ABI_VERSION of the loaded library. */
int mhc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H */

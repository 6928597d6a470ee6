/*
 * gdscan.h -- C ABI of the gfx950 (MI355X) matrix-state affine scan library.
 *
 * The library computes, per head, the prefix scan of the affine monoid
 * (E_t, f_t) acting on a matrix state S (d_v rows = value channels, d_k
 * columns = key channels):
 *
 *     S_t = S_{t-1} E_t + f_t,          o_t = S_t q_t   (inclusive read-out)
 *
 *   SCAN_GDN (gated delta rule):       E_t = alpha_t (I - beta_t k_t k_t^T),
 *                                      f_t = beta_t v_t k_t^T
 *   SCAN_GLA (gated linear attention): E_t = alpha_t I,  f_t = v_t k_t^T
 *   SCAN_GDN_EW (gated delta rule, separate erase and write strengths):
 *                                      E_t = alpha_t (I - be_t k_t k_t^T),
 *                                      f_t = bw_t v_t k_t^T
 *
 *   SCAN_GDN_DIAG (gated delta rule, diagonal gate):
 *                                      E_t = diag(a_t) (I - beta_t k_t k_t^T),
 *                                      f_t = beta_t v_t k_t^T
 *   SCAN_GLA_DIAG (gated linear attention, diagonal gate):
 *                                      E_t = diag(a_t),  f_t = v_t k_t^T
 *   with a_t one decay per key channel (the prefix-scan notes, key design 2,
 *   list the diagonal gate among the forms of E_t).
 *
 * SCAN_GDN_EW is PRISM's write-forget decoupling ("PRISM: Parallel Residual
 * Iterative Sequence Model", gist.science explainer, technical summary 2.1:
 * the forget operator stays the Gated-DeltaNet rank-1 form, the write is
 * free).  An element with alpha = 1, be = 0 is a pure write, so a token's
 * rank-L write becomes L + 1 consecutive elements (see prism_expand below).
 *
 * Sources: "Sequential Parallel Duality in Prefix Scannable Models"
 * (papernotes.org ICLR 2026 notes), key design 2 (affine update
 * s_t = E_t |> s_{t-1} + f_t, monoid combine (E2,f2)+(E1,f1) = (E2 E1, E2 f1 + f2),
 * identity (I,0); gated linear attention is the scalar-gate member) and key
 * design 1 (a parallel training circuit over all positions, plus a per-token
 * state update for inference); "PRISM: Parallel Residual Iterative Sequence
 * Model" (gist.science explainer, technical summary 2.1: S_t = S_{t-1} A_t + B_t
 * with a Gated-DeltaNet rank-1 forget operator; 2.2: S_{t-1} k_t is the value
 * recalled for key k_t) and the PRISM article (banbantang.com, section 1(4):
 * global scalar decay, rank-1 forgetting along k, rank-1 write).  In the
 * right-action form used here E acts on the key index; since every E_t is
 * symmetric this is the left action E_t S^T_{t-1} + f_t^T on the transposed
 * (d_k x d_v) storage.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE memory owned by the caller.  The library
 *    allocates nothing and keeps no pointer after a call returns.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream).  Buffers must stay alive until the stream has completed.
 *  - Arguments are validated on the host before anything is launched; a
 *    non-zero status means nothing was enqueued and nothing was written, and
 *    scan_last_error() (per host thread) describes the problem.
 *  - Data preconditions are documented, not checked on the device: finite
 *    inputs, 0 < alpha <= 1, and for SCAN_GDN 0 <= beta <= 1 with unit-norm keys
 *    recommended (then every E_t has spectral norm <= 1; the same holds for
 *    the erase strengths of SCAN_GDN_EW, whose write strengths are free).
 *  - Layouts are dense and row-major.  q, k, v, o, S0, ST and S must be 16-byte
 *    aligned; alpha and beta 4-byte aligned.
 */
#ifndef GDSCAN_H_
#define GDSCAN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* mode */
#define SCAN_GDN 0
#define SCAN_GLA 1
#define SCAN_GDN_EW 2
#define SCAN_GDN_DIAG 3
#define SCAN_GLA_DIAG 4

/* element type of q, k, v and o (alpha, beta and all states are float32) */
#define SCAN_F32 0
#define SCAN_BF16 1

/* status codes */
#define SCAN_OK 0
#define SCAN_EINVAL 1        /* null required pointer, bad enum, bad size, overlap */
#define SCAN_EUNSUPPORTED 2  /* shape/chunk/dtype combination not built */
#define SCAN_EWORKSPACE 3    /* workspace missing or smaller than required */
#define SCAN_EALIGN 4        /* pointer not aligned as documented above */
#define SCAN_EHIP 5          /* HIP launch/runtime failure (message has the HIP error) */

/* scan_opts.path */
#define SCAN_PATH_AUTO 0
#define SCAN_PATH_SEQUENTIAL 1  /* one pass over the chunks of each head */
#define SCAN_PATH_BLELLOCH 2    /* leaf aggregates + fixed Blelloch tree + output pass */

typedef struct scan_opts {
    int path;         /* SCAN_PATH_*; AUTO picks BLELLOCH when B*H is too small to fill the GPU */
    int leaf_chunks;  /* Blelloch path: chunks per leaf (power of two); 0 = library default */
} scan_opts;

/*
 * Bytes of device workspace scan_fwd needs for these arguments (0 if none).
 * Returns (size_t)-1 if the arguments are invalid or unsupported
 * (scan_last_error() says why).  opts may be NULL (defaults).
 */
size_t scan_fwd_workspace_size(int mode, int dtype, int B, int H, int T, int dk, int dv,
                               int chunk, const scan_opts *opts);

/*
 * Full-sequence forward scan (the parallel training view of key design 1 in
 * the prefix-scan notes; chunked as in their overall framework: every chunk is
 * encoded, chunk states are combined in a fixed order, then each chunk is read
 * out from its exclusive prefix state).
 *
 *   q, k : [B, H, T, dk]  dtype          v, o : [B, H, T, dv]  dtype
 *   alpha: [B, H, T] float32 in (0, 1]; [B, H, T, dk] for SCAN_GDN_DIAG and
 *          SCAN_GLA_DIAG (16-byte aligned), one decay per key channel
 *   beta : [B, H, T] float32 for SCAN_GDN and SCAN_GDN_DIAG; NULL for SCAN_GLA and
 *          SCAN_GLA_DIAG;
 *          [2, B, H, T] float32 for SCAN_GDN_EW (plane 0: erase strengths be,
 *          plane 1: write strengths bw)
 *   S0   : [B, H, dv, dk] float32 initial state, or NULL for the zero state
 *   ST   : [B, H, dv, dk] float32 final state, or NULL to skip writing it.
 *          ST may be the same pointer as S0 (in-place carry); any other overlap
 *          with an input is invalid.
 *   o    : written for every token, o_t = S_t q_t; must not overlap any input.
 *   chunk: tokens per chunk, 16, 32 or 64.  A ragged last chunk behaves as if
 *          padded with identity tokens (alpha = 1, beta = 0, q = k = v = 0);
 *          padded outputs are not written.
 *   workspace / workspace_bytes: device scratch of at least
 *          scan_fwd_workspace_size(...) bytes (may be NULL when that is 0).
 *          Reusable across calls that are ordered on one stream.
 * Supported: dtype SCAN_BF16 with dk = dv = 128 (chunk 64 on the fast path;
 * chunk 16/32 and other sizes take the float32 kernel); dtype SCAN_F32 with
 * dk, dv in {16, 32, 64, 128}.  T >= 1; B, H >= 1.  The diagonal-gate modes
 * run a float32 chunk kernel on the sequential path (its own 32-token chunks;
 * `chunk` is validated but the result does not depend on it) for either dtype
 * with dk in {16, 32, 64, 128} and dv a multiple of 16.
 * Returns SCAN_OK or an error status (see above).
 */
int scan_fwd(int mode, int dtype, int B, int H, int T, int dk, int dv, int chunk,
             const void *q, const void *k, const void *v, const float *alpha,
             const float *beta, const float *S0, void *o, float *ST,
             void *workspace, size_t workspace_bytes, const scan_opts *opts, void *stream);

/* Bytes of the fixed device scratch behind scan_fwd_noalloc (per GPU). */
#define SCAN_NOALLOC_MAX_WORKSPACE (64u << 20)

/*
 * scan_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc.  Same
 * arguments, results and validation as scan_fwd, without the workspace
 * argument: where the chosen path needs scratch (see scan_fwd_workspace_size)
 * the library uses a fixed array of SCAN_NOALLOC_MAX_WORKSPACE bytes in device
 * memory, one per GPU, which that GPU holds from the library's first use on it
 * until the process ends.  The call never allocates or frees device memory.
 *   - Arguments whose workspace size exceeds SCAN_NOALLOC_MAX_WORKSPACE are
 *     rejected with SCAN_EWORKSPACE before anything is launched.
 *   - Every call on one GPU shares that GPU's array: calls that may run at the
 *     same time on one GPU (different streams, or host threads without
 *     ordering) race and give wrong results.  Order them on one stream.
 *   - The array keeps whatever the last call left in it; no path reads it
 *     before writing it.
 *   - The first call on a device looks up the array's device address (a HIP
 *     runtime query, no allocation) and caches it for later calls.
 */
int scan_fwd_noalloc(int mode, int dtype, int B, int H, int T, int dk, int dv, int chunk,
                     const void *q, const void *k, const void *v, const float *alpha,
                     const float *beta, const float *S0, void *o, float *ST,
                     const scan_opts *opts, void *stream);

/*
 * One token for each of N independent states (the sequential view: state
 * update U and read-out F of key design 1 in the prefix-scan notes); exactly
 * scan_fwd with T = 1 applied to each state, state updated in place:
 *
 *   S <- S E + f,   o = S q   (with the updated S)
 *
 *   q, k : [N, dk] dtype     v, o : [N, dv] dtype
 *   alpha: [N] float32 ([N, dk] with diagonal gates)
 *   beta : [N] float32 (SCAN_GDN, SCAN_GDN_DIAG), NULL (SCAN_GLA, SCAN_GLA_DIAG)
 *          or [2, N] float32 (SCAN_GDN_EW: erase, then write)
 *   S    : [N, dv, dk] float32, read and written in place
 * Supported: dk in {16, 32, 64, 128}, dv >= 1, either dtype.
 * o must not overlap any input or S.  Returns SCAN_OK or an error status.
 */
int decode_step(int mode, int dtype, int N, int dk, int dv, const void *q, const void *k,
                const void *v, const float *alpha, const float *beta, float *S, void *o,
                void *stream);

/* Limits of prism_expand */
#define PRISM_MAX_STEPS 8   /* L: refinement steps (rank-1 corrections) per token */
#define PRISM_MAX_WINDOW 8  /* W: taps of the anchor's short convolution */

/*
 * PRISM's rank-L write ("PRISM: Parallel Residual Iterative Sequence Model",
 * gist.science explainer, technical summary 2.2; PRISM article,
 * banbantang.com, section 3(2)-(4)) expanded into a SCAN_GDN_EW element
 * stream.  Per head and token t, from the input only:
 *
 *   u_t       = sum_{j<W} conv[j] * x_{t-j}          (0 before the start)
 *   r^(1)     = v_t - u_t
 *   k^(l)     = Wk[l] u_t,   p^(l) = Wp[l] u_t       (l = 1..L)
 *   delta^(l) = GELU(p^(l) * r^(l)),  r^(l+1) = r^(l) - delta^(l)
 *
 * and the write B_t = beta_t v_t k_t^T + sum_l beta_l[t,l] delta^(l) k^(l)T.
 * Token t becomes elements t(L+1) .. t(L+1)+L of the output stream:
 *   element t(L+1)    : q = 0 (q_t if L = 0), k_t, v_t, alpha_t, erase beta_t, write beta_t
 *   element t(L+1)+l  : q = 0 (q_t for l = L), k^(l), delta^(l), alpha 1, erase 0,
 *                       write beta_l[t, l-1]
 * so scan_fwd(SCAN_GDN_EW, ..., T (L+1), q2, k2, v2, alpha2, beta2, ...) gives
 * o2 with the layer's output o_t = o2[t (L+1) + L] and the same final state.
 * GELU is x (1 + erf(x / sqrt 2)) / 2; the factors are computed in float32
 * (bfloat16 data: the anchor is split into two bfloat16 parts for the MFMA
 * projections) and stored in dtype.
 *
 *   q, k : [B, H, T, dk] dtype      v, x : [B, H, T, dv] dtype (x: the anchor's source)
 *   alpha, beta : [B, H, T] float32  beta_l : [B, H, T, L] float32
 *   conv : [H, W, dv] float32        Wk : [H, L, dk, dv] dtype   Wp : [H, L, dv, dv] dtype
 *   q2, k2 : [B, H, T (L+1), dk] dtype      v2 : [B, H, T (L+1), dv] dtype
 *   alpha2 : [B, H, T (L+1)] float32        beta2 : [2, B, H, T (L+1)] float32
 * x, beta_l, conv, Wk and Wp may be NULL when L = 0.  Outputs must not overlap
 * inputs or each other.  Supported: dk, dv in {16, 32, 64, 128}, either dtype
 * (bfloat16 with dk = dv = 128 projects on the MFMA units).  0 <= L <= 8,
 * 1 <= W <= 8.  Returns SCAN_OK or an error status.
 */
int prism_expand(int dtype, int B, int H, int T, int dk, int dv, int L, int W,
                 const void *q, const void *k, const void *v, const void *x,
                 const float *alpha, const float *beta, const float *beta_l,
                 const float *conv, const void *Wk, const void *Wp,
                 void *q2, void *k2, void *v2, float *alpha2, float *beta2, void *stream);

/*
 * The PRISM layer's scan without a materialised element stream: the element
 * stream that prism_expand would write (same arithmetic, same element order)
 * is scanned in place.  The factor rows k^(l), delta^(l) go to the workspace;
 * the scan reads every other element field from the token arrays (element
 * t(L+1): k_t, v_t, alpha_t, beta_t; elements t(L+1)+l: the factor rows, alpha 1,
 * erase 0, write beta_l[t, l-1]), reads q_t for element t(L+1)+L only, and
 * writes o_t (that element's output) once per token ("PRISM: Parallel Residual
 * Iterative Sequence Model", gist.science explainer, technical summary 2.1-2.2;
 * PRISM article, banbantang.com, section 3(3): the L-step write in one pass).
 *
 *   inputs as prism_expand, plus S0 [B, H, dv, dk] float32 or NULL (zero state)
 *   o    : [B, H, T, dv] bfloat16, o_t = S at token t's last element times q_t
 *   ST   : [B, H, dv, dk] float32 final state, or NULL; may equal S0
 *   workspace: prism_scan_workspace_size(...) bytes (B H T L (dk + dv) bf16
 *          factor rows), 256-byte aligned; NULL when that is 0 (L = 0).
 * Supported: dtype SCAN_BF16, dk = dv = 128, 0 <= L <= 8 (L = 0 is the gated
 * delta rule), 1 <= W <= 8, T (L + 1) < 2^31.  The result equals scan_fwd
 * (SCAN_GDN_EW) over prism_expand's stream bit for bit.  Returns SCAN_OK or an
 * error status; prism_scan_workspace_size returns (size_t)-1 for invalid or
 * unsupported arguments.
 */
size_t prism_scan_workspace_size(int dtype, int B, int H, int T, int dk, int dv, int L);
int prism_scan(int dtype, int B, int H, int T, int dk, int dv, int L, int W,
               const void *q, const void *k, const void *v, const void *x,
               const float *alpha, const float *beta, const float *beta_l,
               const float *conv, const void *Wk, const void *Wp,
               const float *S0, void *o, float *ST, void *workspace, size_t workspace_bytes,
               void *stream);

/*
 * Gradient of scan_fwd (reverse mode through the chunkwise form of the scan;
 * the prefix-scan notes, key design 2, define the affine state update it
 * differentiates).  For incoming gradients dO (at o) and dST (at S_T) it
 * returns the gradients of L = sum <dO, o> + <dST, S_T> with respect to every
 * input of a SCAN_GDN, SCAN_GLA or SCAN_GDN_EW scan_fwd call with the same
 * arguments:
 *   q, k : [B, H, T, dk] dtype       v, dO : [B, H, T, dv] dtype (dO NULL: zero)
 *   alpha: [B, H, T] float32 in (0, 1]    beta: [B, H, T] float32 (SCAN_GDN; NULL for SCAN_GLA;
 *          [2, B, H, T] for SCAN_GDN_EW: erase strengths, then write strengths)
 *   S0, dST: [B, H, dv, dk] float32 or NULL (zero)
 *   dq, dk_out: [B, H, T, dk] float32    dv_out: [B, H, T, dv] float32
 *   dalpha: [B, H, T] float32        dbeta: like beta, float32 (NULL for SCAN_GLA)
 *   dS0: [B, H, dv, dk] float32 (the gradient at the initial state, also when S0 is NULL)
 *   workspace: scan_bwd_workspace_size(...) bytes of device scratch, 256-byte
 *          aligned (the state entering every 32-token chunk and, with more than
 *          two 64-row value slices, per-slice partial sums); reusable across
 *          calls ordered on one stream.
 * All gradients are float32 whatever dtype is.  Outputs may not overlap inputs,
 * each other or the workspace.  Supported: dk in {32, 64, 128}, dv a multiple of
 * 64 (at most 4096).  Three kernels run on `stream`: a forward pass storing the
 * chunk states, the reverse chunk pass, and a reduction over value slices (with
 * dv <= 128 the reverse pass adds the slices' sums into dq, dk_out, dalpha and
 * dbeta itself and the last kernel only divides by alpha; the result is still
 * the same bit for bit from run to run).
 * Returns SCAN_OK or an error status; scan_bwd_workspace_size returns
 * (size_t)-1 for invalid or unsupported arguments.
 */
size_t scan_bwd_workspace_size(int mode, int dtype, int B, int H, int T, int dk, int dv);
int scan_bwd(int mode, int dtype, int B, int H, int T, int dk, int dv,
             const void *q, const void *k, const void *v, const float *alpha, const float *beta,
             const float *S0, const void *dO, const float *dST,
             float *dq, float *dk_out, float *dv_out, float *dalpha, float *dbeta, float *dS0,
             void *workspace, size_t workspace_bytes, void *stream);

/* lact_fwd order */
#define LACT_UPDATE_THEN_APPLY 0  /* chunk b read with W_{b+1}: each token sees its whole chunk */
#define LACT_APPLY_THEN_UPDATE 1  /* chunk b read with W_b: the mask shifted by one chunk */

/*
 * Large-chunk fast-weight update with linear fast weights ("块级更新与端到端
 * TTT", PaperTrace 5.2, opening section; the LaCT news article on
 * senqingzn.com, the large-chunk test-time-training layer and its update/apply
 * paragraph).  Per head a fast weight W (dv x dk, float32) learns the
 * key-value reconstruction loss |W k - v|^2 / 2 with one gradient step per
 * chunk of `chunk` tokens, every gradient of the chunk taken at the chunk's
 * starting weight:
 *
 *   W_{b+1} = W_b - sum_{i in chunk b} eta_i (W_b k_i - v_i) k_i^T
 *   o_i     = W_{b+1} q_i  (LACT_UPDATE_THEN_APPLY)   or   W_b q_i  (LACT_APPLY_THEN_UPDATE)
 *
 * A ragged last chunk holds the remaining tokens.
 *   q, k : [B, H, T, dk] dtype      v, o : [B, H, T, dv] dtype
 *   eta  : [B, H, T] float32 learning rates (a constant array is the pages' scalar)
 *   W0   : [B, H, dv, dk] float32 initial weight, or NULL for zero
 *   WT   : [B, H, dv, dk] float32 final weight, or NULL; may equal W0
 *   workspace: lact_fwd_workspace_size(...) bytes of device scratch (NULL if 0),
 *          256-byte aligned; reusable across calls ordered on one stream.
 * Supported: dtype SCAN_BF16 with dk = dv = 128 and chunk a multiple of 64
 * (MFMA path: chunk statistics G = K^T diag(eta) K and F = V^T diag(eta) K for
 * every chunk in parallel, the chunk recursion per head in float32, then
 * O = Q W^T for every token in parallel), or either dtype with dk, dv in
 * {16, 32, 64} and any chunk >= 1 (plain float32 kernel, one workgroup per head).
 * Returns SCAN_OK or an error status; lact_fwd_workspace_size returns
 * (size_t)-1 for invalid or unsupported arguments.
 */
size_t lact_fwd_workspace_size(int dtype, int B, int H, int T, int dk, int dv, int chunk);
int lact_fwd(int dtype, int B, int H, int T, int dk, int dv, int chunk, int order,
             const void *q, const void *k, const void *v, const float *eta, const float *W0,
             void *o, float *WT, void *workspace, size_t workspace_bytes, void *stream);

/* Message describing the last non-zero status returned on this host thread. */
const char *scan_last_error(void);

/* Library name, version and the GPU architecture it was built for. */
const char *scan_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDSCAN_H_ */

/*
 * gdr.h -- C ABI of the gated delta-rule memory library (libgdr.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * Per head the library runs the recurrent-memory update
 *
 *     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * with the state S in the d_v x d_k orientation (row i = value channel i, so
 * a read at key k returns a value-space vector).  Equivalently
 *     Sbar = S_{t-1} Diag(alpha_t);  u = beta_t (v_t - Sbar k_t);
 *     S_t  = Sbar + u k_t^T;         o_t = S_t q_t.
 * Sources, by title and section:
 *   "Linear Attention Architectures: Mechanisms, Trade-offs, and Cross-Layer
 *   Routing", Sec. 3 (read rule Eq. (8) after the update; prediction and
 *   residual Eqs. (9)-(10); DeltaNet, Gated DeltaNet and Kimi Delta
 *   Attention updates; gates Eqs. (11)-(12));
 *   "linear attention and its gated descendants" (blog), sections
 *   "DeltaNet", "Gated DeltaNet", "Kimi Delta Attention" and "Chunkwise
 *   Parallel Form";
 *   "Linear Attention & DeltaNet" (wiki), "How it works" items 3-4 (the
 *   WY/Householder chunk form).
 *
 * Gate modes:
 *   GDR_ALPHA_NONE    alpha = 1 (DeltaNet)
 *   GDR_ALPHA_SCALAR  one alpha per head and token (Gated DeltaNet)
 *   GDR_ALPHA_CHANNEL one alpha per head, token and key channel (Kimi-style)
 * Gates are passed as beta itself (already in (0,1), no clamping) and as
 * log(alpha) (<= 0); the feature map is the identity (callers pass q and k
 * already normalised) and there is no 1/sqrt(d) scale.
 *
 * Conventions shared by every entry point:
 *  - All arrays are dense, contiguous, row-major in the index order given
 *    beside each argument, and live in device memory of the current HIP
 *    device.  The caller owns every buffer; the library allocates nothing
 *    and keeps no global state (thread-safe per stream).
 *  - Work is enqueued on `stream` (0 = the null stream) and is asynchronous;
 *    results are valid after the caller synchronises with the stream.
 *  - `dtype` selects the type of q, k, v and o: GDR_F32 (float) or GDR_BF16
 *    (bfloat16).  beta, log_alpha and the state are always float32.
 *  - Pointers passed to q, k, v, o, S0, S_final, S and the workspace must be
 *    16-byte aligned; beta 4-byte aligned; log_alpha 4-byte aligned, or
 *    16-byte aligned in GDR_ALPHA_CHANNEL mode.
 *  - Return value: GDR_OK or an error status.  Arguments are validated
 *    before anything is enqueued; on an error status nothing has been
 *    written.  GDR_ERR_HIP reports a failed launch (hipGetLastError).
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *    NaN or Inf inputs are not checked and propagate.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 1

enum gdr_status {
    GDR_OK = 0,
    GDR_ERR_INVALID_ARG = 1,          /* NULL required pointer, negative size,
                                         misaligned pointer, mode/pointer mismatch,
                                         o aliasing an input */
    GDR_ERR_UNSUPPORTED = 2,          /* d_k, d_v, C or dtype outside the domain */
    GDR_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below the queried size */
    GDR_ERR_HIP = 4,                  /* a HIP launch failed */
    GDR_ERR_SCRATCH_TOO_SMALL = 5     /* gdr_fwd_chunked_noalloc: the call needs more
                                         than GDR_NOALLOC_SCRATCH_BYTES of workspace */
};

/* Bytes of the fixed per-device scratch array of gdr_fwd_chunked_noalloc. */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

enum gdr_dtype { GDR_F32 = 0, GDR_BF16 = 1 };

enum gdr_alpha_mode { GDR_ALPHA_NONE = 0, GDR_ALPHA_SCALAR = 1, GDR_ALPHA_CHANNEL = 2 };

/*
 * Input-side steps the *_ex entry points apply themselves (a bit set; 0 =
 * none, which makes them identical to the plain entry points):
 *   GDR_PRO_L2NORM_QK  q and k are raw; every token's q and k is divided by
 *                      max(||.||_2, 1e-6) before use (recall by a key is
 *                      exact for normalised, orthogonal keys: "linear
 *                      attention and its gated descendants", "DeltaNet").
 *   GDR_PRO_GATES      beta and log_alpha hold raw pre-activations b and a:
 *                      the library uses beta = sigmoid(b) and
 *                      alpha = sigmoid(a), i.e. log alpha = -softplus(-a)
 *                      (the sigmoid gates of "Linear Attention & DeltaNet",
 *                      "Minimal pseudocode"; channel a gives one sigmoid per
 *                      key channel).  With channel alpha the floor of
 *                      gdr_fwd_chunked applies after the activation.
 * Other bits are rejected with GDR_ERR_INVALID_ARG.
 */
enum gdr_prologue { GDR_PRO_L2NORM_QK = 1, GDR_PRO_GATES = 2 };

/* Version of this ABI (GDR_ABI_VERSION). */
int gdr_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *gdr_status_string(int status);

/*
 * Bytes of device workspace gdr_fwd_chunked needs for these sizes (0 when
 * the call would do no chunk work).  Returns (size_t)-1 when the sizes are
 * invalid or unsupported.  The workspace holds one record per chunk of 32
 * tokens (16 for GDR_F32 or C == 16): the chunk's triangular WY factor
 * (I + A)^-1 diag(beta); with scalar alpha, and with alpha = 1 (run as
 * log alpha = 0), also its decay matrix and decay factors; with channel
 * alpha also its masked decayed score block, the chunk's total per-channel
 * decay and three decayed copies of its keys and queries.  When there are too few (batch, head) chains to occupy the GPU
 * and many chunks (bf16 only), the scan runs several segments of each chain
 * at once and the workspace also holds, per segment, its end state, its
 * transition and its entry state, plus d_k values per token.  It is scratch
 * only: written and read within the call, its contents are not part of the
 * result.
 */
size_t gdr_fwd_chunked_workspace_size(int B, int H, int L, int d_k, int d_v, int C,
                                      int dtype, int alpha_mode);

/*
 * Tokens per state step that gdr_fwd_chunked (and gdr_fwd_varlen) execute
 * for chunk length C, dtype and gate mode: the block size of the chunk
 * algebra the kernels actually run ("linear attention and its gated
 * descendants", "Chunkwise Parallel Form": C tokens per block, the state
 * carried between blocks).  The result does not depend on it beyond
 * rounding.  Returns 0 for arguments outside the domain.
 */
int gdr_fwd_chunked_token_step(int C, int dtype, int alpha_mode);

/*
 * Chunkwise forward (training / prefill form): runs the recurrence over L
 * tokens for every (batch b, head h) and writes every output and,
 * optionally, the final state.
 * ("linear attention and its gated descendants", "Chunkwise Parallel Form":
 * the sequence is cut into chunks of C tokens; the state is carried across
 * chunk boundaries and each chunk's outputs are dense block products.  The
 * product of a chunk's (I - beta k k^T) factors is kept in the compact
 * WY/Householder form named in "Linear Attention & DeltaNet", item 3.)
 *
 *   B, H       batch and heads (>= 0; 0 => nothing to do)
 *   L          tokens per sequence (>= 0).  L == 0 only copies S0 (or zeros)
 *              to S_final.  L need not be a multiple of C.
 *   d_k, d_v   key and value head dims, each 64 or 128
 *   C          chunk length: 16, 32 or 64.  The result does not depend on C
 *              beyond rounding.  The kernels run the chunk algebra in steps
 *              of gdr_fwd_chunked_token_step(C, dtype, alpha_mode) tokens.
 *   dtype      GDR_F32 or GDR_BF16 (type of q, k, v, o)
 *   q, k       [B][H][L][d_k]
 *   v          [B][H][L][d_v]
 *   beta       [B][H][L] float, the write strength in (0,1)
 *   alpha_mode GDR_ALPHA_NONE:    log_alpha must be NULL
 *              GDR_ALPHA_SCALAR:  log_alpha [B][H][L] float
 *              GDR_ALPHA_CHANNEL: log_alpha [B][H][L][d_k] float.  In this
 *              mode log_alpha values below -10 (alpha < 4.5e-5 per token
 *              and channel) are treated as -10, so that every intermediate
 *              exponential stays finite.  Each such (token, channel) then
 *              keeps at most e^-10 (4.5e-5) of the decayed state column
 *              that the recurrence would have emptied: the result departs
 *              from the unbounded recurrence (and from gdr_decode_step,
 *              which has no floor) by at most that fraction per floored
 *              value.
 *   S0         NULL => zero initial state, else [B][H][d_v][d_k] float
 *   o          [B][H][L][d_v] (dtype); must not overlap any input
 *   S_final    NULL => not written, else [B][H][d_v][d_k] float; may be the
 *              same pointer as S0 (updated in place) but must not partially
 *              overlap it
 *   workspace  device scratch of at least
 *              gdr_fwd_chunked_workspace_size(...) bytes (may be NULL when
 *              that size is 0); must not overlap any other argument
 *   stream     HIP stream to enqueue on
 */
int gdr_fwd_chunked(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                    const void *q, const void *k, const void *v,
                    const float *beta, int alpha_mode, const float *log_alpha,
                    const float *S0, void *o, float *S_final,
                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/* gdr_fwd_chunked with the input-side steps of `prologue` (gdr_prologue);
 * same arguments, layouts, workspace size and errors otherwise. */
int gdr_fwd_chunked_ex(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                       const void *q, const void *k, const void *v,
                       const float *beta, int alpha_mode, const float *log_alpha,
                       const float *S0, void *o, float *S_final,
                       void *workspace, size_t workspace_bytes, hipStream_t stream,
                       unsigned prologue);

/*
 * gdr_fwd_chunked for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, layouts and results as gdr_fwd_chunked, without the
 * workspace: the kernels use a fixed array of GDR_NOALLOC_SCRATCH_BYTES in
 * the library's own device memory, one per GPU, held until the process ends.
 * The call allocates nothing (no hipMalloc, no library allocation); its
 * first call with a device current looks up that device's array address.
 *   Returns GDR_ERR_SCRATCH_TOO_SMALL, before anything is enqueued, when
 *   gdr_fwd_chunked_workspace_size(...) for these sizes exceeds
 *   GDR_NOALLOC_SCRATCH_BYTES (64 MiB: for example B * H = 64 heads of
 *   L = 2048 tokens at d_k = 128, bf16, scalar gates need about 19 MB);
 *   other errors as for gdr_fwd_chunked, GDR_ERR_HIP also if the array's
 *   address cannot be found.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams or host threads) race and must be serialised by
 * the caller.  Nothing in the array needs clearing between calls.
 */
int gdr_fwd_chunked_noalloc(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                            const void *q, const void *k, const void *v,
                            const float *beta, int alpha_mode, const float *log_alpha,
                            const float *S0, void *o, float *S_final, hipStream_t stream);

/*
 * Bytes of device workspace gdr_bwd_chunked needs (0 when B * H == 0 or
 * L == 0), or (size_t)-1 for invalid or unsupported sizes.  It holds the
 * forward's chunk records, every chunk's (I + A)^-1 (fp32), the state
 * gradient at every chunk's end and entry states (d_v x d_k each, in the
 * dtype of q; chunks of 32 tokens, or 16 for GDR_F32 or C == 16): for bf16
 * on 32-token chunks only the state entering every run of
 * ceil(B * H * chunks / 256) chunks, counted over all heads, else the state
 * entering every chunk.
 */
size_t gdr_bwd_chunked_workspace_size(int B, int H, int L, int d_k, int d_v, int C,
                                      int dtype, int alpha_mode);

/*
 * Backward of gdr_fwd_chunked (training): for a loss with gradient dO with
 * respect to the outputs o and dS_final with respect to the final state,
 * the gradients with respect to q, k, v, beta, log alpha and S0.  The
 * forward is recomputed inside the call from the same inputs (nothing from
 * the forward call is kept).  The result is the derivative of the
 * recurrence of gdr_fwd_chunked, taken chunk by chunk ("linear attention and
 * its gated descendants", "Chunkwise Parallel Form" and "Gated DeltaNet").
 *
 *   B, H, L, d_k, d_v, C, dtype, q, k, v, beta, S0   as for gdr_fwd_chunked
 *   alpha_mode, log_alpha   as for gdr_fwd_chunked (channel alpha: the
 *              floor of log alpha at -10 that the forward applies passes no
 *              gradient, so dlog_alpha is 0 where log alpha < -10)
 *   dO         [B][H][L][d_v] (dtype)
 *   dS_final   NULL (zero) or [B][H][d_v][d_k] float
 *   dq, dk     [B][H][L][d_k] (dtype);  dv [B][H][L][d_v] (dtype)
 *   dbeta      [B][H][L] float
 *   dlog_alpha NULL for GDR_ALPHA_NONE, else the shape of log_alpha:
 *              [B][H][L] (scalar) or [B][H][L][d_k] (channel) float
 *   dS0        NULL (not written) or [B][H][d_v][d_k] float
 *   workspace  at least gdr_bwd_chunked_workspace_size(...) bytes
 * Outputs must not overlap any input, each other or the workspace.  Errors
 * as for gdr_fwd_chunked.
 */
int gdr_bwd_chunked(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                    const void *q, const void *k, const void *v,
                    const float *beta, int alpha_mode, const float *log_alpha,
                    const float *S0, const void *dO, const float *dS_final,
                    void *dq, void *dk, void *dv, float *dbeta, float *dlog_alpha,
                    float *dS0, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The forward of a training step that keeps, in a backward workspace, what
 * gdr_bwd_chunked would otherwise recompute (the chunk records, every
 * chunk's (I + A)^-1 and the entry states), so that gdr_bwd_chunked_kept
 * can start from them (the same chunk algebra as gdr_fwd_chunked: "linear
 * attention and its gated descendants", "Chunkwise Parallel Form").
 *
 * Arguments, alignment, aliasing rules and errors as for gdr_fwd_chunked,
 * except:
 *   workspace  at least gdr_bwd_chunked_workspace_size(...) bytes, for the
 *              same sizes; it is filled here and read by the backward
 * o and S_final are those of gdr_fwd_chunked up to rounding (always one
 * scan chain per (b, h): the segment-parallel scan is not used here).
 */
int gdr_fwd_chunked_keep(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                         const void *q, const void *k, const void *v,
                         const float *beta, int alpha_mode, const float *log_alpha,
                         const float *S0, void *o, float *S_final,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gdr_bwd_chunked without the forward's recomputation, for the workspace a
 * gdr_fwd_chunked_keep call filled: the same sizes, dtype, alpha_mode, C and
 * inputs (q, k, v, beta, log_alpha, S0), the workspace unchanged since.
 * Arguments, checks and errors as for gdr_bwd_chunked, whose results it
 * then gives bit for bit.  A workspace that does not hold what such a call
 * left gives meaningless gradients, but no access outside the arrays.
 */
int gdr_bwd_chunked_kept(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                         const void *q, const void *k, const void *v,
                         const float *beta, int alpha_mode, const float *log_alpha,
                         const float *S0, const void *dO, const float *dS_final,
                         void *dq, void *dk, void *dv, float *dbeta, float *dlog_alpha,
                         float *dS0, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of device workspace gdr_fwd_varlen needs (0 when N * H == 0), or
 * (size_t)-1 for invalid or unsupported sizes.  It is sized for any split
 * of the T tokens into N sequences: chunk records for at most
 * (T + N (C' - 1)) / C' chunks per head (C' = 32, or 16 for GDR_F32 or
 * C == 16), plus three ints per sequence.
 */
size_t gdr_fwd_varlen_workspace_size(int N, int H, int T, int d_k, int d_v, int C,
                                     int dtype, int alpha_mode);

/*
 * Chunkwise forward over a packed batch of N sequences of different lengths
 * (prefill of several prompts in one call).  The sequences lie back to back
 * on one token axis of T tokens per head; sequence n owns tokens
 * [cu_seqlens[n], cu_seqlens[n + 1]) and runs the recurrence of
 * gdr_fwd_chunked from its own initial state to its own final state.  Chunks
 * never straddle two sequences, so each sequence's result is the one a
 * separate call would give, up to rounding.  ("linear attention and its
 * gated descendants", "Chunkwise Parallel Form", applied per sequence; the
 * chunk form itself is that of gdr_fwd_chunked.)
 *
 *   N, H       sequences and heads (>= 0; N * H == 0 => nothing to do)
 *   T          packed tokens per head (>= 0)
 *   cu_seqlens [N + 1] int32 in DEVICE memory, read by the kernels (no host
 *              synchronisation): cumulative offsets, cu_seqlens[0] = 0,
 *              non-decreasing, cu_seqlens[N] = T.  Offsets outside [0, T]
 *              are clamped and a decreasing one gives an empty sequence;
 *              tokens no sequence covers are left unwritten in o.  No such
 *              input makes the library touch memory outside the arrays.
 *   q, k       [H][T][d_k];  v, o [H][T][d_v] (dtype)
 *   beta       [H][T] float
 *   log_alpha  NULL | [H][T] | [H][T][d_k] float, as for gdr_fwd_chunked
 *   S0         NULL => zero initial states, else [N][H][d_v][d_k] float
 *   S_final    NULL or [N][H][d_v][d_k] float (may equal S0); an empty
 *              sequence's final state is its initial state
 *   workspace  at least gdr_fwd_varlen_workspace_size(...) bytes
 *   prologue   gdr_prologue bits, as for gdr_fwd_chunked_ex
 * Other arguments, alignment, aliasing rules and errors as for
 * gdr_fwd_chunked (cu_seqlens 4-byte aligned, and it must not overlap o,
 * S_final or the workspace).  Always one scan chain per (sequence, head):
 * the segment-parallel scan of gdr_fwd_chunked is not used here.
 */
int gdr_fwd_varlen(int N, int H, int T, const int *cu_seqlens, int d_k, int d_v, int C, int dtype,
                   const void *q, const void *k, const void *v,
                   const float *beta, int alpha_mode, const float *log_alpha,
                   const float *S0, void *o, float *S_final,
                   void *workspace, size_t workspace_bytes, hipStream_t stream,
                   unsigned prologue);

/*
 * One recurrent decode step for N sequences x H heads (the constant-memory
 * inference form: "linear attention and its gated descendants", "Recurrent
 * Linear Attention for Inference": O(d^2) work and memory per token).  The
 * state is read and written once; o_t is read after the write.
 *
 *   N, H       sequences and heads (>= 0; 0 => nothing to do)
 *   d_k, d_v   64 or 128
 *   dtype      GDR_F32 or GDR_BF16 (type of q, k, v, o)
 *   q, k       [N][H][d_k];  v [N][H][d_v]
 *   beta       [N][H] float
 *   alpha_mode as for gdr_fwd_chunked; log_alpha NULL | [N][H] | [N][H][d_k]
 *              (no lower bound is needed in this entry point)
 *   S          [N][H][d_v][d_k] float, updated in place
 *   o          [N][H][d_v] (dtype); must not overlap any input or S
 */
int gdr_decode_step(int N, int H, int d_k, int d_v, int dtype,
                    const void *q, const void *k, const void *v,
                    const float *beta, int alpha_mode, const float *log_alpha,
                    float *S, void *o, hipStream_t stream);

/* gdr_decode_step with the input-side steps of `prologue` (gdr_prologue). */
int gdr_decode_step_ex(int N, int H, int d_k, int d_v, int dtype,
                       const void *q, const void *k, const void *v,
                       const float *beta, int alpha_mode, const float *log_alpha,
                       float *S, void *o, hipStream_t stream, unsigned prologue);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */

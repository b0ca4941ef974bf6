/*
 * kdn.h -- C ABI of the MI355X (gfx950) Kalman Delta Network mixer library.
 *
 * The library computes the forward recurrence of the scan-compatible Kalman
 * Delta Network (KDN) mixer and its single-token decode step, as defined in
 * "Kalman Delta Networks: Uncertainty-aware Associative Memory" (summary
 * page, method steps 1-5 and the closing isotropic sentence; English page,
 * section 3).  Per (batch, head) pair and token t, with fp32 state:
 *
 *   Diagonal variant (uncertainty p has one entry per key channel):
 *     p_hat = alpha_t^2 * p + omega_t                       predict
 *     kappa = p_hat * k_t / (r_t + sum_i p_hat_i k_t,i^2)    Kalman gain
 *     S     = diag(alpha_t) S
 *             + kappa (v_t - (diag(alpha_t) S)^T k_t)^T      residual write
 *     o_t   = S^T q_t                                        readout (after the write)
 *     p     = p_hat / (1 + (mu / r_t) k_t^2 * p_hat)         mean-field posterior
 *
 *   Isotropic variant (one uncertainty scalar b per head; alpha_t, omega_t
 *   are scalars per head-token):
 *     b_hat = alpha_t^2 b + omega_t / d_k
 *     kappa = k_t * b_hat / (r_t + b_hat |k_t|^2)
 *     S, o_t as above with the scalar decay alpha_t
 *     b     = b_hat / (1 + (mu / (d_k r_t)) |k_t|^2 b_hat)
 *
 *   Isotropic variant with per-channel decay (KDN_ISOTROPIC_CHANNEL, the
 *   general form of that sentence): alpha_t has one entry per key channel
 *   and the memory decays by diag(alpha_t) as in the diagonal variant;
 *   omega_t and r_t are scalars per head-token; the uncertainty scalar is
 *   predicted with the trace projection a_t = (1/d_k) sum_i alpha_t,i^2:
 *     b_hat = a_t b + omega_t / d_k;  kappa, b as in the isotropic variant.
 *   Shapes: alpha [.., dk], omega [..] (no dk), p [B,H].
 *
 *   Diagonal variant with grouped observation noise (KDN_DIAGONAL_GROUPED;
 *   "Memory by Design: Probabilistic Sequence Layers", per-column and grouped
 *   observation noise): the noise covariance is block diagonal over groups of
 *   64 value columns, diag[r_1 I, ..., r_G I] with G = d_v / 64, so each
 *   group keeps its own uncertainty p_g and gain; the groups share q, k,
 *   alpha, omega, and each is the diagonal recurrence above on its columns
 *   with r_t,g.  Shapes: r [.., G], p0 / p_T / the decode p [B,H,G,dk]
 *   (kdn_backward: dr [.., G], dp_T / dp0 [B,H,G,dk]).
 *
 * Initial state: S_0 = S0 (or zero when S0 is NULL); p_0 = p0 (or c0[h] on
 * every channel when p0 is NULL).  No 1/sqrt(d_k) scaling is applied to q.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers (HIP device memory of the
 *    current device), row-major and contiguous.  The caller owns every buffer;
 *    the library allocates no device memory and keeps no state between calls
 *    apart from a thread-local error message.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream).  KDN_OK means the work was enqueued.
 *  - Arguments are validated on the host before any launch.  On any error
 *    nothing is launched and nothing is written; kdn_last_error() describes
 *    the problem.  No C++ exception crosses the ABI.
 *  - Value preconditions are documented, not checked on the device:
 *    r > 0, c0 > 0 (or p0 > 0), 0 < alpha <= 1, omega >= 0.  Violations give
 *    NaN/Inf results, not errors.  mu must be finite and >= 0 (checked).
 *  - Results are deterministic: repeated calls with the same inputs give
 *    bit-identical outputs.
 *  - dtype KDN_BF16: q, k, v, alpha, omega, r are bfloat16 and o is written
 *    as bfloat16 (round to nearest even).  KDN_F32: all of them are float.
 *    c0, S0, p0, S_T, p_T and the decode state are always float.
 *  - Supported sizes: d_k and d_v in {64, 128}; B, T, H, N >= 0 (zero sizes
 *    are valid: with T = 0 the forward only writes S_T = S_0, p_T = p_0).
 *    Anything else returns KDN_ERR_UNSUPPORTED or KDN_ERR_SHAPE.
 */
#ifndef KDN_H
#define KDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kdn_variant { KDN_DIAGONAL = 0, KDN_ISOTROPIC = 1, KDN_ISOTROPIC_CHANNEL = 2, KDN_DIAGONAL_GROUPED = 3 };
enum kdn_dtype { KDN_F32 = 0, KDN_BF16 = 1 };
enum kdn_status {
    KDN_OK = 0,
    KDN_ERR_NULL = 1,        /* a required pointer is NULL */
    KDN_ERR_SHAPE = 2,       /* a size is negative or the element count overflows */
    KDN_ERR_UNSUPPORTED = 3, /* unsupported variant, dtype, d_k, d_v or algorithm */
    KDN_ERR_VALUE = 4,       /* mu is negative or not finite */
    KDN_ERR_HIP = 5,         /* the HIP runtime refused a launch */
    KDN_ERR_ALIAS = 6,       /* an output overlaps an input it may not overlap */
    KDN_ERR_WORKSPACE = 7    /* the workspace is missing, too small or misaligned */
};
/* forward algorithms (kdn_forward_algo).  The chunked algorithm takes bf16
 * inputs (dk and dv are 64 or 128 for every algorithm), q, k, v, alpha and omega
 * 16-byte aligned and o 8-byte aligned; KDN_ALGO_AUTO uses it whenever these
 * hold and the recurrent kernel otherwise, and an explicit KDN_ALGO_CHUNKED*
 * call outside them returns KDN_ERR_UNSUPPORTED.  One chunked workgroup
 * handles one (batch, head) pair and 64 value columns, or 32 when that
 * leaves more than half of the device's compute units idle (AUTO and
 * CHUNKED choose; _WIDE and _NARROW force a width).  Both algorithms are
 * valid for every 0 < alpha <= 1.  The chunked form scales its matrix
 * operands by the decay over at most one half-chunk (16 tokens); a chunk
 * whose half-chunk decay falls below 2^-96 on some channel (a geometric mean
 * below about 0.015 per token) is outside that form, and its workgroup
 * finishes the sequence with the token recurrence from that chunk on: same
 * results, slower for that (batch, head) pair.  The chunked form's operand
 * scaling leaves 2^31 of headroom for |q|, |k| and p_hat |k|. */
enum kdn_algo {
    KDN_ALGO_AUTO = 0,      /* the library picks (chunked when available) */
    KDN_ALGO_RECURRENT = 1, /* token-by-token recurrence, state in registers */
    KDN_ALGO_CHUNKED = 2,   /* chunkwise WY/UT form on matrix cores */
    KDN_ALGO_CHUNKED_WIDE = 3,   /* chunked, 64 value columns per workgroup */
    KDN_ALGO_CHUNKED_NARROW = 4  /* chunked, 32 value columns per workgroup (not with
                                    grouped observation noise) */
};

/*
 * kdn_forward -- the KDN layer recurrence over a whole sequence batch
 * (summary page, method steps 2-5; isotropic variant per its last sentence).
 *
 *   q, k        [B,T,H,dk]   dtype
 *   v           [B,T,H,dv]   dtype
 *   alpha,omega [B,T,H,dk]   dtype (KDN_ISOTROPIC: [B,T,H]; KDN_ISOTROPIC_CHANNEL:
 *                            alpha [B,T,H,dk], omega [B,T,H])
 *   r           [B,T,H]      dtype
 *   c0          [H]          float, per-head initial uncertainty; may be NULL
 *                            only when p0 is given
 *   mu                       information scale of the posterior update
 *   S0          [B,H,dk,dv]  float or NULL (zero initial memory)
 *   p0          [B,H,dk]     float or NULL (both isotropic variants: [B,H])
 *   o           [B,T,H,dv]   dtype, output
 *   S_T         [B,H,dk,dv]  float, output: memory after the last token
 *   p_T         [B,H,dk]     float, output (both isotropic variants: [B,H])
 * S_T may be the same buffer as S0 (the memory is continued in place).  No
 * other output may overlap an input or another output (KDN_ERR_ALIAS); in
 * particular p_T needs its own buffer.
 */
int kdn_forward(const void* q, const void* k, const void* v, const void* alpha,
                const void* omega, const void* r, const float* c0, float mu, int variant,
                int dtype, int B, int T, int H, int dk, int dv, const float* S0,
                const float* p0, void* o, float* S_T, float* p_T, void* stream);

/* kdn_forward with an explicit algorithm (enum kdn_algo); same arguments and
 * results up to floating-point rounding. */
int kdn_forward_algo(const void* q, const void* k, const void* v, const void* alpha,
                     const void* omega, const void* r, const float* c0, float mu, int variant,
                     int dtype, int B, int T, int H, int dk, int dv, const float* S0,
                     const float* p0, void* o, float* S_T, float* p_T, void* stream, int algo);

/*
 * kdn_forward_gated -- kdn_forward with the step before the recurrence done
 * inside the kernel (summary page, method step 1, and its core-method
 * paragraph: decay, process noise and observation noise come from the token
 * through sigmoid / softplus; the information scaling mu = d_k assumes
 * unit-norm keys).  q and k are raw: each [d_k] row is divided by
 * max(|row|, 1e-6) (queries like keys).  The three gate arguments hold
 * pre-activations, and the kernel uses
 *
 *   alpha = sigmoid(z_alpha)          decay
 *   omega = softplus(z_omega)         process noise
 *   r     = 0.01 + softplus(z_r)      observation noise (r_min = 0.01)
 *
 * in place of alpha, omega and r, in the layouts kdn_forward gives them for
 * the variant (KDN_DIAGONAL, KDN_ISOTROPIC or KDN_ISOTROPIC_CHANNEL;
 * KDN_DIAGONAL_GROUPED returns KDN_ERR_UNSUPPORTED).  Same dtypes, alignment,
 * algorithms, aliasing rules and results as kdn_forward_algo fed with the
 * normalised q, k and those values (up to fp32 rounding: about 1 ulp in each
 * gate and norm, at most about 6e-8 absolute in softplus); no extra memory is
 * read or written.
 */
int kdn_forward_gated(const void* q, const void* k, const void* v, const void* z_alpha,
                      const void* z_omega, const void* z_r, const float* c0, float mu, int variant,
                      int dtype, int B, int T, int H, int dk, int dv, const float* S0,
                      const float* p0, void* o, float* S_T, float* p_T, void* stream, int algo);

/*
 * kdn_forward_split -- kdn_forward (diagonal variant, bf16 inputs, the
 * chunked algorithm's alignment) for batches too small to fill the device:
 * each sequence is cut into segments that run concurrently.  Both
 * recurrences compose across a cut (summary page, method steps 4-5): the
 * uncertainty update of each channel is a Mobius map, so the uncertainty
 * entering a segment is p0 carried through the earlier segments' composed
 * maps; and with the gains known the memory update is affine in S, so over
 * segment g, S_end = Phi_g S_start + Psi_g.  One launch runs every segment
 * from S = 0 on the v columns (Psi_g) and from S = I on d_k extra columns
 * with v = 0 (Phi_g, and Phi_t^T q_t per token); then the segments' start
 * states are chained and o_t += (Phi_t^T q_t)^T S_start is added to the
 * tokens of every segment after the first.  About twice the arithmetic of
 * kdn_forward, spread over segments x (batch, head) x column tiles.
 *
 *   segments           0: chosen from the device (as many as fill its
 *                      compute units with one workgroup each, segments of at
 *                      least 2048 tokens, at most 16); > 0: about that many
 *                      (segment lengths are a multiple of 32 tokens).  When
 *                      the choice is 1 the call is kdn_forward_algo(AUTO).
 *   workspace          device memory of kdn_forward_split_workspace_size()
 *                      bytes (16-byte aligned, overlapping no argument), owned
 *                      by the caller; unused when no split is made.
 * Other arguments, layouts and results as kdn_forward, up to rounding: the
 * corrections add one bf16 rounding of Phi_t^T q_t and of S_start.  Errors
 * as kdn_forward_algo(KDN_ALGO_CHUNKED), plus KDN_ERR_UNSUPPORTED for another
 * variant or dtype, KDN_ERR_VALUE for segments < 0 and KDN_ERR_WORKSPACE /
 * KDN_ERR_ALIAS for the workspace.
 */
int kdn_forward_split(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                      const void* r, const float* c0, float mu, int variant, int dtype, int B, int T, int H, int dk,
                      int dv, const float* S0, const float* p0, void* o, float* S_T, float* p_T, int segments,
                      void* workspace, size_t workspace_bytes, void* stream);
/* Segments kdn_forward_split cuts each sequence into for these sizes and
 * segment request on the current device (1: no split; 0: invalid sizes). */
int kdn_forward_split_segments(int B, int T, int H, int dk, int dv, int segments);
/* Workspace bytes of kdn_forward_split for these sizes and segment request
 * (0 when no split is made or the sizes are invalid). */
size_t kdn_forward_split_workspace_size(int B, int T, int H, int dk, int dv, int segments);
/* The checks of kdn_forward_split without a launch. */
int kdn_validate_forward_split(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                               const void* r, const float* c0, float mu, int variant, int dtype, int B, int T, int H,
                               int dk, int dv, const float* S0, const float* p0, void* o, float* S_T, float* p_T,
                               int segments, void* workspace, size_t workspace_bytes);

/* kdn_forward_varlen with the step of kdn_forward_gated: raw q and k,
 * normalised per row inside the kernel, and z_alpha, z_omega, z_r
 * pre-activations in the layouts of alpha, omega and r (not
 * KDN_DIAGONAL_GROUPED).  Same checks and results as kdn_forward_varlen fed
 * with the normalised and gated values. */
int kdn_forward_varlen_gated(const void* q, const void* k, const void* v, const void* z_alpha,
                             const void* z_omega, const void* z_r, const int* cu_seqlens, const int* order,
                             const float* c0, float mu, int variant, int dtype, int N, int total, int H, int dk,
                             int dv, const float* S0, const float* p0, void* o, float* S_T, float* p_T,
                             void* stream, int algo);

/* kdn_step with the step of kdn_forward_gated: raw q and k, normalised per
 * row inside the kernel, and z_alpha, z_omega, z_r pre-activations in the
 * layouts of alpha, omega and r (not KDN_DIAGONAL_GROUPED).  S and p are
 * updated in place as by kdn_step. */
int kdn_step_gated(const void* q, const void* k, const void* v, const void* z_alpha, const void* z_omega,
                   const void* z_r, float mu, int variant, int dtype, int N, int H, int dk, int dv,
                   float* S, float* p, void* o, void* stream);

/* The host-side checks of kdn_forward_gated, with no device access. */
int kdn_validate_forward_gated(const void* q, const void* k, const void* v, const void* z_alpha,
                               const void* z_omega, const void* z_r, const float* c0, float mu, int variant,
                               int dtype, int B, int T, int H, int dk, int dv, const float* S0,
                               const float* p0, void* o, float* S_T, float* p_T, int algo);

/*
 * kdn_forward_varlen -- kdn_forward over N sequences of different lengths
 * packed along the token axis (a variable-length serving batch, e.g. the
 * prompts of several requests).  Each sequence is run through the same
 * recurrence from its own initial state, exactly as kdn_forward would run
 * it alone (summary page, method steps 2-5; isotropic variant per its last
 * sentence).  Sequence n owns the token rows [cu_seqlens[n],
 * cu_seqlens[n + 1]) of the packed tensors:
 *
 *   q, k        [total,H,dk]   dtype
 *   v           [total,H,dv]   dtype
 *   alpha,omega [total,H,dk]   dtype (KDN_ISOTROPIC: [total,H]; KDN_ISOTROPIC_CHANNEL:
 *                              alpha [total,H,dk], omega [total,H])
 *   r           [total,H]      dtype
 *   cu_seqlens  [N+1]          int32, DEVICE pointer, read by the kernels:
 *                              0 = cu[0] <= cu[1] <= ... <= cu[N] = total
 *   order       [N]            int32, DEVICE pointer or NULL: the order in which
 *                              the sequences are scheduled, a permutation of
 *                              0..N-1 (NULL = 0..N-1).  Longest first spreads
 *                              the work evenly over the GPU; results do not
 *                              depend on it.
 *   c0          [H]            float (as kdn_forward)
 *   S0          [N,H,dk,dv]    float or NULL;  p0 [N,H,dk] (isotropic variants: [N,H]) or NULL
 *   o           [total,H,dv]   dtype, output
 *   S_T         [N,H,dk,dv]    float, output;  p_T [N,H,dk] (isotropic variants: [N,H])
 *   algo                       enum kdn_algo, as kdn_forward_algo
 *
 * The offsets and the order live in device memory and are not inspected on
 * the host.  The kernels clamp every sequence into [0, total) and every order
 * entry into [0, N), so offsets that break the rule above, or an order that
 * is not a permutation, give meaningless values for the sequences involved,
 * never an access outside the tensors.  An empty sequence (cu[n] = cu[n + 1])
 * writes S_T = S_0 and p_T = p_0 for its heads.  Aliasing rules, dtypes and
 * the remaining checks are those of kdn_forward (cu_seqlens counts as an
 * input).
 */
int kdn_forward_varlen(const void* q, const void* k, const void* v, const void* alpha,
                       const void* omega, const void* r, const int* cu_seqlens, const int* order,
                       const float* c0,
                       float mu, int variant, int dtype, int N, int total, int H, int dk, int dv,
                       const float* S0, const float* p0, void* o, float* S_T, float* p_T,
                       void* stream, int algo);

/*
 * kdn_step -- one decode step for N independent sequences: exactly one
 * token of the recurrence applied to the carried state (constant-memory
 * decoding; summary page, prerequisites on linear attention, and English
 * page, introduction).
 *
 *   q, k        [N,H,dk]     dtype
 *   v           [N,H,dv]     dtype
 *   alpha,omega [N,H,dk]     dtype (KDN_ISOTROPIC: [N,H]; KDN_ISOTROPIC_CHANNEL:
 *                            alpha [N,H,dk], omega [N,H])
 *   r           [N,H]        dtype
 *   S           [N,H,dk,dv]  float, read and overwritten in place
 *   p           [N,H,dk]     float, read and overwritten (both isotropic variants: [N,H])
 *   o           [N,H,dv]     dtype, output
 */
int kdn_step(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
             const void* r, float mu, int variant, int dtype, int N, int H, int dk, int dv,
             float* S, float* p, void* o, void* stream);

/*
 * kdn_backward -- gradients of the forward recurrence, for training (the
 * reverse-mode adjoint of method steps 2-5 of the summary page, for all
 * three variants).  The scalar differentiated is
 *     L = sum dO (.) o + sum dS_T (.) S_T + sum dp_T (.) p_T
 * where (o, S_T, p_T) is what kdn_forward returns for the same inputs,
 * c0, mu, S0 and p0.
 *
 *   q, k, v, alpha, omega, r, c0, S0, p0, variant, dtype, sizes: as kdn_forward
 *   dO    [B,T,H,dv]   dtype, may be NULL (zero)
 *   dS_T  [B,H,dk,dv]  float, may be NULL (zero)
 *   dp_T  [B,H,dk]     float ([B,H] for both isotropic variants, [B,H,dv/64,dk] for
 *                      grouped observation noise), may be NULL (zero)
 *   dq, dk, dv, dalpha, domega, dr: float outputs in the layouts of
 *                      q, k, v, alpha, omega, r
 *   dS0   [B,H,dk,dv]  float output (gradient with respect to S0, or to the
 *                      zero initial memory when S0 is NULL)
 *   dp0   [B,H,dk]     float output ([B,H] for both isotropic variants)
 *   dc0   [H]          float output, may be NULL: the sum of dp0 over the
 *                      batch and the channels, which is the gradient with
 *                      respect to c0 when p0 is NULL
 *   workspace          device memory of at least
 *                      kdn_backward_workspace_size_for(variant, dtype, ...)
 *                      bytes, 16-byte aligned (the recomputation checkpoints
 *                      and per-token sums); its contents on entry do not
 *                      matter.  A larger workspace lets the chunked path take
 *                      longer slabs of tokens (fewer launches) and the token
 *                      path more pairs at once; the results do not depend on
 *                      its size
 *
 * S0, dS_T, dS0 and dv must be 8-byte aligned (KDN_ERR_UNSUPPORTED
 * otherwise) and the workspace 16-byte aligned (KDN_ERR_WORKSPACE).  No output may overlap
 * an input, another output or the workspace (KDN_ERR_ALIAS).  The diagonal
 * variant with bf16 inputs and 16-byte aligned q, k, v, alpha, omega and dO
 * runs its memory adjoint in chunk form on the matrix cores (bf16 operands,
 * fp32 accumulation and state), after a checkpoint sweep of the chunked
 * forward.  That sweep keeps the chunk-start states in bf16 (the precision in
 * which the adjoint's products take them), and the adjoint runs over slabs of
 * tokens from the last, so that its per-token buffers hold one slab.
 * (Batch, head) pairs whose decays leave the chunked form's range take the
 * token recurrence's adjoint, as do the other variants and fp32 inputs (fp32
 * throughout); on the chunked path's workspace it takes the pairs in rounds
 * of as many as fit.  Calls are asynchronous on `stream` like kdn_forward,
 * and the results are bitwise repeatable.
 */
int kdn_backward(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                 const void* r, const float* c0, float mu, int variant, int dtype, int B, int T,
                 int H, int dk, int dv, const float* S0, const float* p0, const void* dO,
                 const float* dS_T, const float* dp_T, float* dq, float* dk_out, float* dv_out,
                 float* dalpha, float* domega, float* dr, float* dS0, float* dp0, float* dc0,
                 void* workspace, size_t workspace_bytes, void* stream);
/*
 * kdn_backward_noalloc -- kdn_backward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight training or serving loops,
 * harnesses that forbid hipMalloc.  There is no workspace argument: the
 * library's static device scratch of KDN_NOALLOC_SCRATCH_BYTES takes its
 * place.  Each device holds its own copy of the scratch from the library's
 * loading on that device until the process ends.  Same arguments (minus the
 * workspace), checks, kernels and results (bit for bit) as kdn_backward.
 *  - Sizes whose workspace (kdn_backward_workspace_size_for) exceeds the
 *    scratch return KDN_ERR_WORKSPACE and launch nothing.
 *  - Nothing is allocated: no hipMalloc, hipFree or allocating library call.
 *  - Every call on one device shares that device's scratch and leaves its
 *    contents behind (the kernels need none on entry).  Calls that overlap in
 *    time on one device (two streams, two host threads) race on it and give
 *    undefined results: order them.
 */
#define KDN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int kdn_backward_noalloc(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                         const void* r, const float* c0, float mu, int variant, int dtype, int B, int T,
                         int H, int dk, int dv, const float* S0, const float* p0, const void* dO,
                         const float* dS_T, const float* dp_T, float* dq, float* dk_out, float* dv_out,
                         float* dalpha, float* domega, float* dr, float* dS0, float* dp0, float* dc0,
                         void* stream);

/* Workspace bytes with which kdn_backward runs every variant and dtype at
 * these sizes with all (batch, head) pairs at once (0 when B*H*T == 0):
 * B*H*(dv/64)*(ceil(T/32)*(64*dk + 8*dk) + 32*64*dk + 5*T*dk)*4 plus B*H*4
 * rounded up to 256 (the token path's checkpoints and stash per 64-column
 * tile, its per-token partial sums and uncertainties per tile, and one range
 * flag per (batch, head) pair). */
size_t kdn_backward_workspace_size(int B, int T, int H, int dk, int dv);
/* The smallest workspace kdn_backward accepts for this variant and dtype
 * (0 when B*H*T == 0).  For KDN_DIAGONAL with bf16 inputs and dk, dv in
 * {64, 128}, the chunked path's: with U = B*H pairs, n = ceil(T/32) chunks
 * and a slab of S = min(32*n, max(512, 65536/U rounded up to 512)) tokens,
 * about U*(dv/64)*n*dk*128 (bf16 chunk-start states) + U*n*dk*4 (chunk-start
 * uncertainties) + U*T*32 (per-token sums) + U*dk*dv*4 (the state's
 * cotangent between slabs) + U*S*dk*(dv/4 + 4) (one slab's tile sums and
 * uncertainties) bytes, each region rounded up to 256, and never less than
 * the flags plus one pair's token-path workspace (0.874 GB at B=8, T=4096,
 * H=16, dk=dv=128).  Otherwise kdn_backward_workspace_size(). */
size_t kdn_backward_workspace_size_for(int variant, int dtype, int B, int T, int H, int dk, int dv);
int kdn_validate_backward(const void* q, const void* k, const void* v, const void* alpha,
                          const void* omega, const void* r, const float* c0, float mu, int variant,
                          int dtype, int B, int T, int H, int dk, int dv, const float* S0,
                          const float* p0, const void* dO, const float* dS_T, const float* dp_T,
                          float* dq, float* dk_out, float* dv_out, float* dalpha, float* domega,
                          float* dr, float* dS0, float* dp0, float* dc0, void* workspace,
                          size_t workspace_bytes);

/* Host-only argument checks of kdn_forward / kdn_step / kdn_forward_varlen / kdn_backward: the same checks the
 * entry points run, with no device access and no launch.  Return a status. */
int kdn_validate_forward(const void* q, const void* k, const void* v, const void* alpha,
                         const void* omega, const void* r, const float* c0, float mu,
                         int variant, int dtype, int B, int T, int H, int dk, int dv,
                         const float* S0, const float* p0, void* o, float* S_T, float* p_T,
                         int algo);
int kdn_validate_step(const void* q, const void* k, const void* v, const void* alpha,
                      const void* omega, const void* r, float mu, int variant, int dtype, int N,
                      int H, int dk, int dv, float* S, float* p, void* o);
int kdn_validate_forward_varlen(const void* q, const void* k, const void* v, const void* alpha,
                                const void* omega, const void* r, const int* cu_seqlens,
                                const int* order, const float* c0, float mu, int variant, int dtype, int N, int total,
                                int H, int dk, int dv, const float* S0, const float* p0, void* o,
                                float* S_T, float* p_T, int algo);

/* Static description of a status code (never NULL). */
const char* kdn_status_string(int status);
/*
 * kdn_backward_gated -- kdn_backward of the gated layer (kdn_forward_gated):
 * q and k are raw, z_alpha, z_omega, z_r the gate pre-activations (layouts
 * of alpha, omega and r; not KDN_DIAGONAL_GROUPED).  dq and dk receive the
 * gradients with respect to the raw rows, dz_alpha, dz_omega, dz_r those
 * with respect to the pre-activations (fp32, same layouts):
 *   dx = (dx_hat - x_hat (x_hat . dx_hat)) / |x|   (dx_hat / 1e-6 where
 *        |x| < 1e-6),
 *   dz_alpha = d alpha * sigmoid(z) sigmoid(-z),  dz_omega = d omega * sigmoid(z),
 *   dz_r = d r * sigmoid(z).
 * Everything else as kdn_backward, except the workspace: at least
 * kdn_backward_gated_workspace_size_for(variant, dtype, ...) bytes, 16-byte
 * aligned; the fp32 copies take its last bytes and the adjoint everything
 * before them.
 */
int kdn_backward_gated(const void* q, const void* k, const void* v, const void* z_alpha, const void* z_omega,
                       const void* z_r, const float* c0, float mu, int variant, int dtype, int B, int T,
                       int H, int dk, int dv, const float* S0, const float* p0, const void* dO,
                       const float* dS_T, const float* dp_T, float* dq, float* dk_out, float* dv_out,
                       float* dz_alpha, float* dz_omega, float* dz_r, float* dS0, float* dp0, float* dc0,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of kdn_backward_gated: the adjoint's workspace
 * (kdn_backward_workspace_size) rounded up to 256 bytes, then fp32 copies of
 * the normalised q and k, of v and dO, and the gated alpha, omega, r, each
 * rounded up to 256 bytes.
 * 0 for negative sizes, an unknown variant or grouped noise. */
size_t kdn_backward_gated_workspace_size(int variant, int B, int T, int H, int dk, int dv);
/* The smallest workspace kdn_backward_gated accepts for this variant and
 * dtype: kdn_backward_workspace_size_for(variant, dtype, ...) rounded up to
 * 256 bytes, then the same fp32 copies (2.49 GB for the diagonal bf16 form at
 * B=8, T=4096, H=16, dk=dv=128).  0 as kdn_backward_gated_workspace_size. */
size_t kdn_backward_gated_workspace_size_for(int variant, int dtype, int B, int T, int H, int dk, int dv);

/* Detail of the last error on the calling thread ("" if none). */
const char* kdn_last_error(void);
/* ABI version: major * 10000 + minor * 100 + patch. */
int kdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDN_H */

/*
 * la.h -- C ABI of the MI355X (gfx950) kernelized linear-attention library.
 *
 * The method (Katharopoulos et al., "Transformers are RNNs: Fast
 * Autoregressive Transformers with Linear Attention", ICML 2020), as stated
 * on the pages this library is built from:
 *   [review]  nubint.ai, "[Paper Review] Transformers are RNNs: ...",
 *             section "Proposed method".
 *   [summary] paperlayer.ai, "Transformers are RNNs: ..." summary of arXiv
 *             2006.16236v3, sections 3.2, 3.2.1, 3.3, 3.3.1, 3.3.2, 3.4 and
 *             appendix "A. Gradient Derivation".
 *   [deck]    zhengyuhong.cn, "Transformers are RNNs: ... 解读", slides 3-4.
 *
 * Feature map phi(x) = elu(x) + 1 ([deck] slide 3; [summary] 3.2.1): x + 1
 * for x > 0, exp(x) otherwise.  No 1/sqrt(D) scale and no epsilon: phi > 0
 * keeps every denominator positive.
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, row-major, in device memory owned by the caller:
 *     q, k are [B][H][N][D]; v, out, dout are [B][H][N][M] (decode: no N).
 *     dt gives the element type of q, k, v, out, dout, dq, dk, dv (fp32 or
 *     bf16).  All state and accumulation is fp32 inside the kernels.  Matrix
 *     products take bf16 operands (bf16 I/O: the inputs as they are, the
 *     carried fp32 state rounded once per product); with fp32 I/O the
 *     forwards at every head size and the backwards at D <= 64 split every
 *     fp32 operand into two bf16 parts, x = hi + lo within 2^-16 |x|, and
 *     form the exact product of the split values, while the other kernels
 *     (the backwards at D >= 80, the polynomial kernel, the random-feature
 *     projection) use fp32 products.
 *   - Head sizes: the forwards (la_forward_causal, _state, _features,
 *     _noalloc, _noncausal), the backwards and la_decode_step take D, M (F
 *     for features) any multiple of 16 from 16 to 128 -- D, M in {32, 64}
 *     run the fused single-launch forwards and the two-state backward
 *     kernels, the others a path that splits V (and dout) into 16-column
 *     groups, one wavefront each (forward: per-segment sums, scan, outputs;
 *     backward: the same sums and scan, a dQ pass, the scan in reverse, a
 *     dK/dV pass); the polynomial kernel and the random features take D, M
 *     in {32, 64}.  Other sizes return LA_ERR_UNSUPPORTED.  B, H, N >= 1.
 *   - Every tensor pointer must be 16-byte aligned; outputs must not overlap
 *     any input or each other.
 *   - Calls are asynchronous on `stream` (0 = the null stream).  The library
 *     never allocates, frees or synchronizes; scratch memory is the caller's
 *     `workspace`, at least la_workspace_size(...) bytes, 256-byte aligned.
 *     Workspace contents need no initialization and are clobbered.
 *   - Argument errors are reported before anything is launched and leave all
 *     buffers untouched.  LA_ERR_HIP reports a failed launch.  Non-finite
 *     inputs are not errors; they propagate to every output that depends on
 *     them.  The matrix products also carry them a little further, since
 *     0 * NaN = NaN: a non-finite key or value (or, in the backward, output
 *     gradient) can reach outputs of the other tokens of its 16-token chunk
 *     that do not depend on it; outputs outside that chunk that do not
 *     depend on it are unaffected (bit-identical).
 *   - The library keeps no global state beyond a process-wide call counter
 *     (it tags the forwards' cross-workgroup flags, so the workspace needs
 *     no clearing between calls), the wait limit of la_set_wait_limit and a
 *     per-device cache of the compute-unit count; calls on different streams
 *     are independent as long as their buffers (workspace included) are
 *     disjoint.
 *   - The forwards (la_forward_causal, _state, _features, _noncausal) may be
 *     captured into a HIP graph: a captured call records a small kernel that
 *     clears its hand-off flags before the forward itself, so every replay
 *     is correct even with changed inputs.
 *
 * Co-residency contract of the fused forwards.  Each (b, h) is split into blocks
 * of 8 wavefronts that exchange fp32 state through the workspace and wait for
 * each other with bounded waits.  The plan gives a head at most
 * min(64, number of CUs of the current device) blocks (one CU holds a block,
 * and blocks are dispatched in index order, so every block of a head can be
 * resident once the heads before it are done); the CU count is read from the
 * device that is current when the call is made.  Only other work that keeps
 * most CUs busy for the whole length of a wait (about a second) can make a
 * wait give up; the call then still returns LA_OK but its output is wrong,
 * and la_workspace_check reports LA_ERR_TIMEOUT.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_ABI_VERSION 10

/* The enums are int-sized in C; C++ gets the same fixed underlying type, so
 * any int a C caller passes (an unknown dtype, op or status included) is a
 * valid value to validate rather than undefined behaviour. */
#ifdef __cplusplus
#define LA_ENUM_BASE : int
#else
#define LA_ENUM_BASE
#endif

typedef enum la_dtype_e LA_ENUM_BASE { LA_DTYPE_F32 = 0, LA_DTYPE_BF16 = 1 } la_dtype_t;

typedef enum la_status_e LA_ENUM_BASE {
    LA_OK = 0,
    LA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misalignment, overlap */
    LA_ERR_UNSUPPORTED = 2,      /* D or M outside the supported set, unknown dtype,
                                    or a shape beyond the kernels' plan limits */
    LA_ERR_WORKSPACE = 3,        /* workspace missing, misaligned or too small */
    LA_ERR_HIP = 4,              /* a kernel launch (or a copy) failed */
    LA_ERR_TIMEOUT = 5           /* la_workspace_check: a hand-off wait gave up */
} la_status_t;

typedef enum la_op_e LA_ENUM_BASE {
    LA_OP_FWD_CAUSAL = 0,     /* la_forward_causal, la_forward_causal_state,
                                 la_forward_causal_features (with D = F) */
    LA_OP_FWD_NONCAUSAL = 1,  /* la_forward_noncausal */
    LA_OP_BWD_CAUSAL = 2,     /* la_backward_causal */
    LA_OP_BWD_NONCAUSAL = 3,  /* la_backward_noncausal */
    LA_OP_FWD_CAUSAL_POLY2 = 4,   /* la_forward_causal_poly2, la_forward_causal_poly2_state */
    LA_OP_FWD_NONCAUSAL_POLY2 = 5, /* la_forward_noncausal_poly2 */
    LA_OP_BWD_CAUSAL_POLY2 = 6     /* la_backward_causal_poly2 */
} la_op_t;

/*
 * Causal forward ([deck] slide 4; [review] "Proposed method"; [summary] 3.3,
 * 3.3.2 parallel training-time form):
 *   S_i = S_{i-1} + phi(K_i) V_i^T,  Z_i = Z_{i-1} + phi(K_i),
 *   out_i = phi(Q_i)^T S_i / (phi(Q_i)^T Z_i),   S_0 = 0, Z_0 = 0,
 * independently for each (b, h).  Token i sees itself (j <= i).
 * q, k: [B][H][N][D]; v: [B][H][N][M] (inputs, read only).
 * out: [B][H][N][M] (output, fully written).
 * The workgroups of one (b, h) exchange state through the workspace and
 * wait for each other (see the co-residency contract above).  Diagnostic:
 * if a wait ever gave up, the call or-s 1 into the 32-bit error word at
 * byte 4 of the workspace and its output is wrong; the library never clears
 * that word by itself: la_workspace_check reads (and optionally clears) it.
 */
la_status_t la_forward_causal(const void *q, const void *k, const void *v, void *out,
                              int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                              la_dtype_t dt, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * la_forward_causal for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and kernels, with no workspace argument
 * and no allocation of any kind.  Its workspace is a library-owned static
 * device array of LA_NOALLOC_SCRATCH_BYTES (16 MiB), one per GPU, held until
 * the process ends; shapes whose workspace (la_workspace_size(
 * LA_OP_FWD_CAUSAL, ...)) exceeds it return LA_ERR_WORKSPACE before anything
 * is launched (B1 H8 N65536 D=M=64 needs about 8.1 MiB).  The array keeps
 * the last call's contents and needs no clearing (the hand-off flags are
 * tagged per call).  All calls on one GPU share it: calls that can overlap
 * in time on one GPU (other streams, other threads) race and give wrong
 * results; calls ordered on one stream are safe.  `stream` must belong to
 * the current device.  A hand-off wait that gives up is not reported (the
 * error word lives in the array).  Arguments and errors otherwise as
 * la_forward_causal.
 */
#define LA_NOALLOC_SCRATCH_BYTES (16u << 20)
la_status_t la_forward_causal_noalloc(const void *q, const void *k, const void *v, void *out,
                                      int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                                      la_dtype_t dt, hipStream_t stream);

/*
 * Causal forward continuing from a given recurrent state, and/or returning
 * the state after the last token ([summary] 3.3.2 and 3.4: the memory s_i,
 * z_i is all a step needs; 4.2.1: only s_i and z_i are kept between pixels;
 * 4.2.2: image completion conditions on a prefix and then generates):
 *   S_0 = s0, Z_0 = z0 (zero when s0 = z0 = NULL), then the recurrence of
 *   la_forward_causal for i = 1..N;  s_final = S_N, z_final = Z_N.
 * s0, s_final: [B][H][D][M] fp32; z0, z_final: [B][H][D] fp32 -- the layout
 * of la_decode_step's S and Z, so a prompt's forward hands its state to
 * decode directly, and a sequence split into consecutive pieces gives the
 * same outputs piece by piece.  s0/z0 are both NULL or both set, and so are
 * s_final/z_final (NULL: the final state is not written).  s_final == s0
 * and z_final == z0 update the state in place; any other overlap of a state
 * tensor with another buffer is LA_ERR_INVALID_ARGUMENT.  A start state
 * should be one a recurrence can reach (z0 with phi(q) . z0 + ... > 0);
 * the library does not check it.  Other arguments, workspace and
 * diagnostic word: as la_forward_causal (whose call equals this one with
 * all four state pointers NULL).
 */
la_status_t la_forward_causal_state(const void *q, const void *k, const void *v, void *out,
                                    const float *s0, const float *z0, float *s_final,
                                    float *z_final, int64_t B, int64_t H, int64_t N, int64_t D,
                                    int64_t M, la_dtype_t dt, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/*
 * Causal forward with the degree-2 polynomial kernel ([summary] 3.2.1: a
 * degree-2 polynomial kernel has an exact finite feature map).  Reading:
 * sim(q, k) = (q . k)^2, i.e. phi(x) = vec(x x^T) with D^2 features:
 *   out_i = sum_{j<=i} (q_i . k_j)^2 v_j / sum_{j<=i} (q_i . k_j)^2.
 * No feature map is applied to q, k beyond that (no elu).  q, k:
 * [B][H][N][D]; v, out: [B][H][N][M]; D, M in {32, 64} (LA_ERR_UNSUPPORTED
 * otherwise).  The kernels use the D (D + 1) / 2 distinct products q_a q_b,
 * a <= b, as features (the same sums as vec(x x^T)).  Workspace
 * la_workspace_size(LA_OP_FWD_CAUSAL_POLY2, ...): per segment one fp32 record
 * of the segment's feature state and its D x D normalizer sum (256 bytes when
 * each (b, h) is a single segment).  A query orthogonal to every earlier key
 * has a zero denominator; nothing guards it.  Errors as la_forward_causal.
 */
la_status_t la_forward_causal_poly2(const void *q, const void *k, const void *v, void *out,
                                    int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                                    la_dtype_t dt, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * Floats of one (b, h)'s polynomial-kernel state: the feature state
 * sum_j phi(k_j) v_j^T and the normalizer sum_j k_j k_j^T, in the library's own
 * tiled fp32 layout (opaque: only la_forward_causal_poly2_state and
 * la_decode_step_poly2 read or write it; all zeros is the empty prefix).
 * 0 for unsupported D, M.
 */
int64_t la_poly2_state_floats(int64_t D, int64_t M);

/*
 * la_forward_causal_poly2 that also writes, for every (b, h), the state
 * after its last token into state_final [B][H][la_poly2_state_floats(D, M)]
 * (fp32, caller-owned, 16-byte aligned, overlapping no other buffer), from
 * which la_decode_step_poly2 continues the sequence ([summary] 3.3.2: the
 * causal form is an RNN whose state is updated once per token).  Workspace
 * as la_forward_causal_poly2.  state_final NULL: LA_ERR_INVALID_ARGUMENT.
 */
la_status_t la_forward_causal_poly2_state(const void *q, const void *k, const void *v, void *out,
                                          float *state_final, int64_t B, int64_t H, int64_t N,
                                          int64_t D, int64_t M, la_dtype_t dt, void *workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/*
 * Non-causal forward with the degree-2 polynomial kernel ([summary] 3.2.1;
 * every key attends, as in the non-causal linear form):
 *   out_i = sum_j (q_i . k_j)^2 v_j / sum_j (q_i . k_j)^2.
 * Arguments as la_forward_causal_poly2; workspace
 * la_workspace_size(LA_OP_FWD_NONCAUSAL_POLY2, ...) (one record per segment,
 * also with a single segment: the (b, h) total).
 */
la_status_t la_forward_noncausal_poly2(const void *q, const void *k, const void *v, void *out,
                                       int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                                       la_dtype_t dt, void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * One decode step of the polynomial kernel for B*H streams ([summary] 3.3.2:
 * update the state with the new key and value, then read it out): q, k:
 * [B][H][D]; v, out: [B][H][M]; state [B][H][la_poly2_state_floats(D, M)]
 * fp32, updated in place (zeros for an empty prefix, or the state_final of
 * la_forward_causal_poly2_state).  Out is read after the update, so a run of
 * steps equals the causal forward over the same tokens.  D, M in {32, 64}.
 * The state must not overlap q, k, v or out.  Errors as la_decode_step.
 */
la_status_t la_decode_step_poly2(const void *q, const void *k, const void *v, float *state,
                                 void *out, int64_t B, int64_t H, int64_t D, int64_t M,
                                 la_dtype_t dt, hipStream_t stream);

/*
 * Gradients of sum(dout * out) for out = la_forward_causal_poly2(q, k, v)
 * ([summary] 3.2.1 for the kernel; 3.3.1: the gradient of the linear form in
 * linear time, through running sums in both directions).  With
 * s_ij = (q_i . k_j)^2 (j <= i), d_i = sum_j s_ij, g_i = dout_i / d_i,
 * h_i = -(dout_i . out_i) / d_i, e_ij = g_i . v_j + h_i:
 *   dq_i = 2 sum_{j<=i} e_ij (q_i . k_j) k_j,
 *   dk_j = 2 sum_{i>=j} e_ij (q_i . k_j) q_i,
 *   dv_j = sum_{i>=j} s_ij g_i,
 * computed with the D x D sums sum_j [v_j, 1]_m k_j k_j^T (forwards) and
 * sum_i [g_i, h_i]_m q_i q_i^T (backwards), one per column m.  out and d are
 * recomputed from the same forwards sums (so that the terms of the gradient,
 * which cancel, cancel to the sums' precision); out is not an argument.
 * q, k, dq, dk: [B][H][N][D]; v, dout, dv: [B][H][N][M]; dq, dk, dv are
 * outputs, fully written.  D, M in {32, 64}; bf16 or fp32, fp32 sums.
 * Workspace: la_workspace_size(LA_OP_BWD_CAUSAL_POLY2, ...) bytes (per token
 * the weights [g, h] in fp32, the segments' sums and one partial dq / dk per
 * block of columns m).  Results do not vary from run to run.  A zero
 * denominator (a query orthogonal to every earlier key) is not guarded.
 * Errors as la_backward_causal.
 */
la_status_t la_backward_causal_poly2(const void *q, const void *k, const void *v, const void *dout,
                                     void *dq, void *dk, void *dv,
                                     int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                                     la_dtype_t dt, void *workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * Random Fourier features ([summary] 5: approximating the RBF kernel with
 * random Fourier features is named as a feature map for reusing
 * softmax-pretrained models; the map is the standard construction):
 *   out[row][r] = sqrt(2/R) cos(sum_d x[row][d] omega[d][r] + bias[r]).
 * With omega ~ N(0, 1/sigma^2) and bias ~ U[0, 2 pi), drawn by the caller,
 * out(q) . out(k) estimates exp(-|q - k|^2 / (2 sigma^2)).
 * x: [B][H][N][D] in dt (input); omega: [D][R] fp32, bias: [R] fp32 (inputs);
 * out: [B][H][N][R] in dt (output, fully written).  D, R in {32, 64}.
 * No workspace.  The features can be negative: attention on them
 * (la_forward_causal_features) is only as well conditioned as its
 * denominators.
 */
la_status_t la_rff_features(const void *x, const float *omega, const float *bias, void *out,
                            int64_t B, int64_t H, int64_t N, int64_t D, int64_t R,
                            la_dtype_t dt, hipStream_t stream);

/*
 * Causal forward on features that are already applied ([summary] 3.2: any
 * feature map phi gives a kernel phi(q) . phi(k); 3.2.1: the map can be
 * chosen, e.g. elu + 1, a polynomial, or random features):
 *   out_i = sum_{j<=i} (fq_i . fk_j) v_j / sum_{j<=i} (fq_i . fk_j),
 * i.e. la_forward_causal with phi the identity.  fq, fk: [B][H][N][F]; v,
 * out: [B][H][N][M]; F, M multiples of 16 up to 128; workspace
 * la_workspace_size(LA_OP_FWD_CAUSAL, B, H, N, F, M, dt).  Features of any
 * sign are accepted and nothing guards the denominators: a zero or negative
 * one gives what the division gives.  Errors and diagnostic word as
 * la_forward_causal.
 */
la_status_t la_forward_causal_features(const void *fq, const void *fk, const void *v, void *out,
                                       int64_t B, int64_t H, int64_t N, int64_t F, int64_t M,
                                       la_dtype_t dt, void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * Non-causal forward through associativity ([review] "Proposed method";
 * [summary] 3.2; [deck] slide 3): S = sum_j phi(K_j) V_j^T and
 * Z = sum_j phi(K_j) over all N tokens of each (b, h), then
 * out_i = phi(Q_i)^T S / (phi(Q_i)^T Z).  Same arguments as the causal call,
 * and the same execution: one launch whose workgroups of a (b, h) exchange
 * their partial sums through the workspace and wait for each other (bounded
 * waits; the same co-residency limits and diagnostic word at byte 4).
 */
la_status_t la_forward_noncausal(const void *q, const void *k, const void *v, void *out,
                                 int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                                 la_dtype_t dt, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Causal backward ([summary] 3.3.1 and appendix A: gradients through
 * cumulative sums, in linear time, never storing every S_i).  Given
 * dout = dL/dout for out = la_forward_causal(q, k, v), writes the gradients
 * with respect to the raw inputs (through phi and the denominator):
 *   dq, dk: [B][H][N][D];  dv: [B][H][N][M]  (outputs, fully written).
 * The forward quantities (denominators, out) are recomputed; out is not an
 * argument.  With g_i = dout_i / d_i and h_i = -(dout_i . out_i) / d_i:
 *   dL/dphi(Q_i) = S_i g_i + h_i Z_i,
 *   dL/dphi(K_j) = R_j V_j + u_j,  dv_j = R_j^T phi(K_j),
 *   R_j = sum_{i>=j} phi(Q_i) g_i^T,  u_j = sum_{i>=j} h_i phi(Q_i),
 * and dq = dL/dphi(Q) * phi'(Q), dk = dL/dphi(K) * phi'(K).
 */
la_status_t la_backward_causal(const void *q, const void *k, const void *v, const void *dout,
                               void *dq, void *dk, void *dv,
                               int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                               la_dtype_t dt, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * Non-causal backward: the gradients of la_forward_noncausal with every sum
 * over the whole sequence ([summary] 3.2: the non-causal form through
 * associativity; 3.3.1 and appendix A give the causal case, whose
 * derivation carries over with the mask removed).  With S, Z the full sums,
 * d_i = phi(Q_i) . Z, g_i = dout_i / d_i, h_i = -(dout_i . out_i) / d_i:
 *   dL/dphi(Q_i) = S g_i + h_i Z,
 *   dL/dphi(K_j) = R V_j + u,  dv_j = R^T phi(K_j),
 *   R = sum_i phi(Q_i) g_i^T,  u = sum_i h_i phi(Q_i)  (all i),
 * and dq = dL/dphi(Q) * phi'(Q), dk = dL/dphi(K) * phi'(K).
 * Arguments, layouts and errors as la_backward_causal; workspace sized by
 * la_workspace_size(LA_OP_BWD_NONCAUSAL, ...).
 */
la_status_t la_backward_noncausal(const void *q, const void *k, const void *v, const void *dout,
                                  void *dq, void *dk, void *dv,
                                  int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                                  la_dtype_t dt, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * One RNN-style decode step for B*H independent streams ([review] "Proposed
 * method": attention memory s and normalizer memory z with a two-step update;
 * [summary] 3.3.2 and 3.4; [deck] slide 4):
 *   S += phi(k) v^T;  Z += phi(k);  out = S^T phi(q) / (phi(q)^T Z).
 * The update comes first, so a sequence of steps reproduces the causal
 * forward.  q, k: [B][H][D]; v, out: [B][H][M] in dtype dt.
 * S: [B][H][D][M] fp32 and Z: [B][H][D] fp32 are read and updated in place;
 * the caller zeroes them before the first token and may save/restore them
 * between calls (they are the whole recurrent state).  No workspace.
 */
la_status_t la_decode_step(const void *q, const void *k, const void *v, float *S, float *Z,
                           void *out, int64_t B, int64_t H, int64_t D, int64_t M,
                           la_dtype_t dt, hipStream_t stream);

/*
 * Reads the error word of a forward's workspace (see the co-residency
 * contract): waits for the work queued on `stream` (this call synchronizes,
 * unlike the others), returns LA_ERR_TIMEOUT if a hand-off wait of a call
 * that used this workspace gave up since the word was last cleared, LA_OK
 * otherwise; with `clear` != 0 it then zeroes the word.  A new workspace's
 * word holds whatever the memory held: clear it once (clear = 1, ignoring
 * the result) before relying on the report.  workspace: device memory of at
 * least 256 bytes, 256-byte aligned (else LA_ERR_WORKSPACE); LA_ERR_HIP if
 * the copy or the synchronization failed.
 */
la_status_t la_workspace_check(void *workspace, size_t workspace_bytes, int clear, hipStream_t stream);

/*
 * Process-wide limit on the polls one hand-off wait of the forwards makes
 * before it gives up (default 2^20, about a second; a negative value
 * restores the default); returns the previous limit.  A debugging and
 * testing aid: with 0 every wait that has anything to wait for gives up at
 * once, which lets a test see a give-up reported by la_workspace_check while
 * every kernel still exits normally.  Takes effect for calls made after it.
 */
int64_t la_set_wait_limit(int64_t polls);

/* Bytes of workspace `op` needs for this shape (0 if the shape is invalid).
 * The forwards' plan depends on the current device's CU count. */
size_t la_workspace_size(la_op_t op, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                         la_dtype_t dt);

/* Static, human-readable name of a status code. */
const char *la_status_string(la_status_t s);

/* LA_ABI_VERSION of the loaded library. */
int la_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_H */

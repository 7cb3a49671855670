// la_api.hip -- the C ABI declared in include/la.h: argument validation,
// workspace sizing, dispatch to the kernel launchers, and the forwards'
// diagnostics (error word, wait limit).
#include "la.h"
#include "la_internal.h"
#include "la_poly_grad.h"

namespace {

using la::align256;

struct Span {
    uintptr_t lo = 0, hi = 0;
};

Span span(const void *p, size_t bytes) {
    Span s;
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = s.lo + bytes;
    return s;
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t esize(la_dtype_t dt) { return dt == LA_DTYPE_F32 ? 4 : 2; }

constexpr int64_t kMaxElems = int64_t(1) << 40;

// any_size: every multiple of 16 up to 128 (decode, the forwards, the
// backwards); otherwise D, M in {32, 64} (polynomial and random-feature
// kernels).
la_status_t check_shape(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, la_dtype_t dt, bool any_size = false) {
    if (B < 1 || H < 1 || N < 1 || D < 1 || M < 1) return LA_ERR_INVALID_ARGUMENT;
    if (B > kMaxElems || H > kMaxElems || N > kMaxElems) return LA_ERR_INVALID_ARGUMENT;
    if (B * H > kMaxElems / N) return LA_ERR_INVALID_ARGUMENT;
    if (dt != LA_DTYPE_F32 && dt != LA_DTYPE_BF16) return LA_ERR_UNSUPPORTED;
    if (any_size ? !(la::head_size_ok(D) && la::head_size_ok(M)) : !la::fused_head_sizes(D, M))
        return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

// The forwards: the fused single-launch kernels for D, M in {32, 64}, the
// generic path for the other head sizes.
hipError_t launch_any_forward(bool causal, int dt, const void *q, const void *k, const void *v, void *out, int64_t BH,
                              int64_t N, int64_t D, int64_t M, float *ws, hipStream_t s,
                              la::StateIO sio = la::StateIO()) {
    if (la::fused_head_sizes(D, M)) return la::launch_forward(causal, dt, q, k, v, out, BH, N, D, M, ws, s, sio);
    return la::launch_forward_generic(causal, dt, q, k, v, out, BH, N, D, M, ws, s, sio);
}

bool forward_supported(bool causal, int64_t BH, int64_t N, int64_t D, int64_t M, size_t es) {
    return !la::fused_head_sizes(D, M) || la::forward_plan_supported(BH, N, D, M, es);
}

// Pointers: all non-null and 16-byte aligned; no output overlaps any other
// buffer (inputs may alias each other).
la_status_t check_buffers(const Span *in, int nin, const Span *outs, int nout) {
    for (int i = 0; i < nin; ++i)
        if (in[i].lo == 0 || (in[i].lo & 15)) return LA_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < nout; ++i) {
        if (outs[i].lo == 0 || (outs[i].lo & 15)) return LA_ERR_INVALID_ARGUMENT;
        for (int j = 0; j < nin; ++j)
            if (overlap(outs[i], in[j])) return LA_ERR_INVALID_ARGUMENT;
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], outs[j])) return LA_ERR_INVALID_ARGUMENT;
    }
    return LA_OK;
}

la_status_t check_workspace(void *ws, size_t have, size_t need, const Span *bufs, int nb) {
    if (need == 0) return LA_OK;
    if (ws == nullptr || !aligned(ws, 256) || have < need) return LA_ERR_WORKSPACE;
    const Span w = span(ws, need);
    for (int i = 0; i < nb; ++i)
        if (overlap(w, bufs[i])) return LA_ERR_WORKSPACE;
    return LA_OK;
}

la_status_t forward_common(bool causal, const void *q, const void *k, const void *v, void *out, int64_t B,
                           int64_t H, int64_t N, int64_t D, int64_t M, la_dtype_t dt, void *workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    la_status_t st = check_shape(B, H, N, D, M, dt, true);
    if (st != LA_OK) return st;
    const size_t es = esize(dt);
    const int64_t BH = B * H;
    const Span in[3] = {span(q, size_t(BH * N * D) * es), span(k, size_t(BH * N * D) * es),
                        span(v, size_t(BH * N * M) * es)};
    const Span o[1] = {span(out, size_t(BH * N * M) * es)};
    if ((st = check_buffers(in, 3, o, 1)) != LA_OK) return st;
    const Span all[4] = {in[0], in[1], in[2], o[0]};
    const size_t need = la::causal_workspace_bytes(BH, N, D, M);   // the same plan for both forwards
    if ((st = check_workspace(workspace, workspace_bytes, need, all, 4)) != LA_OK) return st;
    if (!forward_supported(causal, BH, N, D, M, es)) return LA_ERR_UNSUPPORTED;
    const hipError_t e = launch_any_forward(causal, dt == LA_DTYPE_F32 ? 0 : 1, q, k, v, out, BH, N, D, M,
                                            static_cast<float *>(workspace), stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

} // namespace

extern "C" {

la_status_t la_forward_causal(const void *q, const void *k, const void *v, void *out, int64_t B, int64_t H,
                              int64_t N, int64_t D, int64_t M, la_dtype_t dt, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    return forward_common(true, q, k, v, out, B, H, N, D, M, dt, workspace, workspace_bytes, stream);
}

la_status_t la_forward_causal_noalloc(const void *q, const void *k, const void *v, void *out, int64_t B,
                                      int64_t H, int64_t N, int64_t D, int64_t M, la_dtype_t dt,
                                      hipStream_t stream) {
    static_assert(la::kNoAllocScratchBytes == LA_NOALLOC_SCRATCH_BYTES, "scratch size in la.h");
    la_status_t st = check_shape(B, H, N, D, M, dt, true);
    if (st != LA_OK) return st;
    const size_t es = esize(dt);
    const int64_t BH = B * H;
    const Span in[3] = {span(q, size_t(BH * N * D) * es), span(k, size_t(BH * N * D) * es),
                        span(v, size_t(BH * N * M) * es)};
    const Span o[1] = {span(out, size_t(BH * N * M) * es)};
    if ((st = check_buffers(in, 3, o, 1)) != LA_OK) return st;
    if (la::causal_workspace_bytes(BH, N, D, M) > la::kNoAllocScratchBytes) return LA_ERR_WORKSPACE;
    if (!forward_supported(true, BH, N, D, M, es)) return LA_ERR_UNSUPPORTED;
    void *ws = la::noalloc_scratch();
    if (ws == nullptr) return LA_ERR_HIP;
    const hipError_t e = launch_any_forward(true, dt == LA_DTYPE_F32 ? 0 : 1, q, k, v, out, BH, N, D, M,
                                            static_cast<float *>(ws), stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status_t la_forward_causal_state(const void *q, const void *k, const void *v, void *out, const float *s0,
                                    const float *z0, float *s_final, float *z_final, int64_t B, int64_t H, int64_t N,
                                    int64_t D, int64_t M, la_dtype_t dt, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    la_status_t st = check_shape(B, H, N, D, M, dt, true);
    if (st != LA_OK) return st;
    if ((s0 == nullptr) != (z0 == nullptr) || (s_final == nullptr) != (z_final == nullptr))
        return LA_ERR_INVALID_ARGUMENT;
    const size_t es = esize(dt);
    const int64_t BH = B * H;
    const size_t sbytes = size_t(BH * D * M) * 4, zbytes = size_t(BH * D) * 4;
    // inputs: q, k, v and the start state unless it is updated in place (a
    // state tensor passed as both is checked once, as an output)
    Span in[5] = {span(q, size_t(BH * N * D) * es), span(k, size_t(BH * N * D) * es),
                  span(v, size_t(BH * N * M) * es)};
    int nin = 3;
    if (s0 != nullptr && s0 != s_final) in[nin++] = span(s0, sbytes);
    if (z0 != nullptr && z0 != z_final) in[nin++] = span(z0, zbytes);
    Span o[3] = {span(out, size_t(BH * N * M) * es)};
    int nout = 1;
    if (s_final != nullptr) {
        o[nout++] = span(s_final, sbytes);
        o[nout++] = span(z_final, zbytes);
    }
    if ((st = check_buffers(in, nin, o, nout)) != LA_OK) return st;
    Span all[8];
    int nall = 0;
    for (int i = 0; i < nin; ++i) all[nall++] = in[i];
    for (int i = 0; i < nout; ++i) all[nall++] = o[i];
    if ((st = check_workspace(workspace, workspace_bytes, la::causal_workspace_bytes(BH, N, D, M), all, nall)) !=
        LA_OK)
        return st;
    if (!forward_supported(true, BH, N, D, M, es)) return LA_ERR_UNSUPPORTED;
    la::StateIO sio;
    sio.s0 = s0;
    sio.z0 = z0;
    sio.s1 = s_final;
    sio.z1 = z_final;
    const hipError_t e = launch_any_forward(true, dt == LA_DTYPE_F32 ? 0 : 1, q, k, v, out, BH, N, D, M,
                                            static_cast<float *>(workspace), stream, sio);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status_t la_forward_causal_features(const void *fq, const void *fk, const void *v, void *out, int64_t B,
                                       int64_t H, int64_t N, int64_t F, int64_t M, la_dtype_t dt, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    la_status_t st = check_shape(B, H, N, F, M, dt, true);
    if (st != LA_OK) return st;
    const size_t es = esize(dt);
    const int64_t BH = B * H;
    const Span in[3] = {span(fq, size_t(BH * N * F) * es), span(fk, size_t(BH * N * F) * es),
                        span(v, size_t(BH * N * M) * es)};
    const Span o[1] = {span(out, size_t(BH * N * M) * es)};
    if ((st = check_buffers(in, 3, o, 1)) != LA_OK) return st;
    const Span all[4] = {in[0], in[1], in[2], o[0]};
    if ((st = check_workspace(workspace, workspace_bytes, la::causal_workspace_bytes(BH, N, F, M), all, 4)) != LA_OK)
        return st;
    if (!forward_supported(true, BH, N, F, M, es)) return LA_ERR_UNSUPPORTED;
    la::StateIO sio;
    sio.features_given = true;
    const hipError_t e = launch_any_forward(true, dt == LA_DTYPE_F32 ? 0 : 1, fq, fk, v, out, BH, N, F, M,
                                            static_cast<float *>(workspace), stream, sio);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

// The polynomial forwards: shapes, buffers and workspace, then the launch.
static la_status_t poly_forward(bool causal, const void *q, const void *k, const void *v, void *out,
                                float *state_final, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                                la_dtype_t dt, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    la_status_t st = check_shape(B, H, N, D, M, dt, true);
    if (st != LA_OK) return st;
    if (!la::poly_head_sizes(D, M)) return LA_ERR_UNSUPPORTED;
    const size_t es = esize(dt);
    const int64_t BH = B * H;
    const Span in[3] = {span(q, size_t(BH * N * D) * es), span(k, size_t(BH * N * D) * es),
                        span(v, size_t(BH * N * M) * es)};
    const Span o[2] = {span(out, size_t(BH * N * M) * es),
                       span(state_final, size_t(BH * la::poly_state_floats(D, M)) * 4)};
    const int no = state_final ? 2 : 1;
    if ((st = check_buffers(in, 3, o, no)) != LA_OK) return st;
    const Span all[5] = {in[0], in[1], in[2], o[0], o[1]};
    if ((st = check_workspace(workspace, workspace_bytes, la::poly_workspace_bytes(BH, N, D, M, causal), all,
                              3 + no)) != LA_OK)
        return st;
    const hipError_t e = la::launch_poly_forward(causal, dt == LA_DTYPE_F32 ? 0 : 1, q, k, v, out, state_final, BH,
                                                 N, D, M, static_cast<float *>(workspace), stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status_t la_forward_causal_poly2(const void *q, const void *k, const void *v, void *out, int64_t B, int64_t H,
                                    int64_t N, int64_t D, int64_t M, la_dtype_t dt, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    return poly_forward(true, q, k, v, out, nullptr, B, H, N, D, M, dt, workspace, workspace_bytes, stream);
}

la_status_t la_forward_causal_poly2_state(const void *q, const void *k, const void *v, void *out,
                                          float *state_final, int64_t B, int64_t H, int64_t N, int64_t D,
                                          int64_t M, la_dtype_t dt, void *workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
    if (state_final == nullptr) return LA_ERR_INVALID_ARGUMENT;
    return poly_forward(true, q, k, v, out, state_final, B, H, N, D, M, dt, workspace, workspace_bytes, stream);
}

la_status_t la_forward_noncausal_poly2(const void *q, const void *k, const void *v, void *out, int64_t B,
                                       int64_t H, int64_t N, int64_t D, int64_t M, la_dtype_t dt, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    return poly_forward(false, q, k, v, out, nullptr, B, H, N, D, M, dt, workspace, workspace_bytes, stream);
}

la_status_t la_decode_step_poly2(const void *q, const void *k, const void *v, float *state, void *out, int64_t B,
                                 int64_t H, int64_t D, int64_t M, la_dtype_t dt, hipStream_t stream) {
    la_status_t st = check_shape(B, H, 1, D, M, dt);
    if (st != LA_OK) return st;
    if (!la::poly_head_sizes(D, M)) return LA_ERR_UNSUPPORTED;
    const size_t es = esize(dt);
    const int64_t BH = B * H;
    if (BH > int64_t(1) << 31) return LA_ERR_UNSUPPORTED;   // one workgroup per stream
    const Span in[3] = {span(q, size_t(BH * D) * es), span(k, size_t(BH * D) * es), span(v, size_t(BH * M) * es)};
    const Span o[2] = {span(state, size_t(BH * la::poly_state_floats(D, M)) * 4), span(out, size_t(BH * M) * es)};
    if ((st = check_buffers(in, 3, o, 2)) != LA_OK) return st;
    const hipError_t e = la::launch_poly_decode(dt == LA_DTYPE_F32 ? 0 : 1, q, k, v, state, out, BH, D, M, stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

int64_t la_poly2_state_floats(int64_t D, int64_t M) { return la::poly_state_floats(D, M); }

la_status_t la_rff_features(const void *x, const float *omega, const float *bias, void *out, int64_t B, int64_t H,
                            int64_t N, int64_t D, int64_t R, la_dtype_t dt, hipStream_t stream) {
    la_status_t st = check_shape(B, H, N, D, R, dt);
    if (st != LA_OK) return st;
    const size_t es = esize(dt);
    const int64_t rows = B * H * N;
    const Span in[3] = {span(x, size_t(rows * D) * es), span(omega, size_t(D * R) * 4), span(bias, size_t(R) * 4)};
    const Span o[1] = {span(out, size_t(rows * R) * es)};
    if ((st = check_buffers(in, 3, o, 1)) != LA_OK) return st;
    const hipError_t e = la::launch_rff_features(dt == LA_DTYPE_F32 ? 0 : 1, x, omega, bias, out, rows, D, R, stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status_t la_forward_noncausal(const void *q, const void *k, const void *v, void *out, int64_t B, int64_t H,
                                 int64_t N, int64_t D, int64_t M, la_dtype_t dt, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    return forward_common(false, q, k, v, out, B, H, N, D, M, dt, workspace, workspace_bytes, stream);
}

} // extern "C"

namespace {

la_status_t backward_common(bool causal, const void *q, const void *k, const void *v, const void *dout, void *dq,
                            void *dk, void *dv, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                            la_dtype_t dt, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    la_status_t st = check_shape(B, H, N, D, M, dt, true);
    if (st != LA_OK) return st;
    const size_t es = esize(dt);
    const int64_t BH = B * H;
    const Span in[4] = {span(q, size_t(BH * N * D) * es), span(k, size_t(BH * N * D) * es),
                        span(v, size_t(BH * N * M) * es), span(dout, size_t(BH * N * M) * es)};
    const Span o[3] = {span(dq, size_t(BH * N * D) * es), span(dk, size_t(BH * N * D) * es),
                       span(dv, size_t(BH * N * M) * es)};
    if ((st = check_buffers(in, 4, o, 3)) != LA_OK) return st;
    const Span all[7] = {in[0], in[1], in[2], in[3], o[0], o[1], o[2]};
    const size_t need = causal ? la::backward_workspace_bytes(BH, N, D, M, es)
                               : la::backward_noncausal_workspace_bytes(BH, N, D, M);
    if ((st = check_workspace(workspace, workspace_bytes, need, all, 7)) != LA_OK) return st;
    const hipError_t e = la::launch_backward(causal, dt == LA_DTYPE_F32 ? 0 : 1, q, k, v, dout, dq, dk, dv, BH, N, D,
                                             M, static_cast<float *>(workspace), stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

} // namespace

extern "C" {

la_status_t la_backward_causal(const void *q, const void *k, const void *v, const void *dout, void *dq, void *dk,
                               void *dv, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, la_dtype_t dt,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return backward_common(true, q, k, v, dout, dq, dk, dv, B, H, N, D, M, dt, workspace, workspace_bytes, stream);
}

la_status_t la_backward_noncausal(const void *q, const void *k, const void *v, const void *dout, void *dq, void *dk,
                                  void *dv, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, la_dtype_t dt,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return backward_common(false, q, k, v, dout, dq, dk, dv, B, H, N, D, M, dt, workspace, workspace_bytes, stream);
}

la_status_t la_backward_causal_poly2(const void *q, const void *k, const void *v, const void *dout, void *dq,
                                     void *dk, void *dv, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                                     la_dtype_t dt, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    la_status_t st = check_shape(B, H, N, D, M, dt);
    if (st != LA_OK) return st;
    if (!la::poly_head_sizes(D, M)) return LA_ERR_UNSUPPORTED;
    const size_t es = esize(dt);
    const int64_t BH = B * H;
    const Span in[4] = {span(q, size_t(BH * N * D) * es), span(k, size_t(BH * N * D) * es),
                        span(v, size_t(BH * N * M) * es), span(dout, size_t(BH * N * M) * es)};
    const Span o[3] = {span(dq, size_t(BH * N * D) * es), span(dk, size_t(BH * N * D) * es),
                       span(dv, size_t(BH * N * M) * es)};
    if ((st = check_buffers(in, 4, o, 3)) != LA_OK) return st;
    const Span all[7] = {in[0], in[1], in[2], in[3], o[0], o[1], o[2]};
    const size_t need = la::poly_backward_workspace_bytes(BH, N, D, M, es);
    if ((st = check_workspace(workspace, workspace_bytes, need, all, 7)) != LA_OK) return st;
    const hipError_t e = la::launch_poly_backward(dt == LA_DTYPE_F32 ? 0 : 1, q, k, v, dout, dq, dk, dv, BH, N, D, M,
                                                  workspace, stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status_t la_decode_step(const void *q, const void *k, const void *v, float *S, float *Z, void *out, int64_t B,
                           int64_t H, int64_t D, int64_t M, la_dtype_t dt, hipStream_t stream) {
    la_status_t st = check_shape(B, H, 1, D, M, dt, true);
    if (st != LA_OK) return st;
    const size_t es = esize(dt);
    const int64_t BH = B * H;
    const Span in[3] = {span(q, size_t(BH * D) * es), span(k, size_t(BH * D) * es), span(v, size_t(BH * M) * es)};
    const Span o[3] = {span(S, size_t(BH * D * M) * 4), span(Z, size_t(BH * D) * 4), span(out, size_t(BH * M) * es)};
    if ((st = check_buffers(in, 3, o, 3)) != LA_OK) return st;
    const hipError_t e =
        la::launch_decode(dt == LA_DTYPE_F32 ? 0 : 1, q, k, v, S, Z, out, BH, D, M, stream);
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

size_t la_workspace_size(la_op_t op, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, la_dtype_t dt) {
    const bool any_size = op == LA_OP_FWD_CAUSAL || op == LA_OP_FWD_NONCAUSAL || op == LA_OP_BWD_CAUSAL ||
                          op == LA_OP_BWD_NONCAUSAL;
    if (check_shape(B, H, N, D, M, dt, any_size) != LA_OK) return 0;
    switch (op) {
    case LA_OP_FWD_CAUSAL:
        return la::causal_workspace_bytes(B * H, N, D, M);
    case LA_OP_FWD_NONCAUSAL:
        return la::causal_workspace_bytes(B * H, N, D, M);
    case LA_OP_BWD_CAUSAL:
        return la::backward_workspace_bytes(B * H, N, D, M, esize(dt));
    case LA_OP_BWD_NONCAUSAL:
        return la::backward_noncausal_workspace_bytes(B * H, N, D, M);
    case LA_OP_FWD_CAUSAL_POLY2:
        return la::poly_head_sizes(D, M) ? la::poly_workspace_bytes(B * H, N, D, M, true) : 0;
    case LA_OP_FWD_NONCAUSAL_POLY2:
        return la::poly_head_sizes(D, M) ? la::poly_workspace_bytes(B * H, N, D, M, false) : 0;
    case LA_OP_BWD_CAUSAL_POLY2:
        return la::poly_head_sizes(D, M) ? la::poly_backward_workspace_bytes(B * H, N, D, M, esize(dt)) : 0;
    }
    return 0;
}

const char *la_status_string(la_status_t s) {
    switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARGUMENT: return "LA_ERR_INVALID_ARGUMENT";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE";
    case LA_ERR_HIP: return "LA_ERR_HIP";
    case LA_ERR_TIMEOUT: return "LA_ERR_TIMEOUT";
    }
    return "LA_ERR_UNKNOWN";
}

la_status_t la_workspace_check(void *workspace, size_t workspace_bytes, int clear, hipStream_t stream) {
    if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < 256) return LA_ERR_WORKSPACE;
    int word = 0;
    int *err = static_cast<int *>(workspace) + 1;
    if (hipMemcpyAsync(&word, err, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess) return LA_ERR_HIP;
    if (clear) {
        static const int zero = 0;
        if (hipMemcpyAsync(err, &zero, sizeof(int), hipMemcpyHostToDevice, stream) != hipSuccess) return LA_ERR_HIP;
    }
    if (hipStreamSynchronize(stream) != hipSuccess) return LA_ERR_HIP;
    return word != 0 ? LA_ERR_TIMEOUT : LA_OK;
}

int64_t la_set_wait_limit(int64_t polls) { return la::set_wait_limit(polls); }

int la_abi_version(void) { return LA_ABI_VERSION; }

} // extern "C"

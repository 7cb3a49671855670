// la_internal.h -- host-side plan and launcher declarations (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace la {

// Tokens per chunk: the unit of the intra-chunk masked product on the
// matrix cores (two 16-token tiles).
constexpr int64_t kChunk = 16;
// Largest number of segments per (b, h) the segment scan handles.
constexpr int64_t kMaxSegPerHead = 256;
// Aim for about this many independent segments (one wavefront each) so that
// every SIMD of the 256 CUs has work.
constexpr int64_t kTargetSegments = 1024;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Head sizes: the fused forward kernels (and the backward, the polynomial and
// random-feature kernels) take D, M in {32, 64}; decode and the generic
// forward every multiple of 16 up to 128.
inline bool fused_head_sizes(int64_t D, int64_t M) { return (D == 32 || D == 64) && (M == 32 || M == 64); }
inline bool head_size_ok(int64_t x) { return x >= 16 && x <= 128 && x % 16 == 0; }

// How a (B*H, N) problem is cut into segments of whole chunks.  Each
// segment is processed by one wavefront, chunk after chunk, carrying the
// fp32 state; segment states are combined by a scan across segments.
struct SegPlan {
    int64_t seg_tokens = 0;  // tokens per segment (multiple of kChunk)
    int64_t nseg = 0;        // segments per (b, h)
    int64_t rec = 0;         // floats per state record: D*M + D (S then Z)
};

inline SegPlan make_plan(int64_t BH, int64_t N, int64_t D, int64_t M) {
    SegPlan p;
    const int64_t nch = ceil_div(N, kChunk);
    int64_t cps = ceil_div(BH * nch, kTargetSegments);       // chunks per segment
    cps = cps < 1 ? 1 : cps;
    const int64_t min_cps = ceil_div(nch, kMaxSegPerHead);
    if (cps < min_cps) cps = min_cps;
    if (!fused_head_sizes(D, M)) {
        // The column-group kernels' records grow as D M: keep the record
        // traffic (written, scanned in place, read back: four passes of
        // 4 (D M + D) bytes per segment) within half of the bf16 input and
        // output bytes of the segment's tokens, 2 (2 D + 2 M) per token.
        const int64_t rec_cps = ceil_div(ceil_div(16 * (D * M + D), 2 * (D + M)), kChunk);
        if (cps < rec_cps) cps = rec_cps;
    }
    p.seg_tokens = cps * kChunk;
    p.nseg = ceil_div(N, p.seg_tokens);
    p.rec = D * M + D;
    return p;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Both forwards run as one pass: workgroups of kFusedWaves wavefronts,
// each workgroup owning a block of kFusedWaves consecutive sub-segments (one
// per wavefront) of one (b, h).  Blocks exchange fp32 state records through
// the workspace (block totals, then their exclusive prefix sums, computed
// slice by slice by all blocks of the head), so no scan launch is needed.
constexpr int kFusedWaves = 8;
constexpr int64_t kMaxBlkPerHead = 64;   // flags of a head fit one wavefront
constexpr int kFusedDirectBlocks = 8;    // up to this many blocks per head: one exchange, no slices

// Compute units of the current device (queried once per device and cached;
// 256, MI355X's count, when no device can be queried).  The fused forward's
// plan follows it: about two wavefronts per SIMD in all (8 per CU), and at
// most one block per CU for each head, so that all blocks of a head can be
// resident at once (a block always fits a CU by itself).
int device_cus();

struct FusedPlan {
    int64_t sub_tokens = 0;  // tokens per wavefront (multiple of kChunk)
    int64_t nblk = 0;        // blocks per (b, h)
    int64_t rec = 0;         // floats per state record
    size_t flags_off = 0;    // 64-bit flags [BH][2][nblk]: total published, prefix slice published
                             // (after a 256-byte header; int word 1 is the error word)
    size_t recs_off = 0;     // float records [BH][nblk][2][rec]: block total, exclusive prefix
                             // (fragment order: only ever summed elementwise)
    size_t total = 0;
};

inline FusedPlan make_fused_plan(int64_t BH, int64_t N, int64_t D, int64_t M, int cus = device_cus()) {
    FusedPlan p;
    const int64_t target_waves = int64_t(cus) * kFusedWaves;
    const int64_t max_blk = std::min<int64_t>(kMaxBlkPerHead, cus);
    const int64_t nch = ceil_div(N, kChunk);
    int64_t cpw = ceil_div(BH * nch, target_waves);
    if (cpw < 1) cpw = 1;
    const int64_t min_cpw = ceil_div(nch, kFusedWaves * max_blk);
    if (cpw < min_cpw) cpw = min_cpw;
    p.sub_tokens = cpw * kChunk;
    p.nblk = ceil_div(N, kFusedWaves * p.sub_tokens);
    // a short problem that leaves most CUs idle anyway: up to twice the chunks
    // per wavefront if that brings a head within the single-exchange hand-off
    if (p.nblk > kFusedDirectBlocks && p.nblk <= 2 * kFusedDirectBlocks && BH * p.nblk <= cus / 2) {
        cpw = ceil_div(nch, kFusedWaves * kFusedDirectBlocks);
        p.sub_tokens = cpw * kChunk;
        p.nblk = ceil_div(N, kFusedWaves * p.sub_tokens);
    }
    p.rec = D * M + D;
    p.flags_off = 256;
    p.recs_off = p.flags_off + align256(size_t(2 * BH * p.nblk) * sizeof(unsigned long long));
    // a single block per head exchanges nothing: no records
    p.total = p.recs_off + (p.nblk > 1 ? align256(size_t(BH * p.nblk * 2 * p.rec) * sizeof(float)) : 0);
    return p;
}

// Polls a hand-off wait makes before it gives up (process-wide; see
// la_set_wait_limit); set_wait_limit returns the previous value (a negative
// argument restores the default).
int64_t wait_limit();
int64_t set_wait_limit(int64_t polls);

// The library-owned scratch of la_forward_causal_noalloc on the current
// device (device address, 256-byte aligned, kNoAllocScratchBytes long), or
// null if it cannot be resolved.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
void *noalloc_scratch();

// Whether the fused forward's plan for this shape is within the kernel's
// limits (checked by the ABI before any launch).
bool forward_plan_supported(int64_t BH, int64_t N, int64_t D, int64_t M, size_t esize);

// Rows of block totals one thread sums while forming its slice (the kernel
// keeps at most kFusedSliceRows in registers): block sb of nb owns ncol = its
// share of the rec4 float4 columns; nthreads threads cover ncol columns x G
// row groups of the nr totals summed (nb - 1 causal, nb non-causal).
constexpr int kFusedSliceRows = 4;
inline int64_t fused_slice_rows(int64_t nb, int64_t nr, int64_t rec4, int64_t nthreads) {
    int64_t worst = 0;
    const int64_t per = ceil_div(rec4, nb);
    for (int64_t sb = 0; sb < nb && nr > 0; ++sb) {
        const int64_t c0 = std::min(rec4, sb * per), ncol = std::min(rec4, c0 + per) - c0;
        if (ncol <= 0) continue;
        const int64_t G = std::max<int64_t>(1, std::min(nr, nthreads / ncol));
        worst = std::max(worst, ceil_div(nr, G));
    }
    return worst;
}

// A fresh nonzero 64-bit value per call (process-wide counter through a
// bijective mixer, seeded once per process): the causal forward's hand-off
// flags count as set only when they hold the current call's tag.
uint64_t next_call_tag();

// Workspace of the forwards (the fused kernels or the generic path, by head size).
size_t generic_workspace_bytes(int64_t BH, int64_t N, int64_t D, int64_t M);
inline size_t causal_workspace_bytes(int64_t BH, int64_t N, int64_t D, int64_t M) {
    return fused_head_sizes(D, M) ? make_fused_plan(BH, N, D, M).total : generic_workspace_bytes(BH, N, D, M);
}

// Backward workspace, in order: forward state records, reverse state records
// (same size), the per-token reciprocal denominators 1/d_i and
// h_i = -(dout_i . out_i) / d_i ([BH][N] fp32 each).  The reverse pass forms
// g_i = dout_i / d_i from dout and 1/d_i itself, exactly as the forward pass
// does, instead of reading a staged copy of g.
struct BwdLayout {
    size_t states = 0, inv_off = 0, h_off = 0, total = 0;
};

inline BwdLayout backward_layout(int64_t BH, int64_t N, int64_t D, int64_t M, size_t) {
    const SegPlan p = make_plan(BH, N, D, M);
    BwdLayout L;
    L.states = align256(size_t(BH * p.nseg * p.rec) * sizeof(float));
    L.inv_off = 2 * L.states;
    L.h_off = L.inv_off + align256(size_t(BH * N) * sizeof(float));
    L.total = L.h_off + align256(size_t(BH * N) * sizeof(float));
    return L;
}

inline size_t backward_workspace_bytes(int64_t BH, int64_t N, int64_t D, int64_t M, size_t esize) {
    return backward_layout(BH, N, D, M, esize).total;
}

// The non-causal backward keeps only the two record arrays (no g, h).
inline size_t backward_noncausal_workspace_bytes(int64_t BH, int64_t N, int64_t D, int64_t M) {
    return 2 * backward_layout(BH, N, D, M, 4).states;
}

// Options of the causal forward.  Optional fp32 state, [BH][D][M] and
// [BH][D] (the decode layout): s0/z0 start the recurrence (null: zero),
// s1/z1 receive the state after the last token (null: not written); s1 may
// equal s0.  features_given: q and k already hold the features (the feature
// map is not applied).
struct StateIO {
    const float *s0 = nullptr, *z0 = nullptr;
    float *s1 = nullptr, *z1 = nullptr;
    bool features_given = false;
};

// Random Fourier features of rows x [rows][D] into out [rows][R]; omega
// [D][R] and bias [R] fp32.
hipError_t launch_rff_features(int dt, const void *x, const float *omega, const float *bias, void *out, int64_t rows,
                               int64_t D, int64_t R, hipStream_t s);

// Causal forward with the degree-2 polynomial kernel (q . k)^2, D, M in
// {32, 64}; workspace: one fp32 record of the segment's feature state and
// D x D normalizer per segment (256 bytes when a (b, h) is one segment).
bool poly_head_sizes(int64_t D, int64_t M);
size_t poly_workspace_bytes(int64_t BH, int64_t N, int64_t D, int64_t M, bool causal);
// Floats of one (b, h)'s state (feature tiles, then the Z tiles); 0 if D, M
// are not supported.
int64_t poly_state_floats(int64_t D, int64_t M);
// causal or not; state_final (causal only, may be null): the state after the
// last token of every (b, h), poly_state_floats(D, M) floats each.
hipError_t launch_poly_forward(bool causal, int dt, const void *q, const void *k, const void *v, void *out,
                               float *state_final, int64_t BH, int64_t N, int64_t D, int64_t M, float *ws,
                               hipStream_t s);
hipError_t launch_poly_decode(int dt, const void *q, const void *k, const void *v, float *state, void *out,
                              int64_t BH, int64_t D, int64_t M, hipStream_t s);

// The generic forward (la_generic.hip: segment sums, scan, outputs, with V
// and out cut into 16-column groups); its workspace is one row-major record
// (S [D][M], Z [D]) per segment.
hipError_t launch_forward_generic(bool causal, int dt, const void *q, const void *k, const void *v, void *out,
                                  int64_t BH, int64_t N, int64_t D, int64_t M, float *ws, hipStream_t s,
                                  StateIO sio = StateIO());

// Launchers (hipError_t of the last launch).  dt: 0 = fp32, 1 = bf16.
hipError_t launch_forward(bool causal, int dt, const void *q, const void *k, const void *v, void *out,
                          int64_t BH, int64_t N, int64_t D, int64_t M, float *ws, hipStream_t s,
                          StateIO sio = StateIO());
hipError_t launch_segment_state(int dt, const void *k, const void *v, float *ws, int64_t BH, int64_t N, int64_t D,
                                int64_t M, hipStream_t s);
// Optional start state of a scan (added to every exclusive prefix) and final
// state (start + total), per (b, h) as S [srec] then Z [rec - srec] floats in
// separate arrays; s1 may equal s0 and z1 z0.
struct ScanIO {
    const float *s0 = nullptr, *z0 = nullptr;
    float *s1 = nullptr, *z1 = nullptr;
    int64_t srec = 0;
};
// mode 0: exclusive prefix over segments; 1: total into record 0;
// 2: exclusive suffix (sum of the later segments).
hipError_t launch_scan(float *ws, int64_t BH, int64_t nseg, int64_t rec, int mode, hipStream_t s,
                       ScanIO io = ScanIO());
hipError_t launch_backward(bool causal, int dt, const void *q, const void *k, const void *v, const void *dout,
                           void *dq, void *dk, void *dv, int64_t BH, int64_t N, int64_t D, int64_t M, float *ws,
                           hipStream_t s);
// The backward for head sizes outside {32, 64} (la_generic.hip), on the same
// workspace layout (backward_layout).
hipError_t launch_backward_generic(bool causal, int dt, const void *q, const void *k, const void *v,
                                   const void *dout, void *dq, void *dk, void *dv, int64_t BH, int64_t N, int64_t D,
                                   int64_t M, float *ws, hipStream_t s);
hipError_t launch_decode(int dt, const void *q, const void *k, const void *v, float *S, float *Z, void *out,
                         int64_t BH, int64_t D, int64_t M, hipStream_t s);

} // namespace la

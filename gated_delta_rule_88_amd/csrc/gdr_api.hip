// gdr_api.hip -- the C ABI (include/gdr.h): argument validation and
// dispatch to the kernels.  Every check runs on the host before anything is
// enqueued, so an error status means no device memory was touched.
#include "../../include/gdr.h"

#include <stdint.h>

#include "gdr_chunk.h"

#define GDR_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi); empty when lo == hi
};
Range rng(const void* p, size_t bytes) {
    const uintptr_t b = (uintptr_t)p;
    return Range{b, p ? b + bytes : b};
}
bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}
bool supported_dim(int d) { return d == 64 || d == 128; }
bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64; }
size_t elem_size(int dtype) { return dtype == gdr::kBF16 ? 2 : 4; }

// Largest workgroup count along grid x times 256 threads must fit 32 bits.
constexpr size_t kMaxGroups = (size_t)1 << 23;

int check_chunk_sizes(int B, int H, int L, int dk, int dv, int C, int dtype, int mode)
{
    if (B < 0 || H < 0 || L < 0) return GDR_ERR_INVALID_ARG;
    if (mode < GDR_ALPHA_NONE || mode > GDR_ALPHA_CHANNEL) return GDR_ERR_INVALID_ARG;
    if (dtype != GDR_F32 && dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
    if (!supported_dim(dk) || !supported_dim(dv) || !supported_chunk(C)) return GDR_ERR_UNSUPPORTED;
    const size_t nc = ((size_t)L + 15) / 16;   // chunks at the shortest token step
    if ((size_t)B * H * nc > kMaxGroups) return GDR_ERR_UNSUPPORTED;
    return GDR_OK;
}

size_t chunk_workspace(int B, int H, int L, int dk, int dv, int C, int dtype, int mode)
{
    return gdr::chunk_workspace_bytes(B, H, L, dk, dv, C, dtype, mode);
}

int check_varlen_sizes(int N, int H, int T, int dk, int dv, int C, int dtype, int mode)
{
    if (N < 0 || H < 0 || T < 0) return GDR_ERR_INVALID_ARG;
    if (mode < GDR_ALPHA_NONE || mode > GDR_ALPHA_CHANNEL) return GDR_ERR_INVALID_ARG;
    if (dtype != GDR_F32 && dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
    if (!supported_dim(dk) || !supported_dim(dv) || !supported_chunk(C)) return GDR_ERR_UNSUPPORTED;
    // record slots per head at the shortest token step: (T + 15 N) / 16
    const size_t slots = ((size_t)T + 15 * (size_t)N) / 16;
    if ((size_t)H * slots > kMaxGroups || (size_t)N * H * 4 > kMaxGroups) return GDR_ERR_UNSUPPORTED;
    return GDR_OK;
}

}  // namespace

GDR_EXPORT int gdr_abi_version(void) { return GDR_ABI_VERSION; }

GDR_EXPORT const char* gdr_status_string(int status)
{
    switch (status) {
    case GDR_OK: return "GDR_OK: success";
    case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG: invalid argument";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED: sizes or dtype outside the supported domain";
    case GDR_ERR_WORKSPACE_TOO_SMALL: return "GDR_ERR_WORKSPACE_TOO_SMALL: workspace smaller than required";
    case GDR_ERR_HIP: return "GDR_ERR_HIP: a HIP launch failed";
    case GDR_ERR_SCRATCH_TOO_SMALL:
        return "GDR_ERR_SCRATCH_TOO_SMALL: the call needs more scratch than the library's fixed "
               "per-device array holds (GDR_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown gdr status";
    }
}

size_t gdr::fwd_chunked_workspace_checked(int B, int H, int L, int dk, int dv, int C, int dtype, int mode)
{
    if (check_chunk_sizes(B, H, L, dk, dv, C, dtype, mode) != GDR_OK) return (size_t)-1;
    return chunk_workspace(B, H, L, dk, dv, C, dtype, mode);
}

GDR_EXPORT size_t gdr_fwd_chunked_workspace_size(int B, int H, int L, int d_k, int d_v, int C,
                                                 int dtype, int alpha_mode)
{
    return gdr::fwd_chunked_workspace_checked(B, H, L, d_k, d_v, C, dtype, alpha_mode);
}

GDR_EXPORT int gdr_fwd_chunked_token_step(int C, int dtype, int alpha_mode)
{
    if (alpha_mode < GDR_ALPHA_NONE || alpha_mode > GDR_ALPHA_CHANNEL) return 0;
    if ((dtype != GDR_F32 && dtype != GDR_BF16) || !supported_chunk(C)) return 0;
    return gdr::fwd_token_step(C, dtype, alpha_mode);
}

namespace gdr {

// The argument checks of a chunked forward whose workspace must hold `need`
// bytes: GDR_OK, or the status to return.
static int check_fwd_args(int B, int H, int L, int d_k, int d_v, int dtype,
                          const void* q, const void* k, const void* v,
                          const float* beta, int alpha_mode, const float* log_alpha,
                          const float* S0, void* o, float* S_final,
                          void* workspace, size_t workspace_bytes, size_t need)
{
    const size_t BH = (size_t)B * H;
    const size_t es = elem_size(dtype);
    const size_t nt = BH * L;
    const size_t state_bytes = BH * d_v * d_k * 4;
    if (L > 0) {
        if (!q || !k || !v || !beta || !o) return GDR_ERR_INVALID_ARG;
        if ((alpha_mode == GDR_ALPHA_NONE) != (log_alpha == nullptr)) return GDR_ERR_INVALID_ARG;
    }
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(S0, 16) || !aligned(S_final, 16) || !aligned(workspace, 16) ||
        !aligned(beta, 4) || !aligned(log_alpha, alpha_mode == GDR_ALPHA_CHANNEL ? 16 : 4))
        return GDR_ERR_INVALID_ARG;

    const size_t la_bytes = alpha_mode == GDR_ALPHA_CHANNEL ? nt * d_k * 4
                          : alpha_mode == GDR_ALPHA_SCALAR ? nt * 4 : 0;
    const Range rq = rng(q, nt * d_k * es), rk = rng(k, nt * d_k * es), rv = rng(v, nt * d_v * es);
    const Range rb = rng(beta, nt * 4), ra = rng(log_alpha, la_bytes);
    const Range r0 = rng(S0, state_bytes), ro = rng(o, nt * d_v * es);
    const Range rf = rng(S_final, state_bytes);
    const Range rw = rng(workspace, need);
    for (Range x : {rq, rk, rv, rb, ra, r0, rf, rw})
        if (overlap(ro, x)) return GDR_ERR_INVALID_ARG;
    for (Range x : {rq, rk, rv, rb, ra, rw})
        if (overlap(rf, x)) return GDR_ERR_INVALID_ARG;
    if (overlap(rf, r0) && (const void*)S_final != (const void*)S0) return GDR_ERR_INVALID_ARG;
    for (Range x : {rq, rk, rv, rb, ra, r0})
        if (overlap(rw, x)) return GDR_ERR_INVALID_ARG;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GDR_ERR_WORKSPACE_TOO_SMALL;
    return GDR_OK;
}

// gdr_fwd_chunked_ex's checks and launches (shared with the entry point
// that brings its own scratch, gdr_noalloc.hip).
int fwd_chunked_checked(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                        const void* q, const void* k, const void* v,
                        const float* beta, int alpha_mode, const float* log_alpha,
                        const float* S0, void* o, float* S_final,
                        void* workspace, size_t workspace_bytes, hipStream_t stream,
                        unsigned prologue)
{
    if (prologue & ~(unsigned)(GDR_PRO_L2NORM_QK | GDR_PRO_GATES)) return GDR_ERR_INVALID_ARG;
    int st = check_chunk_sizes(B, H, L, d_k, d_v, C, dtype, alpha_mode);
    if (st != GDR_OK) return st;
    if ((size_t)B * H == 0) return GDR_OK;
    st = check_fwd_args(B, H, L, d_k, d_v, dtype, q, k, v, beta, alpha_mode, log_alpha, S0, o, S_final,
                        workspace, workspace_bytes, chunk_workspace(B, H, L, d_k, d_v, C, dtype, alpha_mode));
    if (st != GDR_OK) return st;
    gdr::ChunkArgs a{B, H, L, d_k, d_v, C, dtype, alpha_mode, q, k, v, beta, log_alpha, S0, o,
                     S_final, workspace, stream, prologue};
    return gdr::launch_fwd_chunked(a) == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

}  // namespace gdr

GDR_EXPORT int gdr_fwd_chunked_ex(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                                  const void* q, const void* k, const void* v,
                                  const float* beta, int alpha_mode, const float* log_alpha,
                                  const float* S0, void* o, float* S_final,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream,
                                  unsigned prologue)
{
    return gdr::fwd_chunked_checked(B, H, L, d_k, d_v, C, dtype, q, k, v, beta, alpha_mode, log_alpha,
                                    S0, o, S_final, workspace, workspace_bytes, stream, prologue);
}

GDR_EXPORT int gdr_fwd_chunked(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                               const void* q, const void* k, const void* v,
                               const float* beta, int alpha_mode, const float* log_alpha,
                               const float* S0, void* o, float* S_final,
                               void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return gdr_fwd_chunked_ex(B, H, L, d_k, d_v, C, dtype, q, k, v, beta, alpha_mode, log_alpha, S0, o,
                              S_final, workspace, workspace_bytes, stream, 0u);
}

GDR_EXPORT int gdr_decode_step_ex(int N, int H, int d_k, int d_v, int dtype,
                                  const void* q, const void* k, const void* v,
                                  const float* beta, int alpha_mode, const float* log_alpha,
                                  float* S, void* o, hipStream_t stream, unsigned prologue)
{
    if (prologue & ~(unsigned)(GDR_PRO_L2NORM_QK | GDR_PRO_GATES)) return GDR_ERR_INVALID_ARG;
    if (N < 0 || H < 0) return GDR_ERR_INVALID_ARG;
    if (alpha_mode < GDR_ALPHA_NONE || alpha_mode > GDR_ALPHA_CHANNEL) return GDR_ERR_INVALID_ARG;
    if (dtype != GDR_F32 && dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return GDR_ERR_UNSUPPORTED;
    const size_t NH = (size_t)N * H;
    if (NH * 4 > kMaxGroups) return GDR_ERR_UNSUPPORTED;
    if (NH == 0) return GDR_OK;
    if (!q || !k || !v || !beta || !S || !o) return GDR_ERR_INVALID_ARG;
    if ((alpha_mode == GDR_ALPHA_NONE) != (log_alpha == nullptr)) return GDR_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(S, 16) || !aligned(beta, 4) || !aligned(log_alpha, alpha_mode == GDR_ALPHA_CHANNEL ? 16 : 4))
        return GDR_ERR_INVALID_ARG;
    const size_t es = elem_size(dtype);
    const size_t la_bytes = alpha_mode == GDR_ALPHA_CHANNEL ? NH * d_k * 4
                          : alpha_mode == GDR_ALPHA_SCALAR ? NH * 4 : 0;
    const Range rq = rng(q, NH * d_k * es), rk = rng(k, NH * d_k * es), rv = rng(v, NH * d_v * es);
    const Range rb = rng(beta, NH * 4), ra = rng(log_alpha, la_bytes);
    const Range rs = rng(S, NH * d_v * d_k * 4), ro = rng(o, NH * d_v * es);
    for (Range x : {rq, rk, rv, rb, ra, rs})
        if (overlap(ro, x)) return GDR_ERR_INVALID_ARG;
    for (Range x : {rq, rk, rv, rb, ra})
        if (overlap(rs, x)) return GDR_ERR_INVALID_ARG;

    gdr::DecodeArgs a{N, H, d_k, d_v, dtype, alpha_mode, q, k, v, beta, log_alpha, S, o, stream, prologue};
    return gdr::launch_decode_step(a) == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

GDR_EXPORT int gdr_decode_step(int N, int H, int d_k, int d_v, int dtype,
                               const void* q, const void* k, const void* v,
                               const float* beta, int alpha_mode, const float* log_alpha,
                               float* S, void* o, hipStream_t stream)
{
    return gdr_decode_step_ex(N, H, d_k, d_v, dtype, q, k, v, beta, alpha_mode, log_alpha, S, o, stream, 0u);
}

GDR_EXPORT size_t gdr_fwd_varlen_workspace_size(int N, int H, int T, int d_k, int d_v, int C,
                                                int dtype, int alpha_mode)
{
    if (check_varlen_sizes(N, H, T, d_k, d_v, C, dtype, alpha_mode) != GDR_OK) return (size_t)-1;
    return gdr::varlen_workspace_bytes(N, H, T, d_k, d_v, C, dtype, alpha_mode);
}

GDR_EXPORT int gdr_fwd_varlen(int N, int H, int T, const int* cu_seqlens, int d_k, int d_v, int C,
                              int dtype, const void* q, const void* k, const void* v,
                              const float* beta, int alpha_mode, const float* log_alpha,
                              const float* S0, void* o, float* S_final,
                              void* workspace, size_t workspace_bytes, hipStream_t stream,
                              unsigned prologue)
{
    if (prologue & ~(unsigned)(GDR_PRO_L2NORM_QK | GDR_PRO_GATES)) return GDR_ERR_INVALID_ARG;
    int st = check_varlen_sizes(N, H, T, d_k, d_v, C, dtype, alpha_mode);
    if (st != GDR_OK) return st;
    const size_t NH = (size_t)N * H;
    if (NH == 0) return GDR_OK;
    if (!cu_seqlens || !aligned(cu_seqlens, 4)) return GDR_ERR_INVALID_ARG;
    const size_t es = elem_size(dtype);
    const size_t nt = (size_t)H * T;
    const size_t state_bytes = NH * d_v * d_k * 4;
    if (T > 0) {
        if (!q || !k || !v || !beta || !o) return GDR_ERR_INVALID_ARG;
        if ((alpha_mode == GDR_ALPHA_NONE) != (log_alpha == nullptr)) return GDR_ERR_INVALID_ARG;
    }
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(S0, 16) || !aligned(S_final, 16) || !aligned(workspace, 16) ||
        !aligned(beta, 4) || !aligned(log_alpha, alpha_mode == GDR_ALPHA_CHANNEL ? 16 : 4))
        return GDR_ERR_INVALID_ARG;

    const size_t la_bytes = alpha_mode == GDR_ALPHA_CHANNEL ? nt * d_k * 4
                          : alpha_mode == GDR_ALPHA_SCALAR ? nt * 4 : 0;
    const Range rq = rng(q, nt * d_k * es), rk = rng(k, nt * d_k * es), rv = rng(v, nt * d_v * es);
    const Range rb = rng(beta, nt * 4), ra = rng(log_alpha, la_bytes);
    const Range r0 = rng(S0, state_bytes), ro = rng(o, nt * d_v * es);
    const Range rf = rng(S_final, state_bytes), rc = rng(cu_seqlens, ((size_t)N + 1) * 4);
    const size_t need = gdr::varlen_workspace_bytes(N, H, T, d_k, d_v, C, dtype, alpha_mode);
    const Range rw = rng(workspace, need);
    for (Range x : {rq, rk, rv, rb, ra, r0, rf, rw, rc})
        if (overlap(ro, x)) return GDR_ERR_INVALID_ARG;
    for (Range x : {rq, rk, rv, rb, ra, rw, rc})
        if (overlap(rf, x)) return GDR_ERR_INVALID_ARG;
    if (overlap(rf, r0) && (const void*)S_final != (const void*)S0) return GDR_ERR_INVALID_ARG;
    for (Range x : {rq, rk, rv, rb, ra, r0, rc})
        if (overlap(rw, x)) return GDR_ERR_INVALID_ARG;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GDR_ERR_WORKSPACE_TOO_SMALL;

    gdr::ChunkArgs a{1, H, T, d_k, d_v, C, dtype, alpha_mode, q, k, v, beta, log_alpha, S0, o,
                     S_final, workspace, stream, prologue, cu_seqlens, N, gdr::Varlen{}};
    return gdr::launch_fwd_varlen(a) == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

GDR_EXPORT size_t gdr_bwd_chunked_workspace_size(int B, int H, int L, int d_k, int d_v, int C,
                                                 int dtype, int alpha_mode)
{
    if (check_chunk_sizes(B, H, L, d_k, d_v, C, dtype, alpha_mode) != GDR_OK) return (size_t)-1;
    return gdr::bwd_workspace_bytes(B, H, L, d_k, d_v, C, dtype, alpha_mode);
}

// gdr_bwd_chunked's checks and launches; part: gdr::kBwdAll or gdr::kBwdKept
static int bwd_checked(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                       const void* q, const void* k, const void* v,
                       const float* beta, int alpha_mode, const float* log_alpha,
                       const float* S0, const void* dO, const float* dS_final,
                       void* dq, void* dk, void* dv, float* dbeta, float* dlog_alpha,
                       float* dS0, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, int part)
{
    int st = check_chunk_sizes(B, H, L, d_k, d_v, C, dtype, alpha_mode);
    if (st != GDR_OK) return st;
    const size_t BH = (size_t)B * H;
    if (BH == 0) return GDR_OK;
    const size_t es = elem_size(dtype);
    const size_t nt = BH * L;
    const size_t state_bytes = BH * d_v * d_k * 4;
    if (L > 0) {
        if (!q || !k || !v || !beta || !dO || !dq || !dk || !dv || !dbeta) return GDR_ERR_INVALID_ARG;
        if ((alpha_mode == GDR_ALPHA_NONE) != (log_alpha == nullptr)) return GDR_ERR_INVALID_ARG;
        if ((alpha_mode == GDR_ALPHA_NONE) != (dlog_alpha == nullptr)) return GDR_ERR_INVALID_ARG;
    }
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dO, 16) || !aligned(dq, 16) ||
        !aligned(dk, 16) || !aligned(dv, 16) || !aligned(S0, 16) || !aligned(dS_final, 16) ||
        !aligned(dS0, 16) || !aligned(workspace, 16) || !aligned(beta, 4) ||
        !aligned(log_alpha, alpha_mode == GDR_ALPHA_CHANNEL ? 16 : 4) || !aligned(dbeta, 4) ||
        !aligned(dlog_alpha, 4))
        return GDR_ERR_INVALID_ARG;

    const size_t la_bytes = alpha_mode == GDR_ALPHA_SCALAR ? nt * 4
                            : alpha_mode == GDR_ALPHA_CHANNEL ? nt * d_k * 4 : 0;
    const Range rq = rng(q, nt * d_k * es), rk = rng(k, nt * d_k * es), rv = rng(v, nt * d_v * es);
    const Range rb = rng(beta, nt * 4), ra = rng(log_alpha, la_bytes), r0 = rng(S0, state_bytes);
    const Range rdo = rng(dO, nt * d_v * es), rdf = rng(dS_final, state_bytes);
    const Range oq = rng(dq, nt * d_k * es), ok = rng(dk, nt * d_k * es), ov = rng(dv, nt * d_v * es);
    const Range ob = rng(dbeta, nt * 4), oa = rng(dlog_alpha, la_bytes), o0 = rng(dS0, state_bytes);
    const size_t need = gdr::bwd_workspace_bytes(B, H, L, d_k, d_v, C, dtype, alpha_mode);
    const Range rw = rng(workspace, need);
    const Range ins[] = {rq, rk, rv, rb, ra, r0, rdo, rdf};
    const Range outs[] = {oq, ok, ov, ob, oa, o0, rw};
    for (int i = 0; i < 7; ++i) {
        for (Range x : ins)
            if (overlap(outs[i], x)) return GDR_ERR_INVALID_ARG;
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], outs[j])) return GDR_ERR_INVALID_ARG;
    }
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GDR_ERR_WORKSPACE_TOO_SMALL;

    gdr::BwdArgs a{B, H, L, d_k, d_v, C, dtype, alpha_mode, q, k, v, beta, log_alpha, S0, dO, dS_final,
                   dq, dk, dv, dbeta, dlog_alpha, dS0, workspace, stream, part};
    return gdr::launch_bwd_chunked(a) == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

GDR_EXPORT int gdr_bwd_chunked(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                               const void* q, const void* k, const void* v,
                               const float* beta, int alpha_mode, const float* log_alpha,
                               const float* S0, const void* dO, const float* dS_final,
                               void* dq, void* dk, void* dv, float* dbeta, float* dlog_alpha,
                               float* dS0, void* workspace, size_t workspace_bytes,
                               hipStream_t stream)
{
    return bwd_checked(B, H, L, d_k, d_v, C, dtype, q, k, v, beta, alpha_mode, log_alpha, S0, dO, dS_final,
                       dq, dk, dv, dbeta, dlog_alpha, dS0, workspace, workspace_bytes, stream, gdr::kBwdAll);
}

GDR_EXPORT int gdr_bwd_chunked_kept(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                                    const void* q, const void* k, const void* v,
                                    const float* beta, int alpha_mode, const float* log_alpha,
                                    const float* S0, const void* dO, const float* dS_final,
                                    void* dq, void* dk, void* dv, float* dbeta, float* dlog_alpha,
                                    float* dS0, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream)
{
    return bwd_checked(B, H, L, d_k, d_v, C, dtype, q, k, v, beta, alpha_mode, log_alpha, S0, dO, dS_final,
                       dq, dk, dv, dbeta, dlog_alpha, dS0, workspace, workspace_bytes, stream, gdr::kBwdKept);
}

GDR_EXPORT int gdr_fwd_chunked_keep(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                                    const void* q, const void* k, const void* v,
                                    const float* beta, int alpha_mode, const float* log_alpha,
                                    const float* S0, void* o, float* S_final,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    int st = check_chunk_sizes(B, H, L, d_k, d_v, C, dtype, alpha_mode);
    if (st != GDR_OK) return st;
    if ((size_t)B * H == 0) return GDR_OK;
    st = gdr::check_fwd_args(B, H, L, d_k, d_v, dtype, q, k, v, beta, alpha_mode, log_alpha, S0, o, S_final,
                             workspace, workspace_bytes,
                             gdr::bwd_workspace_bytes(B, H, L, d_k, d_v, C, dtype, alpha_mode));
    if (st != GDR_OK) return st;
    gdr::BwdArgs a{B, H, L, d_k, d_v, C, dtype, alpha_mode, q, k, v, beta, log_alpha, S0, nullptr, nullptr,
                   nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, workspace, stream, gdr::kBwdKeep,
                   o, S_final};
    return gdr::launch_bwd_chunked(a) == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

// gdr_fwd.hip -- the chunked forward's host side: workspace size and the
// launch sequence (prepass over every chunk, the chunk scan, and for a
// segment-parallel scan the combination of the segments).
#include "gdr_chunk.h"

namespace gdr {

__global__ void copy_state_kernel(const float* __restrict__ S0, float* __restrict__ S, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) S[i] = S0 ? S0[i] : 0.f;
}

static size_t record_bytes(int B, int H, int L, int dk, int CK, int dtype, int mode)
{
    const size_t nc = (size_t)((L + CK - 1) / CK);
    const int es = dtype == kBF16 ? 2 : 4;
    return (size_t)B * H * nc * (size_t)ws_layout(es, dk, CK, mode).bytes;
}

size_t chunk_workspace_bytes(int B, int H, int L, int dk, int dv, int C, int dtype, int mode)
{
    const int CK = chunk_step(C, dtype);
    const size_t rec = record_bytes(B, H, L, dk, CK, dtype, mode);
    const SegPlan sp = seg_plan(B, H, L, dk, dv, CK, dtype, rec);
    return sp.SEG > 1 ? sp.bytes : rec;
}

hipError_t launch_fwd_chunked(const ChunkArgs& a)
{
    const size_t BH = (size_t)a.B * a.H;
    if (BH == 0) return hipSuccess;
    if (a.L == 0) {
        // no tokens: the final state is the initial state
        if (!a.S_final || a.S0 == a.S_final) return hipSuccess;
        const size_t n = BH * a.dv * a.dk;
        hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, a.stream, a.S0,
                           a.S_final, n);
        return hipGetLastError();
    }
    const int CK = chunk_step(a.C, a.dtype);
    const SegPlan sp = seg_plan(a.B, a.H, a.L, a.dk, a.dv, CK, a.dtype,
                                record_bytes(a.B, a.H, a.L, a.dk, CK, a.dtype, a.mode));
    hipError_t err = launch_wy(a, CK);
    if (err != hipSuccess) return err;
    err = launch_scan(a, CK, sp);
    if (err != hipSuccess || sp.SEG == 1) return err;
    return launch_seg_combine(a, CK, sp);
}

}  // namespace gdr

// gdr_fwd.hip -- the chunked forward's host side: workspace size and the
// launch sequence (prepass over every chunk, then the chunk scan).
#include "gdr_chunk.h"

namespace gdr {

__global__ void copy_state_kernel(const float* __restrict__ S0, float* __restrict__ S, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) S[i] = S0 ? S0[i] : 0.f;
}

size_t chunk_workspace_bytes(int B, int H, int L, int dk, int C, int dtype, int mode)
{
    const int CK = chunk_step(C, dtype);
    const size_t nc = (size_t)((L + CK - 1) / CK);
    const int es = dtype == kBF16 ? 2 : 4;
    return (size_t)B * H * nc * (size_t)ws_layout(es, dk, CK, mode).bytes;
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
    hipError_t err = launch_wy(a, CK);
    if (err != hipSuccess) return err;
    return launch_scan(a, CK);
}

}  // namespace gdr

// gdr_fwd.hip -- the chunked forward's host side: workspace size and the
// launch sequence (prepass over every chunk, the chunk scan, and for a
// segment-parallel scan the combination of the segments), for fixed-length
// batches and for packed variable-length batches.
#include "gdr_chunk.h"
#include "gdr_device.h"

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
    const int CK = fwd_token_step(C, dtype, mode);
    const size_t rec = record_bytes(B, H, L, dk, CK, dtype, mode);
    const SegPlan sp = seg_plan(B, H, L, dk, dv, CK, dtype, rec);
    return sp.SEG > 1 ? sp.bytes : rec;
}

// ---------------------------------------------------------------- varlen
// Workspace of a packed variable-length batch: the chunk records [H][NCmax],
// then per sequence its first token, length and first chunk (ints).
struct VarlenWs {
    int NCmax;
    size_t off_start, off_len, off_choff, bytes;
};

static VarlenWs varlen_ws(int NS, int H, int T, int dk, int CK, int dtype, int mode)
{
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    VarlenWs w{};
    // sum over sequences of ceil(len / CK) <= (T + NS (CK - 1)) / CK
    w.NCmax = (int)(((long long)T + (long long)NS * (CK - 1)) / CK);
    const int es = dtype == kBF16 ? 2 : 4;
    size_t o = al((size_t)H * w.NCmax * (size_t)ws_layout(es, dk, CK, mode).bytes);
    w.off_start = o; o = al(o + (size_t)NS * 4);
    w.off_len = o; o = al(o + (size_t)NS * 4);
    w.off_choff = o; o = al(o + (size_t)(NS + 1) * 4);
    w.bytes = o;
    return w;
}

size_t varlen_workspace_bytes(int NS, int H, int T, int dk, int dv, int C, int dtype, int mode)
{
    (void)dv;
    if ((size_t)NS * H == 0) return 0;
    return varlen_ws(NS, H, T, dk, fwd_token_step(C, dtype, mode), dtype, mode).bytes;
}

// One workgroup of NT threads: every sequence's first token and length, its
// offsets clamped into [0, T] (and its end to at least its start), and the
// exclusive prefix sum of the sequences' chunk counts.  NT = 64 (one wave, no
// barriers) when the batch has at most 64 sequences.
template <int NT>
__global__ __launch_bounds__(NT) void varlen_plan_kernel(const int* __restrict__ cu, int NS, int T, int CK,
                                                         int* __restrict__ start, int* __restrict__ len,
                                                         int* __restrict__ choff)
{
    constexpr int NW = NT / kWave;
    __shared__ int wsum[NW];
    const int tid = threadIdx.x, l = lane_id(), w = tid / kWave;
    int carry = 0;   // chunks of the sequences before this tile
    for (int base = 0; base < NS; base += NT) {
        const int n = base + tid;
        int nc = 0;
        if (n < NS) {
            const int s0 = min(max(cu[n], 0), T);
            const int e0 = min(max(cu[n + 1], s0), T);
            start[n] = s0;
            len[n] = e0 - s0;
            nc = (e0 - s0 + CK - 1) / CK;
        }
        int x = nc;   // inclusive scan within the wave
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(x, d, kWave);
            if (l >= d) x += y;
        }
        int before = carry, tile = __shfl(x, kWave - 1, kWave);
        if constexpr (NW > 1) {
            if (l == kWave - 1) wsum[w] = x;
            __syncthreads();
            tile = 0;
            for (int i = 0; i < NW; ++i) {
                if (i < w) before += wsum[i];
                tile += wsum[i];
            }
            __syncthreads();   // wsum is rewritten by the next tile
        }
        if (n < NS) choff[n] = before + x - nc;
        carry += tile;
    }
    if (tid == 0) choff[NS] = carry;
}

hipError_t launch_fwd_varlen(ChunkArgs a)
{
    if ((size_t)a.NS * a.H == 0) return hipSuccess;
    const int CK = fwd_token_step(a.C, a.dtype, a.mode);
    const VarlenWs w = varlen_ws(a.NS, a.H, a.L, a.dk, CK, a.dtype, a.mode);
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    int* start = reinterpret_cast<int*>(ws + w.off_start);
    int* len = reinterpret_cast<int*>(ws + w.off_len);
    int* choff = reinterpret_cast<int*>(ws + w.off_choff);
    if (a.NS <= kWave)
        hipLaunchKernelGGL(varlen_plan_kernel<kWave>, dim3(1), dim3(kWave), 0, a.stream, a.cu_seqlens, a.NS, a.L,
                           CK, start, len, choff);
    else
        hipLaunchKernelGGL(varlen_plan_kernel<1024>, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens, a.NS, a.L,
                           CK, start, len, choff);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    a.vl = Varlen{start, len, choff, a.NS, w.NCmax};
    // (no tokens: every sequence is empty and the scan only copies S0; the
    // prepass reads a token of every slot, so it runs only when there is one)
    if (w.NCmax > 0 && a.L > 0) {
        err = launch_wy(a, CK);
        if (err != hipSuccess) return err;
    }
    const int NC = (a.L + CK - 1) / CK;
    SegPlan one{1, NC, NC, 0, 0, 0, 0, 0};
    return launch_scan(a, CK, one);
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
    const int CK = fwd_token_step(a.C, a.dtype, a.mode);
    const SegPlan sp = seg_plan(a.B, a.H, a.L, a.dk, a.dv, CK, a.dtype,
                                record_bytes(a.B, a.H, a.L, a.dk, CK, a.dtype, a.mode));
    hipError_t err = launch_wy(a, CK);
    if (err != hipSuccess) return err;
    err = launch_scan(a, CK, sp);
    if (err != hipSuccess || sp.SEG == 1) return err;
    return launch_seg_combine(a, CK, sp);
}

}  // namespace gdr

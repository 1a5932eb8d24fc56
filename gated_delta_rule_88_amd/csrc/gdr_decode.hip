// gdr_decode.hip -- single-token decode step of the gated delta-rule memory.
//
// For every (sequence, head) and every value channel i (row i of S):
//   a        = exp(log alpha)            (scalar, per key channel, or 1)
//   sk_i     = sum_j S[i,j] a_j k_j      prediction from the decayed memory
//   sq_i     = sum_j S[i,j] a_j q_j
//   u_i      = beta (v_i - sk_i)
//   S[i,j]  <- S[i,j] a_j + u_i k_j      erase-then-write
//   o_i      = sq_i + u_i (k . q)        = (S_new q)_i, read after the write
// ("linear attention and its gated descendants", sections "Recurrent Linear
// Attention for Inference", "Gated DeltaNet" and "Kimi Delta Attention";
// "Linear Attention Architectures ...", Sec. 3, Eq. (8).)
//
// Rows of S are independent given q, k, v, beta and alpha, so the kernel
// streams S exactly once: each row of d_k floats is read by d_k/4 lanes
// (16 B per lane), reduced across those lanes, updated and written back.
// The step moves 2 * 4 * d_k * d_v bytes of state per head and does 6 d^2
// flops, so it is bound by HBM bandwidth; the launch shape keeps several
// 16-byte loads per lane in flight.  The optional input-side prologue
// (gdr_decode_step_ex) costs nothing measurable on top: each row group
// already holds all of q and k, so their norms are one more lane reduction,
// and the gates are two activations per head (per key channel).
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

// Rows in flight per lane: 8 at d_k = 128 (measured 1.7 % faster than 4 on
// the 512 MiB state stream), 4 at d_k = 64; rows per block then divide d_v.
template <int DK> constexpr int decode_passes() { return DK == 128 ? 8 : 4; }
template <int DK> constexpr int decode_rows_per_block() { return 4 * (kWave / (DK / 4)) * decode_passes<DK>(); }

template <typename T, int DK, int MODE>
__global__ __launch_bounds__(256) void decode_step_kernel(
    int DV, const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ log_alpha,
    float* __restrict__ S, T* __restrict__ o, unsigned pro)
{
    constexpr int LPR = DK / 4;              // lanes per row
    constexpr int RPW = kWave / LPR;         // rows per wave per pass
    constexpr int U = decode_passes<DK>();   // passes (rows in flight per lane)
    constexpr int RB = 4 * RPW * U;          // rows per block
    static_assert(RB == decode_rows_per_block<DK>() && 64 % RB == 0, "blocks tile d_v = 64, 128");
    const int blocks_per_head = DV / RB;
    const int head = blockIdx.x / blocks_per_head;
    const int rb = blockIdx.x - head * blocks_per_head;
    const int l = lane_id(), w = wave_id();
    const int c = l % LPR, sub = l / LPR;

    // this lane's 4 key channels
    float kk[4], qq[4], ak[4], aq[4], a[4];
    {
        const T* kp = k + (size_t)head * DK + 4 * c;
        const T* qp = q + (size_t)head * DK + 4 * c;
#pragma unroll
        for (int j = 0; j < 4; ++j) { kk[j] = to_f32(kp[j]); qq[j] = to_f32(qp[j]); }
        if (pro & kProNorm) {
            // the row group's lanes together hold all d_k channels
            float nk = kk[0] * kk[0] + kk[1] * kk[1] + kk[2] * kk[2] + kk[3] * kk[3];
            float nq = qq[0] * qq[0] + qq[1] * qq[1] + qq[2] * qq[2] + qq[3] * qq[3];
#pragma unroll
            for (int m = LPR / 2; m >= 1; m >>= 1) {
                nk += __shfl_xor(nk, m, kWave);
                nq += __shfl_xor(nq, m, kWave);
            }
            const float sk = 1.f / fmaxf(sqrtf(nk), kNormEps), sq = 1.f / fmaxf(sqrtf(nq), kNormEps);
#pragma unroll
            for (int j = 0; j < 4; ++j) { kk[j] *= sk; qq[j] *= sq; }
        }
        const bool gates = (pro & kProGates) != 0;
        if (MODE == kAlphaChannel) {
            float4 la = *reinterpret_cast<const float4*>(log_alpha + (size_t)head * DK + 4 * c);
            if (gates) {
                la.x = log_sigmoid_f(la.x); la.y = log_sigmoid_f(la.y);
                la.z = log_sigmoid_f(la.z); la.w = log_sigmoid_f(la.w);
            }
            a[0] = __expf(la.x); a[1] = __expf(la.y); a[2] = __expf(la.z); a[3] = __expf(la.w);
        } else if (MODE == kAlphaScalar) {
            const float la = log_alpha[head];
            const float s = __expf(gates ? log_sigmoid_f(la) : la);
            a[0] = a[1] = a[2] = a[3] = s;
        } else {
            a[0] = a[1] = a[2] = a[3] = 1.0f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) { ak[j] = a[j] * kk[j]; aq[j] = a[j] * qq[j]; }
    }
    float kq = kk[0] * qq[0] + kk[1] * qq[1] + kk[2] * qq[2] + kk[3] * qq[3];
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) kq += __shfl_xor(kq, m, kWave);
    const float b = (pro & kProGates) ? sigmoid_f(beta[head]) : beta[head];

    float4 s[U];
    int row[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        row[u] = rb * RB + u * (4 * RPW) + w * RPW + sub;
        s[u] = *reinterpret_cast<const float4*>(S + ((size_t)head * DV + row[u]) * DK + 4 * c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float sk = s[u].x * ak[0] + s[u].y * ak[1] + s[u].z * ak[2] + s[u].w * ak[3];
        float sq = s[u].x * aq[0] + s[u].y * aq[1] + s[u].z * aq[2] + s[u].w * aq[3];
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) {
            sk += __shfl_xor(sk, m, kWave);
            sq += __shfl_xor(sq, m, kWave);
        }
        const float vi = to_f32(v[(size_t)head * DV + row[u]]);
        const float ui = b * (vi - sk);
        float4 ns;
        ns.x = s[u].x * a[0] + ui * kk[0];
        ns.y = s[u].y * a[1] + ui * kk[1];
        ns.z = s[u].z * a[2] + ui * kk[2];
        ns.w = s[u].w * a[3] + ui * kk[3];
        // the new state is not read again in this step: a non-temporal store
        // (measured 3 % faster per step than a plain one; non-temporal reads
        // of the state were 12 % slower)
        __builtin_nontemporal_store(f32x4{ns.x, ns.y, ns.z, ns.w},
                                    reinterpret_cast<f32x4*>(S + ((size_t)head * DV + row[u]) * DK + 4 * c));
        if (c == 0) o[(size_t)head * DV + row[u]] = from_f32<T>(sq + ui * kq);
    }
}

template <typename T, int DK, int MODE>
static hipError_t launch_decode(int NH, int DV, const void* q, const void* k, const void* v,
                                const float* beta, const float* log_alpha, float* S, void* o,
                                hipStream_t stream, unsigned pro)
{
    constexpr int RB = decode_rows_per_block<DK>();
    const int blocks = NH * (DV / RB);
    hipLaunchKernelGGL((decode_step_kernel<T, DK, MODE>), dim3(blocks), dim3(256), 0, stream,
                       DV, (const T*)q, (const T*)k, (const T*)v, beta, log_alpha, S, (T*)o, pro);
    return hipGetLastError();
}

template <typename T, int DK>
static hipError_t dispatch_mode(int mode, int NH, int DV, const void* q, const void* k,
                                const void* v, const float* beta, const float* la, float* S,
                                void* o, hipStream_t st, unsigned pro)
{
    switch (mode) {
    case kAlphaNone: return launch_decode<T, DK, kAlphaNone>(NH, DV, q, k, v, beta, la, S, o, st, pro);
    case kAlphaScalar: return launch_decode<T, DK, kAlphaScalar>(NH, DV, q, k, v, beta, la, S, o, st, pro);
    default: return launch_decode<T, DK, kAlphaChannel>(NH, DV, q, k, v, beta, la, S, o, st, pro);
    }
}

hipError_t launch_decode_step(const DecodeArgs& a)
{
    const int NH = a.N * a.H;
    if (a.dtype == kBF16) {
        if (a.dk == 128) return dispatch_mode<bf16, 128>(a.mode, NH, a.dv, a.q, a.k, a.v, a.beta, a.log_alpha, a.S, a.o, a.stream, a.pro);
        return dispatch_mode<bf16, 64>(a.mode, NH, a.dv, a.q, a.k, a.v, a.beta, a.log_alpha, a.S, a.o, a.stream, a.pro);
    }
    if (a.dk == 128) return dispatch_mode<float, 128>(a.mode, NH, a.dv, a.q, a.k, a.v, a.beta, a.log_alpha, a.S, a.o, a.stream, a.pro);
    return dispatch_mode<float, 64>(a.mode, NH, a.dv, a.q, a.k, a.v, a.beta, a.log_alpha, a.S, a.o, a.stream, a.pro);
}

}  // namespace gdr

// gdr_bwd.hip -- chunked backward (the gradients training needs) of the
// gated delta-rule memory, for alpha = 1 and scalar alpha.
//
// Forward over one chunk of C tokens with entry state S0 (notation of
// gdr_scan.hip; g = in-chunk cumulative log alpha, gamma = e^g,
// D = e^{g_C - g}, Gamma_rs = e^{g_r - g_s}):
//   A = strictly-lower(diag(beta)(K K^T . Gamma)),  T = (I + A)^{-1},
//   T~ = T diag(beta),  X = K S0^T,  R = V - diag(gamma) X,  U = T~ R,
//   P = Q K^T . Gamma . M_incl,  O = diag(gamma) Q S0^T + P U,
//   S_end = gamma_C S0 + U^T diag(D) K.
// Reverse mode, given dO and dS_end (derived by the chain rule from these
// lines; the per-token form is the fp64 oracle's):
//   dU = P^T dO + diag(D) K dS_end^T,   dR = T~^T dU,   dV = dR,
//   dX = -diag(gamma) dR,
//   dS0 = gamma_C dS_end + dO^T diag(gamma) Q + dX^T K            (the chain)
//   dQ = diag(gamma) dO S0 + (dO U^T . Gamma . M_incl) K
//   dK = (dO U^T . Gamma . M_incl)^T Q + diag(D) U dS_end + dX S0 + dG K + dG^T K
//   with dT~ = dU R^T, dbeta_s = sum_r T_rs dT~_rs + sum_s' dA_ss' (K K^T . Gamma)_ss',
//   dA = strictly-lower(-T^T (dT~ diag(beta)) T^T), dG = dA . diag(beta) Gamma,
//   and for the log-decay every place g enters (gamma, D, gamma_C, Gamma)
//   gives a term of dg; d log alpha_t = sum_{r >= t} dg_r within the chunk.
// ("linear attention and its gated descendants", "Chunkwise Parallel Form"
// and "Gated DeltaNet"; the WY factor of "Linear Attention & DeltaNet",
// "How it works", item 3.)
//
// Launches: the forward prepass and scan run again (the scan keeping the
// state entering every chunk), then
//   chunk_bwd_chain_kernel  one workgroup per (b, h, 32 value channels)
//                           walks the chunks backwards carrying dS (the
//                           only sequential part) and keeps dS_end of every
//                           chunk;
//   chunk_bwd_grad_kernel   one workgroup per chunk: every gradient of the
//                           chunk's tokens from S0, dS_end and its inputs.
// The products run on MFMA (bf16 operands for bf16 inputs, fp32 otherwise;
// fp32 accumulation); the triangular parts (T, dA) stay in fp32.
#include "gdr_device.h"
#include "gdr_chunk.h"
#include "gdr_tri.h"

namespace gdr {

namespace {

constexpr int kBV = 32;   // value channels per block

template <typename E>
__device__ __forceinline__ void pack_frag(Frag<E>& f, const float* x);
template <>
__device__ __forceinline__ void pack_frag<bf16>(Frag<bf16>& f, const float* x) {
    f.v = __builtin_bit_cast(bf16x8, Pack<bf16>::pack(x));
}
template <>
__device__ __forceinline__ void pack_frag<float>(Frag<float>& f, const float* x) {
    f.lo = f32x4{x[0], x[1], x[2], x[3]};
    f.hi = f32x4{x[4], x[5], x[6], x[7]};
}

// acc += A B^T on one 16 x 16 tile: A(m, k) = A[m * ars + k * aks] for rows
// m0 .. m0 + 15, B(n, k) = B[n * brs + k * bks] for rows n0 .. n0 + 15, over
// k < K (zero-filled up to the next multiple of 32).  Operands are gathered
// element by element, so any layout serves; lane (g, c) ends with
// acc[e] = (A B^T)[m0 + 4 g + e][n0 + c].
template <typename E, typename TA, typename TB>
__device__ __forceinline__ void tmma(f32x4& acc, const TA* A, int ars, int aks, int m0,
                                     const TB* B, int brs, int bks, int n0, int K)
{
    const int l = lane_id(), r = l & 15, g = l >> 4;
    for (int k0 = 0; k0 < K; k0 += 32) {
        float xa[8], xb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = k0 + 8 * g + j;
            xa[j] = k < K ? to_f32(A[(m0 + r) * ars + k * aks]) : 0.f;
            xb[j] = k < K ? to_f32(B[(n0 + r) * brs + k * bks]) : 0.f;
        }
        Frag<E> fa, fb;
        pack_frag<E>(fa, xa);
        pack_frag<E>(fb, xb);
        mma(acc, fa, fb);
    }
}

// Sum of x over the 16 lanes that share l / 16 (one tile row).
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

struct BwdParams {
    const void *q, *k, *v, *dO;
    const float *beta, *log_alpha;   // log_alpha NULL: alpha = 1
    const float* dS_final;           // [B*H][d_v][d_k] or null
    const unsigned char* ws;         // forward prepass records
    const float* Sck;                // [B*H][NC][d_v][d_k]: state entering each chunk
    float* dSck;                     // [B*H][NC][d_v][d_k]: dS at each chunk's end
    void *dq, *dk, *dv;
    float *dbeta, *dlog_alpha, *dS0;
    int L, NC, DV, total;
};

// ---------------------------------------------------------------- chain
template <typename E, int DK, int CK>
struct ChainLds {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int off_K = 0;                          // [CK][DK] E
    static constexpr int off_Q = off_K + CK * DK * ES;       // [CK][DK] E
    static constexpr int off_dO = off_Q + CK * DK * ES;      // [CK][kBV] E
    static constexpr int off_gdO = off_dO + CK * kBV * ES;   // gamma . dO
    static constexpr int off_T = off_gdO + CK * kBV * ES;    // [CK][CK] f32, T~
    static constexpr int off_M = off_T + CK * CK * 4;        // [CK][CK] f32, Gamma . M_incl
    static constexpr int off_P = off_M + CK * CK * 4;        // [CK][CK] f32
    static constexpr int off_f = off_P + CK * CK * 4;        // gamma [CK], D [CK], gamma_C
    static constexpr int off_w = off_f + (2 * CK + 4) * 4;   // per wave: dS [16][DK], dU, -gamma dR [CK][16]
    static constexpr int wbytes = 16 * DK * ES + 2 * CK * 16 * ES;
    static constexpr int bytes = off_w + 2 * wbytes;
};

template <typename E, int DK, int CK>
__global__ __launch_bounds__(128) void chunk_bwd_chain_kernel(BwdParams p)
{
    using LY = ChainLds<E, DK, CK>;
    constexpr int NJ = DK / 16, NB = CK / 16;
    constexpr WsLayout WL = ws_layout((int)sizeof(E), DK, CK, kAlphaScalar);
    extern __shared__ __align__(16) unsigned char smem[];
    E* Ks = reinterpret_cast<E*>(smem + LY::off_K);
    E* Qs = reinterpret_cast<E*>(smem + LY::off_Q);
    E* dOs = reinterpret_cast<E*>(smem + LY::off_dO);
    E* gdOs = reinterpret_cast<E*>(smem + LY::off_gdO);
    float* Ts = reinterpret_cast<float*>(smem + LY::off_T);
    float* Ms = reinterpret_cast<float*>(smem + LY::off_M);
    float* Ps = reinterpret_cast<float*>(smem + LY::off_P);
    float* gam = reinterpret_cast<float*>(smem + LY::off_f);
    float* Dd = gam + CK;
    const int tid = threadIdx.x, w = wave_id(), l = lane_id(), g4 = l >> 4, c16 = l & 15;
    E* dSw = reinterpret_cast<E*>(smem + LY::off_w + w * LY::wbytes);   // [16][DK]
    E* dUw = dSw + 16 * DK;                                             // [CK][16]
    E* dRw = dUw + CK * 16;                                             // -gamma dR, [CK][16]

    const int nvb = p.DV / kBV;
    const int bh = blockIdx.x / nvb, v0 = (blockIdx.x % nvb) * kBV;
    const int i0 = v0 + 16 * w;   // this wave's first value channel

    // dS rows i0 + 4 g4 + e, key channels 16 jb + c16
    f32x4 dS[NJ];
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
        dS[jb] = zero4();
        if (p.dS_final)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dS[jb][e] = p.dS_final[((size_t)bh * p.DV + i0 + 4 * g4 + e) * DK + 16 * jb + c16];
    }

    for (int n = p.NC - 1; n >= 0; --n) {
        const int t0 = n * CK, valid = min(CK, p.L - t0);
        const size_t tok = (size_t)bh * p.L + t0;
        const unsigned char* rec = p.ws + ((size_t)bh * p.NC + n) * WL.bytes;
        // ---- stage the chunk; keep dS at the chunk's end
        const E* kg = reinterpret_cast<const E*>(p.k) + tok * DK;
        const E* qg = reinterpret_cast<const E*>(p.q) + tok * DK;
        const E* dog = reinterpret_cast<const E*>(p.dO) + tok * p.DV + v0;
        const E* Tg = reinterpret_cast<const E*>(rec + WL.T);
        const E* Mg = reinterpret_cast<const E*>(rec + WL.M);
        const float* Fg = reinterpret_cast<const float*>(rec + WL.F);
        if (tid < CK) {
            gam[tid] = Fg[tid];
            Dd[tid] = Fg[CK + tid];
        }
        if (tid == 0) gam[2 * CK] = Fg[2 * CK];
        for (int x = tid; x < CK * DK; x += 128) {
            const int r = x / DK;
            Ks[x] = r < valid ? kg[x] : from_f32<E>(0.f);
            Qs[x] = r < valid ? qg[x] : from_f32<E>(0.f);
        }
        for (int x = tid; x < CK * CK; x += 128) {
            const int r = x / CK, mc = x % CK, t = tok_of_col(CK, mc);
            Ts[r * CK + t] = to_f32(Tg[x]);
            Ms[r * CK + t] = to_f32(Mg[x]);
        }
        float* dsk = p.dSck + (((size_t)bh * p.NC + n) * p.DV + i0) * DK;
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * g4 + e, j = 16 * jb + c16;
                dsk[(size_t)i * DK + j] = dS[jb][e];
                dSw[i * DK + j] = from_f32<E>(dS[jb][e]);
            }
        __syncthreads();
        for (int x = tid; x < CK * kBV; x += 128) {
            const int r = x / kBV, i = x % kBV;
            const float d = r < valid ? to_f32(dog[(size_t)r * p.DV + i]) : 0.f;
            dOs[x] = from_f32<E>(d);
            gdOs[x] = from_f32<E>(gam[r] * d);
        }
        // ---- P = Q K^T . Gamma . M_incl (tiles on or below the diagonal)
        for (int tl = w; tl < NB * NB; tl += 2) {
            const int rb = tl / NB, ib = tl % NB;
            f32x4 acc = zero4();
            if (ib <= rb) tmma<E>(acc, Qs, DK, 1, 16 * rb, Ks, DK, 1, 16 * ib, DK);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e, s = 16 * ib + c16;
                Ps[r * CK + s] = acc[e] * Ms[r * CK + s];
            }
        }
        __syncthreads();
        // ---- dU = P^T dO + diag(D) K dS^T  (token r, value channel 16 w + c)
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            f32x4 kds = zero4(), y = zero4();
            tmma<E>(kds, Ks, DK, 1, 16 * rb, dSw, DK, 1, 0, DK);
            tmma<E>(y, Ps, 1, CK, 16 * rb, dOs + 16 * w, 1, kBV, 0, CK);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e;
                dUw[r * 16 + c16] = from_f32<E>(y[e] + Dd[r] * kds[e]);
            }
        }
        wave_lds_fence();
        // ---- dR = T~^T dU, kept as -gamma dR
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            f32x4 dr = zero4();
            tmma<E>(dr, Ts, 1, CK, 16 * rb, dUw, 1, 16, 0, CK);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e;
                dRw[r * 16 + c16] = from_f32<E>(-gam[r] * dr[e]);
            }
        }
        wave_lds_fence();
        // ---- dS <- gamma_C dS + (gamma . dO)^T Q - (gamma . dR)^T K
        const float gC = gam[2 * CK];
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
            f32x4 acc = dS[jb];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] *= gC;
            tmma<E>(acc, gdOs + 16 * w, 1, kBV, 0, Qs, 1, DK, 16 * jb, CK);
            tmma<E>(acc, dRw, 1, 16, 0, Ks, 1, DK, 16 * jb, CK);
            dS[jb] = acc;
        }
        __syncthreads();   // the LDS is restaged for the previous chunk
    }
    if (p.dS0) {
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.dS0[((size_t)bh * p.DV + i0 + 4 * g4 + e) * DK + 16 * jb + c16] = dS[jb][e];
    }
}

// ---------------------------------------------------------------- grads
template <typename E, int DK, int CK>
struct GradLds {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int LF = CK + 4;                        // fp32 C x C row stride
    static constexpr int off_K = 0;                          // [CK][DK] E
    static constexpr int off_Q = off_K + CK * DK * ES;
    static constexpr int off_S0 = off_Q + CK * DK * ES;      // [kBV][DK] E (one value block)
    static constexpr int off_dS = off_S0 + kBV * DK * ES;
    static constexpr int off_dO = off_dS + kBV * DK * ES;    // [CK][kBV] E
    static constexpr int off_gdO = off_dO + CK * kBV * ES;
    static constexpr int off_R = off_gdO + CK * kBV * ES;
    static constexpr int off_U = off_R + CK * kBV * ES;
    static constexpr int off_DU = off_U + CK * kBV * ES;
    static constexpr int off_dU = off_DU + CK * kBV * ES;
    static constexpr int off_dX = off_dU + CK * kBV * ES;
    static constexpr int off_V = off_dX + CK * kBV * ES;     // [CK][kBV] f32
    static constexpr int off_X = off_V + CK * kBV * 4;
    static constexpr int off_KdS = off_X + CK * kBV * 4;
    static constexpr int off_Bm = off_KdS + CK * kBV * 4;    // [CK][LF] f32 each
    static constexpr int off_A = off_Bm + CK * LF * 4;
    static constexpr int off_T = off_A + CK * LF * 4;
    static constexpr int off_Tt = off_T + CK * LF * 4;       // T~ = T diag(beta)
    static constexpr int off_P = off_Tt + CK * LF * 4;
    static constexpr int off_dPW = off_P + CK * LF * 4;
    static constexpr int off_Em = off_dPW + CK * LF * 4;     // dP . P, then dA . A
    static constexpr int off_dTb = off_Em + CK * LF * 4;     // dT~ diag(beta)
    static constexpr int off_dTt = off_dTb + CK * LF * 4;
    static constexpr int off_Y1 = off_dTt + CK * LF * 4;
    static constexpr int off_dA = off_Y1 + CK * LF * 4;
    static constexpr int off_dG = off_dA + CK * LF * 4;
    static constexpr int off_vec = off_dG + CK * LF * 4;     // g, gamma, D, beta, dg [CK]; parts
    static constexpr int NVEC = 5 * CK + 4 * (2 * CK) + 8;
    static constexpr int bytes = off_vec + NVEC * 4;
};

template <typename E, int DK, int CK>
__global__ __launch_bounds__(256) void chunk_bwd_grad_kernel(BwdParams p)
{
    using LY = GradLds<E, DK, CK>;
    constexpr int LF = LY::LF, NB = CK / 16, NJ = DK / 16;
    constexpr int NQT = NB * NJ;                 // C x DK tiles
    constexpr int NQW = (NQT + 3) / 4;           // per wave
    constexpr int NCB = NB * (kBV / 16);         // C x kBV tiles (<= 4)
    constexpr int NCC = NB * NB;                 // C x C tiles (<= 4)
    extern __shared__ __align__(16) unsigned char smem[];
    E* Ks = reinterpret_cast<E*>(smem + LY::off_K);
    E* Qs = reinterpret_cast<E*>(smem + LY::off_Q);
    E* S0s = reinterpret_cast<E*>(smem + LY::off_S0);
    E* dSs = reinterpret_cast<E*>(smem + LY::off_dS);
    E* dOs = reinterpret_cast<E*>(smem + LY::off_dO);
    E* gdOs = reinterpret_cast<E*>(smem + LY::off_gdO);
    E* Rs = reinterpret_cast<E*>(smem + LY::off_R);
    E* Us = reinterpret_cast<E*>(smem + LY::off_U);
    E* DUs = reinterpret_cast<E*>(smem + LY::off_DU);
    E* dUs = reinterpret_cast<E*>(smem + LY::off_dU);
    E* dXs = reinterpret_cast<E*>(smem + LY::off_dX);
    float* Vs = reinterpret_cast<float*>(smem + LY::off_V);
    float* Xs = reinterpret_cast<float*>(smem + LY::off_X);
    float* KdSs = reinterpret_cast<float*>(smem + LY::off_KdS);
    float* Bm = reinterpret_cast<float*>(smem + LY::off_Bm);
    float* Af = reinterpret_cast<float*>(smem + LY::off_A);
    float* Tf = reinterpret_cast<float*>(smem + LY::off_T);
    float* Tt = reinterpret_cast<float*>(smem + LY::off_Tt);
    float* Pf = reinterpret_cast<float*>(smem + LY::off_P);
    float* dPW = reinterpret_cast<float*>(smem + LY::off_dPW);
    float* Em = reinterpret_cast<float*>(smem + LY::off_Em);
    float* dTb = reinterpret_cast<float*>(smem + LY::off_dTb);
    float* dTt = reinterpret_cast<float*>(smem + LY::off_dTt);
    float* Y1 = reinterpret_cast<float*>(smem + LY::off_Y1);
    float* dAf = reinterpret_cast<float*>(smem + LY::off_dA);
    float* dGf = reinterpret_cast<float*>(smem + LY::off_dG);
    float* gs = reinterpret_cast<float*>(smem + LY::off_vec);
    float* gam = gs + CK;
    float* Dd = gam + CK;
    float* bs = Dd + CK;
    float* dg = bs + CK;
    float* hgp = dg + CK;        // [4][CK] per-wave partial sums of the gamma terms
    float* frp = hgp + 4 * CK;   // [4][CK] per-wave partial sums of the D terms
    float* red = frp + 4 * CK;   // [8]: per-wave <dS_end, S0>

    const int cid = blockIdx.x;
    const int tid = threadIdx.x, w = wave_id(), l = lane_id(), g4 = l >> 4, c16 = l & 15;
    const int bh = cid / p.NC, n = cid % p.NC;
    const int t0 = n * CK, valid = min(CK, p.L - t0);
    const size_t tok = (size_t)bh * p.L + t0;
    const E* kg = reinterpret_cast<const E*>(p.k) + tok * DK;
    const E* qg = reinterpret_cast<const E*>(p.q) + tok * DK;

    // ---- the chunk's keys, queries and gates
    for (int x = tid; x < CK * DK; x += 256) {
        const int r = x / DK;
        Ks[x] = r < valid ? kg[x] : from_f32<E>(0.f);
        Qs[x] = r < valid ? qg[x] : from_f32<E>(0.f);
    }
    for (int x = tid; x < 8 * CK; x += 256) hgp[x] = 0.f;   // hgp and frp
    if (w == 0) {
        float la = 0.f, bt = 0.f;
        if (l < valid) {
            bt = p.beta[tok + l];
            if (p.log_alpha) la = p.log_alpha[tok + l];
        }
        const float g = wave_incl_scan(la);
        const float gC = __shfl(g, CK - 1, kWave);
        if (l < CK) {
            gs[l] = g;
            gam[l] = __expf(g);
            Dd[l] = __expf(gC - g);
            bs[l] = bt;
        }
    }
    __syncthreads();
    // ---- Gram and score tiles: Bm = strictly-lower(K K^T . Gamma),
    // A = diag(beta) Bm, P = Q K^T . Gamma (diagonal included)
    if (w < NCC) {
        const int rb = w / NB, ib = w % NB;
        f32x4 kk = zero4(), qk = zero4();
        if (ib <= rb) {
            tmma<E>(kk, Ks, DK, 1, 16 * rb, Ks, DK, 1, 16 * ib, DK);
            tmma<E>(qk, Qs, DK, 1, 16 * rb, Ks, DK, 1, 16 * ib, DK);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e, s = 16 * ib + c16;
            const float G = r >= s ? __expf(gs[r] - gs[s]) : 0.f;
            Bm[r * LF + s] = r > s ? kk[e] * G : 0.f;
            Af[r * LF + s] = r > s ? bs[r] * kk[e] * G : 0.f;
            Pf[r * LF + s] = qk[e] * G;
        }
    }
    __syncthreads();
    if (w == 0) unit_lower_inverse<CK, LF>(Af, Tf);
    __syncthreads();
    // the inverse leaves the block above the diagonal unwritten
    for (int x = tid; x < CK * CK; x += 256) {
        const int r = x / CK, s = x % CK;
        const float t = s <= r ? Tf[r * LF + s] : 0.f;
        Tf[r * LF + s] = t;
        Tt[r * LF + s] = t * bs[s];
    }

    f32x4 dQa[NQW], dKa[NQW];
#pragma unroll
    for (int u = 0; u < NQW; ++u) { dQa[u] = zero4(); dKa[u] = zero4(); }
    f32x4 dPa = zero4(), dTa = zero4();   // C x C tile w (w < NCC)
    float hS = 0.f;                       // this thread's part of <dS_end, S0>

    const float* S0g = p.Sck + (size_t)cid * p.DV * DK;
    const float* dSg = p.dSck + (size_t)cid * p.DV * DK;
    for (int v0 = 0; v0 < p.DV; v0 += kBV) {
        __syncthreads();   // the previous block's operands are consumed
        // ---- one block of value channels: S0, dS_end rows, V and dO columns
        for (int x = tid; x < kBV * DK; x += 256) {
            const float a = S0g[(size_t)v0 * DK + x], b = dSg[(size_t)v0 * DK + x];
            S0s[x] = from_f32<E>(a);
            dSs[x] = from_f32<E>(b);
            hS += a * b;
        }
        const E* vg = reinterpret_cast<const E*>(p.v) + tok * p.DV + v0;
        const E* dog = reinterpret_cast<const E*>(p.dO) + tok * p.DV + v0;
        for (int x = tid; x < CK * kBV; x += 256) {
            const int r = x / kBV, i = x % kBV;
            const bool ok = r < valid;
            const float vv = ok ? to_f32(vg[(size_t)r * p.DV + i]) : 0.f;
            const float d = ok ? to_f32(dog[(size_t)r * p.DV + i]) : 0.f;
            Vs[x] = vv;
            dOs[x] = from_f32<E>(d);
            gdOs[x] = from_f32<E>(gam[r] * d);
        }
        __syncthreads();
        // ---- X = K S0^T, R = V - gamma X; K dS^T; the gamma . dO . Q S0^T term
        if (w < NCB) {
            const int rb = w / 2, cb = w % 2;
            f32x4 x = zero4(), qs = zero4(), kds = zero4();
            tmma<E>(x, Ks, DK, 1, 16 * rb, S0s, DK, 1, 16 * cb, DK);
            tmma<E>(qs, Qs, DK, 1, 16 * rb, S0s, DK, 1, 16 * cb, DK);
            tmma<E>(kds, Ks, DK, 1, 16 * rb, dSs, DK, 1, 16 * cb, DK);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e, i = 16 * cb + c16;
                Xs[r * kBV + i] = x[e];
                KdSs[r * kBV + i] = kds[e];
                Rs[r * kBV + i] = from_f32<E>(Vs[r * kBV + i] - gam[r] * x[e]);
                const float h = row16_sum(to_f32(gdOs[r * kBV + i]) * qs[e]);
                if (c16 == 0) hgp[w * CK + r] += h;
            }
        }
        __syncthreads();
        // ---- U = T~ R, dU = P^T dO + D . K dS^T
        if (w < NCB) {
            const int rb = w / 2, cb = w % 2;
            f32x4 u = zero4(), du = zero4();
            tmma<E>(u, Tt, LF, 1, 16 * rb, Rs + 16 * cb, 1, kBV, 0, CK);
            tmma<E>(du, Pf, 1, LF, 16 * rb, dOs + 16 * cb, 1, kBV, 0, CK);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e, i = 16 * cb + c16;
                const float kds = KdSs[r * kBV + i];
                Us[r * kBV + i] = from_f32<E>(u[e]);
                DUs[r * kBV + i] = from_f32<E>(Dd[r] * u[e]);
                dUs[r * kBV + i] = from_f32<E>(du[e] + Dd[r] * kds);
                const float f = row16_sum(Dd[r] * u[e] * kds);
                if (c16 == 0) frp[w * CK + r] += f;
            }
        }
        __syncthreads();
        // ---- dR = T~^T dU (= dV), dX = -gamma dR
        if (w < NCB) {
            const int rb = w / 2, cb = w % 2;
            f32x4 dr = zero4();
            tmma<E>(dr, Tt, 1, LF, 16 * rb, dUs + 16 * cb, 1, kBV, 0, CK);
            E* dvg = reinterpret_cast<E*>(p.dv) + tok * p.DV + v0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e, i = 16 * cb + c16;
                if (r < valid) dvg[(size_t)r * p.DV + i] = from_f32<E>(dr[e]);
                dXs[r * kBV + i] = from_f32<E>(-gam[r] * dr[e]);
                const float h = row16_sum(-gam[r] * dr[e] * Xs[r * kBV + i]);
                if (c16 == 0) hgp[w * CK + r] += h;
            }
        }
        __syncthreads();
        // ---- accumulate over the block's value channels
#pragma unroll
        for (int u = 0; u < NQW; ++u) {
            const int t = w + 4 * u;
            if (t < NQT) {
                const int rb = t / NJ, jb = t % NJ;
                tmma<E>(dQa[u], gdOs, kBV, 1, 16 * rb, S0s, 1, DK, 16 * jb, kBV);
                tmma<E>(dKa[u], DUs, kBV, 1, 16 * rb, dSs, 1, DK, 16 * jb, kBV);
                tmma<E>(dKa[u], dXs, kBV, 1, 16 * rb, S0s, 1, DK, 16 * jb, kBV);
            }
        }
        if (w < NCC) {
            const int rb = w / NB, sb = w % NB;
            tmma<E>(dPa, dOs, kBV, 1, 16 * rb, Us, kBV, 1, 16 * sb, kBV);
            tmma<E>(dTa, dUs, kBV, 1, 16 * rb, Rs, kBV, 1, 16 * sb, kBV);
        }
    }

    // ---- C x C terms
    if (w < NCC) {
        const int rb = w / NB, sb = w % NB;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e, s = 16 * sb + c16;
            const float W = r >= s ? __expf(gs[r] - gs[s]) : 0.f;
            dPW[r * LF + s] = dPa[e] * W;
            Em[r * LF + s] = dPa[e] * Pf[r * LF + s];
            dTt[r * LF + s] = dTa[e];
            dTb[r * LF + s] = dTa[e] * bs[s];
        }
    }
    {
        // <dS_end, S0> over the whole state
        float x = hS;
#pragma unroll
        for (int m = kWave / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
        if (l == 0) red[w] = x;
    }
    __syncthreads();
    // dQ += (dP . W) K, dK += (dP . W)^T Q; Y1 = dT~ diag(beta) T^T
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        const int t = w + 4 * u;
        if (t < NQT) {
            const int rb = t / NJ, jb = t % NJ;
            tmma<E>(dQa[u], dPW, LF, 1, 16 * rb, Ks, 1, DK, 16 * jb, CK);
            tmma<E>(dKa[u], dPW, 1, LF, 16 * rb, Qs, 1, DK, 16 * jb, CK);
        }
    }
    if (w < NCC) {
        const int rb = w / NB, sb = w % NB;
        f32x4 y = zero4();
        tmma<float>(y, dTb, LF, 1, 16 * rb, Tf, LF, 1, 16 * sb, CK);
#pragma unroll
        for (int e = 0; e < 4; ++e) Y1[(16 * rb + 4 * g4 + e) * LF + 16 * sb + c16] = y[e];
    }
    // the dg terms of dP . P
    if (tid < CK) {
        float a = 0.f;
        for (int s = 0; s < CK; ++s) a += Em[tid * LF + s] - Em[s * LF + tid];
        dg[tid] = a;
    }
    __syncthreads();
    // dA = strictly-lower(-T^T Y1); dG = dA . diag(beta) Gamma; dA . A
    if (w < NCC) {
        const int rb = w / NB, sb = w % NB;
        f32x4 y = zero4();
        tmma<float>(y, Tf, 1, LF, 16 * rb, Y1, 1, LF, 16 * sb, CK);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e, s = 16 * sb + c16;
            const float da = r > s ? -y[e] : 0.f;
            dAf[r * LF + s] = da;
            dGf[r * LF + s] = r > s ? da * bs[r] * __expf(gs[r] - gs[s]) : 0.f;
            Em[r * LF + s] = da * Af[r * LF + s];
        }
    }
    __syncthreads();
    // dK += dG K + dG^T K
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        const int t = w + 4 * u;
        if (t < NQT) {
            const int rb = t / NJ, jb = t % NJ;
            tmma<E>(dKa[u], dGf, LF, 1, 16 * rb, Ks, 1, DK, 16 * jb, CK);
            tmma<E>(dKa[u], dGf, 1, LF, 16 * rb, Ks, 1, DK, 16 * jb, CK);
        }
    }
    // dbeta and dg per token, then d log alpha = suffix sums of dg
    if (w == 0) {
        float db = 0.f, dgl = 0.f, fr = 0.f;
        if (l < CK) {
            for (int u = 0; u < CK; ++u) db += Tf[u * LF + l] * dTt[u * LF + l];
            for (int s = 0; s < CK; ++s) db += dAf[l * LF + s] * Bm[l * LF + s];
            float fa = 0.f, hg = 0.f;
            for (int s = 0; s < CK; ++s) fa += Em[l * LF + s] - Em[s * LF + l];
            for (int x = 0; x < 4; ++x) {
                fr += frp[x * CK + l];
                hg += hgp[x * CK + l];
            }
            dgl = dg[l] + fa + hg - fr;
        }
        // g_C enters gamma_C S0 and every D_r = e^{g_C - g_r}
        float fsum = fr;
#pragma unroll
        for (int m = kWave / 2; m >= 1; m >>= 1) fsum += __shfl_xor(fsum, m, kWave);
        if (l == CK - 1) dgl += gam[CK - 1] * (red[0] + red[1] + red[2] + red[3]) + fsum;
        const float incl = wave_incl_scan(dgl);
        const float total = __shfl(incl, CK - 1, kWave);
        if (l < valid) {
            p.dbeta[tok + l] = db;
            if (p.dlog_alpha) p.dlog_alpha[tok + l] = total - incl + dgl;
        }
    }
    // ---- dq, dk
    E* dqg = reinterpret_cast<E*>(p.dq) + tok * DK;
    E* dkg = reinterpret_cast<E*>(p.dk) + tok * DK;
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        const int t = w + 4 * u;
        if (t < NQT) {
            const int rb = t / NJ, jb = t % NJ;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e, j = 16 * jb + c16;
                if (r < valid) {
                    dqg[(size_t)r * DK + j] = from_f32<E>(dQa[u][e]);
                    dkg[(size_t)r * DK + j] = from_f32<E>(dKa[u][e]);
                }
            }
        }
    }
}

template <typename E, int DK, int CK>
static hipError_t launch_bwd_t(const BwdParams& bp, int BH, hipStream_t stream)
{
    using CL = ChainLds<E, DK, CK>;
    using GL = GradLds<E, DK, CK>;
    static_assert(CL::bytes <= 160 * 1024 && GL::bytes <= 160 * 1024, "LDS budget");
    auto* chain = chunk_bwd_chain_kernel<E, DK, CK>;
    hipError_t err = hipFuncSetAttribute((const void*)chain, hipFuncAttributeMaxDynamicSharedMemorySize, CL::bytes);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(chain, dim3(BH * (bp.DV / kBV)), dim3(128), CL::bytes, stream, bp);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    auto* grad = chunk_bwd_grad_kernel<E, DK, CK>;
    err = hipFuncSetAttribute((const void*)grad, hipFuncAttributeMaxDynamicSharedMemorySize, GL::bytes);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(grad, dim3(bp.total), dim3(256), GL::bytes, stream, bp);
    return hipGetLastError();
}

}  // namespace

// Workspace of the backward: the forward's chunk records, the state entering
// every chunk, dS at every chunk's end, and the recomputed outputs.
struct BwdWs {
    size_t off_Sck, off_dSck, off_o, bytes;
};

static BwdWs bwd_ws(int B, int H, int L, int dk, int dv, int C, int dtype)
{
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const int CK = chunk_step(C, dtype);
    const size_t BH = (size_t)B * H, NC = (size_t)((L + CK - 1) / CK);
    const int es = dtype == kBF16 ? 2 : 4;
    BwdWs w{};
    size_t o = al(BH * NC * (size_t)ws_layout(es, dk, CK, kAlphaScalar).bytes);
    w.off_Sck = o; o = al(o + BH * NC * dv * dk * 4);
    w.off_dSck = o; o = al(o + BH * NC * dv * dk * 4);
    w.off_o = o; o = al(o + BH * (size_t)L * dv * es);
    w.bytes = o;
    return w;
}

size_t bwd_workspace_bytes(int B, int H, int L, int dk, int dv, int C, int dtype)
{
    if ((size_t)B * H == 0 || L == 0) return 0;
    return bwd_ws(B, H, L, dk, dv, C, dtype).bytes;
}

__global__ void copy_grad_state_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_bwd_chunked(const BwdArgs& b)
{
    const size_t BH = (size_t)b.B * b.H;
    if (BH == 0) return hipSuccess;
    if (b.L == 0) {
        // no tokens: the gradient reaching S0 is the one given for S_final
        if (!b.dS0) return hipSuccess;
        const size_t n = BH * b.dv * b.dk;
        hipLaunchKernelGGL(copy_grad_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, b.stream,
                           b.dS_final, b.dS0, n);
        return hipGetLastError();
    }
    const int CK = chunk_step(b.C, b.dtype);
    const int NC = (b.L + CK - 1) / CK;
    const BwdWs w = bwd_ws(b.B, b.H, b.L, b.dk, b.dv, b.C, b.dtype);
    unsigned char* ws = static_cast<unsigned char*>(b.workspace);
    // forward again: the prepass records and every chunk's entry state
    ChunkArgs a{b.B, b.H, b.L, b.dk, b.dv, b.C, b.dtype, b.mode, b.q, b.k, b.v, b.beta, b.log_alpha, b.S0,
                ws + w.off_o, nullptr, ws, b.stream, 0u, nullptr, 0, Varlen{}, reinterpret_cast<float*>(ws + w.off_Sck)};
    hipError_t err = launch_wy(a, CK);
    if (err != hipSuccess) return err;
    SegPlan one{1, NC, 0, 0, 0, 0, 0};
    err = launch_scan(a, CK, one);
    if (err != hipSuccess) return err;
    BwdParams bp{b.q, b.k, b.v, b.dO, b.beta, b.log_alpha, b.dS_final, ws,
                 reinterpret_cast<const float*>(ws + w.off_Sck), reinterpret_cast<float*>(ws + w.off_dSck),
                 b.dq, b.dk_out, b.dv_out, b.dbeta, b.dlog_alpha, b.dS0, b.L, NC, b.dv, (int)(BH * NC)};
    if (b.dtype == kBF16) {
        if (b.dk == 128) return CK == 16 ? launch_bwd_t<bf16, 128, 16>(bp, (int)BH, b.stream)
                                         : launch_bwd_t<bf16, 128, 32>(bp, (int)BH, b.stream);
        return CK == 16 ? launch_bwd_t<bf16, 64, 16>(bp, (int)BH, b.stream) : launch_bwd_t<bf16, 64, 32>(bp, (int)BH, b.stream);
    }
    return b.dk == 128 ? launch_bwd_t<float, 128, 16>(bp, (int)BH, b.stream) : launch_bwd_t<float, 64, 16>(bp, (int)BH, b.stream);
}

}  // namespace gdr

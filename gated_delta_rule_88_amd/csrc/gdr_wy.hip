// gdr_wy.hip -- per-chunk prepass of the chunked forward: everything about a
// chunk that does not depend on the state entering it.
//
// For a chunk of CK tokens of one (b, h) (notation of gdr_scan.hip):
//   g_r = sum_{s<=r} log alpha_s           in-chunk cumulative log-decay
//   A   = strictly-lower( diag(beta) (K K^T . Gamma) ),  Gamma_ri = exp(g_r - g_i)
//   T~  = (I + A)^{-1} diag(beta)          the WY factor of the chunk's
//                                          (I - beta k k^T) products
// ("Linear Attention & DeltaNet", "How it works", item 3: the chunk's
// Householder-like factors kept in compact WY form; "linear attention and its
// gated descendants", "Gated DeltaNet": the decay multiplies the state before
// the delta update, which is where Gamma comes from.)
//
// Chunks are independent, so the whole grid runs at once: this is the part
// of the method that is parallel over the sequence.  Two kernels:
//   chunk_wy_kernel          alpha = 1 or scalar alpha; one wave per chunk.
//                            Writes T~, and for scalar alpha the masked decay
//                            matrix Gamma and gamma_r, exp(g_C - g_r), gamma_C.
//   chunk_wy_channel_kernel  per-channel alpha; one workgroup per chunk.  The
//                            decay sits inside the channel sums,
//                            A_ri = beta_r sum_c k_rc k_ic exp(G_rc - G_ic), so
//                            it also forms the decayed operands the scan needs
//                            (K . exp(G), Q . exp(G), K . exp(G_C - G)), the
//                            masked score block P and exp(G_C).
// The inverse is taken in fp32 on every path: 16 x 16 diagonal blocks by
// forward substitution (one lane per column), the block below the diagonal
// as T_10 = -T_11 (A_10 T_00) with fp32 MFMA.
//
// The optional input-side prologue (gdr_fwd_chunked_ex) lives here too: the
// gate activations beta = sigmoid(b), log alpha = log sigmoid(a) are applied
// where beta and log alpha are first read, and the unit-norm q and k are
// never written out: the key tiles are rescaled in registers for the Gram
// products, and 1 / ||k||, 1 / ||q|| are folded into the per-token factors
// and score masks the scan reads.  Each kernel has a PRO = false
// instantiation that compiles all of it out.
#include "gdr_device.h"
#include "gdr_chunk.h"
#include "gdr_tri.h"

#include <algorithm>

namespace gdr {

namespace {

// K fragment (ldfrag convention) straight from global memory.  The read is
// unconditional, from row min(r, valid - 1) (row 0 when valid = 0): a read
// under a condition makes the compiler wait for it where the branches join,
// which would serialise a wave's reads.  gmask() zeroes the rows at or past
// `valid` once the data is used.
template <typename E>
__device__ __forceinline__ Frag<E> gfrag(const E* base, int ld, int row0, int k0, int valid) {
    const int l = lane_id(), r = max(min(row0 + (l & 15), valid - 1), 0);
    const E* p = base + (size_t)r * ld + k0 + 8 * (l >> 4);
    Frag<E> f;
    if constexpr (sizeof(E) == 2) {
        f.v = *reinterpret_cast<const bf16x8*>(p);
    } else {
        f.lo = *reinterpret_cast<const f32x4*>(p);
        f.hi = *reinterpret_cast<const f32x4*>(p + 4);
    }
    return f;
}
template <typename E>
__device__ __forceinline__ void gmask(Frag<E>& f, int row0, int valid) {
    if (row0 + (lane_id() & 15) < valid) return;
    if constexpr (sizeof(E) == 2) {
        f.v = bf16x8{};
    } else {
        f.lo = zero4();
        f.hi = zero4();
    }
}

// Per-wave LDS scratch of chunk_wy_kernel.
template <typename E, int CK>
struct WyScratch {
    static constexpr int VE = Vec<E>::n;
    static constexpr int LF = CK + 4;    // fp32 row stride
    static constexpr int off_A = 0;
    static constexpr int off_Tf = off_A + CK * LF * 4;
    static constexpr int off_g = off_Tf + CK * LF * 4;
    static constexpr int off_b = off_g + CK * 4;
    static constexpr int off_nk = off_b + CK * 4;    // 1 / ||k||, 1 / ||q|| per token
    static constexpr int off_nq = off_nk + CK * 4;
    static constexpr int bytes = (off_nq + CK * 4 + 15) / 16 * 16;
};

// 1 / max(||row||, eps) for the row 16 tb + (lane % 16) of the fragments
// f[tb][*] (every lane of the row's four lane groups gets the value).
template <typename E, int NB, int NKS>
__device__ __forceinline__ void row_inv_norms(const Frag<E> (&f)[NB][NKS], float (&inv)[NB]) {
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
        float ss = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            float x[8];
            if constexpr (sizeof(E) == 2) {
                Pack<bf16>::unpack(__builtin_bit_cast(u32x4, f[tb][ks].v), x);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) { x[i] = f[tb][ks].lo[i]; x[4 + i] = f[tb][ks].hi[i]; }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
        }
        ss += __shfl_xor(ss, 16, kWave);
        ss += __shfl_xor(ss, 32, kWave);
        inv[tb] = 1.f / fmaxf(sqrtf(ss), kNormEps);
    }
}

template <typename E>
__device__ __forceinline__ void scale_frag(Frag<E>& f, float s) {
    if constexpr (sizeof(E) == 2) {
        float x[8];
        Pack<bf16>::unpack(__builtin_bit_cast(u32x4, f.v), x);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] *= s;
        f.v = __builtin_bit_cast(bf16x8, Pack<bf16>::pack(x));
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) { f.lo[i] *= s; f.hi[i] *= s; }
    }
}

}  // namespace

// ======================================================================
// alpha = 1 and scalar alpha (alpha = 1 runs as log alpha = 0): one wave per
// chunk, four chunks per workgroup.  PRO = false compiles the input-side
// prologue out (it costs registers, hence occupancy, even when unused).
// ======================================================================
template <typename E, int DK, int CK, bool PRO>
__global__ __launch_bounds__(256) void chunk_wy_kernel(WyParams p)
{
    const unsigned pro = PRO ? p.pro : 0u;
    using SC = WyScratch<E, CK>;
    constexpr int VE = SC::VE, LF = SC::LF;
    constexpr int NB = CK / 16, NKS = DK / 32;
    constexpr WsLayout WL = ws_layout((int)sizeof(E), DK, CK, kAlphaScalar);
    extern __shared__ __align__(16) unsigned char smem[];

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int cid = blockIdx.x * 4 + w;
    if (cid >= p.total) return;   // wave-uniform; this kernel has no block barrier
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15;
    const ChunkSlot cs = chunk_slot(p.vl, p.L, p.NC, CK, cid);
    const size_t tok = cs.tok;   // first token on the token axis
    const int valid = cs.valid;

    unsigned char* sw = smem + w * SC::bytes;
    float* Af = reinterpret_cast<float*>(sw + SC::off_A);
    float* Tf = reinterpret_cast<float*>(sw + SC::off_Tf);
    float* gs = reinterpret_cast<float*>(sw + SC::off_g);
    float* bs = reinterpret_cast<float*>(sw + SC::off_b);
    float* nks = reinterpret_cast<float*>(sw + SC::off_nk);
    float* nqs = reinterpret_cast<float*>(sw + SC::off_nq);

    // input-side prologue, queries first: only their norms are needed here
    // (the scan applies 1 / ||q|| through the decay factors and Gamma), so
    // their tiles are dropped before the key tiles are loaded
    float nk = 1.f, nq = 1.f;   // for token l
    if (pro & kProNorm) {
        const E* qc = reinterpret_cast<const E*>(p.q) + tok * DK;
        Frag<E> qf[NB][NKS];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qf[tb][ks] = gfrag<E>(qc, DK, 16 * tb, 32 * ks, valid);
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) gmask(qf[tb][ks], 16 * tb, valid);
        float iq[NB];
        row_inv_norms<E, NB, NKS>(qf, iq);
        nq = iq[min(g4, NB - 1)];
    }

    // K tiles of the chunk as MFMA operands, straight from global memory
    // (scaled to unit rows by the prologue)
    const E* kc = reinterpret_cast<const E*>(p.k) + tok * DK;
    Frag<E> kf[NB][NKS];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) kf[tb][ks] = gfrag<E>(kc, DK, 16 * tb, 32 * ks, valid);
    // beta and log alpha of token l, read with the keys (clamped index; zero
    // past the end of the sequence below)
    const int lt = max(min(l, valid - 1), 0);
    float bt = p.beta[tok + lt];
    float la = p.log_alpha ? p.log_alpha[tok + lt] : 0.f;
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) gmask(kf[tb][ks], 16 * tb, valid);
    if (pro & kProNorm) {
        float ik[NB];
        row_inv_norms<E, NB, NKS>(kf, ik);
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) scale_frag(kf[tb][ks], ik[tb]);
        nk = ik[min(g4, NB - 1)];
    }

    // beta (zero past the end of the sequence) and the cumulative log-decay
    // (log alpha = 0 for alpha = 1)
    if (l < valid) {
        if (pro & kProGates) {
            bt = sigmoid_f(bt);
            if (p.log_alpha) la = log_sigmoid_f(la);
        }
    } else {
        bt = 0.f;
        la = 0.f;
    }
    const float g = scan32(la);
    const float glast = lane_value(g, CK - 1);
    if (l < CK) {
        gs[l] = g;
        bs[l] = bt;
        if (PRO) { nks[l] = nk; nqs[l] = nq; }
    }
    wave_lds_fence();

    // Gram tiles -> A
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
        for (int ib = 0; ib <= rb; ++ib) {
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) mma(acc, kf[rb][ks], kf[ib][ks]);
            const int i = 16 * ib + c16, r0 = 16 * rb + 4 * g4;
            const float gi = gs[i];
            const f32x4 gr = *reinterpret_cast<const f32x4*>(gs + r0);
            const f32x4 br = *reinterpret_cast<const f32x4*>(bs + r0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float d = __expf(fminf(gr[e] - gi, 0.f));
                Af[(r0 + e) * LF + i] = (r0 + e > i) ? br[e] * d * acc[e] : 0.f;
            }
        }
    }
    wave_lds_fence();
    unit_lower_inverse<CK, LF>(Af, Tf);
    if (p.Tout) store_T<CK, LF>(Tf, p.Tout + (size_t)cid * CK * CK, lane_id(), kWave);

    // T~ = T diag(beta) (and Gamma) to the workspace, zero above the diagonal;
    // 16-byte row vectors of memory columns c0.., four consecutive tokens at a time
    unsigned char* rec = p.ws + (size_t)cid * WL.bytes;
    E* Tg = reinterpret_cast<E*>(rec + WL.T);
    E* Mg = reinterpret_cast<E*>(rec + WL.M);
    constexpr int RV = CK / VE, TV = CK * RV;
#pragma unroll
    for (int x0 = 0; x0 < TV; x0 += kWave) {
        const int x = x0 + l;
        if (x < TV) {
            const int r = x / RV, c0 = (x % RV) * VE;
            float tv[VE], mv[VE];
#pragma unroll
            for (int q = 0; q < VE; q += 4) {
                const int t = tok_of_col(CK, c0 + q);
                const f32x4 a = *reinterpret_cast<const f32x4*>(Tf + r * LF + t);
                const f32x4 b = *reinterpret_cast<const f32x4*>(bs + t);
#pragma unroll
                for (int e = 0; e < 4; ++e) tv[q + e] = (t + e <= r) ? a[e] * b[e] : 0.f;
                // Gamma, with the token norms of the scores q_r . k_t folded in
                const float gr = gs[r], qn = PRO ? nqs[r] : 1.f;
                const f32x4 gt = *reinterpret_cast<const f32x4*>(gs + t);
                const f32x4 kn = PRO ? *reinterpret_cast<const f32x4*>(nks + t) : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    mv[q + e] = (t + e <= r) ? __expf(fminf(gr - gt[e], 0.f)) * qn * kn[e] : 0.f;
            }
            // non-temporal: the scan streams the records in later
            st16_nt(Tg + r * CK + c0, Pack<E>::pack(tv));
            st16_nt(Mg + r * CK + c0, Pack<E>::pack(mv));
        }
    }
    if (l < CK) {
        // gamma_r and exp(g_C - g_r) scaled by 1 / ||k_r|| (they multiply the
        // key-side products), gamma_C, and gamma_r / ||q_r|| for the outputs
        float* F = reinterpret_cast<float*>(rec + WL.F);
        F[l] = __expf(g) * nk;
        F[CK + l] = __expf(glast - g) * nk;
        F[2 * CK + l] = (l == 0) ? __expf(glast) : 0.f;
        F[3 * CK + l] = __expf(g) * nq;
    }
}

// ======================================================================
// Per-channel alpha: one workgroup (4 waves) per chunk.
// ======================================================================
template <typename E, int DK, int CK>
struct WyChannelLayout {
    static constexpr int VE = Vec<E>::n, ES = (int)sizeof(E);
    static constexpr int DKP = DK + VE;   // row stride of the K, Q copies
    static constexpr int GP = DK + 4;     // fp32 [CK][DK] cumulative decay
    static constexpr int LF = CK + 4;
    static constexpr int LP = CK + VE;
    static constexpr int off_K = 0;
    static constexpr int off_Q = off_K + CK * DKP * ES;
    static constexpr int off_G = off_Q + CK * DKP * ES;
    static constexpr int off_A = off_G + CK * GP * 4;
    static constexpr int off_Tf = off_A + CK * LF * 4;
    static constexpr int off_P = off_Tf + CK * LF * 4;
    static constexpr int off_b = off_P + CK * LP * ES;
    static constexpr int off_nk = off_b + CK * 4;    // 1 / ||k||, 1 / ||q|| per token
    static constexpr int off_nq = off_nk + CK * 4;
    static constexpr int bytes = off_nq + CK * 4;
};

// Three workgroups fit a CU's LDS at d_k = 128, C = 32; the second bound
// holds the register budget to three waves per SIMD to match, which the
// prologue's extra code would otherwise exceed.
template <typename E, int DK, int CK, bool PRO>
__global__ __launch_bounds__(256, 3) void chunk_wy_channel_kernel(WyParams p)
{
    const unsigned pro = PRO ? p.pro : 0u;
    using LY = WyChannelLayout<E, DK, CK>;
    constexpr int VE = LY::VE, DKP = LY::DKP, GP = LY::GP, LF = LY::LF, LP = LY::LP;
    constexpr int NB = CK / 16, NKS = DK / 32;
    constexpr WsLayout WL = ws_layout((int)sizeof(E), DK, CK, kAlphaChannel);
    extern __shared__ __align__(16) unsigned char smem[];
    E* Ks = reinterpret_cast<E*>(smem + LY::off_K);
    E* Qs = reinterpret_cast<E*>(smem + LY::off_Q);
    float* Gs = reinterpret_cast<float*>(smem + LY::off_G);
    float* Af = reinterpret_cast<float*>(smem + LY::off_A);
    float* Tf = reinterpret_cast<float*>(smem + LY::off_Tf);
    E* Ps = reinterpret_cast<E*>(smem + LY::off_P);
    float* bs = reinterpret_cast<float*>(smem + LY::off_b);
    float* nks = reinterpret_cast<float*>(smem + LY::off_nk);
    float* nqs = reinterpret_cast<float*>(smem + LY::off_nq);
    const bool gates = (pro & kProGates) != 0;

    const int tid = threadIdx.x, l = lane_id(), g4 = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    // Each workgroup walks chunks blockIdx.x, + gridDim.x, ...; the next
    // chunk's K, Q, log alpha and beta are fetched into registers while the
    // current one is worked on, so loads and compute overlap.
    constexpr int RV = DK / VE, RF = DK / 4;
    constexpr int NKV = (CK * RV + 255) / 256, NGV = (CK * RF + 255) / 256;
    u32x4 kr[NKV], qr[NKV];
    f32x4 gr[NGV];
    float br = 0.f;
    auto fetch = [&](int cid) {
        const ChunkSlot cs = chunk_slot(p.vl, p.L, p.NC, CK, cid);
        const int valid = cs.valid;
        const E* kc = reinterpret_cast<const E*>(p.k) + cs.tok * DK;
        const E* qc = reinterpret_cast<const E*>(p.q) + cs.tok * DK;
        const float* lac = p.log_alpha + cs.tok * DK;
        // every read unconditional, from clamped indices (a conditional read
        // would make the compiler wait for it here); rows past the end are
        // zeroed when staged
#pragma unroll
        for (int j = 0; j < NKV; ++j) {
            const int i = min(tid + 256 * j, CK * RV - 1), r = max(min(i / RV, valid - 1), 0), c = (i % RV) * VE;
            kr[j] = ld16(kc + (size_t)r * DK + c);
            qr[j] = ld16(qc + (size_t)r * DK + c);
        }
#pragma unroll
        for (int j = 0; j < NGV; ++j) {
            const int i = min(tid + 256 * j, CK * RF - 1), r = max(min(i / RF, valid - 1), 0), c = (i % RF) * 4;
            gr[j] = *reinterpret_cast<const f32x4*>(lac + (size_t)r * DK + c);
        }
        br = p.beta[cs.tok + max(min(tid, valid - 1), 0)];
    };
    if ((int)blockIdx.x < p.total) fetch(blockIdx.x);
    for (int cid = blockIdx.x; cid < p.total; cid += gridDim.x) {
    unsigned char* rec = p.ws + (size_t)cid * WL.bytes;

    // ---- stage K, Q and log alpha (floored; zero past the end), beta; the
    // prologue's gate activations apply to the chunk's valid tokens
    const int valid = chunk_slot(p.vl, p.L, p.NC, CK, cid).valid;
#pragma unroll
    for (int j = 0; j < NKV; ++j) {
        const int i = tid + 256 * j, r = i / RV, c = (i % RV) * VE;
        if (r >= valid) {
            kr[j] = u32x4{0u, 0u, 0u, 0u};
            qr[j] = u32x4{0u, 0u, 0u, 0u};
        }
        if (i < CK * RV) {
            st16(Ks + r * DKP + c, kr[j]);
            st16(Qs + r * DKP + c, qr[j]);
        }
        if (PRO) {
            // the prologue's 1 / max(||row||, eps) for K and Q row r: the row
            // is spread over RV consecutive lanes, a whole aligned lane group
            // (1 when the norms are not asked for)
            float sk = 1.f, sq = 1.f;
            if (pro & kProNorm) {
                float x[VE], y[VE];
                Pack<E>::unpack(kr[j], x);
                Pack<E>::unpack(qr[j], y);
                sk = 0.f;
                sq = 0.f;
#pragma unroll
                for (int e = 0; e < VE; ++e) { sk += x[e] * x[e]; sq += y[e] * y[e]; }
#pragma unroll
                for (int m = RV / 2; m >= 1; m >>= 1) {
                    sk += __shfl_xor(sk, m, kWave);
                    sq += __shfl_xor(sq, m, kWave);
                }
                sk = 1.f / fmaxf(sqrtf(sk), kNormEps);
                sq = 1.f / fmaxf(sqrtf(sq), kNormEps);
            }
            if (i < CK * RV && c == 0) { nks[r] = sk; nqs[r] = sq; }
        }
    }
#pragma unroll
    for (int j = 0; j < NGV; ++j) {
        const int i = tid + 256 * j, r = i / RF, c = (i % RF) * 4;
        if (i < CK * RF) {
            f32x4 x = r < valid ? gr[j] : zero4();
            if (gates && r < valid) {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = log_sigmoid_f(x[e]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = fmaxf(x[e], kChannelLogAlphaMin);
            *reinterpret_cast<f32x4*>(Gs + r * GP + c) = x;
        }
    }
    if (tid < CK) bs[tid] = tid < valid ? (gates ? sigmoid_f(br) : br) : 0.f;
    if (cid + (int)gridDim.x < p.total) fetch(cid + gridDim.x);
    __syncthreads();
    // cumulative sum down each key channel (the column is read whole first,
    // so the reads are in flight together)
    for (int c = tid; c < DK; c += 256) {
        float col[CK];
#pragma unroll
        for (int r = 0; r < CK; ++r) col[r] = Gs[r * GP + c];
#pragma unroll
        for (int r = 1; r < CK; ++r) col[r] += col[r - 1];
#pragma unroll
        for (int r = 0; r < CK; ++r) Gs[r * GP + c] = col[r];
    }
    __syncthreads();

    // ---- decayed operands for the scan and exp(G_C)
    {
        const float* GL = Gs + (CK - 1) * GP;
        E* KGg = reinterpret_cast<E*>(rec + WL.KG);
        E* QGg = reinterpret_cast<E*>(rec + WL.QG);
        E* KDg = reinterpret_cast<E*>(rec + WL.KD);
        for (int i = tid; i < CK * RV; i += 256) {
            const int r = i / RV, c0 = (i % RV) * VE;
            float kx[VE], qx[VE], a[VE], b[VE], d[VE];
            Pack<E>::unpack(ld16(Ks + r * DKP + c0), kx);
            Pack<E>::unpack(ld16(Qs + r * DKP + c0), qx);
#pragma unroll
            for (int j = 0; j < VE; ++j) {
                const float gg = Gs[r * GP + c0 + j];
                const float eg = __expf(gg), ed = __expf(GL[c0 + j] - gg);
                a[j] = kx[j] * eg * (PRO ? nks[r] : 1.f);
                b[j] = qx[j] * eg * (PRO ? nqs[r] : 1.f);
                d[j] = kx[j] * ed * (PRO ? nks[r] : 1.f);
            }
            // non-temporal: 24 KiB per chunk that the scan streams in later;
            // left dirty in the caches their write-back slowed the scan's
            // copies by 15 %
            st16_nt(KGg + r * DK + c0, Pack<E>::pack(a));
            st16_nt(QGg + r * DK + c0, Pack<E>::pack(b));
            st16_nt(KDg + r * DK + c0, Pack<E>::pack(d));
        }
        float* F = reinterpret_cast<float*>(rec + WL.F);
        for (int c = tid; c < DK; c += 256) F[c] = __expf(GL[c]);
    }

    // ---- Gram and score tiles.  The decay exp(G_rc - G_ic) sits inside the
    // channel sum; each operand row is scaled relative to a reference row m:
    // the left row r by exp(G_r - G_m), the right row i by exp(G_m - G_i).
    // Below the diagonal m = 16 rb - 1 (both factors <= 1); on a diagonal
    // block m = 16 rb + 7, so no factor exceeds exp(8 * 10) in fp32.
    constexpr int NTILE = NB * (NB + 1) / 2;
    if (w < NTILE) {
        const int rb = (w == 0) ? 0 : 1, ib = (w == 2) ? 1 : 0;
        const int m = (rb == ib) ? 16 * rb + 7 : 16 * rb - 1;
        const int rl = 16 * rb + c16, rr = 16 * ib + c16;
        f32x4 accA = zero4(), accP = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int c0 = 32 * ks + 8 * g4;
            float fk[8], fq[8], fr[8];
            const float nkl = PRO ? nks[rl] : 1.f, nql = PRO ? nqs[rl] : 1.f, nkr = PRO ? nks[rr] : 1.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float gm = Gs[m * GP + c0 + j];
                const float fl = __expf(Gs[rl * GP + c0 + j] - gm);
                fk[j] = fl * nkl;
                fq[j] = fl * nql;
                fr[j] = __expf(gm - Gs[rr * GP + c0 + j]) * nkr;
            }
            Frag<E> kl, ql, kr;
            load_scaled_frag(kl, Ks + rl * DKP + c0, fk);
            load_scaled_frag(ql, Qs + rl * DKP + c0, fq);
            load_scaled_frag(kr, Ks + rr * DKP + c0, fr);
            mma(accA, kl, kr);   // A tile: lane holds [16rb + 4g + e][16ib + c]
            mma(accP, kr, ql);   // P^T tile: lane holds P[16rb + c][16ib + 4g + e]
        }
        {
            const int i = 16 * ib + c16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e;
                Af[r * LF + i] = (r > i) ? bs[r] * accA[e] : 0.f;
            }
        }
        {
            const int r = 16 * rb + c16, i0 = 16 * ib + 4 * g4;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (r >= i0 + e) ? accP[e] : 0.f;
            st4(Ps + r * LP + i0, x[0], x[1], x[2], x[3]);
        }
    }
    __syncthreads();
    if (w == 0) unit_lower_inverse<CK, LF>(Af, Tf);
    __syncthreads();
    if (p.Tout) store_T<CK, LF>(Tf, p.Tout + (size_t)cid * CK * CK, tid, 256);

    // ---- T~ = T diag(beta) and P to the workspace, zero above the diagonal
    // (columns in tok_of_col order)
    E* Tg = reinterpret_cast<E*>(rec + WL.T);
    E* Pg = reinterpret_cast<E*>(rec + WL.M);
    constexpr int CV = CK / VE;
    for (int idx = tid; idx < CK * CV; idx += 256) {
        const int r = idx / CV, c0 = (idx % CV) * VE;
        float x[VE], y[VE];
#pragma unroll
        for (int q = 0; q < VE; q += 4) {
            const int t = tok_of_col(CK, c0 + q);
            const f32x4 pv = load4f(Ps + r * LP + t);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[q + e] = (t + e <= r) ? Tf[r * LF + t + e] * bs[t + e] : 0.f;
                y[q + e] = (t + e <= r) ? pv[e] : 0.f;
            }
        }
        st16(Tg + r * CK + c0, Pack<E>::pack(x));
        st16(Pg + r * CK + c0, Pack<E>::pack(y));
    }
    __syncthreads();   // the LDS is restaged for the next chunk
    }
}

// ------------------------------------------------------------------ host side
int compute_units()
{
    static int n = 0;
    if (n == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
    }
    return n;
}

template <typename K>
static hipError_t launch_with_lds(K* kern, int grid, int lds, hipStream_t stream, const WyParams& wp)
{
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, stream, wp);
    return hipGetLastError();
}

template <typename E, int DK, int CK>
static hipError_t launch_wy_t(const ChunkArgs& a)
{
    const int NC = (a.L + CK - 1) / CK;
    const int total = a.vl.start ? a.H * a.vl.NCmax : a.B * a.H * NC;   // record slots
    WyParams wp{a.q, a.k, a.beta, a.log_alpha, static_cast<unsigned char*>(a.workspace), a.L, NC,
                total, a.pro, a.vl, a.Tout};
    if (a.mode == kAlphaChannel) {
        using LY = WyChannelLayout<E, DK, CK>;
        static_assert(LY::bytes <= 160 * 1024, "LDS budget");
        // persistent: as many workgroups as fit the CUs at once
        const int per_cu = (160 * 1024) / LY::bytes;
        const int grid = std::min(wp.total, per_cu * compute_units());
        return a.pro ? launch_with_lds(chunk_wy_channel_kernel<E, DK, CK, true>, grid, LY::bytes, a.stream, wp)
                     : launch_with_lds(chunk_wy_channel_kernel<E, DK, CK, false>, grid, LY::bytes, a.stream, wp);
    }
    constexpr int bytes = 4 * WyScratch<E, CK>::bytes;
    static_assert(bytes <= 160 * 1024, "LDS budget");
    const int grid = (wp.total + 3) / 4;
    // alpha = 1 runs the scalar path with log alpha = 0 (log_alpha is NULL)
    return a.pro ? launch_with_lds(chunk_wy_kernel<E, DK, CK, true>, grid, bytes, a.stream, wp)
                 : launch_with_lds(chunk_wy_kernel<E, DK, CK, false>, grid, bytes, a.stream, wp);
}

hipError_t launch_wy(const ChunkArgs& a, int CK)
{
    if (a.dtype == kBF16) {
        if (a.dk == 128) return CK == 16 ? launch_wy_t<bf16, 128, 16>(a) : launch_wy_t<bf16, 128, 32>(a);
        return CK == 16 ? launch_wy_t<bf16, 64, 16>(a) : launch_wy_t<bf16, 64, 32>(a);
    }
    return a.dk == 128 ? launch_wy_t<float, 128, 16>(a) : launch_wy_t<float, 64, 16>(a);
}

}  // namespace gdr

// gdr_chunk.hip -- chunkwise forward of the gated delta-rule memory.
//
// Chunk algebra (one head, one chunk of C tokens, entry state S0, d_v x d_k).
// The pages give the chunkwise form for plain linear attention ("linear
// attention and its gated descendants", "Chunkwise Parallel Form": boundary
// state plus a C x C masked block) and name the WY/Householder compact form
// of a chunk's (I - beta k k^T) factors for the delta rule ("Linear
// Attention & DeltaNet", item 3).  Written out for the gated update:
//
//   g_r     = sum_{s<=r} log alpha_s   (in-chunk cumulative log-decay;
//             per key channel, G_{r,c}, in channel mode)
//   A       = strictly-lower( diag(beta) (K K^T . Gamma) ),
//             Gamma_{ri} = exp(g_r - g_i)        (channel mode: the decay sits
//             inside the sum, A_ri = beta_r sum_c k_rc k_ic exp(G_rc - G_ic))
//   T       = (I + A)^{-1}                        unit lower triangular
//   W       = T diag(beta) (diag(gamma) K)        gamma_r = exp(g_r)
//   U~      = T diag(beta) V
//   U       = U~ - W S0^T                         the chunk's delta residuals
//   O       = diag(gamma) Q S0^T + (Q K^T . Gamma . M_incl) U
//   S_exit  = gamma_C S0 + U^T diag(exp(g_C - g)) K
//
// (Substituting S_{r-1} = gamma_{r-1} S0 + sum_{i<r} Gamma_{r-1,i} u_i k_i^T
// into u_r = beta_r (v_r - alpha_r S_{r-1} k_r) gives (I + A) U =
// diag(beta) V - diag(beta gamma) K S0^T.)  Every exponential has a
// non-positive argument except inside the channel-mode diagonal blocks,
// which use a mid-block reference (see chunk_prep_kernel).
//
// Kernel P (chunk_prep_kernel) runs once per chunk, fully parallel: it forms
// the decay, the Gram and score blocks with MFMA, inverts I + A in fp32 and
// writes T diag(beta) and the masked score block P to the workspace.
// Kernel S (chunk_scan_kernel) runs one workgroup per (batch, head, d_v
// block); it walks the chunks in order with the state block in registers,
// forms W and U~ from T, then U, O and the next state, all with MFMA.  Rows
// of S (value channels) evolve independently, which is what lets the value
// dimension be split across workgroups.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

// ------------------------------------------------------------------ helpers
__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr int align_up(int x, int a) { return (x + a - 1) / a * a; }

// 32-wide k-steps that cover k in [0, 16*(tt+1)) (lower-triangular operands).
__device__ __forceinline__ constexpr int ksteps_tri(int tt) { return (16 * (tt + 1) + 31) / 32; }

// Multiply the VE elements of a 16-byte vector by f[0..VE).
template <typename E>
__device__ __forceinline__ u32x4 scale_vec(u32x4 v, const float* f) {
    float x[Vec<E>::n];
    Pack<E>::unpack(v, x);
#pragma unroll
    for (int j = 0; j < Vec<E>::n; ++j) x[j] *= f[j];
    return Pack<E>::pack(x);
}

// ======================================================================
// Kernel P: per-chunk WY factor and masked scores.
// ======================================================================
struct PrepParams {
    const void *q, *k;
    const float *beta, *log_alpha;
    void *Tws, *Pws;   // [BH][NC][C][C] each, element type E
    int L, NC;
};

template <typename E, int DK, int C, int MODE>
struct PrepLayout {
    static constexpr int VE = Vec<E>::n;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int DKP = DK + VE;          // row stride of K/Q copies
    static constexpr int CF = C + 4;             // fp32 C x C buffers
    static constexpr int CP = C + VE;            // E  C x C staging
    static constexpr int GP = DK + 4;            // fp32 [C][DK] log-decay
    // Region 1, tile phase: K, Q (and G in channel mode).  After the tile
    // phase the same bytes hold T, T^T and the per-wave Y scratch.
    static constexpr int off_K = 0;
    static constexpr int off_Q = off_K + C * DKP * ES;
    static constexpr int off_G = off_Q + C * DKP * ES;
    static constexpr int endA = off_G + (MODE == kAlphaChannel ? C * GP * 4 : 0);
    static constexpr int off_T = 0;
    static constexpr int off_Tt = off_T + C * CF * 4;
    static constexpr int off_Y = off_Tt + C * CF * 4;
    static constexpr int endB = off_Y + 4 * 16 * 20 * 4;
    static constexpr int off_A = align_up(cmax(endA, endB), 16);
    static constexpr int off_P = off_A + C * CF * 4;
    static constexpr int off_g = off_P + C * CP * ES;
    static constexpr int off_b = off_g + C * 4;
    static constexpr int bytes = off_b + C * 4;
};

template <typename E, int DK, int C, int MODE>
__global__ __launch_bounds__(256) void chunk_prep_kernel(PrepParams p)
{
    using LY = PrepLayout<E, DK, C, MODE>;
    constexpr int VE = LY::VE, DKP = LY::DKP, CF = LY::CF, CP = LY::CP, GP = LY::GP;
    constexpr int NB = C / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    E* Ks = reinterpret_cast<E*>(smem + LY::off_K);
    E* Qs = reinterpret_cast<E*>(smem + LY::off_Q);
    float* Gs = reinterpret_cast<float*>(smem + LY::off_G);
    float* Af = reinterpret_cast<float*>(smem + LY::off_A);
    float* Tf = reinterpret_cast<float*>(smem + LY::off_T);
    float* Tt = reinterpret_cast<float*>(smem + LY::off_Tt);
    float* Ys = reinterpret_cast<float*>(smem + LY::off_Y);
    E* Ps = reinterpret_cast<E*>(smem + LY::off_P);
    float* gs = reinterpret_cast<float*>(smem + LY::off_g);
    float* bs = reinterpret_cast<float*>(smem + LY::off_b);

    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int n = blockIdx.x % p.NC, bh = blockIdx.x / p.NC;
    const int t0 = n * C;
    const int valid = min(C, p.L - t0);
    const E* kg = reinterpret_cast<const E*>(p.k) + ((size_t)bh * p.L + t0) * DK;
    const E* qg = reinterpret_cast<const E*>(p.q) + ((size_t)bh * p.L + t0) * DK;

    // ---- stage K, Q rows (zero past the end of the sequence)
    constexpr int RV = DK / VE;  // vectors per row
    for (int i = tid; i < C * RV; i += 256) {
        const int r = i / RV, c = (i % RV) * VE;
        u32x4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
        if (r < valid) { kv = ld16(kg + (size_t)r * DK + c); qv = ld16(qg + (size_t)r * DK + c); }
        st16(Ks + r * DKP + c, kv);
        st16(Qs + r * DKP + c, qv);
    }
    if (MODE == kAlphaChannel) {
        constexpr int RF = DK / 4;
        const float* lag = p.log_alpha + ((size_t)bh * p.L + t0) * DK;
        for (int i = tid; i < C * RF; i += 256) {
            const int r = i / RF, c = (i % RF) * 4;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < valid) {
                x = *reinterpret_cast<const float4*>(lag + (size_t)r * DK + c);
                x.x = fmaxf(x.x, kChannelLogAlphaMin); x.y = fmaxf(x.y, kChannelLogAlphaMin);
                x.z = fmaxf(x.z, kChannelLogAlphaMin); x.w = fmaxf(x.w, kChannelLogAlphaMin);
            }
            *reinterpret_cast<float4*>(Gs + r * GP + c) = x;
        }
    }
    if (w == 0) {
        // beta and (scalar mode) the in-chunk cumulative log-decay
        float bta = 0.f, la = 0.f;
        if (l < valid) {
            bta = p.beta[(size_t)bh * p.L + t0 + l];
            if (MODE == kAlphaScalar) la = p.log_alpha[(size_t)bh * p.L + t0 + l];
        }
        const float g = wave_incl_scan(la);
        if (l < C) { gs[l] = g; bs[l] = bta; }
    }
    __syncthreads();
    if (MODE == kAlphaChannel) {
        // cumulative sum down each key channel: thread c owns channel c
        for (int c = tid; c < DK; c += 256) {
            float acc = 0.f;
#pragma unroll 8
            for (int r = 0; r < C; ++r) { acc += Gs[r * GP + c]; Gs[r * GP + c] = acc; }
        }
        __syncthreads();
    }

    // ---- Gram tiles -> A (fp32), and score tiles -> P.
    // Tile (rb, ib), rb >= ib: rows of block rb against rows of block ib.
    constexpr int NTILE = NB * (NB + 1) / 2;
    auto tile_of = [](int t, int& rb, int& ib) {
        rb = 0;
        while ((rb + 1) * (rb + 2) / 2 <= t) ++rb;
        ib = t - rb * (rb + 1) / 2;
    };
    if (MODE != kAlphaChannel) {
        // A tiles: all waves.
        for (int t = w; t < NTILE; t += 4) {
            int rb, ib; tile_of(t, rb, ib);
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < DK / 32; ++s)
                mma(acc, ldfrag(Ks, DKP, 16 * rb, 32 * s), ldfrag(Ks, DKP, 16 * ib, 32 * s));
            const int i = 16 * ib + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * (l >> 4) + e;
                float a = 0.f;
                if (r > i) a = bs[r] * (MODE == kAlphaScalar ? __expf(gs[r] - gs[i]) : 1.f) * acc[e];
                Af[r * CF + i] = a;
            }
        }
        // P tiles as P^T = K_ib Q_rb^T: lane holds P[r][i..i+3].
        for (int t = w; t < NTILE; t += 4) {
            int rb, ib; tile_of(t, rb, ib);
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < DK / 32; ++s)
                mma(acc, ldfrag(Ks, DKP, 16 * ib, 32 * s), ldfrag(Qs, DKP, 16 * rb, 32 * s));
            const int r = 16 * rb + (l & 15);
            const int i0 = 16 * ib + 4 * (l >> 4);
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = i0 + e;
                x[e] = (r >= i) ? (MODE == kAlphaScalar ? __expf(gs[r] - gs[i]) : 1.f) * acc[e] : 0.f;
            }
            st4(Ps + r * CP + i0, x[0], x[1], x[2], x[3]);
        }
    } else {
        // Channel mode: the decay exp(G_rc - G_ic) sits inside the channel
        // sum.  Each operand row is scaled relative to a reference row m:
        // left row r by exp(G_r - G_m), right row i by exp(G_m - G_i).  For
        // rb > ib, m = 16 rb - 1 (both factors <= 1).  On a diagonal block,
        // m = 16 rb + 7 (mid-block), so no factor exceeds exp(8 * 10).
        for (int t = w; t < NTILE; t += 4) {
            int rb, ib; tile_of(t, rb, ib);
            const int m = (rb == ib) ? 16 * rb + 7 : 16 * rb - 1;
            const int rl = 16 * rb + (l & 15);   // left operand row (this lane)
            const int rr = 16 * ib + (l & 15);   // right operand row (this lane)
            f32x4 accA = zero4(), accP = zero4();
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                const int c0 = 32 * s + 8 * (l >> 4);
                float fl[8], fr[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float gm = Gs[m * GP + c0 + j];
                    fl[j] = __expf(Gs[rl * GP + c0 + j] - gm);
                    fr[j] = __expf(gm - Gs[rr * GP + c0 + j]);
                }
                Frag<E> kl, ql, kr;
                load_scaled_frag(kl, Ks + rl * DKP + c0, fl);
                load_scaled_frag(ql, Qs + rl * DKP + c0, fl);
                load_scaled_frag(kr, Ks + rr * DKP + c0, fr);
                mma(accA, kl, kr);   // A tile: [r][i]
                mma(accP, kr, ql);   // P^T tile: [i][r]
            }
            {
                const int i = 16 * ib + (l & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * (l >> 4) + e;
                    Af[r * CF + i] = (r > i) ? bs[r] * accA[e] : 0.f;
                }
            }
            {
                const int r = 16 * rb + (l & 15);
                const int i0 = 16 * ib + 4 * (l >> 4);
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (r >= i0 + e) ? accP[e] : 0.f;
                st4(Ps + r * CP + i0, x[0], x[1], x[2], x[3]);
            }
        }
    }
    __syncthreads();

    // ---- T = (I + A)^{-1}, blocked: 16x16 diagonal blocks by forward
    // substitution (wave 0, one lane per (block, column)), then the
    // off-diagonal blocks by distance d from the diagonal:
    //   T_ij = -T_ii * sum_{k=j}^{i-1} A_ik T_kj   (fp32 MFMA).
    if (w == 0) {
        const int b = l >> 4, j = l & 15;
        if (b < NB) {
            float t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == j) ? 1.f : 0.f;
                const float* arow = Af + (16 * b + r) * CF + 16 * b;
#pragma unroll
                for (int i = 0; i < r; ++i) s -= arow[i] * t[i];
                t[r] = s;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Tf[(16 * b + r) * CF + 16 * b + j] = t[r];
#pragma unroll
            for (int r = 0; r < 16; r += 4)
                *reinterpret_cast<f32x4*>(Tt + (16 * b + j) * CF + 16 * b + r) =
                    f32x4{t[r], t[r + 1], t[r + 2], t[r + 3]};
        }
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < NB; ++d) {
        const int i = d + w, j = w;   // block (i, j), one per wave
        const bool act = (i < NB);
        float* Yw = Ys + w * 16 * 20;
        if (act) {
            // Y^T[c][r] = sum_x T^T[16j + c][x] A[16i + r][x], x in [16j, 16i)
            f32x4 acc = zero4();
            for (int kb = j; kb < i; ++kb) mma_k16(acc, Tt, CF, 16 * j, Af, CF, 16 * i, 16 * kb);
#pragma unroll
            for (int e = 0; e < 4; ++e) Yw[(4 * (l >> 4) + e) * 20 + (l & 15)] = acc[e];
        }
        __syncthreads();
        if (act) {
            // Z^T[c][r'] = sum_r Y^T[c][r] T_ii[r'][r];  T_ij = -Z
            f32x4 acc = zero4();
            mma_k16(acc, Yw, 20, 0, Tf + 16 * i, CF, 16 * i, 0);
            const int rr = 16 * i + (l & 15);
            const int c0 = 16 * j + 4 * (l >> 4);
            *reinterpret_cast<f32x4*>(Tf + rr * CF + c0) = f32x4{-acc[0], -acc[1], -acc[2], -acc[3]};
#pragma unroll
            for (int e = 0; e < 4; ++e) Tt[(c0 + e) * CF + rr] = -acc[e];
        }
        __syncthreads();
    }

    // ---- write T diag(beta) and P (upper triangles zero) to the workspace
    E* Tg = reinterpret_cast<E*>(p.Tws) + ((size_t)bh * p.NC + n) * C * C;
    E* Pg = reinterpret_cast<E*>(p.Pws) + ((size_t)bh * p.NC + n) * C * C;
    constexpr int CV = C / VE;
    for (int idx = tid; idx < C * CV; idx += 256) {
        const int r = idx / CV, c0 = (idx % CV) * VE;
        // blocks above the diagonal were never computed: write zeros there
        float x[VE], y[VE];
        Pack<E>::unpack(ld16(Ps + r * CP + c0), y);
#pragma unroll
        for (int j = 0; j < VE; ++j) {
            const int c = c0 + j;
            x[j] = (c <= r) ? Tf[r * CF + c] * bs[c] : 0.f;
            y[j] = (c <= r) ? y[j] : 0.f;
        }
        st16(Tg + (size_t)r * C + c0, Pack<E>::pack(x));
        st16(Pg + (size_t)r * C + c0, Pack<E>::pack(y));
    }
}

// ======================================================================
// Kernel S: sequential chunk scan, one workgroup per (bh, d_v block).
// ======================================================================
struct ScanParams {
    const void *q, *k, *v;
    const float *log_alpha, *S0;
    const void *Tws, *Pws;
    void* o;
    float* S_final;
    int L, NC, DV, NVB, total;
};

template <typename E, int DK, int BV, int C, int MODE>
struct ScanLayout {
    static constexpr int VE = Vec<E>::n;
    static constexpr int CK = cmax(C, 32);       // k extent over tokens
    static constexpr int CKP = CK + VE;
    static constexpr int DKP = DK + VE;
    static constexpr int ES = (int)sizeof(E);
    static constexpr bool CH = (MODE == kAlphaChannel);
    // [DK][CKP]: K^T (scalar/none) or (K . exp(G))^T (channel)
    static constexpr int off_Kt = 0;
    // [DK][CKP]: (K . exp(G_C - G))^T, channel mode only
    static constexpr int off_Kd = off_Kt + DK * CKP * ES;
    static constexpr int off_Q = off_Kd + (CH ? DK * CKP * ES : 0);
    static constexpr int off_Vt = off_Q + C * DKP * ES;
    static constexpr int off_Tb = off_Vt + BV * CKP * ES;
    static constexpr int off_Tg = off_Tb + C * CKP * ES;          // scalar/none only
    static constexpr int off_P = off_Tg + (CH ? 0 : C * CKP * ES);
    static constexpr int off_W = off_P + C * CKP * ES;
    static constexpr int off_Sb = off_W + C * DKP * ES;
    static constexpr int off_Ut = off_Sb + BV * DKP * ES;
    static constexpr int off_Us = off_Ut + BV * CKP * ES;           // scalar/none only
    static constexpr int off_G = off_Us + (CH ? 0 : BV * CKP * ES); // channel: [C][DK+4] fp32
    static constexpr int GP = DK + 4;
    static constexpr int off_g = off_G + (CH ? C * GP * 4 : 0);
    static constexpr int bytes = off_g + 3 * 64 * 4 + 16;
};

template <typename E, int DK, int BV, int C, int MODE>
__global__ __launch_bounds__(256) void chunk_scan_kernel(ScanParams p)
{
    using LY = ScanLayout<E, DK, BV, C, MODE>;
    constexpr int VE = LY::VE, CK = LY::CK, CKP = LY::CKP, DKP = LY::DKP, GP = LY::GP;
    constexpr bool CH = LY::CH;
    constexpr int NB = C / 16, NKT = DK / 16, NVT = BV / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    E* Kt = reinterpret_cast<E*>(smem + LY::off_Kt);
    E* Kd = reinterpret_cast<E*>(smem + LY::off_Kd);
    E* Qs = reinterpret_cast<E*>(smem + LY::off_Q);
    E* Vt = reinterpret_cast<E*>(smem + LY::off_Vt);
    E* Tb = reinterpret_cast<E*>(smem + LY::off_Tb);
    E* Tg = reinterpret_cast<E*>(smem + LY::off_Tg);
    E* Ps = reinterpret_cast<E*>(smem + LY::off_P);
    E* Ws = reinterpret_cast<E*>(smem + LY::off_W);
    E* Sb = reinterpret_cast<E*>(smem + LY::off_Sb);
    E* Ut = reinterpret_cast<E*>(smem + LY::off_Ut);
    E* Us = reinterpret_cast<E*>(smem + LY::off_Us);
    float* Gs = reinterpret_cast<float*>(smem + LY::off_G);
    float* gam = reinterpret_cast<float*>(smem + LY::off_g);   // exp(g_r)
    float* dec = gam + 64;                                       // exp(g_last - g_r)
    float* misc = dec + 64;                                      // [0] = exp(g_last)

    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    // Spread the d_v blocks of one head over one XCD (consecutive block ids
    // go to different XCDs), so they share that XCD's L2 for K, Q, T, P.
    int lid = blockIdx.x;
    if (p.total % 8 == 0) lid = (blockIdx.x % 8) * (p.total / 8) + blockIdx.x / 8;
    const int bh = lid / p.NVB, vb = lid % p.NVB;
    const int v0 = vb * BV;
    const E* kg = reinterpret_cast<const E*>(p.k) + (size_t)bh * p.L * DK;
    const E* qg = reinterpret_cast<const E*>(p.q) + (size_t)bh * p.L * DK;
    const E* vg = reinterpret_cast<const E*>(p.v) + (size_t)bh * p.L * p.DV + v0;
    E* og = reinterpret_cast<E*>(p.o) + (size_t)bh * p.L * p.DV + v0;
    const E* Tw = reinterpret_cast<const E*>(p.Tws) + (size_t)bh * p.NC * C * C;
    const E* Pw = reinterpret_cast<const E*>(p.Pws) + (size_t)bh * p.NC * C * C;

    // zero the token padding columns [C, CK) once (only when C < 32)
    if (CK > C) {
        constexpr int PADC = CK > C ? CK - C : 1;
        auto zero_cols = [&](E* buf, int rows) {
            for (int i = tid; i < rows * PADC; i += 256) buf[(i / PADC) * CKP + C + i % PADC] = from_f32<E>(0.f);
        };
        zero_cols(Kt, DK); if (CH) zero_cols(Kd, DK);
        zero_cols(Vt, BV); zero_cols(Tb, C); if (!CH) zero_cols(Tg, C);
        zero_cols(Ps, C); zero_cols(Ut, BV); if (!CH) zero_cols(Us, BV);
    }

    // ---- state block S^T tiles (dk-tile a, v-tile vt) in registers
    constexpr int NT5 = NKT * NVT, MT5 = (NT5 + 3) / 4;
    f32x4 sacc[MT5];
#pragma unroll
    for (int i = 0; i < MT5; ++i) {
        sacc[i] = zero4();
        const int t = w + 4 * i;
        if (t < NT5 && p.S0) {
            const int a = t / NVT, vt = t % NVT;
            const float* src = p.S0 + ((size_t)bh * p.DV + v0 + 16 * vt + (l & 15)) * DK + 16 * a + 4 * (l >> 4);
            sacc[i] = *reinterpret_cast<const f32x4*>(src);
        }
    }

    // ---- prefetch registers for one chunk
    constexpr int KBLK = (C / VE) * (DK / VE);     // VE x VE blocks of K
    constexpr int VBLK = (C / VE) * (BV / VE);     // VE x VE blocks of the V block
    constexpr int QVEC = C * DK / VE;
    constexpr int TVEC = C * C / VE;
    constexpr int NKB = (KBLK + 255) / 256, NVB_ = (VBLK + 255) / 256;
    constexpr int NQV = (QVEC + 255) / 256, NTV = (TVEC + 255) / 256;
    u32x4 rk[NKB][VE], rv[NVB_][VE], rq[NQV], rt[NTV], rp[NTV];
    constexpr int GVEC = CH ? C * DK / 4 : 0;
    constexpr int NGV = CH ? (GVEC + 255) / 256 : 1;
    float4 rg[NGV];
    float rla = 0.f;

    auto load_chunk = [&](int n) {
        const int t0 = n * C;
        const int valid = min(C, p.L - t0);
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
            const int b = tid + 256 * i;
            if (b < KBLK) {
                const int r0 = (b / (DK / VE)) * VE, c0 = (b % (DK / VE)) * VE;
#pragma unroll
                for (int r = 0; r < VE; ++r)
                    rk[i][r] = (r0 + r < valid) ? ld16(kg + (size_t)(t0 + r0 + r) * DK + c0) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < NVB_; ++i) {
            const int b = tid + 256 * i;
            if (b < VBLK) {
                const int r0 = (b / (BV / VE)) * VE, c0 = (b % (BV / VE)) * VE;
#pragma unroll
                for (int r = 0; r < VE; ++r)
                    rv[i][r] = (r0 + r < valid) ? ld16(vg + (size_t)(t0 + r0 + r) * p.DV + c0) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < NQV; ++i) {
            const int x = tid + 256 * i;
            if (x < QVEC) {
                const int r = x / (DK / VE), c0 = (x % (DK / VE)) * VE;
                rq[i] = (r < valid) ? ld16(qg + (size_t)(t0 + r) * DK + c0) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < NTV; ++i) {
            const int x = tid + 256 * i;
            if (x < TVEC) {
                rt[i] = ld16(Tw + (size_t)n * C * C + x * VE);
                rp[i] = ld16(Pw + (size_t)n * C * C + x * VE);
            }
        }
        if (CH) {
#pragma unroll
            for (int i = 0; i < NGV; ++i) {
                const int x = tid + 256 * i;
                if (x < GVEC) {
                    const int r = x / (DK / 4), c0 = (x % (DK / 4)) * 4;
                    float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (r < valid) {
                        g = *reinterpret_cast<const float4*>(p.log_alpha + ((size_t)bh * p.L + t0 + r) * DK + c0);
                        g.x = fmaxf(g.x, kChannelLogAlphaMin); g.y = fmaxf(g.y, kChannelLogAlphaMin);
                        g.z = fmaxf(g.z, kChannelLogAlphaMin); g.w = fmaxf(g.w, kChannelLogAlphaMin);
                    }
                    rg[i] = g;
                }
            }
        } else {
            rla = (MODE == kAlphaScalar && l < valid) ? p.log_alpha[(size_t)bh * p.L + t0 + l] : 0.f;
        }
    };

    load_chunk(0);
    for (int n = 0; n < p.NC; ++n) {
        const int t0 = n * C;
        const int valid = min(C, p.L - t0);
        // ---------------- (A) stage chunk n into LDS; S block as E
#pragma unroll
        for (int i = 0; i < MT5; ++i) {
            const int t = w + 4 * i;
            if (t < NT5) {
                const int a = t / NVT, vt = t % NVT;
                st4(Sb + (16 * vt + (l & 15)) * DKP + 16 * a + 4 * (l >> 4), sacc[i][0], sacc[i][1], sacc[i][2], sacc[i][3]);
            }
        }
        if (!CH) {
            // every wave scans the chunk's log-decay itself (lane = token)
            const float g = wave_incl_scan(rla);
            const float glast = __shfl(g, C - 1, kWave);
            if (w == 0 && l < C) { gam[l] = __expf(g); dec[l] = __expf(glast - g); }
            if (w == 0 && l == 0) misc[0] = __expf(glast);
            // T diag(beta) as is, and with its columns scaled by gamma
            // (the shuffles run on every lane, outside the bounds test)
#pragma unroll
            for (int i = 0; i < NTV; ++i) {
                const int x = tid + 256 * i;
                const int r = x / (C / VE), c0 = (x % (C / VE)) * VE;
                float f[VE];
#pragma unroll
                for (int j = 0; j < VE; ++j) f[j] = __expf(__shfl(g, c0 + j, kWave));
                if (x < TVEC) {
                    st16(Tb + r * CKP + c0, rt[i]);
                    st16(Tg + r * CKP + c0, scale_vec<E>(rt[i], f));
                    st16(Ps + r * CKP + c0, rp[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < NKB; ++i) {
                const int b = tid + 256 * i;
                if (b < KBLK) {
                    const int r0 = (b / (DK / VE)) * VE, c0 = (b % (DK / VE)) * VE;
                    u32x4 o[VE];
                    transpose_block(rk[i], o, (E*)nullptr);
#pragma unroll
                    for (int j = 0; j < VE; ++j) st16(Kt + (c0 + j) * CKP + r0, o[j]);
                }
            }
#pragma unroll
            for (int i = 0; i < NQV; ++i) {
                const int x = tid + 256 * i;
                if (x < QVEC) {
                    const int r = x / (DK / VE), c0 = (x % (DK / VE)) * VE;
                    st16(Qs + r * DKP + c0, rq[i]);
                }
            }
        } else {
            // channel mode: cumulative log-decay per key channel first
#pragma unroll
            for (int i = 0; i < NGV; ++i) {
                const int x = tid + 256 * i;
                if (x < GVEC) {
                    const int r = x / (DK / 4), c0 = (x % (DK / 4)) * 4;
                    *reinterpret_cast<float4*>(Gs + r * GP + c0) = rg[i];
                }
            }
#pragma unroll
            for (int i = 0; i < NTV; ++i) {
                const int x = tid + 256 * i;
                if (x < TVEC) {
                    const int r = x / (C / VE), c0 = (x % (C / VE)) * VE;
                    st16(Tb + r * CKP + c0, rt[i]);
                    st16(Ps + r * CKP + c0, rp[i]);
                }
            }
            __syncthreads();
            for (int c = tid; c < DK; c += 256) {
                float acc = 0.f;
#pragma unroll 8
                for (int r = 0; r < C; ++r) { acc += Gs[r * GP + c]; Gs[r * GP + c] = acc; }
            }
            __syncthreads();
            // K^T scaled by exp(G) and by exp(G_last - G); Q scaled by exp(G)
#pragma unroll
            for (int i = 0; i < NKB; ++i) {
                const int b = tid + 256 * i;
                if (b < KBLK) {
                    const int r0 = (b / (DK / VE)) * VE, c0 = (b % (DK / VE)) * VE;
                    u32x4 o[VE];
                    transpose_block(rk[i], o, (E*)nullptr);
#pragma unroll
                    for (int j = 0; j < VE; ++j) {
                        const int c = c0 + j;
                        const float glast = Gs[(C - 1) * GP + c];
                        float fa[VE], fb[VE];
#pragma unroll
                        for (int r = 0; r < VE; ++r) {
                            const float g = Gs[(r0 + r) * GP + c];
                            fa[r] = __expf(g);
                            fb[r] = __expf(glast - g);
                        }
                        st16(Kt + c * CKP + r0, scale_vec<E>(o[j], fa));
                        st16(Kd + c * CKP + r0, scale_vec<E>(o[j], fb));
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < NQV; ++i) {
                const int x = tid + 256 * i;
                if (x < QVEC) {
                    const int r = x / (DK / VE), c0 = (x % (DK / VE)) * VE;
                    float f[VE];
#pragma unroll
                    for (int j = 0; j < VE; ++j) f[j] = __expf(Gs[r * GP + c0 + j]);
                    st16(Qs + r * DKP + c0, scale_vec<E>(rq[i], f));
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NVB_; ++i) {
            const int b = tid + 256 * i;
            if (b < VBLK) {
                const int r0 = (b / (BV / VE)) * VE, c0 = (b % (BV / VE)) * VE;
                u32x4 o[VE];
                transpose_block(rv[i], o, (E*)nullptr);
#pragma unroll
                for (int j = 0; j < VE; ++j) st16(Vt + (c0 + j) * CKP + r0, o[j]);
            }
        }
        __syncthreads();  // B1
        if (n + 1 < p.NC) load_chunk(n + 1);

        // ---------------- (1) W^T = K^T (T diag(beta gamma))^T  -> Ws [tok][dk]
        {
            const E* Aop = Kt;                 // channel: (K . exp(G))^T
            const E* Bop = CH ? Tb : Tg;
            constexpr int NT1 = NKT * NB, MT1 = (NT1 + 3) / 4;
#pragma unroll
            for (int i = 0; i < MT1; ++i) {
                const int t = w + 4 * i;
                if (t < NT1) {
                    const int a = t / NB, tt = t % NB;
                    f32x4 acc = zero4();
                    const int ks = ksteps_tri(tt);
                    for (int s = 0; s < ks; ++s) mma(acc, ldfrag(Aop, CKP, 16 * a, 32 * s), ldfrag(Bop, CKP, 16 * tt, 32 * s));
                    st4(Ws + (16 * tt + (l & 15)) * DKP + 16 * a + 4 * (l >> 4), acc[0], acc[1], acc[2], acc[3]);
                }
            }
        }
        // ---------------- (2) U~ = (T diag(beta)) V  (registers)
        constexpr int NT2 = NB * NVT, MT2 = (NT2 + 3) / 4;
        f32x4 uacc[MT2];
#pragma unroll
        for (int i = 0; i < MT2; ++i) {
            uacc[i] = zero4();
            const int t = w + 4 * i;
            if (t < NT2) {
                const int tt = t / NVT, vt = t % NVT;
                const int ks = ksteps_tri(tt);
                for (int s = 0; s < ks; ++s) mma(uacc[i], ldfrag(Tb, CKP, 16 * tt, 32 * s), ldfrag(Vt, CKP, 16 * vt, 32 * s));
            }
        }
        __syncthreads();  // B2: Ws complete
        // ---------------- (3) U = U~ - W S^T;  O^T = S Q^T (inter-chunk part)
        f32x4 oacc[MT2];
#pragma unroll
        for (int i = 0; i < MT2; ++i) {
            oacc[i] = zero4();
            const int t = w + 4 * i;
            if (t < NT2) {
                const int tt = t / NVT, vt = t % NVT;
                f32x4 z = zero4();
#pragma unroll
                for (int s = 0; s < DK / 32; ++s) {
                    const Frag<E> sf = ldfrag(Sb, DKP, 16 * vt, 32 * s);
                    mma(z, ldfrag(Ws, DKP, 16 * tt, 32 * s), sf);
                    mma(oacc[i], sf, ldfrag(Qs, DKP, 16 * tt, 32 * s));
                }
                float u[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) u[e] = uacc[i][e] - z[e];
                const int tok0 = 16 * tt + 4 * (l >> 4);
                const int vr = 16 * vt + (l & 15);
                st4(Ut + vr * CKP + tok0, u[0], u[1], u[2], u[3]);
                if (!CH) {
                    st4(Us + vr * CKP + tok0, u[0] * dec[tok0], u[1] * dec[tok0 + 1],
                        u[2] * dec[tok0 + 2], u[3] * dec[tok0 + 3]);
                }
                if (!CH) {
                    const float gmy = gam[16 * tt + (l & 15)];
#pragma unroll
                    for (int e = 0; e < 4; ++e) oacc[i][e] *= gmy;
                }
            }
        }
        __syncthreads();  // B3: Ut/Us complete
        // ---------------- (4) O^T += U^T P^T; write O
#pragma unroll
        for (int i = 0; i < MT2; ++i) {
            const int t = w + 4 * i;
            if (t < NT2) {
                const int tt = t / NVT, vt = t % NVT;
                const int ks = ksteps_tri(tt);
                for (int s = 0; s < ks; ++s) mma(oacc[i], ldfrag(Ut, CKP, 16 * vt, 32 * s), ldfrag(Ps, CKP, 16 * tt, 32 * s));
                const int tok = 16 * tt + (l & 15);
                if (tok < valid)
                    st4(og + (size_t)(t0 + tok) * p.DV + 16 * vt + 4 * (l >> 4), oacc[i][0], oacc[i][1], oacc[i][2], oacc[i][3]);
            }
        }
        // ---------------- (5) S^T <- decay S^T + K~^T U^T
        {
            const E* Aop = CH ? Kd : Kt;
            const E* Bop = CH ? Ut : Us;
            const float gl = CH ? 0.f : misc[0];
#pragma unroll
            for (int i = 0; i < MT5; ++i) {
                const int t = w + 4 * i;
                if (t < NT5) {
                    const int a = t / NVT, vt = t % NVT;
                    if (CH) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sacc[i][e] *= __expf(Gs[(C - 1) * GP + 16 * a + 4 * (l >> 4) + e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) sacc[i][e] *= gl;
                    }
#pragma unroll
                    for (int s = 0; s < CK / 32; ++s) mma(sacc[i], ldfrag(Aop, CKP, 16 * a, 32 * s), ldfrag(Bop, CKP, 16 * vt, 32 * s));
                }
            }
        }
        __syncthreads();  // B4: all reads of this chunk's LDS done
    }

    // ---- final state
    if (p.S_final) {
#pragma unroll
        for (int i = 0; i < MT5; ++i) {
            const int t = w + 4 * i;
            if (t < NT5) {
                const int a = t / NVT, vt = t % NVT;
                float* dst = p.S_final + ((size_t)bh * p.DV + v0 + 16 * vt + (l & 15)) * DK + 16 * a + 4 * (l >> 4);
                *reinterpret_cast<f32x4*>(dst) = sacc[i];
            }
        }
    }
}

// L == 0: S_final = S0 (or zero).
__global__ void copy_state_kernel(const float* __restrict__ S0, float* __restrict__ S, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) S[i] = S0 ? S0[i] : 0.f;
}

// ------------------------------------------------------------------ host side
template <typename E>
static constexpr int scan_bv(int DK) { return (sizeof(E) == 4 && DK == 128) ? 16 : 32; }

// fp32 operands with d_k = 128 do not fit a 64-token chunk's staging in
// the 160 KiB of LDS, so that combination runs 32-token chunks; the result
// is the same up to rounding.
int effective_chunk(int C, int dtype, int dk)
{
    return (dtype == kF32 && dk == 128 && C > 32) ? 32 : C;
}

size_t chunk_workspace_bytes_per_chunk(int C, int dtype)
{
    return (size_t)2 * C * C * (dtype == kBF16 ? 2 : 4);
}

template <typename E, int DK, int C, int MODE>
static hipError_t launch_chunk(const ChunkArgs& a)
{
    constexpr int BV = scan_bv<E>(DK);
    const int BH = a.B * a.H;
    const int NC = (a.L + C - 1) / C;
    const size_t per = (size_t)C * C;
    E* Tws = reinterpret_cast<E*>(a.workspace);
    E* Pws = Tws + (size_t)BH * NC * per;

    using PL = PrepLayout<E, DK, C, MODE>;
    static_assert(PL::bytes <= 160 * 1024, "prep LDS");
    PrepParams pp{a.q, a.k, a.beta, a.log_alpha, Tws, Pws, a.L, NC};
    auto* pk = chunk_prep_kernel<E, DK, C, MODE>;
    hipError_t err = hipFuncSetAttribute((const void*)pk, hipFuncAttributeMaxDynamicSharedMemorySize, PL::bytes);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(pk, dim3(NC * BH), dim3(256), PL::bytes, a.stream, pp);
    err = hipGetLastError();
    if (err != hipSuccess) return err;

    using SL = ScanLayout<E, DK, BV, C, MODE>;
    static_assert(SL::bytes <= 160 * 1024, "scan LDS");
    const int NVB = a.dv / BV;
    ScanParams sp{a.q, a.k, a.v, a.log_alpha, a.S0, Tws, Pws, a.o, a.S_final, a.L, NC, a.dv, NVB, BH * NVB};
    auto* sk = chunk_scan_kernel<E, DK, BV, C, MODE>;
    err = hipFuncSetAttribute((const void*)sk, hipFuncAttributeMaxDynamicSharedMemorySize, SL::bytes);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(sk, dim3(BH * NVB), dim3(256), SL::bytes, a.stream, sp);
    return hipGetLastError();
}

template <typename E, int DK, int C>
static hipError_t by_mode(const ChunkArgs& a)
{
    switch (a.mode) {
    case kAlphaNone: return launch_chunk<E, DK, C, kAlphaNone>(a);
    case kAlphaScalar: return launch_chunk<E, DK, C, kAlphaScalar>(a);
    default: return launch_chunk<E, DK, C, kAlphaChannel>(a);
    }
}

template <typename E, int DK>
static hipError_t by_chunk(const ChunkArgs& a)
{
    switch (effective_chunk(a.C, a.dtype, a.dk)) {
    case 16: return by_mode<E, DK, 16>(a);
    case 32: return by_mode<E, DK, 32>(a);
    default:
        if constexpr (sizeof(E) == 4 && DK == 128) return hipErrorInvalidValue;
        else return by_mode<E, DK, 64>(a);
    }
}

hipError_t launch_fwd_chunked(const ChunkArgs& a)
{
    if (a.mode != kAlphaChannel && a.L > 0 && (size_t)a.B * a.H > 0) return launch_pipe_chunked(a);
    const size_t BH = (size_t)a.B * a.H;
    if (BH == 0) return hipSuccess;
    if (a.L == 0) {
        if (!a.S_final) return hipSuccess;
        const size_t n = BH * a.dv * a.dk;
        if (a.S0 == a.S_final) return hipSuccess;
        hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, a.stream, a.S0, a.S_final, n);
        return hipGetLastError();
    }
    if (a.dtype == kBF16) return a.dk == 128 ? by_chunk<bf16, 128>(a) : by_chunk<bf16, 64>(a);
    return a.dk == 128 ? by_chunk<float, 128>(a) : by_chunk<float, 64>(a);
}

}  // namespace gdr

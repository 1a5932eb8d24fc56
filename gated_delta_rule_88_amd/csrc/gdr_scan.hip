// gdr_scan.hip -- the sequential part of the chunked forward: one workgroup
// per (batch, head, 32 value channels) walks the chunks in order with its
// block of the state in registers.
//
// Chunk algebra (one head, chunk of CK tokens, entry state S, d_v x d_k;
// T~, Gamma, gamma come from the prepass in gdr_wy.hip):
//   X = K S^T;   R = V - diag(gamma) X;   U = T~ R        (delta residuals)
//   O = diag(gamma) Q S^T + (Q K^T . Gamma . M_incl) U
//   S <- gamma_C S + U^T diag(exp(g_C - g)) K
// Substituting the recurrence into itself over one chunk gives
// (I + A) U = diag(beta) (V - diag(gamma) K S^T), hence U = T~ R.  ("linear
// attention and its gated descendants", "Chunkwise Parallel Form": boundary
// state plus a masked intra-chunk block, with the output read after the
// write so the mask includes the diagonal; "Gated DeltaNet": decay then
// delta update.)  Per-channel alpha replaces gamma K by K . exp(G), gamma Q
// by Q . exp(G), exp(g_C - g) K by K . exp(G_C - G), gamma_C S by
// S Diag(exp(G_C)) ("Kimi Delta Attention": the decay acts on the key
// dimension), and the score block P comes precomputed.
//
// Rows of S (value channels) evolve independently given K, beta and alpha,
// which is what lets the value dimension be split across workgroups and
// waves.  Five waves, one barrier per chunk step, four rotating LDS slots:
//   waves 0, 1  (state owners)  each holds the state of 16 value channels
//               (d_k x 16 fp32) in registers; for chunk n it publishes S as
//               an MFMA operand, forms X, R, U (published too) and the next
//               state.  Only this chain is sequential.
//   waves 2, 3  (output waves)  for chunk n - 1, from the published S and U:
//               the inter-chunk output diag(gamma) Q S^T, the masked score
//               block P (MFMA), P U, and the store of o.
//   wave 4      (copier)        direct global->LDS copies of chunk n + 2 (K,
//               Q, the V block, T~, Gamma or P, the decay factors), 16 bytes
//               per lane, then waits until chunk n + 1 has landed.
// Every product is v_mfma_f32_16x16x32_bf16 (fp32: 16x16x4f32) in NT form;
// result tiles feed the next product straight from registers (tile-pair
// operands, gdr_device.h), K^T and V are read with transposing LDS loads.
// K, Q, V, T~ and Gamma/P sit in LDS row-major with their 16-byte chunks
// XOR-swizzled by row: the copier applies the permutation by choosing each
// lane's source address, every reader undoes it.
#include "gdr_device.h"
#include "gdr_chunk.h"

namespace gdr {

namespace {
__host__ __device__ constexpr int align16(int x) { return (x + 15) / 16 * 16; }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Row-major LDS tile of W elements per row whose 16-byte chunks are permuted
// within each row by XOR with swz(row).
template <typename E, int W>
struct Swz {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int RB = W * ES;      // bytes per row
    static constexpr int NCH = RB / 16;    // 16-byte chunks per row
    static_assert(NCH == 2 || NCH == 4 || NCH == 8 || NCH == 16 || NCH == 32, "row width");
    __device__ static __forceinline__ int swz(int r) {
        if (NCH == 2) return (r >> 2) & 1;
        if (NCH == 4) return (r >> 2) & 3;
        if (NCH == 8) return (r >> 1) & 7;
        if (NCH == 16) return ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3);
        return r & 15;
    }
    // byte offset of element (r, c); an access of up to 16 bytes starting at
    // c must not cross a 16-byte boundary
    __device__ static __forceinline__ int off(int r, int c) {
        const int cb = c * ES;
        return r * RB + ((((cb >> 4) ^ swz(r))) << 4) + (cb & 15);
    }
};

__device__ __forceinline__ u32x4 lds16(const unsigned char* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 lds8(const unsigned char* p) { return *reinterpret_cast<const u32x2*>(p); }

// Tile-pair fragment: lane reads row r0 + l%16, k = k0 + 16p + 4(l/16) + e.
template <typename E, int W>
__device__ __forceinline__ Frag<E> ldfrag_pair_swz(const unsigned char* base, int r0, int k0) {
    using S = Swz<E, W>;
    const int l = lane_id(), r = r0 + (l & 15), k = k0 + 4 * (l >> 4);
    Frag<E> f;
    if constexpr (sizeof(E) == 2) {
        const u32x2 lo = lds8(base + S::off(r, k)), hi = lds8(base + S::off(r, k + 16));
        f.v = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
    } else {
        f.lo = __builtin_bit_cast(f32x4, lds16(base + S::off(r, k)));
        f.hi = __builtin_bit_cast(f32x4, lds16(base + S::off(r, k + 16)));
    }
    return f;
}
// 16-wide k-step fragment: lane reads row r0 + l%16, k = k0 + 4(l/16) + e.
template <typename E, int W>
__device__ __forceinline__ Frag16<E> ldfrag16_swz(const unsigned char* base, int r0, int k0) {
    using S = Swz<E, W>;
    const int l = lane_id(), r = r0 + (l & 15), k = k0 + 4 * (l >> 4);
    Frag16<E> f;
    if constexpr (sizeof(E) == 2) {
        f.v = __builtin_bit_cast(s16x4, lds8(base + S::off(r, k)));
    } else {
        f.v = __builtin_bit_cast(f32x4, lds16(base + S::off(r, k)));
    }
    return f;
}
// Four consecutive elements of row r from column c (c % 4 == 0), as fp32.
template <typename E, int W>
__device__ __forceinline__ f32x4 ld4_swz(const unsigned char* base, int r, int c) {
    using S = Swz<E, W>;
    if constexpr (sizeof(E) == 2) {
        const u32x2 w = lds8(base + S::off(r, c));
        return f32x4{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
    } else {
        return __builtin_bit_cast(f32x4, lds16(base + S::off(r, c)));
    }
}
// Transposed read: lane (g, c) = (l/16, l%16) receives M[r0 + 4g + q][c0 + c]
// for q = 0..3.  bf16 uses the transposing LDS load (lane 16h + i supplies
// the address of M[r0 + 4h + i/4][c0 + 4(i%4) .. +3]); fp32 reads the four
// elements one by one.
template <typename E, int W>
__device__ __forceinline__ f32x4 ld_tr(const unsigned char* base, int r0, int c0, s16x4* raw = nullptr) {
    using S = Swz<E, W>;
    const int l = lane_id(), g = l >> 4, i = l & 15;
    if constexpr (sizeof(E) == 2) {
        const unsigned char* a = base + S::off(r0 + 4 * g + (i >> 2), c0 + 4 * (i & 3));
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(a));
        if (raw) *raw = v;
        const u32x2 w = __builtin_bit_cast(u32x2, v);
        return f32x4{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
    } else {
        f32x4 r;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            r[q] = *reinterpret_cast<const float*>(base + S::off(r0 + 4 * g + q, c0 + i));
        return r;
    }
}

// Direct global->LDS copies, 16 bytes per lane: the instruction's lane l
// writes LDS bytes [dst + 16 l, +16).
template <int NBYTES>
struct CopyCount { static constexpr int n = (NBYTES + 1023) / 1024; };

// [CK][W] row-major tile, global row stride gstride bytes, into a swizzled
// LDS region; rows at or past `valid` repeat row valid - 1.
template <typename E, int W, int CK>
__device__ __forceinline__ void copy_tile(unsigned char* dst, const unsigned char* src, size_t gstride, int valid) {
    using S = Swz<E, W>;
    constexpr int TB = CK * S::RB;
    const int l = lane_id();
#pragma unroll
    for (int j = 0; j < CopyCount<TB>::n; ++j) {
        const int b = 1024 * j + 16 * l;
        if (TB % 1024 == 0 || b < TB) {
            const int row = b / S::RB, pch = (b % S::RB) / 16;
            const int lch = pch ^ S::swz(row);
            const unsigned char* g = src + (size_t)min(row, valid - 1) * gstride + lch * 16;
            __builtin_amdgcn_global_load_lds((const glb_void_t*)g, (lds_void_t*)(dst + 1024 * j), 16, 0, 0);
        }
    }
}
template <int NBYTES>
__device__ __forceinline__ void copy_flat(unsigned char* dst, const unsigned char* src) {
    const int l = lane_id();
#pragma unroll
    for (int j = 0; j < CopyCount<NBYTES>::n; ++j) {
        const int b = 1024 * j + 16 * l;
        if (NBYTES % 1024 == 0 || b < NBYTES)
            __builtin_amdgcn_global_load_lds((const glb_void_t*)(src + b), (lds_void_t*)(dst + 1024 * j), 16, 0, 0);
    }
}

// Barrier for the pipeline: this wave's LDS accesses are complete, then all
// waves meet.  It does not wait for outstanding global->LDS copies: the
// copier waits for those explicitly.
__device__ __forceinline__ void step_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
}  // namespace

template <typename E, int DK, int CK, int MODE>
struct ScanLayout {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int BV = 32;             // value channels per workgroup
    static constexpr int NSLOT = 4;
    static constexpr bool CH = (MODE == kAlphaChannel);
    static constexpr int FB = MODE == kAlphaScalar ? 4 * CK * 4 : (CH ? DK * 4 : 0);
    // one chunk slot
    static constexpr int s_KX = 0;                                   // K or K.exp(G) [CK][DK]
    static constexpr int s_KU = s_KX + CK * DK * ES;                 // K.exp(G_C-G) (channel)
    static constexpr int s_Q = s_KU + (CH ? CK * DK * ES : 0);       // Q or Q.exp(G) [CK][DK]
    static constexpr int s_V = s_Q + CK * DK * ES;                   // V block [CK][BV]
    static constexpr int s_T = s_V + CK * BV * ES;                   // T~ [CK][CK]
    static constexpr int s_M = s_T + CK * CK * ES;                   // Gamma or P [CK][CK]
    static constexpr int s_F = s_M + (MODE != kAlphaNone ? CK * CK * ES : 0);
    static constexpr int slot = align16(s_F + FB);
    // exchange buffers (two steps deep): S operands and U operands of each
    // state owner, one fragment per lane
    static constexpr int NKS = DK / 32;
    static constexpr int FS = (int)sizeof(Frag<E>);
    static constexpr int off_xS = NSLOT * slot;
    static constexpr int off_xU = off_xS + 2 * 2 * NKS * kWave * FS;
    static constexpr int bytes = off_xU + 2 * 2 * kWave * FS;
    // copy instructions per chunk
    static constexpr int NOPS = (CH ? 3 : 2) * CopyCount<CK * DK * ES>::n + CopyCount<CK * BV * ES>::n +
                                CopyCount<CK * CK * ES>::n * (MODE != kAlphaNone ? 2 : 1) +
                                (FB ? CopyCount<(FB ? FB : 1)>::n : 0);
    static_assert(NOPS < 64, "vmcnt range");
};

template <typename E, int DK, int CK, int MODE>
__global__ __launch_bounds__(320) void chunk_scan_kernel(ScanParams p)
{
    using LY = ScanLayout<E, DK, CK, MODE>;
    constexpr int ES = LY::ES, BV = LY::BV;
    constexpr int NB = CK / 16, NKT = DK / 16, NKS = DK / 32;
    constexpr bool GATED = (MODE == kAlphaScalar), CH = LY::CH;
    constexpr WsLayout WL = ws_layout(ES, DK, CK, MODE);
    extern __shared__ __align__(16) unsigned char smem[];

    // wave index as a scalar: the role branches below are wave-uniform
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15;
    int lid = blockIdx.x;
    // consecutive block ids land on different XCDs: give the value blocks of
    // one head neighbouring logical ids on one XCD so they share its L2
    if (p.total % 8 == 0) lid = (blockIdx.x % 8) * (p.total / 8) + blockIdx.x / 8;
    const int bh = lid / p.NVB, vb = lid % p.NVB;
    const int v0 = vb * BV;

    struct Slot {
        unsigned char *KX, *KU, *Q, *V, *T, *M;
        float* F;
    };
    auto slot = [&](int m) {
        unsigned char* b = smem + (m % LY::NSLOT) * LY::slot;
        Slot s;
        s.KX = b + LY::s_KX;
        s.KU = CH ? b + LY::s_KU : b + LY::s_KX;
        s.Q = b + LY::s_Q;
        s.V = b + LY::s_V;
        s.T = b + LY::s_T;
        s.M = b + LY::s_M;
        s.F = reinterpret_cast<float*>(b + LY::s_F);
        return s;
    };
    Frag<E>* xS = reinterpret_cast<Frag<E>*>(smem + LY::off_xS);   // [buf][owner][ks][lane]
    Frag<E>* xU = reinterpret_cast<Frag<E>*>(smem + LY::off_xU);   // [buf][owner][lane]

    if (w < 2) {
        // ===================================================== state owners
        const int vw = v0 + 16 * w;
        f32x4 sT[NKT];   // S^T[16a + 4g + e][v = vw + c16]
#pragma unroll
        for (int a = 0; a < NKT; ++a) {
            sT[a] = zero4();
            if (p.S0)
                sT[a] = *reinterpret_cast<const f32x4*>(p.S0 + ((size_t)bh * p.DV + vw + c16) * DK + 16 * a + 4 * g4);
        }
        auto own = [&](int m) {
            const Slot s = slot(m);
            Frag<E> sop[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                frag_of_tiles(sop[ks], sT[2 * ks], sT[2 * ks + 1]);
                xS[(((m & 1) * 2 + w) * NKS + ks) * kWave + l] = sop[ks];
            }
            // X = K S^T and R = V - diag(gamma) X: token 16tt + 4g + e, channel c16
            f32x4 r[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                f32x4 x = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) mma(x, ldfrag_pair_swz<E, DK>(s.KX, 16 * tt, 32 * ks), sop[ks]);
                const f32x4 vv = ld_tr<E, BV>(s.V, 16 * tt, 16 * w);
                const f32x4 gm = GATED ? *reinterpret_cast<const f32x4*>(s.F + 16 * tt + 4 * g4)
                                       : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int e = 0; e < 4; ++e) r[tt][e] = vv[e] - gm[e] * x[e];
            }
            // decay of the state over the chunk
            if (GATED) {
                const float gC = s.F[2 * CK];
#pragma unroll
                for (int a = 0; a < NKT; ++a)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sT[a][e] *= gC;
            } else if (CH) {
#pragma unroll
                for (int a = 0; a < NKT; ++a) {
                    const f32x4 ec = *reinterpret_cast<const f32x4*>(s.F + 16 * a + 4 * g4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) sT[a][e] *= ec[e];
                }
            }
            // U = T~ R (published for the output wave), then
            // S^T += K'^T (dec . U), K' = K (channel: K . exp(G_C - G), dec = 1)
            if constexpr (NB == 2) {
                Frag<E> rop;
                frag_of_tiles(rop, r[0], r[1]);
                f32x4 u[2];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    u[tt] = zero4();
                    mma(u[tt], ldfrag_pair_swz<E, CK>(s.T, 16 * tt, 0), rop);
                }
                Frag<E> uop;
                frag_of_tiles(uop, u[0], u[1]);
                xU[((m & 1) * 2 + w) * kWave + l] = uop;
                if (GATED) {
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        const f32x4 dc = *reinterpret_cast<const f32x4*>(s.F + CK + 16 * tt + 4 * g4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) u[tt][e] *= dc[e];
                    }
                    frag_of_tiles(uop, u[0], u[1]);
                }
#pragma unroll
                for (int a = 0; a < NKT; ++a) {
                    Frag<E> kt;
                    if constexpr (sizeof(E) == 2) {
                        s16x4 k0, k1;
                        ld_tr<E, DK>(s.KU, 0, 16 * a, &k0);
                        ld_tr<E, DK>(s.KU, 16, 16 * a, &k1);
                        const u32x2 a0 = __builtin_bit_cast(u32x2, k0), a1 = __builtin_bit_cast(u32x2, k1);
                        kt.v = __builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y});
                    } else {
                        kt.lo = ld_tr<E, DK>(s.KU, 0, 16 * a);
                        kt.hi = ld_tr<E, DK>(s.KU, 16, 16 * a);
                    }
                    mma(sT[a], kt, uop);
                }
            } else {
                Frag16<E> rop;
                frag16_of_tile(rop, r[0]);
                f32x4 u = zero4();
                mma16(u, ldfrag16_swz<E, CK>(s.T, 0, 0), rop);
                Frag16<E> uop;
                frag16_of_tile(uop, u);
                *reinterpret_cast<Frag16<E>*>(xU + ((m & 1) * 2 + w) * kWave + l) = uop;
                if (GATED) {
                    const f32x4 dc = *reinterpret_cast<const f32x4*>(s.F + CK + 4 * g4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) u[e] *= dc[e];
                    frag16_of_tile(uop, u);
                }
#pragma unroll
                for (int a = 0; a < NKT; ++a) {
                    Frag16<E> kt;
                    if constexpr (sizeof(E) == 2) {
                        ld_tr<E, DK>(s.KU, 0, 16 * a, &kt.v);
                    } else {
                        kt.v = ld_tr<E, DK>(s.KU, 0, 16 * a);
                    }
                    mma16(sT[a], kt, uop);
                }
            }
        };
        step_barrier();
        for (int s = 0; s <= p.NC; ++s) {
            if (s < p.NC) own(s);
            step_barrier();
        }
        if (p.S_final) {
#pragma unroll
            for (int a = 0; a < NKT; ++a)
                *reinterpret_cast<f32x4*>(p.S_final + ((size_t)bh * p.DV + vw + c16) * DK + 16 * a + 4 * g4) = sT[a];
        }
    } else if (w < 4) {
        // ===================================================== output waves
        const int c = w - 2, vw = v0 + 16 * c;
        E* og = reinterpret_cast<E*>(p.o) + (size_t)bh * p.L * p.DV;
        auto out = [&](int m) {
            const Slot s = slot(m);
            const int t0 = m * CK, valid = min(CK, p.L - t0);
            Frag<E> sop[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) sop[ks] = xS[(((m & 1) * 2 + c) * NKS + ks) * kWave + l];
            Frag<E> qf[NB][NKS];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) qf[tt][ks] = ldfrag_pair_swz<E, DK>(s.Q, 16 * tt, 32 * ks);
            // inter-chunk part: O^T = S Q^T, lane holds O[16tt + c16][vw + 4g + e]
            f32x4 oi[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                oi[tt] = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) mma(oi[tt], sop[ks], qf[tt][ks]);
                if (GATED) {
                    const float gq = s.F[16 * tt + c16];
#pragma unroll
                    for (int e = 0; e < 4; ++e) oi[tt][e] *= gq;
                }
            }
            // masked score tile (rb, ib): lane holds P[16rb + c16][16ib + 4g + e]
            auto score = [&](int rb, int ib) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    mma(acc, ldfrag_pair_swz<E, DK>(s.KX, 16 * ib, 32 * ks), qf[rb][ks]);
                const int r = 16 * rb + c16, i0 = 16 * ib + 4 * g4;
                if (GATED) {
                    const f32x4 gm = ld4_swz<E, CK>(s.M, r, i0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] *= gm[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = (r >= i0 + e) ? acc[e] : 0.f;
                }
                return acc;
            };
            // intra-chunk part: O^T += U^T P^T
            if constexpr (NB == 2) {
                Frag<E> pf[2];
                if constexpr (CH) {
                    pf[0] = ldfrag_pair_swz<E, CK>(s.M, 0, 0);
                    pf[1] = ldfrag_pair_swz<E, CK>(s.M, 16, 0);
                } else {
                    frag_of_tiles(pf[0], score(0, 0), zero4());
                    frag_of_tiles(pf[1], score(1, 0), score(1, 1));
                }
                const Frag<E> uop = xU[((m & 1) * 2 + c) * kWave + l];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) mma(oi[tt], uop, pf[tt]);
            } else {
                Frag16<E> pf;
                if constexpr (CH) pf = ldfrag16_swz<E, CK>(s.M, 0, 0);
                else frag16_of_tile(pf, score(0, 0));
                const Frag16<E> uop = *reinterpret_cast<const Frag16<E>*>(xU + ((m & 1) * 2 + c) * kWave + l);
                mma16(oi[0], uop, pf);
            }
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                const int tok = 16 * tt + c16;
                if (tok < valid)
                    st4(og + (size_t)(t0 + tok) * p.DV + vw + 4 * g4, oi[tt][0], oi[tt][1], oi[tt][2], oi[tt][3]);
            }
        };
        step_barrier();
        for (int s = 0; s <= p.NC; ++s) {
            if (s >= 1) out(s - 1);
            step_barrier();
        }
    } else {
        // ===================================================== copier
        const unsigned char* kb = static_cast<const unsigned char*>(p.k);
        const unsigned char* qb = static_cast<const unsigned char*>(p.q);
        const unsigned char* vbase = static_cast<const unsigned char*>(p.v);
        auto issue = [&](int m) {
            const Slot s = slot(m);
            const int t0 = m * CK, valid = min(CK, p.L - t0);
            const unsigned char* rec = p.ws + ((size_t)bh * p.NC + m) * WL.bytes;
            const size_t row0 = (size_t)bh * p.L + t0;
            if constexpr (CH) {
                copy_tile<E, DK, CK>(s.KX, rec + WL.KG, DK * ES, CK);
                copy_tile<E, DK, CK>(s.KU, rec + WL.KD, DK * ES, CK);
                copy_tile<E, DK, CK>(s.Q, rec + WL.QG, DK * ES, CK);
            } else {
                copy_tile<E, DK, CK>(s.KX, kb + row0 * DK * ES, DK * ES, valid);
                copy_tile<E, DK, CK>(s.Q, qb + row0 * DK * ES, DK * ES, valid);
            }
            copy_tile<E, BV, CK>(s.V, vbase + (row0 * p.DV + v0) * ES, (size_t)p.DV * ES, valid);
            copy_tile<E, CK, CK>(s.T, rec + WL.T, CK * ES, CK);
            if constexpr (MODE != kAlphaNone) copy_tile<E, CK, CK>(s.M, rec + WL.M, CK * ES, CK);
            if constexpr (LY::FB > 0) copy_flat<LY::FB>(reinterpret_cast<unsigned char*>(s.F), rec + WL.F);
        };
        issue(0);
        if (p.NC > 1) {
            issue(1);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LY::NOPS) : "memory");   // chunk 0 landed
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        step_barrier();
        for (int s = 0; s <= p.NC; ++s) {
            if (s + 2 < p.NC) {
                issue(s + 2);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LY::NOPS) : "memory");   // chunk s + 1 landed
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            step_barrier();
        }
    }
}

// ------------------------------------------------------------------ host side
template <typename E, int DK, int CK, int MODE>
static hipError_t launch_scan_t(const ChunkArgs& a)
{
    using LY = ScanLayout<E, DK, CK, MODE>;
    static_assert(LY::bytes <= 160 * 1024, "LDS budget");
    const int BH = a.B * a.H;
    const int NC = (a.L + CK - 1) / CK;
    const int NVB = a.dv / LY::BV;
    ScanParams sp{a.q, a.k, a.v, a.S0, static_cast<const unsigned char*>(a.workspace), a.o, a.S_final,
                  a.L, NC, a.dv, NVB, BH * NVB};
    auto* kern = chunk_scan_kernel<E, DK, CK, MODE>;
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LY::bytes);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(BH * NVB), dim3(320), LY::bytes, a.stream, sp);
    return hipGetLastError();
}

template <typename E, int DK, int CK>
static hipError_t launch_scan_m(const ChunkArgs& a)
{
    if (a.mode == kAlphaChannel) return launch_scan_t<E, DK, CK, kAlphaChannel>(a);
    if (a.mode == kAlphaScalar) return launch_scan_t<E, DK, CK, kAlphaScalar>(a);
    return launch_scan_t<E, DK, CK, kAlphaNone>(a);
}

hipError_t launch_scan(const ChunkArgs& a, int CK)
{
    if (a.dtype == kBF16) {
        if (a.dk == 128) return CK == 16 ? launch_scan_m<bf16, 128, 16>(a) : launch_scan_m<bf16, 128, 32>(a);
        return CK == 16 ? launch_scan_m<bf16, 64, 16>(a) : launch_scan_m<bf16, 64, 32>(a);
    }
    return a.dk == 128 ? launch_scan_m<float, 128, 16>(a) : launch_scan_m<float, 64, 16>(a);
}

}  // namespace gdr

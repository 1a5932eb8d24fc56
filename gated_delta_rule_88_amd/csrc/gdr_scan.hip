// gdr_scan.hip -- fused, pipelined chunkwise forward for DeltaNet (alpha = 1)
// and Gated DeltaNet (scalar alpha).
//
// Chunk algebra (one head, chunk of CK tokens, entry state S, d_v x d_k; see
// the header of gdr_chunk.hip for the derivation):
//   A  = strictly-lower( diag(beta) (K K^T . Gamma) ),  Gamma_ri = exp(g_r - g_i)
//   T  = (I + A)^{-1} diag(beta)                         (WY factor)
//   X  = K S^T;   R = V - diag(gamma) X;   U = T R       (delta residuals)
//   O  = diag(gamma) Q S^T + (Q K^T . Gamma . M_incl) U
//   S <- gamma_C S + U^T diag(exp(g_C - g)) K
// ("linear attention and its gated descendants", "Chunkwise Parallel Form":
// boundary state plus a masked intra-chunk block; "Linear Attention &
// DeltaNet", item 3: the chunk's (I - beta k k^T) factors kept in WY form.)
//
// One workgroup owns one (batch, head) and a block of 32 value channels and
// walks the chunks in order.  Its four waves form a pipeline with one
// barrier per chunk step; chunk data lives in four rotating LDS slots:
//   wave 2 (stager)    issues the direct global->LDS copies of K, Q and the
//                      V block of chunk n+3, then, for chunk n+2 (whose
//                      copies have landed), the in-chunk cumulative
//                      log-decay and the masked decayed score block
//                      P = Q K^T . Gamma . M_incl (MFMA);
//   wave 3 (WY)        chunk n+1: the Gram block, A, and T = (I + A)^{-1}
//                      diag(beta) (fp32: 16x16 diagonal blocks by forward
//                      substitution, the off-diagonal block with MFMA);
//   waves 0, 1         chunk n: each owns 16 value channels of the state in
//   (consumers)        registers and runs X, R, U, the outputs and the state
//                      update with MFMA.  Every product's result tile feeds
//                      the next product straight from registers (tile-pair
//                      operands, gdr_device.h); K^T and V are read with
//                      transposing LDS loads, so no transposed copy exists.
// K, Q and V sit in LDS row-major with their 16-byte chunks XOR-swizzled by
// row; the swizzle is applied when each lane picks the global address of
// the chunk it copies, and undone by every reader.
// Rows of S (value channels) evolve independently given K, beta and alpha,
// which is what allows the value dimension to be split across waves and
// workgroups.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {
__host__ __device__ constexpr int align16(int x) { return (x + 15) / 16 * 16; }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Row-major LDS buffer of W elements per row whose 16-byte chunks are
// permuted within each row by XOR with swz(row); the permutation keeps the
// fragment reads (16 rows, one chunk) and the transposing reads (4 rows,
// two chunks) free of bank conflicts.
template <typename E, int W>
struct Swz {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int RB = W * ES;      // bytes per row
    static constexpr int NCH = RB / 16;    // 16-byte chunks per row
    static_assert(NCH == 4 || NCH == 8 || NCH == 16 || NCH == 32, "row width");
    __device__ static __forceinline__ int swz(int r) {
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

// Fragment (ldfrag convention: lane reads row r0 + l%16, k = k0 + 8(l/16)..+7)
template <typename E, int W>
__device__ __forceinline__ Frag<E> ldfrag_swz(const unsigned char* base, int r0, int k0) {
    using S = Swz<E, W>;
    const int l = lane_id(), r = r0 + (l & 15), k = k0 + 8 * (l >> 4);
    Frag<E> f;
    if constexpr (sizeof(E) == 2) {
        f.v = __builtin_bit_cast(bf16x8, lds16(base + S::off(r, k)));
    } else {
        f.lo = __builtin_bit_cast(f32x4, lds16(base + S::off(r, k)));
        f.hi = __builtin_bit_cast(f32x4, lds16(base + S::off(r, k + 4)));
    }
    return f;
}
// Tile-pair fragment: lane reads row r0 + l%16, k = k0 + 16p + 4(l/16) + e
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

// Barrier for the pipeline: this wave's LDS writes are complete, then all
// waves meet.  Unlike __syncthreads() it does not wait for outstanding
// global->LDS copies, which are waited for explicitly before their data is
// read.
__device__ __forceinline__ void step_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
}  // namespace

template <typename E, int DK, int CK>
struct PipeLayout {
    static constexpr int VE = Vec<E>::n;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int BV = 32;             // value channels per workgroup
    static constexpr int LTK = CK + VE;       // row stride of [*][token] buffers (T, P)
    static constexpr int LF = CK + 4;         // row stride of fp32 scratch
    static constexpr int NSLOT = 4;
    // one chunk slot
    static constexpr int s_K = 0;                          // K [CK][DK], swizzled
    static constexpr int s_Q = s_K + CK * DK * ES;         // Q [CK][DK], swizzled
    static constexpr int s_V = s_Q + CK * DK * ES;         // V [CK][BV], swizzled
    static constexpr int s_T = s_V + CK * BV * ES;         // T diag(beta) [CK][LTK]
    static constexpr int s_P = s_T + CK * LTK * ES;        // P [CK][LTK]
    static constexpr int s_f = s_P + CK * LTK * ES;        // g, gamma, dec, beta [CK]; gamma_C
    static constexpr int slot = align16(s_f + (4 * CK + 4) * 4);
    // WY-wave scratch (fp32)
    static constexpr int off_A = NSLOT * slot;
    static constexpr int off_Tf = off_A + CK * LF * 4;
    static constexpr int off_Tt = off_Tf + CK * LF * 4;
    static constexpr int bytes = off_Tt + CK * LF * 4;
    static_assert((CK * DK * ES) % 1024 == 0 && (CK * BV * ES) % 1024 == 0, "copy granule");
};

struct PipeParams {
    const void *q, *k, *v;
    const float *beta, *log_alpha, *S0;
    void* o;
    float* S_final;
    int L, NC, DV, NVB, total;
};

template <typename E, int DK, int CK, int MODE>
__global__ __launch_bounds__(256) void chunk_pipe_kernel(PipeParams p)
{
    using LY = PipeLayout<E, DK, CK>;
    using SK = Swz<E, DK>;
    using SV = Swz<E, LY::BV>;
    constexpr int VE = LY::VE, ES = LY::ES, BV = LY::BV, LTK = LY::LTK, LF = LY::LF;
    constexpr int NB = CK / 16, NKT = DK / 16, NKS = DK / 32;
    constexpr bool GATED = (MODE == kAlphaScalar);
    extern __shared__ __align__(16) unsigned char smem[];

    // wave index as a scalar: the role branches below are wave-uniform
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15;
    int lid = blockIdx.x;
    // consecutive block ids land on different XCDs: give the d_v blocks of
    // one head neighbouring logical ids on one XCD so they share its L2.
    if (p.total % 8 == 0) lid = (blockIdx.x % 8) * (p.total / 8) + blockIdx.x / 8;
    const int bh = lid / p.NVB, vb = lid % p.NVB;
    const int v0 = vb * BV;

    struct Slot {
        unsigned char *K, *Q, *V;
        E *T, *P;
        float *gs, *gam, *dec, *bet, *misc;
    };
    auto slot = [&](int m) {
        unsigned char* b = smem + (m % LY::NSLOT) * LY::slot;
        Slot s;
        s.K = b + LY::s_K;
        s.Q = b + LY::s_Q;
        s.V = b + LY::s_V;
        s.T = reinterpret_cast<E*>(b + LY::s_T);
        s.P = reinterpret_cast<E*>(b + LY::s_P);
        float* f = reinterpret_cast<float*>(b + LY::s_f);
        s.gs = f; s.gam = f + CK; s.dec = f + 2 * CK; s.bet = f + 3 * CK; s.misc = f + 4 * CK;
        return s;
    };

    const E* kg = reinterpret_cast<const E*>(p.k) + (size_t)bh * p.L * DK;
    const E* qg = reinterpret_cast<const E*>(p.q) + (size_t)bh * p.L * DK;
    const E* vg = reinterpret_cast<const E*>(p.v) + (size_t)bh * p.L * p.DV + v0;

    if (w == 2) {
        // ============================================================ stager
        float rla = 0.f, rbt = 0.f;
        // copy a [CK][W] row-major tile (row stride gstride elements) into a
        // swizzled LDS region, 1 KiB per instruction; rows past the end of the
        // sequence repeat its last row (their contributions are cancelled by
        // beta = 0 and are never stored).
        auto copy_tile = [&](unsigned char* dst, const E* src, int gstride, int t0, int valid, auto sw) {
            using S = decltype(sw);
            constexpr int TB = CK * S::RB;
#pragma unroll
            for (int j = 0; j < TB / 1024; ++j) {
                const int b = 1024 * j + 16 * l;
                const int row = b / S::RB, pch = (b % S::RB) / 16;
                const int lch = pch ^ S::swz(row);
                const E* gsrc = src + (size_t)(t0 + min(row, valid - 1)) * gstride + lch * (16 / ES);
                __builtin_amdgcn_global_load_lds((const glb_void_t*)gsrc, (lds_void_t*)(dst + 1024 * j), 16, 0, 0);
            }
        };
        auto issue = [&](int m) {
            const Slot s = slot(m);
            const int t0 = m * CK, valid = min(CK, p.L - t0);
            copy_tile(s.K, kg, DK, t0, valid, SK{});
            copy_tile(s.Q, qg, DK, t0, valid, SK{});
            copy_tile(s.V, vg, p.DV, t0, valid, SV{});
            const int tl = t0 + min(l, valid - 1);
            rla = GATED ? p.log_alpha[(size_t)bh * p.L + tl] : 0.f;
            rbt = p.beta[(size_t)bh * p.L + tl];
        };
        auto decay = [&](int m) {
            const Slot s = slot(m);
            const int valid = min(CK, p.L - m * CK);
            const float la = (l < valid) ? rla : 0.f;
            const float gg = wave_incl_scan(la);
            const float glast = __shfl(gg, CK - 1, kWave);
            if (l < CK) {
                s.gs[l] = gg;
                s.gam[l] = __expf(gg);
                s.dec[l] = __expf(glast - gg);
                s.bet[l] = (l < valid) ? rbt : 0.f;
            }
            if (l == 0) s.misc[0] = __expf(glast);
        };
        // P = Q K^T . Gamma . M_incl (P^T tiles: lane holds P[r][i0..i0+3])
        auto scores = [&](int m) {
            const Slot s = slot(m);
            wave_lds_fence();
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
                for (int ib = 0; ib < NB; ++ib) {
                    const int r = 16 * rb + c16, i0 = 16 * ib + 4 * g4;
                    float x[4] = {0.f, 0.f, 0.f, 0.f};
                    if (ib <= rb) {   // compile-time
                        f32x4 acc = zero4();
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks)
                            mma(acc, ldfrag_swz<E, DK>(s.K, 16 * ib, 32 * ks), ldfrag_swz<E, DK>(s.Q, 16 * rb, 32 * ks));
                        const float gr = s.gs[r];
                        const f32x4 gi = *reinterpret_cast<const f32x4*>(s.gs + i0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float d = GATED ? __expf(fminf(gr - gi[e], 0.f)) : 1.f;
                            x[e] = (r >= i0 + e) ? d * acc[e] : 0.f;
                        }
                    }
                    st4(s.P + r * LTK + i0, x[0], x[1], x[2], x[3]);
                }
            }
        };
        issue(0);
        for (int it = -3; it < p.NC; ++it) {
            const int m = it + 2;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // chunk m has landed
            if (m >= 0 && m < p.NC) decay(m);
            if (m + 1 >= 1 && m + 1 < p.NC) issue(m + 1);
            if (m >= 0 && m < p.NC) scores(m);
            step_barrier();
        }
    } else if (w == 3) {
        // ============================================================ WY wave
        float* Af = reinterpret_cast<float*>(smem + LY::off_A);
        float* Tf = reinterpret_cast<float*>(smem + LY::off_Tf);
        float* Tt = reinterpret_cast<float*>(smem + LY::off_Tt);
        auto wy = [&](int m) {
            const Slot s = slot(m);
            // A = strictly-lower(diag(beta) (K K^T . Gamma))
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
                for (int ib = 0; ib <= rb; ++ib) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        mma(acc, ldfrag_swz<E, DK>(s.K, 16 * rb, 32 * ks), ldfrag_swz<E, DK>(s.K, 16 * ib, 32 * ks));
                    const int i = 16 * ib + c16, r0 = 16 * rb + 4 * g4;
                    const float gi = s.gs[i];
                    const f32x4 gr = *reinterpret_cast<const f32x4*>(s.gs + r0);
                    const f32x4 br = *reinterpret_cast<const f32x4*>(s.bet + r0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float d = GATED ? __expf(fminf(gr[e] - gi, 0.f)) : 1.f;
                        Af[(r0 + e) * LF + i] = (r0 + e > i) ? br[e] * d * acc[e] : 0.f;
                    }
                }
            }
            wave_lds_fence();
            // diagonal 16x16 blocks of (I + A)^{-1}: lane = (block, column).
            // Lanes of one block read the same rows of A (broadcast); row r+1
            // is fetched while row r is being solved.
            {
                const int b = min(g4, NB - 1), j = c16;
                const float* ab = Af + 16 * b * LF + 16 * b;
                float t[16];
                f32x4 cur[4], nxt[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) cur[q] = *reinterpret_cast<const f32x4*>(ab + 4 * q);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (r + 1 < 16) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) nxt[q] = *reinterpret_cast<const f32x4*>(ab + (r + 1) * LF + 4 * q);
                    }
                    float acc[4] = {(r == j) ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < r; ++i) acc[i & 3] -= cur[i >> 2][i & 3] * t[i];
                    t[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
                    if (r + 1 < 16) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
                    }
                }
                if (g4 < NB) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) Tf[(16 * b + r) * LF + 16 * b + j] = t[r];
#pragma unroll
                    for (int r = 0; r < 16; r += 4)
                        *reinterpret_cast<f32x4*>(Tt + (16 * b + j) * LF + 16 * b + r) =
                            f32x4{t[r], t[r + 1], t[r + 2], t[r + 3]};
                }
            }
            wave_lds_fence();
            if constexpr (NB == 2) {
                // T_10 = -T_11 (A_10 T_00):  Y[r][c] = sum_x A_10[r][x] T_00[x][c]
                f32x4 y = zero4();
                mma_k16(y, Af, LF, 16, Tt, LF, 0, 0);       // lane: Y[4g + e][c]
                const f32x4 t11 = *reinterpret_cast<const f32x4*>(Tf + (16 + c16) * LF + 16 + 4 * g4);
                f32x4 z = zero4();                          // Z[r'][c] = sum_r T_11[r'][r] Y[r][c]
#pragma unroll
                for (int e = 0; e < 4; ++e) z = __builtin_amdgcn_mfma_f32_16x16x4f32(t11[e], y[e], z, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) Tf[(16 + 4 * g4 + e) * LF + c16] = -z[e];
                wave_lds_fence();
            }
            // T diag(beta) into the slot, zeros above the diagonal
            constexpr int TV = CK * CK / VE;
#pragma unroll
            for (int x0 = 0; x0 < TV; x0 += 64) {
                const int x = min(x0 + l, TV - 1);
                const int r = x / (CK / VE), c0 = (x % (CK / VE)) * VE;
                float tv[VE], bv[VE], v[VE];
#pragma unroll
                for (int q = 0; q < VE; q += 4) {
                    const f32x4 a = *reinterpret_cast<const f32x4*>(Tf + r * LF + c0 + q);
                    const f32x4 bb = *reinterpret_cast<const f32x4*>(s.bet + c0 + q);
#pragma unroll
                    for (int e = 0; e < 4; ++e) { tv[q + e] = a[e]; bv[q + e] = bb[e]; }
                }
#pragma unroll
                for (int jj = 0; jj < VE; ++jj) v[jj] = (c0 + jj <= r) ? tv[jj] * bv[jj] : 0.f;
                if (x0 + l < TV) st16(s.T + r * LTK + c0, Pack<E>::pack(v));
            }
        };
        for (int it = -3; it < p.NC; ++it) {
            const int m = it + 1;
            if (m >= 0 && m < p.NC) wy(m);
            step_barrier();
        }
    } else {
        // ============================================================ consumers
        f32x4 sT[NKT];   // S^T[16a + 4g + e][v = c16] for this wave's 16 value channels
        const int vw = v0 + 16 * w;
        E* og = reinterpret_cast<E*>(p.o) + (size_t)bh * p.L * p.DV;
#pragma unroll
        for (int a = 0; a < NKT; ++a) {
            sT[a] = zero4();
            if (p.S0)
                sT[a] = *reinterpret_cast<const f32x4*>(
                    p.S0 + ((size_t)bh * p.DV + vw + c16) * DK + 16 * a + 4 * g4);
        }
        auto consume = [&](int m) {
            const Slot s = slot(m);
            const int t0 = m * CK, valid = min(CK, p.L - t0);
            // the entry state as an operand (contraction over d_k)
            Frag<E> sop[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) frag_of_tiles(sop[ks], sT[2 * ks], sT[2 * ks + 1]);
            // X = K S^T and the inter-chunk output O^T = S Q^T
            f32x4 x[NB], oi[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                x[tt] = zero4();
                oi[tt] = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    mma(x[tt], ldfrag_pair_swz<E, DK>(s.K, 16 * tt, 32 * ks), sop[ks]);
                    mma(oi[tt], sop[ks], ldfrag_pair_swz<E, DK>(s.Q, 16 * tt, 32 * ks));
                }
                if (GATED) {
                    const float gq = s.gam[16 * tt + c16];
#pragma unroll
                    for (int e = 0; e < 4; ++e) oi[tt][e] *= gq;
                }
            }
            // R = V - diag(gamma) X   (element: token 16tt + 4g + e, channel c16)
            f32x4 r[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                const f32x4 vv = ld_tr<E, BV>(s.V, 16 * tt, 16 * w);
                const f32x4 gm = GATED ? *reinterpret_cast<const f32x4*>(s.gam + 16 * tt + 4 * g4)
                                       : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int e = 0; e < 4; ++e) r[tt][e] = vv[e] - gm[e] * x[tt][e];
            }
            // U = T R, then O^T += U^T P^T and the state update
            f32x4 u[NB], ud[NB];
            if constexpr (NB == 2) {
                Frag<E> rop;
                frag_of_tiles(rop, r[0], r[1]);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    u[tt] = zero4();
                    mma(u[tt], ldfrag_pair(s.T, LTK, 16 * tt, 0), rop);
                }
                Frag<E> uop;
                frag_of_tiles(uop, u[0], u[1]);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) mma(oi[tt], uop, ldfrag_pair(s.P, LTK, 16 * tt, 0));
            } else {
                Frag16<E> rop;
                frag16_of_tile(rop, r[0]);
                u[0] = zero4();
                mma16(u[0], ldfrag16(s.T, LTK, 0, 0), rop);
                Frag16<E> uop;
                frag16_of_tile(uop, u[0]);
                mma16(oi[0], uop, ldfrag16(s.P, LTK, 0, 0));
            }
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                const int tok = 16 * tt + c16;
                if (tok < valid)
                    st4(og + (size_t)(t0 + tok) * p.DV + vw + 4 * g4, oi[tt][0], oi[tt][1], oi[tt][2], oi[tt][3]);
                const f32x4 dc = GATED ? *reinterpret_cast<const f32x4*>(s.dec + 16 * tt + 4 * g4)
                                       : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int e = 0; e < 4; ++e) ud[tt][e] = u[tt][e] * dc[e];
            }
            // S^T <- gamma_C S^T + K^T (dec . U): K^T read transposed from K
            const float gC = GATED ? s.misc[0] : 1.f;
            if constexpr (NB == 2) {
                Frag<E> udop;
                frag_of_tiles(udop, ud[0], ud[1]);
#pragma unroll
                for (int a = 0; a < NKT; ++a) {
                    Frag<E> kt;
                    if constexpr (sizeof(E) == 2) {
                        s16x4 k0, k1;
                        ld_tr<E, DK>(s.K, 0, 16 * a, &k0);
                        ld_tr<E, DK>(s.K, 16, 16 * a, &k1);
                        const u32x2 a0 = __builtin_bit_cast(u32x2, k0), a1 = __builtin_bit_cast(u32x2, k1);
                        kt.v = __builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y});
                    } else {
                        kt.lo = ld_tr<E, DK>(s.K, 0, 16 * a);
                        kt.hi = ld_tr<E, DK>(s.K, 16, 16 * a);
                    }
                    if (GATED) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) sT[a][e] *= gC;
                    }
                    mma(sT[a], kt, udop);
                }
            } else {
                Frag16<E> udop;
                frag16_of_tile(udop, ud[0]);
#pragma unroll
                for (int a = 0; a < NKT; ++a) {
                    Frag16<E> kt;
                    if constexpr (sizeof(E) == 2) {
                        ld_tr<E, DK>(s.K, 0, 16 * a, &kt.v);
                    } else {
                        kt.v = ld_tr<E, DK>(s.K, 0, 16 * a);
                    }
                    if (GATED) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) sT[a][e] *= gC;
                    }
                    mma16(sT[a], kt, udop);
                }
            }
        };
        for (int it = -3; it < p.NC; ++it) {
            if (it >= 0) consume(it);
            step_barrier();
        }
        if (p.S_final) {
#pragma unroll
            for (int a = 0; a < NKT; ++a)
                *reinterpret_cast<f32x4*>(p.S_final + ((size_t)bh * p.DV + vw + c16) * DK + 16 * a + 4 * g4) = sT[a];
        }
    }
}

// ------------------------------------------------------------------ host side
int pipe_chunk(int C, int dtype, int dk)
{
    if (dtype == kF32 && dk == 128) return 16;
    return C < 32 ? C : 32;
}

template <typename E, int DK, int CK, int MODE>
static hipError_t launch_pipe(const ChunkArgs& a)
{
    using LY = PipeLayout<E, DK, CK>;
    static_assert(LY::bytes <= 160 * 1024, "LDS budget");
    const int BH = a.B * a.H;
    const int NC = (a.L + CK - 1) / CK;
    const int NVB = a.dv / LY::BV;
    PipeParams pp{a.q, a.k, a.v, a.beta, a.log_alpha, a.S0, a.o, a.S_final, a.L, NC, a.dv, NVB,
                  BH * NVB};
    auto* kern = chunk_pipe_kernel<E, DK, CK, MODE>;
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LY::bytes);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(BH * NVB), dim3(256), LY::bytes, a.stream, pp);
    return hipGetLastError();
}

template <typename E, int DK>
static hipError_t pipe_by_chunk_mode(const ChunkArgs& a)
{
    const int ck = pipe_chunk(a.C, a.dtype, a.dk);
    if constexpr (sizeof(E) == 4 && DK == 128) {
        return a.mode == kAlphaNone ? launch_pipe<E, DK, 16, kAlphaNone>(a)
                                    : launch_pipe<E, DK, 16, kAlphaScalar>(a);
    } else {
        if (ck == 16)
            return a.mode == kAlphaNone ? launch_pipe<E, DK, 16, kAlphaNone>(a)
                                        : launch_pipe<E, DK, 16, kAlphaScalar>(a);
        return a.mode == kAlphaNone ? launch_pipe<E, DK, 32, kAlphaNone>(a)
                                    : launch_pipe<E, DK, 32, kAlphaScalar>(a);
    }
}

hipError_t launch_pipe_chunked(const ChunkArgs& a)
{
    if (a.dtype == kBF16) return a.dk == 128 ? pipe_by_chunk_mode<bf16, 128>(a) : pipe_by_chunk_mode<bf16, 64>(a);
    return a.dk == 128 ? pipe_by_chunk_mode<float, 128>(a) : pipe_by_chunk_mode<float, 64>(a);
}

}  // namespace gdr

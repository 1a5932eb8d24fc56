// gdr_bwd_chain.hip -- the backward's sequential part for bf16 operands and
// 32-token steps: dS carried backwards over the chunks of a head, on the
// chunk-pipelined layout of the forward scan (gdr_scan.hip).
//
// Per chunk, walking from the last to the first (notation of gdr_bwd.hip;
// gamma = e^g, D = e^{g_C - g}, P = Q K^T . Gamma . M_incl):
//   Y = K dS^T,  dU = P^T dO + diag(D) Y,  dR = T~^T dU,
//   dS <- gamma_C dS + Q^T diag(gamma) dO - K^T diag(gamma) dR.
// Channel alpha (the records' decayed operands and score block P):
//   Y = (K . e^{G_C - G}) dS^T,  dU = P^T dO + Y,  dR = T~^T dU,
//   dS <- dS Diag(e^{G_C}) + (Q . e^G)^T dO - (K . e^G)^T dR.
// ("linear attention and its gated descendants", "Chunkwise Parallel Form",
// "Gated DeltaNet" and "Kimi Delta Attention"; reverse mode of the chunk
// algebra by the chain rule.)
//
// This is the forward scan's step (X = K S^T, R = V - gamma X, U = T~ R,
// S <- gamma_C S + K^T D U) with T~^T in place of T~ and one more product,
// Q^T diag(gamma) dO, that does not depend on dS.  So the roles are the
// scan's:
//   waves 0, 1 (owners)  each holds dS of 16 value channels (d_k x 16 fp32)
//                        in registers, publishes it at every chunk's end and
//                        does the products above; the dS-free product is
//                        issued while Y is in flight;
//   waves 2, 3 (pre)     one chunk ahead of the owners: P^T dO for their 16
//                        value channels (scalar alpha: P from Q K^T and the
//                        record's Gamma; channel: the record's P), handed to
//                        the owners through LDS;
//   waves 4, 5 (copiers) direct global->LDS copies of the chunk three steps
//                        ahead;
//   wave 6 (storer)      the store of the dS the owners published a step
//                        before (the gradient kernel reads it).
// T~^T, P^T (channel), Gamma^T, Q^T, K^T and dO^T come from transposing LDS
// reads (ds_read_b64_tr_b16), so nothing is transposed on its way in.  The
// compiler makes a transposing read wait for every outstanding global memory
// operation of its wave, so the waves that use them issue no global stores:
// the dS stores have a wave of their own.
#include "gdr_device.h"
#include "gdr_chunk.h"
#include "gdr_pipe.h"
#include "gdr_bwd.h"

namespace gdr {

namespace {

// Slots and exchange buffers: the forward scan's regions (K or K.exp(G),
// channel K.exp(G_C - G), Q or Q.exp(G), the dO block in the V region, T~,
// Gamma or P, the decay factors), then dS operands [parity][owner][ks][lane]
// and P^T dO [parity][owner][tt][lane] (fp32 tiles).
template <int DK, int MODE>
struct ChainPipeLayout {
    using LY = ScanLayout<bf16, DK, 32, MODE>;
    static constexpr int rxS = LY::rxS, XSB = LY::XSB;
    static constexpr int rxV = rxS + 2 * XSB;
    static constexpr int XVB = 2 * 2 * kWave * 16;
    static constexpr int bytes = rxV + 2 * XVB;
};

// A 16x16x32 operand from two transposing reads 16 rows apart (rows 4g + q
// and 16 + 4g + q of the addressed block).
template <int N0, int N1>
__device__ __forceinline__ Frag<bf16> tr_pair(const unsigned char* base, int off) {
    const u32x2 a0 = __builtin_bit_cast(u32x2, ld_tr16<N0>(base, off));
    const u32x2 a1 = __builtin_bit_cast(u32x2, ld_tr16<N1>(base, off));
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y});
    return f;
}

template <int DK, int MODE>
__global__ __launch_bounds__(64 * 7) void chunk_bwd_chain_pipe_kernel(BwdParams p)
{
    using E = bf16;
    constexpr int CK = 32;
    using CL = ChainPipeLayout<DK, MODE>;
    using LY = typename CL::LY;
    using SK = Swz<E, DK>;
    using SV = Swz<E, LY::BV>;
    using ST = Swz<E, CK>;
    constexpr int ES = 2, BV = LY::BV, NSLOT = LY::NSLOT;
    constexpr int NB = 2, NKT = DK / 16, NKS = DK / 32;
    constexpr bool CH = LY::CH;
    constexpr int szK = LY::szK, szV = LY::szV, szT = LY::szT, szF = LY::szF, FS = LY::FS;
    constexpr int RBK = SK::RB, RBV = SV::RB, RBT = ST::RB;
    constexpr int XSB = CL::XSB, XVB = CL::XVB;
    constexpr WsLayout WL = ws_layout(ES, DK, CK, MODE);
    static_assert(NSLOT == 4, "slot ring");
    constexpr int LEADC = NSLOT - 2;   // the copier fills step u + LEADC in iteration u
    extern __shared__ __align__(16) unsigned char smem[];

    // Role index w: 0, 1 owners, 2, 3 pre, 4, 5 copiers, 6 storer; wave i runs
    // on SIMD i % 4, so waves 2, 3 take the owners (a SIMD each).
    const int hw = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int w = hw < 2 ? hw + 2 : (hw < 4 ? hw - 2 : hw);
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15;
    // consecutive block ids land on different XCDs: the value blocks of one
    // head get neighbouring logical ids on one XCD so they share its L2
    int lid = blockIdx.x;
    if (gridDim.x % 8 == 0) lid = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
    const int NVB = p.DV / BV;
    const int bh = lid / NVB, v0 = (lid % NVB) * BV;
    const int NC = p.NC, L = p.L;
    const size_t tok0 = (size_t)bh * L, rec0 = (size_t)bh * NC;

    // K / Q operand rows: row c16 (+16 tt), key channels 32 ks + 8 g4 .. + 7
    int oKQ[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) oKQ[ks] = SK::off(c16, 32 * ks + 8 * g4);
    // transposing reads of a [CK][CK] block: address lane (g, 4q + m) names
    // row 4g + q, memory columns 8m .. 8m + 3 (tokens 4m ..; + 8 bytes for
    // tokens 16 + 4m ..); lane (g, c) then holds rows 4g + q of token column c
    const int oTr = ST::off(4 * g4 + (c16 >> 2), 8 * (c16 & 3));

    if (w < 2) {
        // ========================================================= owners
        const int vw = v0 + 16 * w;
        int oKX[NKS], oKt[NKT], oQt[NKT];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) oKX[ks] = lane_base((CH ? LY::rKU : LY::rK) + oKQ[ks]);
        // transposing reads of K^T / Q^T tile a: address lane (g, i) names
        // token 4g + i/4 (+16), key channels 32ks + 4pa + 8(i%4) .. +3
#pragma unroll
        for (int a = 0; a < NKT; ++a) {
            const int o = SK::off(4 * g4 + (c16 >> 2), 32 * (a >> 1) + 4 * (a & 1) + 8 * (c16 & 3));
            oKt[a] = lane_base(LY::rK + o);
            oQt[a] = lane_base(LY::rQ + o);
        }
        // dO block, transposed: token 4g + i/4 (+16 tt), channels 16w + 4(i%4)
        const int oVt = lane_base(LY::rV + SV::off(4 * g4 + (c16 >> 2), 16 * w + 4 * (c16 & 3)));
        const int oTt = lane_base(LY::rT + oTr);
        const int oXS = lane_base(CL::rxS + (w * NKS * kWave + l) * FS);
        const int oXV = lane_base(CL::rxV + (w * NB * kWave + l) * 16);
        const int oFg = lane_base(LY::rF + 16 * g4);
        const int oF0 = lane_base(LY::rF);

        f32x4 sT[NKT];   // dS^T[key 32ks + 8g + 4p + e][v = vw + c16], a = 2ks + p
        if (p.dS_final) {
            const float* s0 = p.dS_final + ((size_t)bh * p.DV + vw + c16) * DK + 8 * g4;
#pragma unroll
            for (int a = 0; a < NKT; ++a) sT[a] = *reinterpret_cast<const f32x4*>(s0 + 32 * (a >> 1) + 4 * (a & 1));
        } else {
#pragma unroll
            for (int a = 0; a < NKT; ++a) sT[a] = zero4();
        }

        // step s: chunk NC - 1 - s, from slot J = s % NSLOT
        auto own = [&](auto jc, int s) {
            constexpr int J = decltype(jc)::value;
            constexpr int cK = J * szK;   // slot offset within each K / Q region
            constexpr int cV = J * szV, cT = J * szT, cF = J * szF;
            constexpr int pS = (J & 1) * XSB, pV = (J & 1) * XVB;   // s & 1 == J & 1
            const int n = NC - 1 - s, valid = min(CK, L - n * CK);
            // ---- rows for Y; dS as an operand, published for the store
            Frag<E> kx[NB][NKS];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) kx[tt][ks] = ld_frag<E, 0>(smem + cK + 16 * tt * RBK, oKX[ks], oKX[ks]);
            Frag<E> sop[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                frag_of_tiles(sop[ks], sT[2 * ks], sT[2 * ks + 1]);
                *reinterpret_cast<Frag<E>*>(smem + oXS + pS + ks * kWave * FS) = sop[ks];
            }
            // ---- Y = K dS^T (lane: token 16tt + 4g + e, value channel c16)
            f32x4 y[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                y[tt] = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) mma(y[tt], kx[tt][ks], sop[ks]);
            }
            sched_fence();
            // ---- the dS-free product, issued while Y is in flight:
            // dS^T <- decay . dS^T + Q^T (gamma . dO)
            Frag<E> qt[NKT];
#pragma unroll
            for (int a = 0; a < NKT; ++a) qt[a] = tr_pair<0, 16 * RBK>(smem + cK, oQt[a]);
            f32x4 gm[NB], dc[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                gm[tt] = CH ? f32x4{1.f, 1.f, 1.f, 1.f} : ldf4<0>(smem + cF + 64 * tt, oFg);
                dc[tt] = CH ? f32x4{1.f, 1.f, 1.f, 1.f} : ldf4<0>(smem + cF + 4 * CK + 64 * tt, oFg);
            }
            f32x4 gd[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                const f32x4 d = unpack4(ld_tr16<0>(smem + cV + 16 * tt * RBV, oVt));
#pragma unroll
                for (int e = 0; e < 4; ++e) gd[tt][e] = (16 * tt + 4 * g4 + e < valid) ? gm[tt][e] * d[e] : 0.f;
            }
            if constexpr (CH) {
#pragma unroll
                for (int a = 0; a < NKT; ++a) {
                    const f32x4 dk = ldf4<0>(smem + cF + 4 * (32 * (a >> 1) + 4 * (a & 1)), oF0 + 32 * g4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) sT[a][e] *= dk[e];
                }
            } else {
                const float gC = ldf<8 * CK>(smem + cF, oF0);
#pragma unroll
                for (int a = 0; a < NKT; ++a)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sT[a][e] *= gC;
            }
            Frag<E> gdo;
            frag_of_tiles(gdo, gd[0], gd[1]);
#pragma unroll
            for (int a = 0; a < NKT; ++a) mma(sT[a], qt[a], gdo);
            sched_fence();
            // ---- dU = P^T dO + diag(D) Y, dR = T~^T dU
            Frag<E> tq[NB];
            tq[0] = tr_pair<0, 16 * RBT>(smem + cT, oTt);
            tq[1] = tr_pair<8, 16 * RBT + 8>(smem + cT, oTt);
            f32x4 du[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                const f32x4 vp = *reinterpret_cast<const f32x4*>(smem + oXV + pV + tt * kWave * 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) du[tt][e] = vp[e] + dc[tt][e] * y[tt][e];
            }
            Frag<E> duop;
            frag_of_tiles(duop, du[0], du[1]);
            f32x4 dr[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                dr[tt] = zero4();
                mma(dr[tt], tq[tt], duop);
            }
            Frag<E> kt[NKT];
#pragma unroll
            for (int a = 0; a < NKT; ++a) kt[a] = tr_pair<0, 16 * RBK>(smem + cK, oKt[a]);
            // ---- dS^T += K^T (-gamma . dR)  (rows of dR past the chunk's end are
            // zero: so are those columns of T~)
#pragma unroll
            for (int tt = 0; tt < NB; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) dr[tt][e] *= -gm[tt][e];
            Frag<E> drop;
            frag_of_tiles(drop, dr[0], dr[1]);
#pragma unroll
            for (int a = 0; a < NKT; ++a) mma(sT[a], kt[a], drop);
        };
        step_barrier();
        // iteration u: step u - 1 (the pre waves prepared step u - 1 in iteration u - 1)
        for (int u0 = 0; u0 <= NC; u0 += NSLOT) {
            auto step = [&](auto jc) {
                constexpr int J = decltype(jc)::value;
                const int u = u0 + J;
                if (u <= NC) {
                    if (u >= 1) own(std::integral_constant<int, (J + NSLOT - 1) % NSLOT>{}, u - 1);
                    step_barrier();
                }
            };
            StaticFor<0, NSLOT>::run(step);
        }
        if (p.dS0) {
            float* d0 = p.dS0 + ((size_t)bh * p.DV + vw + c16) * DK + 8 * g4;
#pragma unroll
            for (int a = 0; a < NKT; ++a) *reinterpret_cast<f32x4*>(d0 + 32 * (a >> 1) + 4 * (a & 1)) = sT[a];
        }
    } else if (w < 4) {
        // ========================================================= pre waves
        const int c = w - 2, vw = v0 + 16 * c;
        const int oXV = lane_base(CL::rxV + (c * NB * kWave + l) * 16);
        const int oVt = lane_base(LY::rV + SV::off(4 * g4 + (c16 >> 2), 16 * c + 4 * (c16 & 3)));
        const int oMt = lane_base(LY::rM + oTr);
        int oQ[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) oQ[ks] = lane_base(LY::rQ + oKQ[ks]);

        // P^T dO of step j (slot J) for value channels 16c .., into parity J & 1:
        // lane holds (P^T dO)[16tt + 4g + e][16c + c16]
        auto pre = [&](auto jc, int j) {
            constexpr int J = decltype(jc)::value;
            constexpr int cK = J * szK, cM = J * szT, cV = J * szV, pV = (J & 1) * XVB;
            const int n = NC - 1 - j, valid = min(CK, L - n * CK);
            // P^T rows 16tt + c16 over tokens (4g + q | 16 + 4g + q)
            Frag<E> pt[NB];
            if constexpr (CH) {
                pt[0] = tr_pair<0, 16 * RBT>(smem + cM, oMt);
                pt[1] = tr_pair<8, 16 * RBT + 8>(smem + cM, oMt);
            } else {
                Frag<E> qf[NB][NKS], kf[NB][NKS];
#pragma unroll
                for (int pp = 0; pp < NB; ++pp)
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        qf[pp][ks] = ld_frag<E, 0>(smem + cK + 16 * pp * RBK, oQ[ks], oQ[ks]);
                        kf[pp][ks] = ld_frag<E, 0>(smem + LY::rK + cK + 16 * pp * RBK, oKQ[ks], oKQ[ks]);
                    }
                // Gamma[16pp + 4g + q][16tt + c16], q = 0..3 (zero above the diagonal)
                const f32x4 g00 = unpack4(ld_tr16<0>(smem + cM, oMt));
                const f32x4 g10 = unpack4(ld_tr16<16 * RBT>(smem + cM, oMt));
                const f32x4 g11 = unpack4(ld_tr16<16 * RBT + 8>(smem + cM, oMt));
                sched_fence();
                // (Q K^T)[16pp + 4g + e][16tt + c16] . Gamma
                auto tile = [&](int pp, int tt, f32x4 gmv) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) mma(acc, qf[pp][ks], kf[tt][ks]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] *= gmv[e];
                    return acc;
                };
                frag_of_tiles(pt[0], tile(0, 0, g00), tile(1, 0, g10));
                frag_of_tiles(pt[1], zero4(), tile(1, 1, g11));
            }
            // dO of value channel 16c + c16 at tokens 4g + q and 16 + 4g + q
            // (zero past the chunk's end)
            f32x4 d0 = unpack4(ld_tr16<0>(smem + cV, oVt));
            f32x4 d1 = unpack4(ld_tr16<16 * RBV>(smem + cV, oVt));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d0[e] = (4 * g4 + e < valid) ? d0[e] : 0.f;
                d1[e] = (16 + 4 * g4 + e < valid) ? d1[e] : 0.f;
            }
            Frag<E> dof;
            frag_of_tiles(dof, d0, d1);
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                f32x4 v = zero4();
                mma(v, pt[tt], dof);
                *reinterpret_cast<f32x4*>(smem + oXV + pV + tt * kWave * 16) = v;
            }
        };
        step_barrier();
        // iteration u: P^T dO of step u
        for (int u0 = 0; u0 <= NC; u0 += NSLOT) {
            auto step = [&](auto jc) {
                constexpr int J = decltype(jc)::value;
                const int u = u0 + J;
                if (u <= NC) {
                    if (u < NC) pre(jc, u);
                    step_barrier();
                }
            };
            StaticFor<0, NSLOT>::run(step);
        }
    } else if (w == 6) {
        // ========================================================= storer
        // the dS the owners published at step s (chunk NC - 1 - s), parity PC:
        // value rows v0 .. v0 + 31 are one contiguous run of the [d_v][d_k]
        // block, so each store writes 1 KiB of it, gathered from the owners'
        // fragments
        auto store_dS = [&](auto pc, int s) {
            constexpr int PS = decltype(pc)::value * XSB;
            constexpr int NI = 32 * DK * (int)sizeof(E) / 1024;
            const int n = NC - 1 - s;
            unsigned char* ck = static_cast<unsigned char*>(p.dSck) +
                                (((size_t)bh * NC + n) * p.DV + v0) * DK * sizeof(E) + 16 * l;
            u32x4 x[NI];
#pragma unroll
            for (int j = 0; j < NI; ++j) x[j] = *reinterpret_cast<const u32x4*>(smem + CL::rxS + PS + xs_piece<E, DK>(64 * j + l));
#pragma unroll
            for (int j = 0; j < NI; ++j) st16(ck + 1024 * j, x[j]);
        };
        step_barrier();
        // iteration u: the store of step u - 2's dS
        for (int u0 = 0; u0 <= NC; u0 += NSLOT) {
            auto step = [&](auto jc) {
                constexpr int J = decltype(jc)::value;
                const int u = u0 + J;
                if (u <= NC) {
                    if (u >= 2) store_dS(std::integral_constant<int, J & 1>{}, u - 2);
                    step_barrier();
                }
            };
            StaticFor<0, NSLOT>::run(step);
        }
        // the last published dS (step NC - 1: the first chunk's end)
        if ((NC - 1) & 1) store_dS(std::integral_constant<int, 1>{}, NC - 1);
        else store_dS(std::integral_constant<int, 0>{}, NC - 1);
    } else {
        // ========================================================= copiers
        // As the forward scan's copiers (instruction j, lane l fills LDS bytes
        // 1024 j + 16 l of a region; the source offsets apply the swizzle),
        // with the dO block in the V region.  Step j's chunk is NC - 1 - j.
        auto tile_off = [&](auto sw, int j, int gstride, int valid) {
            using S = decltype(sw);
            const int b = 1024 * j + 16 * l;
            const int row = b / S::RB, pch = (b % S::RB) / 16;
            return (uint32_t)(min(row, valid - 1) * gstride + ((pch ^ S::swz(row)) << 4));
        };
        uint32_t offK[LY::NCK], offV[LY::NCV], offT[LY::NCT];
#pragma unroll
        for (int j = 0; j < LY::NCK; ++j) offK[j] = tile_off(SK{}, j, DK * ES, CK);
#pragma unroll
        for (int j = 0; j < LY::NCV; ++j) offV[j] = tile_off(SV{}, j, p.DV * ES, CK);
#pragma unroll
        for (int j = 0; j < LY::NCT; ++j) offT[j] = tile_off(ST{}, j, CK * ES, CK);

        const int cw = w - 4;
        const unsigned char* kb = static_cast<const unsigned char*>(p.k);
        const unsigned char* qb = static_cast<const unsigned char*>(p.q);
        const unsigned char* db = static_cast<const unsigned char*>(p.dO);
        const uint32_t sbase = (uint32_t)(uintptr_t)(lds_void_t*)smem;
        auto copy = [&](int dst, const unsigned char* src, const uint32_t* off, auto ni, int total) {
            constexpr int NI = decltype(ni)::value;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if (total % 1024 == 0 || 1024 * j + 16 * l < total)
                    __builtin_amdgcn_global_load_lds((const glb_void_t*)(src + off[j]),
                                                     (lds_void_t*)(uintptr_t)(sbase + (uint32_t)(dst + 1024 * j)), 16, 0, 0);
            }
        };
        auto issue = [&](auto jc, int j) {
            constexpr int J = decltype(jc)::value;
            const int n = NC - 1 - j, t0 = n * CK, valid = min(CK, L - t0);
            const unsigned char* rec = p.ws + (rec0 + n) * WL.bytes;
            const size_t row0 = tok0 + t0;
            using NK = std::integral_constant<int, LY::NCK>;
            using NV = std::integral_constant<int, LY::NCV>;
            using NT = std::integral_constant<int, LY::NCT>;
            const bool vt = (cw == (CH ? 1 : 0));   // copier of the dO block and T~
            if constexpr (CH) {
                if (cw == 0) {
                    copy(LY::rK + J * szK, rec + WL.KG, offK, NK{}, szK);
                    copy(LY::rKU + J * szK, rec + WL.KD, offK, NK{}, szK);
                } else {
                    copy(LY::rQ + J * szK, rec + WL.QG, offK, NK{}, szK);
                }
            }
            if (valid == CK) {
                if constexpr (!CH) {
                    if (cw == 0) copy(LY::rK + J * szK, kb + row0 * DK * ES, offK, NK{}, szK);
                    else copy(LY::rQ + J * szK, qb + row0 * DK * ES, offK, NK{}, szK);
                }
                if (vt) copy(LY::rV + J * szV, db + (row0 * p.DV + v0) * ES, offV, NV{}, szV);
            } else {
                // the last, partial chunk: rows past the end repeat the last row
                // (the readers zero their dO and the records' columns do the rest)
                uint32_t rK[LY::NCK], rV[LY::NCV];
#pragma unroll
                for (int jj = 0; jj < LY::NCK; ++jj) rK[jj] = tile_off(SK{}, jj, DK * ES, valid);
#pragma unroll
                for (int jj = 0; jj < LY::NCV; ++jj) rV[jj] = tile_off(SV{}, jj, p.DV * ES, valid);
                if constexpr (!CH) {
                    if (cw == 0) copy(LY::rK + J * szK, kb + row0 * DK * ES, rK, NK{}, szK);
                    else copy(LY::rQ + J * szK, qb + row0 * DK * ES, rK, NK{}, szK);
                }
                if (vt) copy(LY::rV + J * szV, db + (row0 * p.DV + v0) * ES, rV, NV{}, szV);
            }
            if (vt) copy(LY::rT + J * szT, rec + WL.T, offT, NT{}, szT);
            if (cw == 1) copy(LY::rM + J * szT, rec + WL.M, offT, NT{}, szT);
            if (cw == 0) {
#pragma unroll
                for (int jj = 0; jj < LY::NCF; ++jj) {
                    if (LY::FB % 1024 == 0 || 1024 * jj + 16 * l < LY::FB)
                        __builtin_amdgcn_global_load_lds((const glb_void_t*)(rec + WL.F + 1024 * jj + 16 * l),
                                                         (lds_void_t*)(uintptr_t)(sbase + (uint32_t)(LY::rF + J * szF + 1024 * jj)),
                                                         16, 0, 0);
                }
            }
        };
        // wait until at most k chunks' copies of this copier are in flight
        static_assert((NSLOT - 3) * LY::NOPS0 < 64 && (NSLOT - 3) * LY::NOPS1 < 64, "vmcnt range");
        auto wait_k = [&](int k) {
            auto one = [&](auto kc) {
                constexpr int K = decltype(kc)::value;
                if (k == K) {
                    if (cw == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K * LY::NOPS0) : "memory");
                    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K * LY::NOPS1) : "memory");
                }
            };
            StaticFor<0, NSLOT - 2>::run(one);
        };
        // prologue: steps 0 .. LEADC - 1, then wait for step 0
        auto pro = [&](auto kc) {
            constexpr int K = decltype(kc)::value;
            if (K < NC) issue(kc, K);
        };
        StaticFor<0, LEADC>::run(pro);
        wait_k(min(LEADC - 1, NC - 1));
        step_barrier();
        // iteration u: fill step u + LEADC into slot (u + LEADC) % NSLOT, then
        // wait for step u + 1
        for (int u0 = 0; u0 <= NC; u0 += NSLOT) {
            auto step = [&](auto jc) {
                constexpr int J = decltype(jc)::value;
                const int u = u0 + J;
                if (u <= NC) {
                    if (u + LEADC < NC) issue(std::integral_constant<int, (J + LEADC) % NSLOT>{}, u + LEADC);
                    wait_k(max(0, min(LEADC - 1, NC - 2 - u)));
                    step_barrier();
                }
            };
            StaticFor<0, NSLOT>::run(step);
        }
    }
}

template <int DK, int MODE>
hipError_t launch_t(const BwdParams& bp, int BH, hipStream_t stream)
{
    using CL = ChainPipeLayout<DK, MODE>;
    static_assert(CL::bytes <= 160 * 1024, "LDS budget");
    auto* kern = chunk_bwd_chain_pipe_kernel<DK, MODE>;
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, CL::bytes);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(BH * (bp.DV / 32)), dim3(64 * 7), CL::bytes, stream, bp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_chain_pipe(const BwdParams& bp, int BH, int dk, bool channel, hipStream_t stream)
{
    if (dk == 128) return channel ? launch_t<128, kAlphaChannel>(bp, BH, stream) : launch_t<128, kAlphaScalar>(bp, BH, stream);
    return channel ? launch_t<64, kAlphaChannel>(bp, BH, stream) : launch_t<64, kAlphaScalar>(bp, BH, stream);
}

}  // namespace gdr

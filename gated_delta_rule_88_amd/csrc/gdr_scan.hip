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
// When the library normalises q and k itself (gdr_fwd_chunked_ex), K and Q
// reach this kernel raw: the prepass has folded 1 / ||k_t|| into gamma and
// exp(g_C - g) (and into K . exp(G) etc. per channel) and 1 / ||q_t|| into a
// second copy of gamma and into Gamma, so the scan's arithmetic is unchanged.
//
// Rows of S (value channels) evolve independently given K, beta and alpha,
// which is what lets the value dimension be split across workgroups and
// waves.  Six waves, one barrier per chunk step, four rotating LDS slots:
//   waves 0, 1  (state owners)  each holds the state of 16 value channels
//               (d_k x 16 fp32) in registers; for chunk n it publishes S as
//               an MFMA operand, forms X, R, U (published too) and the next
//               state.  Only this chain is sequential.
//   waves 2, 3  (output waves)  for chunk n - 1, from the published S and U:
//               the inter-chunk output diag(gamma) Q S^T, the masked score
//               block P (MFMA), P U, and the store of o.
//   waves 4 ..  (copiers)       direct global->LDS copies of chunk n + 2 (K,
//               Q, the V block, T~, Gamma or P, the decay factors; two
//               copiers split the regions, four for bf16 channel alpha), 16
//               bytes per lane, then wait until chunk n + 1 has landed.
// Every product is v_mfma_f32_16x16x32_bf16 (fp32: 16x16x4f32) in NT form;
// result tiles feed the next product straight from registers (tile-pair
// operands, gdr_device.h).
//
// Layout choices that keep the per-step instruction count low:
//  - d_k order inside the state.  Element e of state tile a = 2ks + p held by
//    lane group g is key channel 32ks + 8g + 4p + e, so the eight key
//    channels a lane group contracts over are contiguous in K and Q: every
//    K or Q operand is one 16-byte LDS read.  K^T comes from transposing LDS
//    reads whose per-lane addresses follow the same order.
//  - LDS is region-major ([K: 4 slots][Q: 4 slots][V]...) and the step loop
//    is unrolled over the four slots, so slot and tile offsets are
//    instruction immediates; per-lane addresses are computed once.
//  - K and Q rows are XOR-swizzled by (r & 15) ^ ((r & 2) << 2) on 16-byte
//    chunks, which keeps both the 16-byte fragment reads and the
//    transposing reads at the LDS's conflict-free rate; the copier applies
//    the permutation by its choice of source addresses.
#include "gdr_device.h"
#include "gdr_chunk.h"
#include "gdr_pipe.h"

namespace gdr {

// AH: chunks the copiers run ahead of the state owners (the slot ring holds
// AH + 2 chunks).
template <typename E, int DK, int CK, int MODE, int AH>
__global__ __launch_bounds__(64 * 8) void chunk_scan_kernel(ScanParams p)
{
    using LY = ScanLayout<E, DK, CK, MODE, AH>;
    using SK = Swz<E, DK>;
    using SV = Swz<E, LY::BV>;
    using ST = Swz<E, CK>;
    constexpr int ES = LY::ES, BV = LY::BV, NSLOT = LY::NSLOT, AHEAD = LY::AHEAD;
    constexpr int NB = CK / 16, NKT = DK / 16, NKS = DK / 32;
    constexpr bool GATED = (MODE == kAlphaScalar), CH = LY::CH;
    constexpr int szK = LY::szK, szV = LY::szV, szT = LY::szT, szF = LY::szF, FS = LY::FS;
    constexpr int RBK = SK::RB, RBV = SV::RB, RBT = ST::RB;
    constexpr WsLayout WL = ws_layout(ES, DK, CK, MODE);
    static_assert(sizeof(E) == 2 || CK == 16, "fp32 operands run 16-token steps");
    extern __shared__ __align__(16) unsigned char smem[];

    // wave index as a scalar: the role branches below are wave-uniform
    // Role index w: 0, 1 state owners, 2, 3 output waves, 4 .. copiers.  The
    // hardware places wave i of a workgroup on SIMD i % 4, so waves 2, 3 run
    // the owners (a SIMD each) and copiers 4, 5 share SIMDs 0, 1 with the
    // output waves (copiers 6, 7, when there are four, share the owners'
    // SIMDs: they issue copies and wait, little else).
    const int hw = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int w = hw < 2 ? hw + 2 : (hw < 4 ? hw - 2 : hw);
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15;
    int lid = blockIdx.x;
    // consecutive block ids land on different XCDs: give the value blocks of
    // one head neighbouring logical ids on one XCD so they share its L2
    if (p.total % 8 == 0) lid = (blockIdx.x % 8) * (p.total / 8) + blockIdx.x / 8;
    // This workgroup's job.  Segment 0 (the whole sequence unless the scan is
    // split into p.SEG segments) runs value blocks from the true initial
    // state.  Every later segment runs its value blocks from a zero state and,
    // as further rows of the same recurrence, d_k key rows started from the
    // identity: those rows give the segment's transition matrix and
    // (transition so far) q_t, from which the segment's true result follows
    // once its entry state is known.
    int bh, vb, sg = 0;
    bool keyrows = false;
    if (p.vl.start) {
        // packed variable-length batch: chain bh = n * H + h, one segment
        bh = lid / p.NVB;
        vb = lid % p.NVB;
    } else {
        const int per_seg = p.NVB + p.NMB;
        const int later = (p.SEG - 1) * per_seg;        // later-segment workgroups per chain
        const int units = p.NVB + later;
        const int nbh = p.total / units;
        int u;
        if (p.SEG > 1 && nbh % 8 == 0) {
            // eight groups of chains, one per XCD (the order above); in each
            // group every segment-0 workgroup comes first, so that when the
            // plan holds more workgroups than the CUs run at once, the ones
            // that wait for a free CU belong to the (shorter) later segments
            const int cpg = nbh / 8, r = lid % (cpg * units);
            bh = (lid / (cpg * units)) * cpg;
            if (r < cpg * p.NVB) {
                bh += r / p.NVB;
                u = r % p.NVB;
            } else {
                bh += (r - cpg * p.NVB) / later;
                u = p.NVB + (r - cpg * p.NVB) % later;
            }
        } else {
            bh = lid / units;
            u = lid % units;
        }
        if (u < p.NVB) {
            vb = u;
        } else {
            u -= p.NVB;
            sg = 1 + u / per_seg;
            const int r = u % per_seg;
            keyrows = r >= p.NVB;
            vb = keyrows ? r - p.NVB : r;
        }
    }
    const int v0 = vb * BV;                            // first value channel (key row for key rows)
    const int c0 = sg == 0 ? 0 : p.N0 + (sg - 1) * p.NCS;   // first chunk
    // the chain's tokens: head row start on the token axis, length, first record
    size_t tok0 = (size_t)bh * p.L, rec0 = (size_t)bh * p.NC;
    int len = p.L;
    int NC = min(sg == 0 ? p.N0 : p.NCS, p.NC - c0);   // chunks this workgroup walks
    // a recomputation that keeps only every sck_every-th entry state and forms
    // no outputs stops at the last chunk of the head whose entry state it keeps
    if (p.Sck && p.sck_every > 1 && !p.o && !p.S_final && p.SEG == 1 && !p.vl.start)
        NC = max(1, NC - (int)((rec0 + NC - 1) % p.sck_every));
    if (p.vl.start) {
        const int n = bh / p.H, h = bh % p.H;
        const int cb = p.vl.choff[n];
        tok0 = (size_t)h * p.L + p.vl.start[n];
        len = p.vl.len[n];
        rec0 = (size_t)h * p.vl.NCmax + cb;
        NC = min((len + CK - 1) / CK, max(0, p.vl.NCmax - cb));
        if (NC == 0) {
            // an empty sequence: its final state is its initial state
            if (w < 2 && p.S_final) {
                const size_t r = ((size_t)bh * p.DV + v0 + 16 * w + c16) * DK;
                for (int c = 4 * g4; c < DK; c += 16)
                    *reinterpret_cast<f32x4*>(p.S_final + r + c) =
                        p.S0 ? *reinterpret_cast<const f32x4*>(p.S0 + r + c) : zero4();
            }
            return;   // workgroup-uniform, before any barrier
        }
    }
    if (keyrows) {
        // key rows carry no values: the V slots stay zero
        for (int i = threadIdx.x; i < NSLOT * szV / 16; i += 64 * LY::NWAVES)
            *reinterpret_cast<u32x4*>(smem + LY::rV + 16 * i) = u32x4{0u, 0u, 0u, 0u};
    }

    // per-lane LDS offsets shared by the readers
    // K / Q operand: row c16 (+16 tt), key channels 32 ks + 8 g4 .. +7
    int oKQ[NKS], oKQh[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        oKQ[ks] = SK::off(c16, 32 * ks + 8 * g4);
        oKQh[ks] = sizeof(E) == 4 ? SK::off(c16, 32 * ks + 8 * g4 + 4) : 0;
    }
    // T~ (and channel P) operand: row c16 (+16 tt), memory columns 8 g4 ..
    // (CK = 16: 4 g4 ..)
    const int oT = ST::off(c16, (CK == 32 ? 8 : 4) * g4);

    if (w < 2) {
        // ===================================================== state owners
        const int vw = v0 + 16 * w;
        // transposing reads of K' (per dk tile a): address lane (g, i) names
        // token 4g + i/4 (+16 p), key channels 32ks + 4pa + 8(i%4) .. +3
        int oKt[NKT];
#pragma unroll
        for (int a = 0; a < NKT; ++a)
            oKt[a] = SK::off(4 * g4 + (c16 >> 2), 32 * (a >> 1) + 4 * (a & 1) + 8 * (c16 & 3));
        // V block, transposed: token 4g + i/4 (+16 tt), channels 16w + 4(i%4)
        const int oVt = lane_base(LY::rV + SV::off(4 * g4 + (c16 >> 2), 16 * w + 4 * (c16 & 3)));
        const int oXS = lane_base(LY::rxS + (w * NKS * kWave + l) * FS);   // + parity XSB + ks 64 FS
        const int oXU = lane_base(LY::rxU + (w * kWave + l) * FS);         // + parity XUB
        const int oTo = lane_base(LY::rT + oT);
        const int oFg = lane_base(LY::rF + 16 * g4);
        const int oF0 = lane_base(LY::rF);

        f32x4 sT[NKT];   // S^T[key 32ks + 8g + 4p + e][v = vw + c16], a = 2ks + p
        // (one branch around all reads of S0, so that they are in flight together)
        if (keyrows) {
#pragma unroll
            for (int a = 0; a < NKT; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sT[a][e] = (32 * (a >> 1) + 8 * g4 + 4 * (a & 1) + e == vw + c16) ? 1.f : 0.f;
        } else if (sg == 0 && p.S0) {
            const float* s0 = p.S0 + ((size_t)bh * p.DV + vw + c16) * DK + 8 * g4;
#pragma unroll
            for (int a = 0; a < NKT; ++a)
                sT[a] = *reinterpret_cast<const f32x4*>(s0 + 32 * (a >> 1) + 4 * (a & 1));
        } else {
#pragma unroll
            for (int a = 0; a < NKT; ++a) sT[a] = zero4();
        }

        // operands of one chunk, read from its slot
        struct In {
            Frag<E> kx[NB][NKS];      // K rows (X = K S^T)
            Frag<E> kt[NKT];          // K'^T, tokens 0-31 (state update)
            Frag16<E> kt16[NKT];      //   tokens 0-15 (16-token steps)
            Frag<E> tf[NB];           // T~ rows
            Frag16<E> tf16;
            s16x4 vraw[NB];           // V^T (bf16)
            f32x4 vv[NB];             // V^T (fp32)
            f32x4 gm[NB], dc[NB];     // gamma, exp(g_C - g) per token
            f32x4 dS[NKT];            // decay of the state rows
        };
        auto load_in = [&](auto jc, In& in) {
            constexpr int J = decltype(jc)::value;
            constexpr int cK = LY::rK + J * szK, cKU = (CH ? LY::rKU : LY::rK) + J * szK;
            // slot offsets relative to the lane bases above
            constexpr int cV = J * szV, cT = J * szT, cF = J * szF;
#pragma unroll
            for (int tt = 0; tt < NB; ++tt)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) in.kx[tt][ks] = ld_frag<E, 0>(smem + cK + 16 * tt * RBK, oKQ[ks], oKQh[ks]);
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                if constexpr (sizeof(E) == 2) {
                    in.vraw[tt] = ld_tr16<0>(smem + cV + 16 * tt * RBV, oVt);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        in.vv[tt][q] = ldf<0>(smem + LY::rV + cV, SV::off(16 * tt + 4 * g4 + q, 16 * w + c16));
                }
                in.gm[tt] = GATED ? ldf4<0>(smem + cF + 64 * tt, oFg) : f32x4{1.f, 1.f, 1.f, 1.f};
                in.dc[tt] = GATED ? ldf4<0>(smem + cF + 4 * CK + 64 * tt, oFg) : f32x4{1.f, 1.f, 1.f, 1.f};
            }
            if constexpr (NB == 2) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) in.tf[tt] = ld_frag<E, 0>(smem + cT + 16 * tt * RBT, oTo, oTo);
            } else {
                in.tf16 = ld_frag16<E, 0>(smem + cT, oTo);
            }
            if constexpr (GATED) {
                const float gC = ldf<8 * CK>(smem + cF, oF0);
#pragma unroll
                for (int a = 0; a < NKT; ++a) in.dS[a] = f32x4{gC, gC, gC, gC};
            } else if constexpr (CH) {
#pragma unroll
                for (int a = 0; a < NKT; ++a)
                    in.dS[a] = ldf4<0>(smem + cF + 4 * (32 * (a >> 1) + 4 * (a & 1)), oF0 + 32 * g4);
            }
        };
        // K'^T for the state update: read once the X products are issued
        auto load_kt = [&](auto jc, In& in) {
            constexpr int J = decltype(jc)::value;
            constexpr int cKU = (CH ? LY::rKU : LY::rK) + J * szK;
#pragma unroll
            for (int a = 0; a < NKT; ++a) {
                if constexpr (sizeof(E) == 2) {
                    const s16x4 k0 = ld_tr16<0>(smem + cKU, oKt[a]);
                    if constexpr (NB == 2) {
                        const s16x4 k1 = ld_tr16<16 * RBK>(smem + cKU, oKt[a]);
                        const u32x2 a0 = __builtin_bit_cast(u32x2, k0), a1 = __builtin_bit_cast(u32x2, k1);
                        in.kt[a].v = __builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y});
                    } else {
                        in.kt16[a].v = k0;
                    }
                } else {
                    // fp32: lane (g, r) reads tokens 4g + q (+16) of key channel
                    // 32ks + 4pa + 8(r/4) + r%4 one by one
                    const int kc = 32 * (a >> 1) + 4 * (a & 1) + 8 * (c16 >> 2) + (c16 & 3);
                    f32x4 lo, hi;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        lo[q] = ldf<0>(smem + cKU, SK::off(4 * g4 + q, kc));
                        if constexpr (NB == 2) hi[q] = ldf<0>(smem + cKU, SK::off(16 + 4 * g4 + q, kc));
                    }
                    if constexpr (NB == 2) { in.kt[a].lo = lo; in.kt[a].hi = hi; }
                    else in.kt16[a].v = lo;
                }
            }
        };
        // chunk m, from slot J
        auto own = [&](auto jc, int m) {
            constexpr int J = decltype(jc)::value;
            In in;
            load_in(jc, in);
            constexpr int pS = (J & 1) * LY::XSB, pU = (J & 1) * LY::XUB;   // m & 1 == J & 1
            // ---- S as an operand, published for the output wave
            Frag<E> sop[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                frag_of_tiles(sop[ks], sT[2 * ks], sT[2 * ks + 1]);
                *reinterpret_cast<Frag<E>*>(smem + oXS + pS + ks * kWave * FS) = sop[ks];
            }
            // ---- X = K S^T
            f32x4 x[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                x[tt] = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) mma(x[tt], in.kx[tt][ks], sop[ks]);
            }
            sched_fence();
            load_kt(jc, in);
            sched_fence();
            // ---- R = V - diag(gamma) X (token 16tt + 4g + e, channel c16)
            f32x4 r[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                const f32x4 vv = sizeof(E) == 2 ? unpack4(in.vraw[tt]) : in.vv[tt];
#pragma unroll
                for (int e = 0; e < 4; ++e) r[tt][e] = vv[e] - in.gm[tt][e] * x[tt][e];
            }
            // ---- decay of the state over the chunk
            if constexpr (GATED || CH) {
#pragma unroll
                for (int a = 0; a < NKT; ++a)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sT[a][e] *= in.dS[a][e];
            }
            // ---- U = T~ R (published), then S^T += K'^T (dec . U)
            Frag<E> uop;
            Frag16<E> uop16;
            if constexpr (NB == 2) {
                Frag<E> rop;
                frag_of_tiles(rop, r[0], r[1]);
                f32x4 u[2];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    u[tt] = zero4();
                    mma(u[tt], in.tf[tt], rop);
                }
                frag_of_tiles(uop, u[0], u[1]);
                *reinterpret_cast<Frag<E>*>(smem + oXU + pU) = uop;
                if constexpr (GATED) {
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) u[tt][e] *= in.dc[tt][e];
                    frag_of_tiles(uop, u[0], u[1]);
                }
            } else {
                Frag16<E> rop;
                frag16_of_tile(rop, r[0]);
                f32x4 u = zero4();
                mma16(u, in.tf16, rop);
                frag16_of_tile(uop16, u);
                *reinterpret_cast<Frag16<E>*>(smem + oXU + pU) = uop16;
                if constexpr (GATED) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) u[e] *= in.dc[0][e];
                    frag16_of_tile(uop16, u);
                }
            }
#pragma unroll
            for (int a = 0; a < NKT; ++a) {
                if constexpr (NB == 2) mma(sT[a], in.kt[a], uop);
                else mma16(sT[a], in.kt16[a], uop16);
            }
        };
        step_barrier();
        for (int s0 = 0; s0 <= NC; s0 += NSLOT) {
            auto step = [&](auto jc) {
                constexpr int J = decltype(jc)::value;
                const int s = s0 + J;
                if (s <= NC) {
                    if (s < NC) own(jc, s);
                    step_barrier();
                }
            };
            StaticFor<0, NSLOT>::run(step);
        }
        // final state: S_final, or this segment's end state; key rows store
        // the segment's transition transposed (row k' of P^T, column vw + c16)
        if (keyrows) {
            float* pt = p.Pseg + ((size_t)bh * p.SEG + sg) * DK * DK + vw + c16;
#pragma unroll
            for (int a = 0; a < NKT; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) pt[(size_t)(32 * (a >> 1) + 8 * g4 + 4 * (a & 1) + e) * DK] = sT[a][e];
        } else {
            float* sf = p.S_final ? p.S_final + ((size_t)bh * p.DV + vw + c16) * DK : nullptr;
            if (p.SEG > 1) sf = p.Sseg + (((size_t)bh * p.SEG + sg) * p.DV + vw + c16) * DK;
            if (sf) {
#pragma unroll
                for (int a = 0; a < NKT; ++a)
                    *reinterpret_cast<f32x4*>(sf + 32 * (a >> 1) + 8 * g4 + 4 * (a & 1)) = sT[a];
            }
        }
    } else if (w < 4) {
        // ===================================================== output waves
        const int c = w - 2, vw = v0 + 16 * c;
        // key rows write (transition so far) q_t, d_k per token, to p.qt
        const int ostride = keyrows ? DK : p.DV;
        // (no output array: the backward's recomputation, which keeps only the
        // states entering the chunks)
        E* const ob = keyrows ? reinterpret_cast<E*>(p.qt) : reinterpret_cast<E*>(p.o);
        E* og = ob ? ob + tok0 * ostride : nullptr;
        const int oXS = lane_base(LY::rxS + (c * NKS * kWave + l) * FS);
        const int oXU = lane_base(LY::rxU + (c * kWave + l) * FS);
        // Gamma tile (rb, ib): row c16 (+16 rb), tokens 16ib + 4g .. +3
        int oG[NB];
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) oG[ib] = lane_base(LY::rM + ST::off(c16, col_of_tok(CK, 16 * ib + 4 * g4)));
        const int oMo = lane_base(LY::rM + oT);
        const int oFq = lane_base(LY::rF + 12 * CK + 4 * c16);   // gamma / ||q||
        int oQ[NKS], oQh[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            oQ[ks] = lane_base(LY::rQ + oKQ[ks]);
            oQh[ks] = sizeof(E) == 4 ? lane_base(LY::rQ + oKQh[ks]) : 0;
        }

        auto out = [&](auto jc, int m) {
            constexpr int J = decltype(jc)::value;
            // slot offsets relative to the lane bases above (K: region at 0)
            constexpr int cK = LY::rK + J * szK, cQ = J * szK;
            constexpr int cM = J * szT, cF = J * szF;
            constexpr int pS = (J & 1) * LY::XSB, pU = (J & 1) * LY::XUB;   // m & 1 == J & 1
            const int t0 = (c0 + m) * CK, valid = min(CK, len - t0);
            // ---- reads
            Frag<E> sop[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) sop[ks] = *reinterpret_cast<const Frag<E>*>(smem + oXS + pS + ks * kWave * FS);
            const size_t fc = rec0 + c0 + m;   // chunk index over all heads
            if (p.Sck && fc % p.sck_every == 0) {
                // the state entering chunk m, for the backward, from the
                // operand owner c published -- kept off the owners' chain.
                // This wave's 16 value rows are one contiguous run of the
                // [d_v][d_k] state: each store writes 1 KiB of it, gathered
                // from the fragments that hold those key channels.
                constexpr int NI = 16 * DK * ES / 1024;
                unsigned char* ck = static_cast<unsigned char*>(p.Sck) +
                                    ((fc / p.sck_every) * p.DV + vw) * DK * ES + 16 * l;
                const unsigned char* xs = smem + LY::rxS + pS + c * NKS * kWave * FS;
                u32x4 pc[NI];
#pragma unroll
                for (int j = 0; j < NI; ++j) pc[j] = *reinterpret_cast<const u32x4*>(xs + xs_piece<E, DK>(64 * j + l));
#pragma unroll
                for (int j = 0; j < NI; ++j) st16(ck + 1024 * j, pc[j]);
            }
            if (!og) return;   // states only
            Frag<E> qf[NB][NKS], kf[NB][NKS];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    qf[tt][ks] = ld_frag<E, 0>(smem + cQ + 16 * tt * RBK, oQ[ks], oQh[ks]);
                    if constexpr (!CH) kf[tt][ks] = ld_frag<E, 0>(smem + cK + 16 * tt * RBK, oKQ[ks], oKQh[ks]);
                }
            f32x4 gmask[NB][NB];
            Frag<E> pf[NB];
            Frag16<E> pf16;
            if constexpr (CH) {
                if constexpr (NB == 2) {
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) pf[tt] = ld_frag<E, 0>(smem + cM + 16 * tt * RBT, oMo, oMo);
                } else {
                    pf16 = ld_frag16<E, 0>(smem + cM, oMo);
                }
            } else if constexpr (GATED) {
#pragma unroll
                for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                    for (int ib = 0; ib <= rb; ++ib) gmask[rb][ib] = ld_4f<E, 0>(smem + cM + 16 * rb * RBT, oG[ib]);
            }
            float gq[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) gq[tt] = GATED ? ldf<0>(smem + cF + 64 * tt, oFq) : 1.f;
            Frag<E> uop;
            Frag16<E> uop16;
            if constexpr (NB == 2) uop = *reinterpret_cast<const Frag<E>*>(smem + oXU + pU);
            else uop16 = *reinterpret_cast<const Frag16<E>*>(smem + oXU + pU);
            sched_fence();
            // ---- inter-chunk part: O^T = S Q^T, lane holds O[16tt + c16][vw + 4g + e]
            f32x4 oi[NB];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                oi[tt] = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) mma(oi[tt], sop[ks], qf[tt][ks]);
            }
            // ---- masked score tile (rb, ib): lane holds P[16rb + c16][16ib + 4g + e]
            auto score = [&](int rb, int ib) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) mma(acc, kf[ib][ks], qf[rb][ks]);
                if constexpr (GATED) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] *= gmask[rb][ib][e];
                } else {
                    const int r = 16 * rb + c16, i0 = 16 * ib + 4 * g4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = (r >= i0 + e) ? acc[e] : 0.f;
                }
                return acc;
            };
            if constexpr (!CH) {
                if constexpr (NB == 2) {
                    frag_of_tiles(pf[0], score(0, 0), zero4());
                    frag_of_tiles(pf[1], score(1, 0), score(1, 1));
                } else {
                    frag16_of_tile(pf16, score(0, 0));
                }
            }
#pragma unroll
            for (int tt = 0; tt < NB; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) oi[tt][e] *= gq[tt];
            // ---- intra-chunk part: O^T += U^T P^T
            if constexpr (NB == 2) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) mma(oi[tt], uop, pf[tt]);
            } else {
                // own accumulator: fed straight into a 16x16x16 product as its
                // accumulator input, the 16x16x32 result above was read before
                // all its rows were written (gfx950, this compiler)
                f32x4 oin = zero4();
                mma16(oin, uop16, pf16);
#pragma unroll
                for (int e = 0; e < 4; ++e) oi[0][e] += oin[e];
            }
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                const int tok = 16 * tt + c16;
                if (tok < valid)
                    st4(og + (size_t)(t0 + tok) * ostride + vw + 4 * g4, oi[tt][0], oi[tt][1], oi[tt][2], oi[tt][3]);
            }
        };
        step_barrier();
        for (int s0 = 0; s0 <= NC; s0 += NSLOT) {
            // step s works on chunk s - 1, in slot (s - 1) % NSLOT
            auto step = [&](auto jc) {
                constexpr int J = decltype(jc)::value;
                const int s = s0 + J;
                if (s <= NC) {
                    if (s >= 1) out(std::integral_constant<int, (J + NSLOT - 1) % NSLOT>{}, s - 1);
                    step_barrier();
                }
            };
            StaticFor<0, NSLOT>::run(step);
        }
    } else {
        // ===================================================== copiers (waves 4 ..)
        // Per-lane source offsets of one chunk's tiles, as for a full chunk:
        // instruction j, lane l fills LDS bytes 1024 j + 16 l of the region,
        // i.e. row b / RB, physical chunk (b % RB) / 16, which holds logical
        // chunk physical ^ swz(row).
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

        const int cw = w - 4;   // which copier
        // Q and the score block feed only the outputs: a call that keeps only the
        // states entering the chunks (the backward's recomputation) skips them
        const bool need_q = keyrows || p.o != nullptr;
        const unsigned char* kb = static_cast<const unsigned char*>(p.k);
        const unsigned char* qb = static_cast<const unsigned char*>(p.q);
        const unsigned char* vbs = static_cast<const unsigned char*>(p.v);
        // LDS destinations as 32-bit LDS addresses (no generic-pointer round trip)
        const uint32_t sbase = (uint32_t)(uintptr_t)(lds_void_t*)smem;
        // one region's copies: NI instructions of 1 KiB (the last may be partial)
        auto copy = [&](int dst, const unsigned char* src, const uint32_t* off, auto ni, int total) {
            constexpr int NI = decltype(ni)::value;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if (total % 1024 == 0 || 1024 * j + 16 * l < total)
                    __builtin_amdgcn_global_load_lds((const glb_void_t*)(src + off[j]),
                                                     (lds_void_t*)(uintptr_t)(sbase + (uint32_t)(dst + 1024 * j)), 16, 0, 0);
            }
        };
        auto issue = [&](auto jc, int m) {
            constexpr int J = decltype(jc)::value;
            const int t0 = (c0 + m) * CK, valid = min(CK, len - t0);
            const unsigned char* rec = p.ws + (rec0 + c0 + m) * WL.bytes;
            const size_t row0 = tok0 + t0;
            using NK = std::integral_constant<int, LY::NCK>;
            using NV = std::integral_constant<int, LY::NCV>;
            using NT = std::integral_constant<int, LY::NCT>;
            // V and T~ go with copier 0 unless alpha is per channel or the call
            // keeps only the states (then copier 1 has no Q to copy); key rows
            // have no V to copy
            const bool vt = (cw == ((CH || !need_q) ? 1 : 0));
            if constexpr (CH) {
                if (cw == 0) {
                    copy(LY::rK + J * szK, rec + WL.KG, offK, NK{}, szK);
                    copy(LY::rKU + J * szK, rec + WL.KD, offK, NK{}, szK);
                } else if (need_q) {
                    copy(LY::rQ + J * szK, rec + WL.QG, offK, NK{}, szK);
                }
            }
            if (valid == CK) {
                if constexpr (!CH) {
                    if (cw == 0) copy(LY::rK + J * szK, kb + row0 * DK * ES, offK, NK{}, szK);
                    else if (need_q) copy(LY::rQ + J * szK, qb + row0 * DK * ES, offK, NK{}, szK);
                }
                if (vt && !keyrows) copy(LY::rV + J * szV, vbs + (row0 * p.DV + v0) * ES, offV, NV{}, szV);
            } else {
                // last, partial chunk: rows past the end repeat the last row
                uint32_t rK[LY::NCK], rV[LY::NCV];
#pragma unroll
                for (int j = 0; j < LY::NCK; ++j) rK[j] = tile_off(SK{}, j, DK * ES, valid);
#pragma unroll
                for (int j = 0; j < LY::NCV; ++j) rV[j] = tile_off(SV{}, j, p.DV * ES, valid);
                if constexpr (!CH) {
                    if (cw == 0) copy(LY::rK + J * szK, kb + row0 * DK * ES, rK, NK{}, szK);
                    else if (need_q) copy(LY::rQ + J * szK, qb + row0 * DK * ES, rK, NK{}, szK);
                }
                if (vt && !keyrows) copy(LY::rV + J * szV, vbs + (row0 * p.DV + v0) * ES, rV, NV{}, szV);
            }
            if (vt) copy(LY::rT + J * szT, rec + WL.T, offT, NT{}, szT);
            if (cw == 1 && need_q) copy(LY::rM + J * szT, rec + WL.M, offT, NT{}, szT);
            if (cw == 0) {
#pragma unroll
                for (int j = 0; j < LY::NCF; ++j) {
                    if (LY::FB % 1024 == 0 || 1024 * j + 16 * l < LY::FB)
                        __builtin_amdgcn_global_load_lds((const glb_void_t*)(rec + WL.F + 1024 * j + 16 * l),
                                                         (lds_void_t*)(uintptr_t)(sbase + (uint32_t)(LY::rF + J * szF + 1024 * j)),
                                                         16, 0, 0);
                }
            }
        };
        // four copiers (channel alpha): K.exp(G) | K.exp(G_C - G) and the
        // decay factors | Q.exp(G) | V, T~ and P
        auto issue4 = [&](auto jc, int m) {
            constexpr int J = decltype(jc)::value;
            const int t0 = (c0 + m) * CK, valid = min(CK, len - t0);
            const unsigned char* rec = p.ws + (rec0 + c0 + m) * WL.bytes;
            const size_t row0 = tok0 + t0;
            using NK = std::integral_constant<int, LY::NCK>;
            using NV = std::integral_constant<int, LY::NCV>;
            using NT = std::integral_constant<int, LY::NCT>;
            if (cw == 0) {
                copy(LY::rK + J * szK, rec + WL.KG, offK, NK{}, szK);
            } else if (cw == 1) {
                copy(LY::rKU + J * szK, rec + WL.KD, offK, NK{}, szK);
#pragma unroll
                for (int j = 0; j < LY::NCF; ++j) {
                    if (LY::FB % 1024 == 0 || 1024 * j + 16 * l < LY::FB)
                        __builtin_amdgcn_global_load_lds((const glb_void_t*)(rec + WL.F + 1024 * j + 16 * l),
                                                         (lds_void_t*)(uintptr_t)(sbase + (uint32_t)(LY::rF + J * szF + 1024 * j)),
                                                         16, 0, 0);
                }
            } else if (cw == 2) {
                if (need_q) copy(LY::rQ + J * szK, rec + WL.QG, offK, NK{}, szK);
            } else {
                if (!keyrows) {
                    if (valid == CK) {
                        copy(LY::rV + J * szV, vbs + (row0 * p.DV + v0) * ES, offV, NV{}, szV);
                    } else {
                        // last, partial chunk: rows past the end repeat the last row
                        uint32_t rV[LY::NCV];
#pragma unroll
                        for (int j = 0; j < LY::NCV; ++j) rV[j] = tile_off(SV{}, j, p.DV * ES, valid);
                        copy(LY::rV + J * szV, vbs + (row0 * p.DV + v0) * ES, rV, NV{}, szV);
                    }
                }
                copy(LY::rT + J * szT, rec + WL.T, offT, NT{}, szT);
                if (need_q) copy(LY::rM + J * szT, rec + WL.M, offT, NT{}, szT);
            }
        };
        // this copier's copy instructions per chunk
        int nops;
        if constexpr (LY::NCP == 4) {
            nops = cw == 0 ? LY::NCK
                 : cw == 1 ? LY::NCK + LY::NCF
                 : cw == 2 ? (need_q ? LY::NCK : 0)
                 : (keyrows ? 0 : LY::NCV) + LY::NCT + (need_q ? LY::NCT : 0);
        } else if (!need_q && !CH) {
            nops = cw == 0 ? LY::NCK + LY::NCF : LY::NCV + LY::NCT;
        } else if (cw == 0) {
            nops = LY::NOPS0 - ((!CH && keyrows) ? LY::NCV : 0);
        } else {
            nops = need_q ? LY::NOPS1 - ((CH && keyrows) ? LY::NCV : 0) : LY::NOPS1 - LY::NCK - LY::NCT;
        }
        static_assert((AH - 1) * (LY::NOPS0 > LY::NOPS1 ? LY::NOPS0 : LY::NOPS1) < 64, "vmcnt range");
        // wait until at most k chunks issued after the one needed next are in flight
        auto wait_k = [&](int k) { vm_wait(k * nops); };
        auto issue_any = [&](auto jc, int m) {
            if constexpr (LY::NCP == 4) issue4(jc, m);
            else issue(jc, m);
        };
        {
            auto pro = [&](auto kc) {
                constexpr int K = decltype(kc)::value;
                if (K < NC) issue_any(kc, K);
            };
            StaticFor<0, AHEAD>::run(pro);
        }
        wait_k(min(AHEAD - 1, NC - 1));   // chunk 0 has landed
        step_barrier();
        // step s fills chunk s + AHEAD into slot (s + AHEAD) % NSLOT, then waits
        // for chunk s + 1
        for (int s0 = 0; s0 <= NC; s0 += NSLOT) {
            auto step = [&](auto jc) {
                constexpr int J = decltype(jc)::value;
                const int s = s0 + J;
                if (s <= NC) {
                    if (s + AHEAD < NC) issue_any(std::integral_constant<int, (J + AHEAD) % NSLOT>{}, s + AHEAD);
                    wait_k(max(0, min(AHEAD - 1, NC - 2 - s)));
                    step_barrier();
                }
            };
            StaticFor<0, NSLOT>::run(step);
        }
    }
}

// ------------------------------------------------------------------ host side
template <typename E, int DK, int CK, int MODE, int AH>
static hipError_t launch_scan_t(const ChunkArgs& a, const SegPlan& seg)
{
    using LY = ScanLayout<E, DK, CK, MODE, AH>;
    static_assert(LY::bytes <= 160 * 1024, "LDS budget");
    const int BH = a.B * a.H;
    const int NC = (a.L + CK - 1) / CK;
    const int NVB = a.dv / LY::BV, NMB = DK / 32;
    const int total = a.vl.start ? a.vl.NS * a.H * NVB : BH * (NVB + (seg.SEG - 1) * (NVB + NMB));
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    ScanParams sp{a.q, a.k, a.v, a.S0, ws, a.o, a.S_final, a.L, NC, a.dv, NVB, total,
                  seg.SEG, seg.NCS, NMB, seg.N0, nullptr, nullptr, nullptr, a.H, a.vl, a.Sck};
    sp.sck_every = a.sck_every > 0 ? a.sck_every : 1;
    if (seg.SEG > 1) {
        sp.qt = ws + seg.off_qt;
        sp.Sseg = reinterpret_cast<float*>(ws + seg.off_Z);
        sp.Pseg = reinterpret_cast<float*>(ws + seg.off_P);
    }
    auto* kern = chunk_scan_kernel<E, DK, CK, MODE, AH>;
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LY::bytes);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(total), dim3(64 * LY::NWAVES), LY::bytes, a.stream, sp);
    return hipGetLastError();
}

template <typename E, int DK, int CK>
static hipError_t launch_scan_m(const ChunkArgs& a, const SegPlan& sp)
{
    if (a.mode == kAlphaChannel) return launch_scan_t<E, DK, CK, kAlphaChannel, 2>(a, sp);
    // scalar alpha, and alpha = 1 as log alpha = 0 (the prepass wrote gamma = 1)
    return launch_scan_t<E, DK, CK, kAlphaScalar, 2>(a, sp);
}

hipError_t launch_scan(const ChunkArgs& a, int CK, const SegPlan& sp)
{
    if (a.dtype == kBF16) {
        if (a.dk == 128) return CK == 16 ? launch_scan_m<bf16, 128, 16>(a, sp) : launch_scan_m<bf16, 128, 32>(a, sp);
        return CK == 16 ? launch_scan_m<bf16, 64, 16>(a, sp) : launch_scan_m<bf16, 64, 32>(a, sp);
    }
    return a.dk == 128 ? launch_scan_m<float, 128, 16>(a, sp) : launch_scan_m<float, 64, 16>(a, sp);
}

}  // namespace gdr

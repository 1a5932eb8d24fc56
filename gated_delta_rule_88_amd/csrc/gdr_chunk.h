// gdr_chunk.h -- what the chunked forward's two kernels share: the token step,
// the per-chunk workspace layout and the kernel parameters.
//
// The forward runs in two launches on the caller's stream:
//   chunk_wy_kernel / chunk_wy_channel_kernel (gdr_wy.hip): every chunk of
//     every (b, h) independently -- the in-chunk cumulative log-decay, the
//     Gram block, the WY factor T~ = (I + A)^{-1} diag(beta), and what the
//     scan needs of the decay, into the workspace;
//   chunk_scan_kernel (gdr_scan.hip): one workgroup per (b, h, 32 value
//     channels) walks the chunks in order with the state in registers.
#pragma once

#include "gdr_internal.h"

namespace gdr {

// Tokens per state step of the backward (and of its forward recompute).
// Results do not depend on it beyond rounding (the chunk form is exact); 16
// for fp32 operands, whose pipeline slots would not fit LDS at 32, and where
// the caller asks for 16.
__host__ __device__ constexpr int chunk_step(int C, int dtype)
{
    return (C == 16 || dtype == kF32) ? 16 : 32;
}

// Tokens per state step of the chunked forward.
__host__ __device__ constexpr int fwd_token_step(int C, int dtype, int mode)
{
    (void)mode;
    return chunk_step(C, dtype);
}

// Column order of the [CK][CK] workspace blocks (T~, Gamma, P).  For CK = 32
// memory column 8g + 4p + e holds token 16p + 4g + e: the eight tokens that
// lane group g of a 16x16x32 MFMA contracts over (two 16-token tiles p, four
// consecutive tokens e each) are then one 16-byte read.  For CK = 16 the
// order is the natural one.
__host__ __device__ constexpr int tok_of_col(int CK, int mc)
{
    return CK == 32 ? 16 * ((mc >> 2) & 1) + 4 * (mc >> 3) + (mc & 3) : mc;
}
__host__ __device__ constexpr int col_of_tok(int CK, int t)
{
    return CK == 32 ? 8 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3) : t;
}

// Per-chunk workspace record (byte offsets), CK tokens, element type of size
// ES.  Regions are 16-byte aligned and each is a dense row-major block.
//   T   [CK][CK] E     T~ = (I + A)^{-1} diag(beta), zero above the diagonal
//                      (rows in token order, columns in tok_of_col order)
//   M   [CK][CK] E     scalar alpha: Gamma_ri = exp(g_r - g_i) / (||q_r|| ||k_i||)
//                      on and below the diagonal (norms 1 unless the prologue
//                      normalises q and k), zero above;  channel alpha: the
//                      masked decayed score block P
//   F   fp32           scalar alpha: gamma_r / ||k_r|| [CK], exp(g_C - g_r) / ||k_r||
//                      [CK], gamma_C and zeros [CK], gamma_r / ||q_r|| [CK];
//                      channel alpha: exp(G_C) per key channel [DK]
//   KG, QG, KD [CK][DK] E   channel alpha only: K . exp(G), Q . exp(G),
//                      K . exp(G_C - G)
// alpha = 1 uses the scalar layout with log alpha = 0.
struct WsLayout {
    int T, M, F, KG, QG, KD, bytes;
};

__host__ __device__ constexpr WsLayout ws_layout(int ES, int DK, int CK, int MODE)
{
    const bool channel = (MODE == kAlphaChannel);   // else scalar alpha or alpha = 1
    const int t = 0;
    const int m = t + CK * CK * ES;
    const int f = m + CK * CK * ES;
    const int kg = f + (channel ? DK * 4 : 4 * CK * 4);
    const int ch = channel ? CK * DK * ES : 0;
    return WsLayout{t, m, f, kg, kg + ch, kg + 2 * ch, kg + 3 * ch};
}

// The chunk in record slot cid: its first token on the token axis
// (head-row * L + position) and its number of tokens (0 for a slot no
// sequence fills).
struct ChunkSlot {
    size_t tok;
    int valid;
};

__device__ __forceinline__ ChunkSlot chunk_slot(const Varlen& vl, int L, int NC, int CK, int cid)
{
    if (!vl.start) {
        const int bh = cid / NC, n = cid % NC;
        return ChunkSlot{(size_t)bh * L + (size_t)n * CK, min(CK, L - n * CK)};
    }
    const int h = cid / vl.NCmax, j = cid % vl.NCmax;
    if (j >= vl.choff[vl.NS]) return ChunkSlot{0, 0};
    // the sequence s with choff[s] <= j < choff[s + 1]
    int lo = 0, hi = vl.NS;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (vl.choff[mid] <= j) lo = mid;
        else hi = mid;
    }
    const int c = j - vl.choff[lo];
    return ChunkSlot{(size_t)h * L + vl.start[lo] + (size_t)c * CK, min(CK, vl.len[lo] - c * CK)};
}

struct WyParams {
    const void *q, *k;
    const float *beta, *log_alpha;   // log_alpha NULL: alpha = 1
    unsigned char* ws;
    int L, NC, total;   // total = B * H * NC chunks (varlen: H * NCmax)
    unsigned pro;       // input-side prologue (kProNorm, kProGates)
    Varlen vl;
    float* Tout;        // null, or [total][CK][CK] fp32: T = (I + A)^{-1}, zero above the diagonal
};

struct ScanParams {
    const void *q, *k, *v;
    const float* S0;
    const unsigned char* ws;
    void* o;
    float* S_final;
    int L, NC, DV, NVB, total;   // total = B * H * (NVB + (SEG - 1) * (NVB + NMB)) workgroups
    // Segment-parallel scan (SEG > 1): segment 0 covers chunks [0, N0), segment
    // g >= 1 chunks [N0 + (g - 1) NCS, min(N0 + g NCS, NC)); NMB blocks of 32
    // key rows per later segment.
    int SEG, NCS, NMB, N0;
    void* qt;       // [B*H][L][d_k] (input dtype): (transition from the segment start) q_t
    float* Sseg;    // [B*H][SEG][d_v][d_k]: segment end state from S0 (g = 0) or zero (g > 0)
    float* Pseg;    // [B*H][SEG][d_k][d_k]: segment transition (g > 0)
    // Packed variable-length batch (vl.start != NULL; one segment): chain
    // n * H + h is sequence n of head h, total = NS * H * NVB workgroups.
    int H;
    Varlen vl;
    // [ceil(B*H*NC / sck_every)][d_v][d_k] in the operand type: the state
    // entering chunks 0, sck_every, 2 sck_every, ... counted over all heads
    // (chunk n of head bh is bh * NC + n), kept for the backward; or null
    void* Sck;
    int sck_every;
};

// Segment-parallel scan.  A head's chunk scan is one sequential chain; when
// the batch has too few (b, h) chains to give every CU a workgroup, the chain
// is cut into SEG segments that run at the same time.  Segment 0 runs from
// the true initial state; segment g > 0 runs from a zero state, plus d_k key
// rows started from the identity, whose end values are the segment's
// transition P_g (S_end = S_entry P_g + Z_g, Z_g = its end state from zero)
// and whose outputs are (P up to t) q_t.  Afterwards the entry states follow
// in order, E_1 = Z_0, E_{g+1} = E_g P_g + Z_g, and every output of
// segment g gains E_g (P up to t) q_t.  Only for bf16 operands: the entry
// states enter these last products as bf16 operands.
// The budget is the MI355X's 256 CUs (one scan workgroup each) as a constant,
// not a device query: the plan fixes the workspace size, which the size
// query must report without a device argument.  (The backward's gradient
// walk divides its chunks into as many runs, for the same reason.)
constexpr int kSegWorkgroups = 256;   // scan workgroups the device runs at once (one per CU)
constexpr int kSegMinChunks = 16;     // shortest segment worth splitting off
constexpr int kMaxSeg = 16;
// Chain-chunks of later segments whose output correction (seg_correct_kernel:
// (P up to t) q_t and o read, o written) costs about one scan step of the
// whole batch (measured at B1 H16 L65536: 97 us for 16 x 1024 chain-chunks,
// 0.64 us per scan step).
constexpr int kSegCorrectPerStep = 110;

struct SegPlan {
    int SEG, NCS, N0;                 // segments, chunks per later segment (the last may be
                                      // shorter), chunks of segment 0
    size_t off_Z, off_P, off_E, off_qt, bytes;   // extra workspace after the chunk records
};

// The plan with the shortest estimated time, in scan steps: the longest run
// of chunks any CU walks, plus the later segments' output correction.
//  - When every workgroup fits the budget at once, the segments are equal.
//  - A plan may hold more workgroups than the budget when B*H is a multiple of
//    8: the scan then orders each XCD's workgroups with every segment-0
//    workgroup first (gdr_scan.hip), so the ones left waiting for a free CU are
//    later-segment workgroups, which start when the first of them finish.
//    With segment 0 twice as long as a later segment, those finish together
//    with segment 0: NC = a + (SEG - 1) b with a = 2 b.  This needs the
//    waiting workgroups to be no more than the later-segment workgroups of
//    the first round: W - 256 <= 256 - B*H*NVB.
inline SegPlan seg_plan(int B, int H, int L, int dk, int dv, int CK, int dtype, size_t base)
{
    const int NC = (L + CK - 1) / CK;
    SegPlan sp{1, NC, NC, 0, 0, 0, 0, 0};
    const size_t BH = (size_t)B * H;
    const size_t NVB = dv / 32, NMB = dk / 32;
    const size_t W0 = BH * NVB;
    if (dtype != kBF16 || BH == 0 || W0 > (size_t)kSegWorkgroups || NC < 2 * kSegMinChunks) return sp;
    double best = NC;
    for (int g = 2; g <= kMaxSeg; ++g) {
        const size_t W = BH * (NVB + (g - 1) * (NVB + NMB));
        int n0, ncs, seg = g;
        if (W <= (size_t)kSegWorkgroups) {
            ncs = (NC + g - 1) / g;
            seg = (NC + ncs - 1) / ncs;
            n0 = ncs;
        } else if (BH % 8 == 0 && W + W0 <= 2 * (size_t)kSegWorkgroups) {
            ncs = (NC + g) / (g + 1);
            n0 = NC - (g - 1) * ncs;
            if (n0 < ncs) continue;
        } else {
            break;
        }
        if (seg < 2 || ncs < kSegMinChunks) break;
        const int later = NC - n0;
        const int span = W <= (size_t)kSegWorkgroups ? max(n0, ncs) : max(n0, 2 * ncs);
        const double t = span + (double)BH * later / kSegCorrectPerStep;
        if (t < best) {
            best = t;
            sp.SEG = seg;
            sp.NCS = ncs;
            sp.N0 = n0;
        }
    }
    if (sp.SEG == 1) return sp;
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    size_t o = al(base);
    sp.off_Z = o; o = al(o + BH * sp.SEG * dv * dk * 4);
    sp.off_P = o; o = al(o + BH * sp.SEG * dk * dk * 4);
    sp.off_E = o; o = al(o + BH * sp.SEG * dv * dk * 2);
    sp.off_qt = o; o = al(o + BH * (size_t)L * dk * 2);
    sp.bytes = o;
    return sp;
}

hipError_t launch_wy(const ChunkArgs& a, int CK);
hipError_t launch_scan(const ChunkArgs& a, int CK, const SegPlan& sp);
hipError_t launch_seg_combine(const ChunkArgs& a, int CK, const SegPlan& sp);
// Compute units of the current device (256 if the query fails).
int compute_units();

}  // namespace gdr

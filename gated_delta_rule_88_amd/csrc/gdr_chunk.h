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

// Tokens per state step.  Results do not depend on it beyond rounding (the
// chunk form is exact); 16 for fp32 operands, whose pipeline slots would not
// fit LDS at 32, and where the caller asks for 16.
__host__ __device__ constexpr int chunk_step(int C, int dtype)
{
    return (C == 16 || dtype == kF32) ? 16 : 32;
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
//   M   [CK][CK] E     scalar alpha: Gamma_ri = exp(g_r - g_i) on and below the
//                      diagonal, zero above;  channel alpha: the masked decayed
//                      score block P;  alpha = 1: absent
//   F   fp32           scalar alpha: gamma_r = exp(g_r) [CK], exp(g_C - g_r) [CK],
//                      gamma_C, zero padding (4 CK floats);
//                      channel alpha: exp(G_C) per key channel [DK];  alpha = 1: absent
//   KG, QG, KD [CK][DK] E   channel alpha only: K . exp(G), Q . exp(G),
//                      K . exp(G_C - G)
struct WsLayout {
    int T, M, F, KG, QG, KD, bytes;
};

__host__ __device__ constexpr WsLayout ws_layout(int ES, int DK, int CK, int MODE)
{
    const int t = 0;
    const int m = t + CK * CK * ES;
    const int f = m + (MODE != kAlphaNone ? CK * CK * ES : 0);
    const int kg = f + (MODE == kAlphaScalar ? 4 * CK * 4 : (MODE == kAlphaChannel ? DK * 4 : 0));
    const int ch = (MODE == kAlphaChannel) ? CK * DK * ES : 0;
    return WsLayout{t, m, f, kg, kg + ch, kg + 2 * ch, kg + 3 * ch};
}

struct WyParams {
    const void *q, *k;
    const float *beta, *log_alpha;
    unsigned char* ws;
    int L, NC, total;   // total = B * H * NC chunks
};

struct ScanParams {
    const void *q, *k, *v;
    const float* S0;
    const unsigned char* ws;
    void* o;
    float* S_final;
    int L, NC, DV, NVB, total;   // total = B * H * NVB workgroups
};

hipError_t launch_wy(const ChunkArgs& a, int CK);
hipError_t launch_scan(const ChunkArgs& a, int CK);

}  // namespace gdr

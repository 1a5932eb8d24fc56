// gdr_bwd.h -- what the backward's two translation units share: the kernel
// parameters and the pipelined chain's launcher.
#pragma once

#include "gdr_internal.h"

namespace gdr {

struct BwdParams {
    const void *q, *k, *v, *dO;
    const float *beta, *log_alpha;   // log_alpha NULL: alpha = 1
    const float* dS_final;           // [B*H][d_v][d_k] or null
    const unsigned char* ws;         // forward prepass records
    const void* Sck;                 // (operand type) entry states, as span says
    void* dSck;                      // [B*H][NC][d_v][d_k] (operand type): dS at each chunk's end
    void *dq, *dk, *dv;
    float *dbeta, *dlog_alpha, *dS0;
    int L, NC, DV, total;
    const float* Tck;                // [B*H][NC][CK][CK] fp32: each chunk's T = (I + A)^{-1}
    // span > 0 (bf16 operands on 32-token steps): gradient workgroup b takes
    // chunks b span .. (b + 1) span - 1, counted over all heads (chunk n of
    // head bh is bh * NC + n), in order and carries the state across them;
    // Sck is [ceil(total / span)][d_v][d_k], the state entering chunks 0,
    // span, 2 span, ..., and a head's first chunk starts from S0 (null:
    // zero).  span = 0: Sck is [total][d_v][d_k], every chunk's entry state.
    int span;
    const float* S0;                 // [B*H][d_v][d_k] or null
};

// The chain (dS carried backwards over the chunks of every (b, h)) for bf16
// operands and 32-token steps, d_k = 64 or 128, d_v a multiple of 32:
// one workgroup per (b, h, 32 value channels) on the stream.
hipError_t launch_bwd_chain_pipe(const BwdParams& bp, int BH, int dk, bool channel, hipStream_t stream);

}  // namespace gdr

// gdr_tri.h -- the in-chunk triangular inverse shared by the forward
// prepass and the backward: (I + A)^{-1} for a strictly lower-triangular
// CK x CK block A, in fp32 (the WY factor of a chunk's (I - beta k k^T)
// products, "Linear Attention & DeltaNet", "How it works", item 3).
#pragma once

#include "gdr_device.h"

namespace gdr {

// (I + A)^{-1} for a strictly lower-triangular CK x CK block A (CK = 16 or
// 32) held in LDS (row stride LF), by one wave.  Writes T row-major to Tf
// (stride LF).  Af and Tf belong to this wave.
template <int CK, int LF>
__device__ __forceinline__ void unit_lower_inverse(const float* Af, float* Tf) {
    constexpr int NB = CK / 16;
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15;
    {
        // lane (b, j) solves column j of diagonal block b; row r + 1 of A is
        // fetched while row r is being solved
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
        }
    }
    wave_lds_fence();
    if constexpr (NB == 2) {
        // Y = A_10 T_00 (lane: Y[4g + e][c]), then Z = T_11 Y, T_10 = -Z;
        // step e contracts over k = 4g + e: lane (g, c) supplies A_10[c][k]
        // and T_00[k][c]
        const f32x4 a10 = *reinterpret_cast<const f32x4*>(Af + (16 + c16) * LF + 4 * g4);
        f32x4 y = zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e)
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(a10[e], Tf[(4 * g4 + e) * LF + c16], y, 0, 0, 0);
        const f32x4 t11 = *reinterpret_cast<const f32x4*>(Tf + (16 + c16) * LF + 16 + 4 * g4);
        f32x4 z = zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) z = __builtin_amdgcn_mfma_f32_16x16x4f32(t11[e], y[e], z, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) Tf[(16 + 4 * g4 + e) * LF + c16] = -z[e];
        wave_lds_fence();
    }
}

// T (row stride LF in LDS, as unit_lower_inverse leaves it: the block above
// the diagonal unwritten) to dst as a dense [CK][CK] fp32 block with zeros
// above the diagonal, 16 bytes per thread index i = t, t + n, ...
template <int CK, int LF>
__device__ __forceinline__ void store_T(const float* Tf, float* dst, int t, int n) {
    for (int i = t; i < CK * CK / 4; i += n) {
        const int r = (4 * i) / CK, s0 = (4 * i) % CK;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (s0 + e <= r) ? Tf[r * LF + s0 + e] : 0.f;
        *reinterpret_cast<f32x4*>(dst + 4 * i) = v;
    }
}

}  // namespace gdr

// gdr_device.h -- device helpers for the gfx950 kernels: element types,
// 16-byte vector access, bf16 conversion and 16x16 MFMA fragments.
//
// Fragment convention (used by every tile product in this library):
// products are written in "NT" form, C[m][n] = sum_k A[m][k] * B[n][k], with
// both operands stored in LDS as [outer][k] (k contiguous).  For one 32-wide
// k-step, lane l supplies row (l % 16) of A and row (l % 16) of B, and the 8
// consecutive k values k0 + 8*(l/16) .. +7 of each.  Because A and B use the
// same k mapping the sum over k does not depend on how the hardware orders
// k inside an instruction.  The 16x16 fp32 accumulator holds
// C[4*(l/16) + e][l % 16] in element e (e = 0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace gdr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// ---------------------------------------------------------------- conversion
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Elements per 16-byte vector.
template <typename T> struct Vec { static constexpr int n = 16 / sizeof(T); };

// 16-byte loads and stores (global or LDS; the pointer must be 16-B aligned).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Non-temporal 16-byte store: for data the next kernel streams in, so that it
// does not sit dirty in the caches while that kernel reads other data.
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Unpack / pack a 16-byte vector of T into floats.
template <typename T> struct Pack;
template <> struct Pack<float> {
    static constexpr int n = 4;
    __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
    __device__ static __forceinline__ u32x4 pack(const float* f) {
        u32x4 v; v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
        v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]); return v;
    }
};
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Round two floats to bf16 (nearest even) and pack them: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
template <> struct Pack<bf16> {
    static constexpr int n = 8;
    __device__ static __forceinline__ void unpack(u32x4 v, float* f) {
        f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
        f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
    }
    __device__ static __forceinline__ u32x4 pack(const float* f) {
        u32x4 v; v.x = pack_bf2(f[0], f[1]); v.y = pack_bf2(f[2], f[3]);
        v.z = pack_bf2(f[4], f[5]); v.w = pack_bf2(f[6], f[7]); return v;
    }
};

// Store 4 consecutive elements (from fp32) at p (8 B for bf16, 16 B for f32).
__device__ __forceinline__ void st4(bf16* p, float a, float b, float c, float d) {
    u32x2 v; v.x = pack_bf2(a, b); v.y = pack_bf2(c, d); st8(p, v);
}
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
    u32x4 v; v.x = __float_as_uint(a); v.y = __float_as_uint(b);
    v.z = __float_as_uint(c); v.w = __float_as_uint(d); st16(p, v);
}

// ---------------------------------------------------------------- fragments
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

// Fragment of a matrix stored [row][k] with leading dimension ld (elements):
// lane reads row row0 + l%16, k = k0 + 8*(l/16) .. +7.
__device__ __forceinline__ Frag<bf16> ldfrag(const bf16* base, int ld, int row0, int k0) {
    const int l = lane_id();
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x8*>(base + (row0 + (l & 15)) * ld + k0 + 8 * (l >> 4));
    return f;
}
__device__ __forceinline__ Frag<float> ldfrag(const float* base, int ld, int row0, int k0) {
    const int l = lane_id();
    const float* p = base + (row0 + (l & 15)) * ld + k0 + 8 * (l >> 4);
    Frag<float> f;
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 4);
    return f;
}

// Fragment read from p (8 consecutive elements) with element j multiplied
// by s[j] in fp32 before the operand is formed.
__device__ __forceinline__ void load_scaled_frag(Frag<bf16>& f, const bf16* p, const float* s) {
    float x[8];
    Pack<bf16>::unpack(ld16(p), x);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] *= s[j];
    f.v = __builtin_bit_cast(bf16x8, Pack<bf16>::pack(x));
}
__device__ __forceinline__ void load_scaled_frag(Frag<float>& f, const float* p, const float* s) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    f.lo = f32x4{a.x * s[0], a.y * s[1], a.z * s[2], a.w * s[3]};
    f.hi = f32x4{b.x * s[4], b.y * s[5], b.z * s[6], b.w * s[7]};
}

// acc += A * B^T over one 32-wide k-step.
__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

// fp32 product over one 16-wide k-step (k0 + 4*(l/16) .. +3 per lane), used
// by the triangular inverse, which stays in fp32 on every path.
__device__ __forceinline__ void mma_k16(f32x4& acc, const float* a, int lda, int arow0,
                                        const float* b, int ldb, int brow0, int k0) {
    const int l = lane_id();
    f32x4 x = *reinterpret_cast<const f32x4*>(a + (arow0 + (l & 15)) * lda + k0 + 4 * (l >> 4));
    f32x4 y = *reinterpret_cast<const f32x4*>(b + (brow0 + (l & 15)) * ldb + k0 + 4 * (l >> 4));
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, y.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, y.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, y.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, y.w, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// ------------------------------------------------------ tile-pair operands
// Second operand convention, used where MFMA results feed the next product
// directly from registers.  A 32-wide k-step is two 16-wide k-tiles p = 0, 1;
// element j = 4p + e of lane group g = l/16 holds k = k0 + 16p + 4g + e.  A
// 16x16 fp32 accumulator tile holds rows 4g + e of column l%16, so two such
// tiles (k-tiles p = 0, 1 along their row index) are already an operand for
// a product that contracts over that row index: no LDS round trip.
__device__ __forceinline__ Frag<bf16> ldfrag_pair(const bf16* base, int ld, int row0, int k0) {
    const int l = lane_id();
    const bf16* p = base + (row0 + (l & 15)) * ld + k0 + 4 * (l >> 4);
    const u32x2 lo = ld8(p), hi = ld8(p + 16);
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
    return f;
}
__device__ __forceinline__ Frag<float> ldfrag_pair(const float* base, int ld, int row0, int k0) {
    const int l = lane_id();
    const float* p = base + (row0 + (l & 15)) * ld + k0 + 4 * (l >> 4);
    Frag<float> f;
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 16);
    return f;
}
__device__ __forceinline__ void frag_of_tiles(Frag<bf16>& f, f32x4 t0, f32x4 t1) {
    f.v = __builtin_bit_cast(bf16x8, u32x4{pack_bf2(t0[0], t0[1]), pack_bf2(t0[2], t0[3]),
                                           pack_bf2(t1[0], t1[1]), pack_bf2(t1[2], t1[3])});
}
__device__ __forceinline__ void frag_of_tiles(Frag<float>& f, f32x4 t0, f32x4 t1) {
    f.lo = t0;
    f.hi = t1;
}

// 16-wide k-step: element e of lane group g holds k = k0 + 4g + e.
typedef short s16x4 __attribute__((ext_vector_type(4)));
template <typename T> struct Frag16;
template <> struct Frag16<bf16> { s16x4 v; };
template <> struct Frag16<float> { f32x4 v; };
__device__ __forceinline__ Frag16<bf16> ldfrag16(const bf16* base, int ld, int row0, int k0) {
    const int l = lane_id();
    Frag16<bf16> f;
    f.v = __builtin_bit_cast(s16x4, ld8(base + (row0 + (l & 15)) * ld + k0 + 4 * (l >> 4)));
    return f;
}
__device__ __forceinline__ Frag16<float> ldfrag16(const float* base, int ld, int row0, int k0) {
    const int l = lane_id();
    Frag16<float> f;
    f.v = *reinterpret_cast<const f32x4*>(base + (row0 + (l & 15)) * ld + k0 + 4 * (l >> 4));
    return f;
}
__device__ __forceinline__ void frag16_of_tile(Frag16<bf16>& f, f32x4 t) {
    f.v = __builtin_bit_cast(s16x4, u32x2{pack_bf2(t[0], t[1]), pack_bf2(t[2], t[3])});
}
__device__ __forceinline__ void frag16_of_tile(Frag16<float>& f, f32x4 t) { f.v = t; }
__device__ __forceinline__ void mma16(f32x4& acc, const Frag16<bf16>& a, const Frag16<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const Frag16<float>& a, const Frag16<float>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.x, b.v.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.y, b.v.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.z, b.v.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.w, b.v.w, acc, 0, 0, 0);
}

// Transpose a VE x VE block held as VE 16-byte row vectors (row r = token,
// element j = channel) into VE column vectors (column j, element r).
__device__ __forceinline__ void transpose_block(const u32x4* in, u32x4* out, bf16*) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int d = j >> 1;
        const int sh = (j & 1) * 16;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t a = (in[2 * p][d] >> sh) & 0xffffu;
            const uint32_t b = (in[2 * p + 1][d] >> sh) & 0xffffu;
            w[p] = a | (b << 16);
        }
        out[j] = u32x4{w[0], w[1], w[2], w[3]};
    }
}
__device__ __forceinline__ void transpose_block(const u32x4* in, u32x4* out, float*) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = u32x4{in[0][j], in[1][j], in[2][j], in[3][j]};
}

// Four consecutive elements as fp32 (one 8-byte or 16-byte read).
__device__ __forceinline__ f32x4 load4f(const bf16* p) {
    const u32x2 v = ld8(p);
    return f32x4{bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y)};
}
__device__ __forceinline__ f32x4 load4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Make this wave's earlier LDS accesses complete before its later ones (and
// keep the compiler from moving memory operations across this point).
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Gate activations of the input-side prologue: beta = sigmoid(b) and
// log alpha = log sigmoid(a) = min(a, 0) - log(1 + exp(-|a|)), a form that
// never overflows.  Both use the hardware exp / log: where 1 + exp(-|a|)
// rounds to 1 the dropped tail is below 6e-8 absolute, and the per-channel
// gates run on every key channel of every token, where a full-precision
// log1p would cost more than the rest of the prepass.
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + __expf(-x)); }
__device__ __forceinline__ float log_sigmoid_f(float x) { return fminf(x, 0.f) - __logf(1.f + __expf(-fabsf(x))); }

// 4 x 4 transpose within each quad of lanes (two butterfly stages of quad
// permutes): quad lane b, holding rows 0 .. 3 of column b, ends up holding
// row b, columns 0 .. 3.  A 16 x 16 MFMA result tile (lane (g, c): rows
// 4g .. 4g + 3 of column c) then gives lane (g, c) row 4g + c % 4, columns
// 4 (c / 4) .. + 3, four consecutive elements one store can write.  Every
// lane of a quad must execute it.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 v) {
    const int b = lane_id() & 3;
    auto mv = [](float x, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                     decltype(ctrl)::value, 0xf, 0xf, false));
    };
    using X1 = std::integral_constant<int, 0xB1>;   // quad_perm [1, 0, 3, 2]
    using X2 = std::integral_constant<int, 0x4E>;   // quad_perm [2, 3, 0, 1]
    f32x4 y = {mv(v[1], X1{}), mv(v[0], X1{}), mv(v[3], X1{}), mv(v[2], X1{})};
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = ((e ^ b) & 1) ? y[e] : v[e];
    y = f32x4{mv(v[2], X2{}), mv(v[3], X2{}), mv(v[0], X2{}), mv(v[1], X2{})};
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = ((e ^ b) & 2) ? y[e] : v[e];
    return v;
}

// Inclusive prefix sum over lanes 0 .. 31 of a wave (lanes 32 .. 63 get
// sums of their own rows): four shifts within each 16-lane row, then row 0's
// total added to row 1 -- VALU data moves (DPP), no round trip through the
// LDS unit as lane permutes take.
__device__ __forceinline__ float scan32(float x) {
    auto shr = [](float v, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     decltype(ctrl)::value, 0xf, 0xf, true));
    };
    x += shr(x, std::integral_constant<int, 0x111>{});   // row_shr:1
    x += shr(x, std::integral_constant<int, 0x112>{});   // row_shr:2
    x += shr(x, std::integral_constant<int, 0x114>{});   // row_shr:4
    x += shr(x, std::integral_constant<int, 0x118>{});   // row_shr:8
    // row_bcast:15 into rows 1 and 3 (rows 0 and 2 add 0)
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false));
    return x;
}
// Value of a wave-uniform lane (a scalar read, no lane permute).
__device__ __forceinline__ float lane_value(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

}  // namespace gdr

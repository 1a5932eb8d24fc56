// gdr_pipe.h -- the pieces of the chunk-pipelined kernels (the forward scan
// and the backward chain) that move chunks through LDS: swizzled tiles,
// fragment and transposing reads, the step barrier, the region layout of a
// ring of chunk slots, and the copy-instruction counts.
#pragma once

#include "gdr_device.h"
#include "gdr_chunk.h"

namespace gdr {

namespace {
__host__ __device__ constexpr int align16(int x) { return (x + 15) / 16 * 16; }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Row-major LDS tile of W elements per row whose 16-byte chunks are permuted
// within each row by XOR with swz(row); swz depends only on row % 16.
template <typename E, int W>
struct Swz {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int RB = W * ES;      // bytes per row
    static constexpr int NCH = RB / 16;    // 16-byte chunks per row
    static_assert(NCH == 2 || NCH == 4 || NCH == 8 || NCH == 16 || NCH == 32, "row width");
    __device__ static __forceinline__ int swz(int r) {
        if (NCH == 2) return (r >> 1) & 1;
        if (NCH == 4) return (r >> 1) & 3;
        if (NCH == 8) return (r >> 1) & 7;
        return (r & 15) ^ ((r & 2) << 2);
    }
    // byte offset of element (r, c); an access of up to 16 bytes starting at
    // c must not cross a 16-byte boundary
    __device__ static __forceinline__ int off(int r, int c) {
        const int cb = c * ES;
        return r * RB + ((((cb >> 4) ^ swz(r))) << 4) + (cb & 15);
    }
};

template <int N> __device__ __forceinline__ u32x4 lds16(const unsigned char* base, int off) {
    return *reinterpret_cast<const u32x4*>(base + off + N);
}
template <int N> __device__ __forceinline__ u32x2 lds8(const unsigned char* base, int off) {
    return *reinterpret_cast<const u32x2*>(base + off + N);
}

// MFMA operand of 8 consecutive elements at base + off + N; fp32 takes two
// 16-byte reads, the second at base + off_hi + N (the swizzle may have moved
// it away from the first).
template <typename E, int N>
__device__ __forceinline__ Frag<E> ld_frag(const unsigned char* base, int off, int off_hi) {
    Frag<E> f;
    if constexpr (sizeof(E) == 2) {
        f.v = __builtin_bit_cast(bf16x8, lds16<N>(base, off));
    } else {
        f.lo = __builtin_bit_cast(f32x4, lds16<N>(base, off));
        f.hi = __builtin_bit_cast(f32x4, lds16<N>(base, off_hi));
    }
    return f;
}
// 16-wide k-step operand of 4 consecutive elements.
template <typename E, int N>
__device__ __forceinline__ Frag16<E> ld_frag16(const unsigned char* base, int off) {
    Frag16<E> f;
    if constexpr (sizeof(E) == 2) f.v = __builtin_bit_cast(s16x4, lds8<N>(base, off));
    else f.v = __builtin_bit_cast(f32x4, lds16<N>(base, off));
    return f;
}
// Four consecutive elements as fp32.
template <typename E, int N>
__device__ __forceinline__ f32x4 ld_4f(const unsigned char* base, int off) {
    if constexpr (sizeof(E) == 2) {
        const u32x2 w = lds8<N>(base, off);
        return f32x4{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
    } else {
        return __builtin_bit_cast(f32x4, lds16<N>(base, off));
    }
}
// Transposing read of a 4 x 4 bf16 block per lane group: the lane's address
// (from tr_off) names 4 consecutive elements; lane (g, c) receives element
// c % 4 of the vectors addressed by lanes (g, 4q + c / 4), q = 0..3.
template <int N>
__device__ __forceinline__ s16x4 ld_tr16(const unsigned char* base, int off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + off + N));
}
__device__ __forceinline__ f32x4 unpack4(s16x4 v) {
    const u32x2 w = __builtin_bit_cast(u32x2, v);
    return f32x4{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
}
template <int N> __device__ __forceinline__ float ldf(const unsigned char* base, int off) {
    return *reinterpret_cast<const float*>(base + off + N);
}
template <int N> __device__ __forceinline__ f32x4 ldf4(const unsigned char* base, int off) {
    return *reinterpret_cast<const f32x4*>(base + off + N);
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [LO, HI) (the count is an
// instruction immediate: a binary dispatch over its values).
template <int LO, int HI>
__device__ __forceinline__ void vm_wait_range(int n) {
    if constexpr (HI - LO == 1) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LO) : "memory");
    } else {
        constexpr int MID = (LO + HI) / 2;
        if (n < MID) vm_wait_range<LO, MID>(n);
        else vm_wait_range<MID, HI>(n);
    }
}
__device__ __forceinline__ void vm_wait(int n) { vm_wait_range<0, 64>(n); }

// A block of 16 (or 32) value rows of a state, published as the owners'
// MFMA operands (fragment (ks, lane 16 g + r) of owner o holds row 16 o + r,
// key channels 32 ks + 8 g .. +7), written out row-major [row][d_k]: the LDS
// byte offset, from the first owner's fragments, of flat 16-byte piece f of
// the block, so that lane l of store j takes piece 64 j + l and every store
// covers 1 KiB of contiguous rows.
template <typename E, int DK>
__device__ __forceinline__ int xs_piece(int f) {
    constexpr int ES = (int)sizeof(E), PR = DK * ES / 16;   // pieces per row
    constexpr int NKS = DK / 32, FS = (int)sizeof(Frag<E>);
    const int r = f / PR, kc = (f % PR) * (16 / ES);
    return (((r >> 4) * NKS + (kc >> 5)) * kWave + 16 * ((kc & 31) >> 3) + (r & 15)) * FS + (kc & 7) * ES;
}

// Barrier for the pipeline: this wave's LDS accesses are complete, then all
// waves meet.  It does not wait for outstanding global->LDS copies: the
// copier waits for those explicitly.
__device__ __forceinline__ void step_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// A per-lane LDS offset that already includes a region's base: hidden from
// constant folding so the slot and tile offsets that are added to it stay
// within the 16-bit immediate of the LDS instructions (the regions past
// 64 KiB would otherwise cost an address add per access).
__device__ __forceinline__ int lane_base(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Compile-time loop: f(integral_constant<int, I>) for I = B .. N - 1.
template <int I, int N>
struct StaticFor {
    template <class F>
    __device__ static __forceinline__ void run(F& f) {
        f(std::integral_constant<int, I>{});
        StaticFor<I + 1, N>::run(f);
    }
};
template <int N>
struct StaticFor<N, N> {
    template <class F>
    __device__ static __forceinline__ void run(F&) {}
};

template <int NBYTES>
struct CopyCount { static constexpr int n = (NBYTES + 1023) / 1024; };
}  // namespace

// MODE is kAlphaScalar or kAlphaChannel: alpha = 1 runs as scalar alpha with
// log alpha = 0 (the prepass writes gamma = 1 and Gamma = the causal mask).
template <typename E, int DK, int CK, int MODE, int AHEAD_ = 2>
struct ScanLayout {
    static_assert(MODE == kAlphaScalar || MODE == kAlphaChannel, "gate mode of the scan");
    static constexpr int ES = (int)sizeof(E);
    static constexpr int BV = 32;             // value channels per workgroup
    static constexpr bool CH = (MODE == kAlphaChannel);
    // Ring of chunk slots.  At step s the copier fills chunk s + AHEAD while
    // the state owners work on chunk s and the output waves on chunk s - 1.
    static constexpr int AHEAD = AHEAD_;
    static constexpr int NSLOT = AHEAD + 2;
    static_assert(NSLOT % 2 == 0, "exchange parity follows the slot index");
    static constexpr int FB = CH ? DK * 4 : 4 * CK * 4;
    static constexpr int szK = CK * DK * ES, szV = CK * BV * ES, szT = CK * CK * ES, szF = align16(FB);
    // regions, each NSLOT slots
    static constexpr int rK = 0;                                   // K or K.exp(G)
    static constexpr int rKU = rK + NSLOT * szK;                   // K.exp(G_C - G) (channel)
    static constexpr int rQ = rKU + (CH ? NSLOT * szK : 0);        // Q or Q.exp(G)
    static constexpr int rV = rQ + NSLOT * szK;                    // V block
    static constexpr int rT = rV + NSLOT * szV;                    // T~
    static constexpr int rM = rT + NSLOT * szT;                    // Gamma or P
    static constexpr int rF = rM + NSLOT * szT;
    // exchange buffers (two chunks deep): S and U operands of each state owner
    static constexpr int NKS = DK / 32;
    static constexpr int FS = (int)sizeof(Frag<E>);
    static constexpr int XSB = 2 * NKS * kWave * FS, XUB = 2 * kWave * FS;   // one chunk's worth
    static constexpr int rxS = rF + NSLOT * szF;                   // [parity][owner][ks][lane]
    static constexpr int rxU = rxS + 2 * XSB;                      // [parity][owner][lane]
    static constexpr int bytes = rxU + 2 * XUB;
    // copier waves of the forward scan: four for bf16 operands with channel
    // alpha (whose 30 KiB of copies per step bound the step with two), else two
    static constexpr int NCP = (CH && ES == 2) ? 4 : 2;
    static constexpr int NWAVES = 4 + NCP;
    // copy instructions per chunk.  Two copiers: copier 0 takes K (and
    // K.exp(G_C - G)) and the decay factors, plus V and T~ unless alpha is per
    // channel; copier 1 the rest, which keeps the two within a few KiB of each
    // other.  Four copiers (channel alpha): K.exp(G) | K.exp(G_C - G) and the
    // decay factors | Q.exp(G) | V, T~ and P.
    static constexpr int NCK = CopyCount<szK>::n, NCV = CopyCount<szV>::n, NCT = CopyCount<szT>::n;
    static constexpr int NCF = CopyCount<FB>::n;
    static constexpr int NOPS0 = (CH ? 2 : 1) * NCK + NCF + (CH ? 0 : NCV + NCT);
    static constexpr int NOPS1 = NCK + NCT + (CH ? NCV + NCT : 0);
    static_assert(NOPS0 < 64 && NOPS1 < 64, "vmcnt range");
};

}  // namespace gdr

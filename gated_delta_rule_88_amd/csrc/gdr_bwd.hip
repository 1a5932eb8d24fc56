// gdr_bwd.hip -- chunked backward (the gradients training needs) of the
// gated delta-rule memory, for alpha = 1, scalar alpha and channel alpha.
//
// Forward over one chunk of C tokens with entry state S0 (notation of
// gdr_scan.hip; g = in-chunk cumulative log alpha, gamma = e^g,
// D = e^{g_C - g}, Gamma_rs = e^{g_r - g_s}):
//   A = strictly-lower(diag(beta)(K K^T . Gamma)),  T = (I + A)^{-1},
//   T~ = T diag(beta),  X = K S0^T,  R = V - diag(gamma) X,  U = T~ R,
//   P = Q K^T . Gamma . M_incl,  O = diag(gamma) Q S0^T + P U,
//   S_end = gamma_C S0 + U^T diag(D) K.
// Reverse mode, given dO and dS_end (derived by the chain rule from these
// lines; the per-token form is the fp64 oracle's):
//   dU = P^T dO + diag(D) K dS_end^T,   dR = T~^T dU,   dV = dR,
//   dX = -diag(gamma) dR,
//   dS0 = gamma_C dS_end + dO^T diag(gamma) Q + dX^T K            (the chain)
//   dQ = diag(gamma) dO S0 + (dO U^T . Gamma . M_incl) K
//   dK = (dO U^T . Gamma . M_incl)^T Q + diag(D) U dS_end + dX S0 + dG K + dG^T K
//   with dT~ = dU R^T, dbeta_s = sum_r T_rs dT~_rs + sum_s' dA_ss' (K K^T . Gamma)_ss',
//   dA = strictly-lower(-T^T (dT~ diag(beta)) T^T), dG = dA . diag(beta) Gamma,
//   and for the log-decay every place g enters (gamma, D, gamma_C, Gamma)
//   gives a term of dg; d log alpha_t = sum_{r >= t} dg_r within the chunk.
// ("linear attention and its gated descendants", "Chunkwise Parallel Form"
// and "Gated DeltaNet"; the WY factor of "Linear Attention & DeltaNet",
// "How it works", item 3.)
//
// Launches: the forward prepass and scan run again (the prepass also keeping
// every chunk's T, the scan the entry states the gradient walk starts from:
// every chunk's, or for bf16 on 32-token steps the state entering each run
// of chunks), unless a keeping forward left them; then
//   chunk_bwd_chain_kernel  one workgroup per (b, h, 32 value channels)
//                           walks the chunks backwards carrying dS and
//                           keeps dS_end of every chunk (the pipelined form
//                           for bf16 on 32-token steps is in
//                           gdr_bwd_chain.hip);
//   chunk_bwd_grad_kernel   every gradient of a chunk's tokens from S0,
//                           dS_end and its inputs: for bf16 on 32-token
//                           steps one workgroup per run of consecutive
//                           chunks, carrying the state across it; otherwise
//                           persistent, one workgroup per CU walking the
//                           chunks (chunk_bwd_grad_channel_kernel for
//                           channel alpha, whose chunk algebra is written
//                           out above it).
// The products run on MFMA (bf16 operands for bf16 inputs, fp32 otherwise;
// fp32 accumulation); the triangular parts (T, dA) stay in fp32.
#include "gdr_device.h"
#include "gdr_chunk.h"
#include "gdr_bwd.h"

namespace gdr {

namespace {

constexpr int kBV = 32;   // value channels per block

template <typename E>
__device__ __forceinline__ void pack_frag(Frag<E>& f, const float* x);
template <>
__device__ __forceinline__ void pack_frag<bf16>(Frag<bf16>& f, const float* x) {
    f.v = __builtin_bit_cast(bf16x8, Pack<bf16>::pack(x));
}
template <>
__device__ __forceinline__ void pack_frag<float>(Frag<float>& f, const float* x) {
    f.lo = f32x4{x[0], x[1], x[2], x[3]};
    f.hi = f32x4{x[4], x[5], x[6], x[7]};
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): two bf16 operands
// that carry about 16 bits of x.
__device__ __forceinline__ void split_frag(const float* x, Frag<bf16>& hi, Frag<bf16>& lo) {
    float h[8], r[8];
    const u32x4 hv = Pack<bf16>::pack(x);
    Pack<bf16>::unpack(hv, h);
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = x[j] - h[j];
    hi.v = __builtin_bit_cast(bf16x8, hv);
    lo.v = __builtin_bit_cast(bf16x8, Pack<bf16>::pack(r));
}

// 8 consecutive elements of a row as floats (16-byte aligned reads), zero
// when they lie at or past K.
__device__ __forceinline__ void load8f(const bf16* p, float* x) { Pack<bf16>::unpack(ld16(p), x); }
__device__ __forceinline__ void load8f(const float* p, float* x) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// A value the compiler cannot see through.  A persistent kernel derives its
// lane index from it once per chunk and passes that lane to the fragment
// loads, so that the address arithmetic built on it is not hoisted out of
// the chunk loop (which would hold every such address in a register
// throughout).
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Operand fragment of a row-major [rows][ld] array (contraction index
// contiguous): lane reads row row0 + l % 16, k = k0 + 8 (l / 16) .. + 7.
template <typename E, typename T>
__device__ __forceinline__ Frag<E> cfrag(const T* base, int ld, int row0, int k0, int K, int l = lane_id()) {
    const int k = k0 + 8 * (l >> 4);
    const T* p = base + (row0 + (l & 15)) * ld + k;
    Frag<E> f;
    if constexpr (sizeof(E) == 2 && sizeof(T) == 2) {
        f.v = k < K ? *reinterpret_cast<const bf16x8*>(p) : bf16x8{};
    } else {
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (k < K) load8f(p, x);
        pack_frag<E>(f, x);
    }
    return f;
}

// acc += A B^T on one 16 x 16 tile, A = rows m0.. of a row-major [.][lda]
// array, B = rows n0.. of [.][ldb], contracting over k < K (a multiple of 8,
// zero-filled to the next multiple of 32).  Lane (g, c) ends with
// acc[e] = (A B^T)[m0 + 4 g + e][n0 + c].
template <typename E, typename TA, typename TB>
__device__ __forceinline__ void tmma(f32x4& acc, const TA* A, int lda, int m0, const TB* B, int ldb, int n0,
                                     int K, int l = lane_id())
{
    for (int k0 = 0; k0 < K; k0 += 32) mma(acc, cfrag<E>(A, lda, m0, k0, K, l), cfrag<E>(B, ldb, n0, k0, K, l));
}

// Sum of x over the 16 lanes that share l / 16 (one tile row), in every
// one of them: four DPP moves (swap neighbours, swap pairs, mirror the half
// rows, mirror the rows), no LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm(1, 0, 3, 2)
    x += dpp_mov<0x4E>(x);    // quad_perm(2, 3, 0, 1)
    x += dpp_mov<0x141>(x);   // row_half_mirror
    x += dpp_mov<0x140>(x);   // row_mirror
    return x;
}

// Lanes l and l ^ 1 hold the bf16 entries c .. c + 7 of rows r and r ^ 1,
// packed in v.  Stores them transposed, dst[(c + j) * LT + r], as 4-byte words
// that hold both rows: the two lanes trade halves (a DPP swap of neighbouring
// lanes), then the even lane writes columns c .. c + 3 and the odd lane
// c + 4 .. c + 7 -- half the stores of 2-byte writes, and no two lanes write
// into one word.  Both lanes of a pair must be active; LT is even.
__device__ __forceinline__ void store_t_pair(bf16* dst, int LT, int r, int c, u32x4 v, int l) {
    const bool odd = l & 1;
    const uint32_t s0 = odd ? v.x : v.z, s1 = odd ? v.y : v.w;   // for the partner
    const uint32_t m0 = odd ? v.z : v.x, m1 = odd ? v.w : v.y;   // kept
    const uint32_t p0 = __builtin_amdgcn_mov_dpp((int)s0, 0xB1, 0xF, 0xF, false);   // quad_perm(1, 0, 3, 2)
    const uint32_t p1 = __builtin_amdgcn_mov_dpp((int)s1, 0xB1, 0xF, 0xF, false);
    const uint32_t a0 = odd ? p0 : m0, a1 = odd ? p1 : m1;   // row r & ~1
    const uint32_t b0 = odd ? m0 : p0, b1 = odd ? m1 : p1;   // row r | 1
    uint32_t* d = reinterpret_cast<uint32_t*>(dst + (c + (odd ? 4 : 0)) * LT + (r & ~1));
    const int ld = LT / 2;
    d[0] = (a0 & 0xffffu) | (b0 << 16);
    d[ld] = (a0 >> 16) | (b0 & 0xffff0000u);
    d[2 * ld] = (a1 & 0xffffu) | (b1 << 16);
    d[3 * ld] = (a1 >> 16) | (b1 & 0xffff0000u);
}
// Row (over the tile's 16 columns) and column (over its 16 rows) sums of a
// 16 x 16 tile held as MFMA accumulators (lane (g, c): rows 4 g + e, column
// c), written to rowp[r] (lanes c = 0) and colp[c] (lanes g = 0).
template <bool ROWS, bool COLS>
__device__ __forceinline__ void tile_row_col_sums(const float (&v)[4], float* rowp, float* colp, int g4, int c16) {
    if constexpr (COLS) {
        float cs = (v[0] + v[1]) + (v[2] + v[3]);
        cs += __shfl_xor(cs, 16, kWave);
        cs += __shfl_xor(cs, 32, kWave);
        if (g4 == 0) colp[c16] = cs;
    }
    if constexpr (ROWS) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float rs = row16_sum(v[e]);
            if (c16 == 0) rowp[4 * g4 + e] = rs;
        }
    }
}

// Rows of a [ROWS][ld] global array into registers, 16 bytes per read, NT
// threads (every read of the stage in flight at once); rows at or past
// `valid` read as zero.  Then into LDS, plain [ROWS][COLS] (row stride LD)
// and transposed [COLS][ROWS] (row stride LT).  Consecutive threads take
// consecutive rows, so the transposed 2- or 4-byte stores of a wave land in
// consecutive LDS words.
template <typename E, int ROWS, int COLS, int NT>
struct RowStage {
    static constexpr int VE = Vec<E>::n, PER = COLS / VE, NV = (ROWS * PER + NT - 1) / NT;
    u32x4 v[NV];
    __device__ __forceinline__ void load(const E* src, int ld, int valid, int tid) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int x = tid + NT * j, r = x % ROWS, c = (x / ROWS) * VE;
            v[j] = u32x4{0u, 0u, 0u, 0u};
            if (x < ROWS * PER && r < valid) v[j] = ld16(src + (size_t)r * ld + c);
        }
    }
    // Prefetch form: every read unconditional, from row min(r, valid - 1)
    // (valid >= 1) and a clamped vector index, so that issuing it never
    // waits; mask() zeroes the rows past valid once the data is used.
    __device__ __forceinline__ void prefetch(const E* src, int ld, int valid, int tid) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int x = min(tid + NT * j, ROWS * PER - 1), r = min(x % ROWS, valid - 1), c = (x / ROWS) * VE;
            v[j] = ld16(src + (size_t)r * ld + c);
        }
    }
    __device__ __forceinline__ void mask(int valid, int tid) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int x = tid + NT * j;
            if (x % ROWS >= valid) v[j] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(E* dst, int LD, E* dstT, int LT, int tid) const {
        store_plain(dst, LD, tid);
        store_t(dstT, LT, tid);
    }
    __device__ __forceinline__ void store_plain(E* dst, int LD, int tid) const {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int x = tid + NT * j, r = x % ROWS, c = (x / ROWS) * VE;
            if (x < ROWS * PER) st16(dst + r * LD + c, v[j]);
        }
    }
    __device__ __forceinline__ void store_t(E* dstT, int LT, int tid) const {
        if constexpr (sizeof(E) == 2 && ROWS % 2 == 0 && NT % 2 == 0) {
            // threads tid, tid ^ 1 hold rows r, r ^ 1 of the same columns
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int x = tid + NT * j, r = x % ROWS, c = (x / ROWS) * VE;
                if (x < ROWS * PER) store_t_pair(dstT, LT, r, c, v[j], tid);
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int x = tid + NT * j, r = x % ROWS, c = (x / ROWS) * VE;
            if (x < ROWS * PER) {
                E e[VE];
                __builtin_memcpy(e, &v[j], 16);
#pragma unroll
                for (int i = 0; i < VE; ++i) dstT[(c + i) * LT + r] = e[i];
            }
        }
    }
};


// LDS row strides: every row padded by 16 bytes, so that the 16 rows a
// fragment read touches (and the rows a transposed store walks) fall on
// different banks.
template <typename E, int DK, int CK>
struct Strides {
    static constexpr int PE = 16 / (int)sizeof(E);
    static constexpr int LDK = DK + PE;    // rows of d_k elements
    static constexpr int LCK = CK + PE;    // rows of CK elements
    static constexpr int LBV = kBV + PE;   // rows of kBV elements
    static constexpr int LF = CK + 4;      // fp32 rows of CK
    static constexpr int LBF = kBV + 4;    // fp32 rows of kBV
};

// ---------------------------------------------------------------- chain
// Two LDS buffers of one chunk's operands: the helper waves fill one with
// chunk n - 1 while the owner waves read chunk n from the other.  (Channel
// alpha: K holds K . exp(G_C - G), Kt and Qt the transposes of K . exp(G)
// and Q . exp(G), f holds exp(G_C) per key channel.)
template <typename E, int DK, int CK>
struct ChainLds : Strides<E, DK, CK> {
    using S = Strides<E, DK, CK>;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int b_K = 0;                               // [CK][LDK] E
    static constexpr int b_Kt = b_K + CK * S::LDK * ES;         // [DK][LCK] E
    static constexpr int b_Qt = b_Kt + DK * S::LCK * ES;        // [DK][LCK] E
    static constexpr int b_dOt = b_Qt + DK * S::LCK * ES;       // [kBV][LCK] E, dO^T
    static constexpr int b_gdOt = b_dOt + kBV * S::LCK * ES;    // (gamma . dO)^T
    static constexpr int b_Tt = b_gdOt + kBV * S::LCK * ES;     // [CK][LCK] E, T~^T
    static constexpr int b_Pt = b_Tt + CK * S::LCK * ES;        // [CK][LCK] E, P^T
    static constexpr int b_f = b_Pt + CK * S::LCK * ES;         // gamma [CK], D [CK], gamma_C
    static constexpr int NF = (2 * CK + 4 > DK ? 2 * CK + 4 : DK);
    static constexpr int bbytes = (b_f + NF * 4 + 15) / 16 * 16;
    static constexpr int off_w = 2 * bbytes;                    // per owner wave: dS [16][LDK], dU^T, -gamma dR^T [16][LCK]
    static constexpr int wbytes = 16 * S::LDK * ES + 2 * 16 * S::LCK * ES;
    static constexpr int bytes = off_w + 2 * wbytes;
};

// One 16-row block (rows r0 + l % 16) of a row-major [rows][DK] global array
// as MFMA operand fragments (lane group g: key channels 32 ks + 8 g .. + 7),
// zero at or past `valid`.
template <typename E, int DK>
struct RowFrags {
    static constexpr int NKS = DK / 32;
    Frag<E> f[NKS];
    // Reads row min(r0 + l % 16, rmax) unconditionally: a read under a
    // condition, or a select on its value, makes the compiler wait for it
    // where it is issued; rows past the end are zeroed by mask() once the
    // data is used.
    __device__ __forceinline__ void load(const E* base, int r0, int rmax, int l) {
        const int r = min(r0 + (l & 15), rmax), k = 8 * (l >> 4);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const E* src = base + (size_t)r * DK + 32 * ks + k;
            if constexpr (sizeof(E) == 2) {
                f[ks].v = *reinterpret_cast<const bf16x8*>(src);
            } else {
                f[ks].lo = *reinterpret_cast<const f32x4*>(src);
                f[ks].hi = *reinterpret_cast<const f32x4*>(src + 4);
            }
        }
    }
    __device__ __forceinline__ void mask(int r0, int valid, int l) {
        if (r0 + (l & 15) < valid) return;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (sizeof(E) == 2) f[ks].v = bf16x8{};
            else { f[ks].lo = zero4(); f[ks].hi = zero4(); }
        }
    }
    // Products of these fragments stay after this point (a prefetching loop
    // would otherwise let the compiler compute them right after the reads,
    // waiting for them there).
    __device__ __forceinline__ void pin() {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (sizeof(E) == 2) {
                asm volatile("" : "+v"(f[ks].v));
            } else {
                asm volatile("" : "+v"(f[ks].lo), "+v"(f[ks].hi));
            }
        }
    }
    // rows into LDS, plain [row][LD] and/or transposed [key channel][LT]
    __device__ __forceinline__ void store(E* dst, int LD, int r0, int l) const {
        const int r = r0 + (l & 15), k = 8 * (l >> 4);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            E* d = dst + r * LD + 32 * ks + k;
            if constexpr (sizeof(E) == 2) {
                st16(d, __builtin_bit_cast(u32x4, f[ks].v));
            } else {
                *reinterpret_cast<f32x4*>(d) = f[ks].lo;
                *reinterpret_cast<f32x4*>(d + 4) = f[ks].hi;
            }
        }
    }
    __device__ __forceinline__ void store_t(E* dstT, int LT, int r0, int l) const {
        const int r = r0 + (l & 15), k = 8 * (l >> 4);
        if constexpr (sizeof(E) == 2) {
            // lanes l, l ^ 1 hold rows r, r ^ 1 of the same key channels
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                store_t_pair(dstT, LT, r, 32 * ks + k, __builtin_bit_cast(u32x4, f[ks].v), l);
            return;
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            E e[8];
            if constexpr (sizeof(E) == 2) {
                __builtin_memcpy(e, &f[ks].v, 16);
            } else {
                __builtin_memcpy(e, &f[ks].lo, 16);
                __builtin_memcpy(e + 4, &f[ks].hi, 16);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) dstT[(32 * ks + k + j) * LT + r] = e[j];
        }
    }
};

// What a helper wave reads for one chunk.  Helpers 0, 1 (kb = 0, 1): row
// block kb of K (channel: of K . exp(G_C - G) and K . exp(G)) and, scalar
// alpha, the score tiles (kb, kb) and, helper 0, (1, 0) with the Q rows they
// need; helpers 2, 3: row block kb - 2 of Q (channel: Q . exp(G)), and
// halves of T~, P (channel), the dO block and the decay factors.
template <typename E, int DK, int CK, bool CH>
struct ChainIn {
    RowFrags<E, DK> kf;          // K rows
    RowFrags<E, DK> kg;          // channel: K . exp(G) rows
    RowFrags<E, DK> qa;          // Q rows (scalar helpers 0, 1: block kb; helpers 2, 3: block kb - 2)
    RowFrags<E, DK> qb;          // scalar, helper 0: Q rows 16 ..
    u32x4 tv, mv, ov;            // T~ vector; channel: P vector; dO vector
    float gv, fv;                // gamma of the dO vector's token; decay factor entry
    uint32_t gm[2][4];           // scalar: Gamma entries (raw bits) of the score tiles,
                                 // converted only when used so that reading them does not wait
    __device__ static __forceinline__ float gval(uint32_t x) {
        return __uint_as_float(sizeof(E) == 2 ? x << 16 : x);
    }
};

// dS (d_v x d_k per (b, h)) carried backwards over the chunks.  Owner waves
// 0, 1 each hold the dS rows of 16 value channels in registers and do the
// dependent products of a step (dU, dR, the dS update); helper waves 2 .. 5
// read chunk n - 1 from memory, stage it into the other LDS buffer and (scalar
// alpha) form its masked score block P = Q K^T . Gamma there, so a step costs
// one barrier and no staging on the owners' path.
template <typename E, int DK, int CK, bool CH>
__global__ __launch_bounds__(384, 1) void chunk_bwd_chain_kernel(BwdParams p)
{
    using LY = ChainLds<E, DK, CK>;
    using IN = ChainIn<E, DK, CK, CH>;
    constexpr int NJ = DK / 16, NB = CK / 16, VE = Vec<E>::n;
    constexpr int LDK = LY::LDK, LCK = LY::LCK;
    constexpr WsLayout WL = ws_layout((int)sizeof(E), DK, CK, CH ? kAlphaChannel : kAlphaScalar);
    constexpr int NRV = CK * CK / VE;            // 16-byte vectors of T~ (and of Gamma or P)
    constexpr int PERO = kBV / VE;               // 16-byte vectors per token of the dO block
    constexpr int NFV = CH ? DK : 2 * CK + 1;    // decay factor entries
    static_assert(NRV <= 128 && CK * PERO <= 128 && NFV <= 128, "two helper waves cover a chunk");
    extern __shared__ __align__(16) unsigned char smem[];
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int hr = w - 2;                        // helper role 0 .. 3
    const bool khelp = hr < 2;                   // helpers of K (and the scores)
    const int kb = khelp ? hr : hr - 2;          // the row block it handles
    const int nvb = p.DV / kBV;
    const int bh = blockIdx.x / nvb, v0 = (blockIdx.x % nvb) * kBV;
    const int i0 = v0 + 16 * w;   // owner: first value channel

#define BUF_E(name, n, off) E* name = reinterpret_cast<E*>(smem + ((n) & 1) * LY::bbytes + LY::off)

    // ---- helpers: read chunk n into registers
    auto load = [&](IN& in, int n, auto kh) __attribute__((always_inline)) {
        constexpr bool KH = decltype(kh)::value;
        const int valid = min(CK, p.L - n * CK);
        const size_t tok = (size_t)bh * p.L + (size_t)n * CK;
        const unsigned char* rec = p.ws + ((size_t)bh * p.NC + n) * WL.bytes;
        const E* qc = CH ? reinterpret_cast<const E*>(rec + WL.QG) : reinterpret_cast<const E*>(p.q) + tok * DK;
        const int rmax = CH ? CK - 1 : valid - 1;   // records are zero past the end
        if (16 * kb < CK) in.qa.load(qc, 16 * kb, rmax, l);
        if constexpr (KH) {
            if constexpr (CH) {
                // the forward's decayed operands (zero past the end of the sequence)
                if (16 * kb < CK) {
                    in.kf.load(reinterpret_cast<const E*>(rec + WL.KD), 16 * kb, CK - 1, l);
                    in.kg.load(reinterpret_cast<const E*>(rec + WL.KG), 16 * kb, CK - 1, l);
                }
            } else {
                if (16 * kb < CK) in.kf.load(reinterpret_cast<const E*>(p.k) + tok * DK, 16 * kb, rmax, l);
                if (NB == 2 && kb == 0) in.qb.load(qc, 16, rmax, l);
                // Gamma of the score tiles: tile 0 is (kb, kb), tile 1 (helper 0) is (1, 0)
                const E* mg = reinterpret_cast<const E*>(rec + WL.M);
                // (read unconditionally from an index clamped into the block: a
                // select on a loaded value would wait for the load here; the
                // entries a helper has no tile for are never used)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int rb = t == 0 ? kb : 1, ib = t == 0 ? kb : 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = min(16 * rb + 4 * g4 + e, CK - 1), s = min(16 * ib + c16, CK - 1);
                        const int idx = r * CK + col_of_tok(CK, s);
                        if constexpr (sizeof(E) == 2) in.gm[t][e] = reinterpret_cast<const unsigned short*>(mg)[idx];
                        else in.gm[t][e] = reinterpret_cast<const uint32_t*>(mg)[idx];
                    }
                }
            }
        } else {
            // (every read unconditional from a clamped index; the entries
            // past the ends are dropped or zeroed in stage)
            const int x = 64 * kb + l;
            in.tv = ld16(rec + WL.T + 16 * min(x, NRV - 1));
            if constexpr (CH) in.mv = ld16(rec + WL.M + 16 * min(x, NRV - 1));
            in.fv = reinterpret_cast<const float*>(rec + WL.F)[min(x, NFV - 1)];
            const int xo = min(x, CK * PERO - 1), r = xo % CK, c = (xo / CK) * VE;
            in.ov = ld16(reinterpret_cast<const E*>(p.dO) + (tok + min(r, valid - 1)) * p.DV + v0 + c);
            if constexpr (!CH) in.gv = reinterpret_cast<const float*>(rec + WL.F)[r];
        }
    };
    // ---- helpers: chunk n from registers into its LDS buffer
    auto stage = [&](IN& in, int n, auto kh) __attribute__((always_inline)) {
        constexpr bool KH = decltype(kh)::value;
        BUF_E(Ks, n, b_K); BUF_E(Kt, n, b_Kt); BUF_E(Qt, n, b_Qt); BUF_E(dOt, n, b_dOt);
        BUF_E(gdOt, n, b_gdOt); BUF_E(Tts, n, b_Tt); BUF_E(Pt, n, b_Pt);
        float* f = reinterpret_cast<float*>(smem + (n & 1) * LY::bbytes + LY::b_f);
        const int tvalid = min(CK, p.L - n * CK);
        const int valid = CH ? CK : tvalid;   // K and Q rows (records are zero past the end)
        if constexpr (KH) {
            if constexpr (!CH) {
                in.kf.pin();
                in.qa.pin();
                if (NB == 2) in.qb.pin();
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(in.gm[t][e]));
                in.kf.mask(16 * kb, valid, l);
                in.qa.mask(16 * kb, valid, l);
                if (NB == 2) in.qb.mask(16, valid, l);
            }
            if (16 * kb < CK) {
                in.kf.store(Ks, LDK, 16 * kb, l);
                (CH ? in.kg : in.kf).store_t(Kt, LCK, 16 * kb, l);
            }
            if constexpr (!CH) {
                // P = Q K^T . Gamma . M_incl on and below the diagonal, kept as
                // P^T: tile (kb, kb) and, helper 0, (1, 0); helper 1 zeroes
                // the tile above the diagonal
                if (16 * kb < CK) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int ks = 0; ks < DK / 32; ++ks) mma(acc, in.qa.f[ks], in.kf.f[ks]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 16 * kb + 4 * g4 + e, s = 16 * kb + c16;
                        Pt[s * LCK + r] = from_f32<E>(acc[e] * IN::gval(in.gm[0][e]));
                    }
                }
                if (NB == 2 && kb == 0) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int ks = 0; ks < DK / 32; ++ks) mma(acc, in.qb.f[ks], in.kf.f[ks]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 16 + 4 * g4 + e, s = c16;
                        Pt[s * LCK + r] = from_f32<E>(acc[e] * IN::gval(in.gm[1][e]));
                    }
                }
                if (NB == 2 && kb == 1)
#pragma unroll
                    for (int e = 0; e < 4; ++e) Pt[(16 + c16) * LCK + 4 * g4 + e] = from_f32<E>(0.f);
            }
        } else {
            in.qa.mask(16 * kb, valid, l);
            if (16 * kb < CK) in.qa.store_t(Qt, LCK, 16 * kb, l);
            const int x = 64 * kb + l;
            if (x < NRV) {
                const int r = (VE * x) / CK, mc0 = (VE * x) % CK;
                E te[VE], me[VE];
                __builtin_memcpy(te, &in.tv, 16);
                __builtin_memcpy(me, &in.mv, 16);
#pragma unroll
                for (int j = 0; j < VE; ++j) {
                    const int t = tok_of_col(CK, mc0 + j);
                    Tts[t * LCK + r] = te[j];
                    if constexpr (CH) Pt[t * LCK + r] = me[j];   // the score block, transposed
                }
            }
            if (x < NFV) f[x] = in.fv;   // gamma, D, gamma_C (channel: exp(G_C))
            if (x < CK * PERO) {
                const int r = x % CK, c = (x / CK) * VE;
                if constexpr (sizeof(E) == 2) {
                    // lanes l, l ^ 1 hold tokens r, r ^ 1 of the same value channels
                    const u32x4 dv = r < tvalid ? in.ov : u32x4{0u, 0u, 0u, 0u};
                    store_t_pair(dOt, LCK, r, c, dv, l);
                    if constexpr (!CH) {
                        float d[VE];
                        Pack<bf16>::unpack(dv, d);
#pragma unroll
                        for (int i = 0; i < VE; ++i) d[i] *= in.gv;
                        store_t_pair(gdOt, LCK, r, c, Pack<bf16>::pack(d), l);
                    }
                } else {
                    E d[VE];
                    __builtin_memcpy(d, &in.ov, 16);
                    if (r >= tvalid)
#pragma unroll
                        for (int i = 0; i < VE; ++i) d[i] = from_f32<E>(0.f);
#pragma unroll
                    for (int i = 0; i < VE; ++i) {
                        dOt[(c + i) * LCK + r] = d[i];
                        if constexpr (!CH) gdOt[(c + i) * LCK + r] = from_f32<E>(in.gv * to_f32(d[i]));
                    }
                }
            }
        }
    };

    // ---- owners: dS rows i0 + 4 g4 + e, key channels 16 jb + c16
    E* dSw = reinterpret_cast<E*>(smem + LY::off_w + (w & 1) * LY::wbytes);   // [16][LDK]
    E* dUt = dSw + 16 * LDK;                                                  // [16][LCK]
    E* dRt = dUt + 16 * LCK;                                                  // -gamma dR, [16][LCK]
    f32x4 dS[NJ];
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
        dS[jb] = zero4();
        if (w < 2 && p.dS_final)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dS[jb][e] = p.dS_final[((size_t)bh * p.DV + i0 + 4 * g4 + e) * DK + 16 * jb + c16];
    }
    auto own = [&](int n) __attribute__((always_inline)) {
        BUF_E(Ks, n, b_K); BUF_E(Kt, n, b_Kt); BUF_E(Qt, n, b_Qt); BUF_E(dOt, n, b_dOt);
        BUF_E(gdOt, n, b_gdOt); BUF_E(Tts, n, b_Tt); BUF_E(Pt, n, b_Pt);
        const float* gam = reinterpret_cast<const float*>(smem + (n & 1) * LY::bbytes + LY::b_f);
        const float* Dd = gam + CK;
        // keep dS at the chunk's end (through the wave's LDS rows, 16 bytes per store)
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) dSw[(4 * g4 + e) * LDK + 16 * jb + c16] = from_f32<E>(dS[jb][e]);
        wave_lds_fence();
        E* dsk = static_cast<E*>(p.dSck) + (((size_t)bh * p.NC + n) * p.DV + i0) * DK;
        constexpr int RVS = DK / VE;   // 16-byte vectors per dS row
#pragma unroll
        for (int j = 0; j < 16 * RVS / kWave; ++j) {
            const int v = l + kWave * j, r = v / RVS, c = (v % RVS) * VE;
            st16(dsk + (size_t)r * DK + c, ld16(dSw + r * LDK + c));
        }
        // dU = P^T dO + diag(D) K dS^T  (token r, value channel 16 w + c), kept as dU^T
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            f32x4 kds = zero4(), y = zero4();
            tmma<E>(kds, Ks, LDK, 16 * rb, dSw, LDK, 0, DK);
            tmma<E>(y, Pt, LCK, 16 * rb, dOt + 16 * w * LCK, LCK, 0, CK);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e;
                dUt[c16 * LCK + r] = from_f32<E>(y[e] + (CH ? 1.f : Dd[r]) * kds[e]);
            }
        }
        wave_lds_fence();
        // dR = T~^T dU, kept as -gamma dR (transposed)
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            f32x4 dr = zero4();
            tmma<E>(dr, Tts, LCK, 16 * rb, dUt, LCK, 0, CK);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e;
                dRt[c16 * LCK + r] = from_f32<E>(-(CH ? 1.f : gam[r]) * dr[e]);
            }
        }
        wave_lds_fence();
        // dS <- gamma_C dS + (gamma . dO)^T Q - (gamma . dR)^T K
        // (channel: dS Diag(exp(G_C)) + dO^T (Q . exp(G)) - dR^T (K . exp(G)))
        const float gC = CH ? 0.f : gam[2 * CK];
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
            f32x4 acc = dS[jb];
            const float sc = CH ? gam[16 * jb + c16] : gC;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] *= sc;
            tmma<E>(acc, (CH ? dOt : gdOt) + 16 * w * LCK, LCK, 0, Qt, LCK, 16 * jb, CK);
            tmma<E>(acc, dRt, LCK, 0, Kt, LCK, 16 * jb, CK);
            dS[jb] = acc;
        }
    };

    // One loop per role, each with one barrier per step (so that every wave
    // meets the same barriers), and one register set per helper: a chunk is
    // staged before the next one is read into it.  Separate loops keep each
    // role's prefetched registers apart, so the compiler never has to merge
    // them (which would wait for the reads in flight).
    if (w < 2) {
        __syncthreads();   // the last chunk staged
        for (int n = p.NC - 1; n >= 0; --n) {
            own(n);
            __syncthreads();   // chunk n consumed, chunk n - 1 staged
        }
    } else {
        // The two kinds of helper run loops of their own, for the same reason,
        // with one register set each: a chunk is staged before the next one
        // is read into it.  (Two sets, reading chunk n - 2 before staging
        // chunk n - 1, measured slower; two sets read two steps ahead of
        // staging, no faster.)
        auto helper = [&](auto kh) __attribute__((always_inline)) {
            IN in;
            load(in, p.NC - 1, kh);
            stage(in, p.NC - 1, kh);
            if (p.NC >= 2) load(in, p.NC - 2, kh);
            __syncthreads();
            // step n: stage chunk n - 1 (read during the previous step), read chunk n - 2
            for (int n = p.NC - 1; n >= 0; --n) {
                if (n >= 1) {
                    stage(in, n - 1, kh);
                    if (n >= 2) load(in, n - 2, kh);
                }
                __syncthreads();
            }
        };
        if (khelp) helper(std::true_type{});
        else helper(std::false_type{});
    }
#undef BUF_E
    if (w < 2 && p.dS0) {
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.dS0[((size_t)bh * p.DV + i0 + 4 * g4 + e) * DK + 16 * jb + c16] = dS[jb][e];
    }
}

// ------------------------------------------- value blocks, lean form (bf16, C = 32)
// The value-block pass of the gradient kernels for bf16 operands and 32-token
// chunks.  Per block of 32 value channels (scalar alpha; channel alpha uses
// K . exp(G) for the first K, K . exp(G_C - G) for the second and no gamma, D):
//   A: R = V - gamma . K S0^T (waves 0..3), dU = P^T dO + D . K dS^T (waves 4..7)
//   B: U = T~ R (waves 0..3, which then stage the next block into the free
//      buffer and read the one after it), dR = T~^T dU (waves 4..7, which
//      also store dv)
//   C: dO S0, dR S0, U dS, dO U^T, dU R^T accumulated (all waves)
// R, dU, U, dR are kept as [value channel][token] bf16 rows (one 8-byte store
// per result tile); every operand is a 16-byte row read or a transposing read
// (ds_read_b64_tr_b16) of a padded row-major tile, so no transposed copy is
// staged.  The block inputs are double-buffered; waves 0..3 hold the block
// after next in registers, so its reads have a whole block to land.
template <int DK>
struct LeanVB {
    static constexpr int LDK = DK + 8, LB = 40;       // padded row lengths (elements)
    static constexpr int SZS = 32 * LDK * 2, SZV = 32 * LB * 2;
    static constexpr int oS0 = 0, odS = SZS, oV = 2 * SZS, odO = 2 * SZS + SZV;
    static constexpr int IN = 2 * SZS + 2 * SZV;     // one buffer of block inputs
    static constexpr int SZX = 32 * LB * 2;          // one [32 v][32 tok] intermediate
    static constexpr int oR = 0, odU = SZX, oU = 2 * SZX, odR = 3 * SZX, XB = 4 * SZX;
    static constexpr int NS = 32 * DK / 8;           // 16-byte vectors of one state block
    static constexpr int NPS = NS / 256;             // of them per staging thread
    static constexpr int NPF = NPS + 1;              // registers per staging thread
};

__device__ __forceinline__ Frag<bf16> rowf(const unsigned char* p) {
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8, ld16(p));
    return f;
}
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Operand of X^T from a padded row-major bf16 tile X (row length LD): lane
// (g, c) holds X[row0 + 8g + j][col0 + c], j = 0..7 (two transposing reads:
// address lane (g, i) names row row0 + 8g + i/4 (+4), columns col0 + 4(i%4) ..)
template <int LD>
__device__ __forceinline__ Frag<bf16> trn(const unsigned char* tile, int row0, int col0, int l) {
    const int g = l >> 4, i = l & 15;
    const unsigned char* a = tile + ((row0 + 8 * g + (i >> 2)) * LD + col0 + 4 * (i & 3)) * 2;
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a)));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 8 * LD)));
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
    return f;
}
// X[row0 + 4g + e][col0 + c] in result-tile order (one transposing read)
template <int LD>
__device__ __forceinline__ f32x4 trc(const unsigned char* tile, int row0, int col0, int l) {
    const int g = l >> 4, i = l & 15;
    const unsigned char* a = tile + ((row0 + 4 * g + (i >> 2)) * LD + col0 + 4 * (i & 3)) * 2;
    const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a)));
    return f32x4{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
}
__device__ __forceinline__ bf16x2 bf2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }
__device__ __forceinline__ void st4bf(unsigned char* p, f32x4 x) {
    st8(p, u32x2{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3])});
}

// Block inputs held in registers by a staging thread t (0..255): dS vectors
// t + 256 i of the block, and vector t % 128 of V (t < 128) or dO.  (S0 comes
// from the carried state.)
template <int DK>
struct LeanPf {
    u32x4 r[LeanVB<DK>::NPF];
    int valid;      // token rows of the block's chunk
    int pn, pbh;    // the chunk the loads read: its index within its head, the head
    // position at chunk c (one division), then one chunk on (none)
    __device__ __forceinline__ void at(const BwdParams& p, int c) {
        c = __builtin_amdgcn_readfirstlane(c);
        pn = c % p.NC;
        pbh = c / p.NC;
    }
    __device__ __forceinline__ void step(const BwdParams& p) {
        if (++pn == p.NC) {
            pn = 0;
            ++pbh;
        }
    }
    // chunk c, which at() and step() have positioned
    __device__ __forceinline__ void load(const BwdParams& p, int c, int v0, int t) {
        using LV = LeanVB<DK>;
        constexpr int CK = 32;
        // the block's chunk arithmetic on the scalar unit
        c = __builtin_amdgcn_readfirstlane(c);
        v0 = __builtin_amdgcn_readfirstlane(v0);
        const int n = pn;
        valid = min(CK, p.L - n * CK);
        const size_t tok = (size_t)pbh * p.L + (size_t)n * CK;
        const bf16* ds = static_cast<const bf16*>(p.dSck) + ((size_t)c * p.DV + v0) * DK;
#pragma unroll
        for (int i = 0; i < LV::NPS; ++i) r[i] = ld16(ds + (uint32_t)(8 * (t + 256 * i)));
        // (uniform bases, 32-bit lane offsets: waves 0 and 1 read V, 2 and 3 dO)
        const int x = t & 127, row = min(x >> 2, valid - 1);
        const bool vw = __builtin_amdgcn_readfirstlane(t >> 6) < 2;
        const bf16* src = reinterpret_cast<const bf16*>(vw ? p.v : p.dO) + tok * p.DV + v0;
        r[LV::NPS] = ld16(src + (uint32_t)(row * p.DV + 8 * (x & 3)));
    }
    // into buffer b (rows of V and dO past the chunk's end as zeros)
    __device__ __forceinline__ void store(unsigned char* b, int t) const {
        using LV = LeanVB<DK>;
        constexpr int PR = DK / 8;   // vectors per state row
#pragma unroll
        for (int i = 0; i < LV::NPS; ++i) {
            const int x = t + 256 * i, row = x / PR, ch = x % PR;
            st16(b + LV::odS + (row * LV::LDK + 8 * ch) * 2, r[i]);
        }
        const int x = t & 127, row = x >> 2;
        st16(b + (t < 128 ? LV::oV : LV::odO) + (row * LV::LB + 8 * (x & 3)) * 2,
             row < valid ? r[LV::NPS] : u32x4{0u, 0u, 0u, 0u});
    }
};

// The state a gradient workgroup carries across its chunks (fp32, d_v <= 128
// in blocks of 32 value channels).  Block vb as S^T tiles t = w + 8 u of wave
// w: lane (g4, c16) holds S[16 (t / NJ) + c16][16 (t % NJ) + 4 g4 + e], e =
// 0..3 (value row within the block, key channel), so the key channel
// 16 (t % NJ) + .. is the same for every u.  (Indexed by block only in
// unrolled loops: every entry stays in registers.)
template <int DK>
struct LeanCarry {
    static constexpr int NJ = DK / 16, NQW = (2 * NJ + 7) / 8, MAXVB = 4;
    static_assert(2 * NJ == 8 * NQW, "every wave holds NQW tiles of a block");
    f32x4 s[MAXVB][NQW];
    // the state entering chunk c: S0 (null: zero) at a head's first chunk,
    // else the kept entry c / span (c a multiple of span)
    __device__ __forceinline__ void load(const BwdParams& p, int c, int w, int l) {
        const int g4 = l >> 4, c16 = l & 15, nvb = p.DV / 32;
        const bool first = c % p.NC == 0;
        const size_t row0 = first ? (size_t)(c / p.NC) * p.DV : (size_t)(c / p.span) * p.DV;
#pragma unroll
        for (int vb = 0; vb < MAXVB; ++vb)
#pragma unroll
            for (int u = 0; u < NQW; ++u) {
                const int t = w + 8 * u;
                const size_t e0 = (row0 + 32 * vb + 16 * (t / NJ) + c16) * DK + 16 * (t % NJ) + 4 * g4;
                f32x4 x = zero4();
                if (vb < nvb) {
                    if (!first) {
                        const u32x2 b = *reinterpret_cast<const u32x2*>(static_cast<const bf16*>(p.Sck) + e0);
                        x = f32x4{bf_lo(b.x), bf_hi(b.x), bf_lo(b.y), bf_hi(b.y)};
                    } else if (p.S0) {
                        x = *reinterpret_cast<const f32x4*>(p.S0 + e0);
                    }
                }
                s[vb][u] = x;
            }
        // s_waitcnt vmcnt(0) as an instruction the compiler tracks: the
        // carried registers leave here complete, so no later use of them
        // waits for the loads in flight then
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    // block vb (a constant once unrolled; bf16) into the S0 slot of input buffer b
    __device__ __forceinline__ void stage(int vb, unsigned char* b, int w, int l) const {
        using LV = LeanVB<DK>;
        const int g4 = l >> 4, c16 = l & 15;
#pragma unroll
        for (int u = 0; u < NQW; ++u) {
            const int t = w + 8 * u;
            st4bf(b + LV::oS0 + ((16 * (t / NJ) + c16) * LV::LDK + 16 * (t % NJ) + 4 * g4) * 2, s[vb][u]);
        }
    }
};

// One chunk's value blocks in the lean form, NVB = d_v / 32 of them (2 or 4,
// unrolled; block vb in input buffer vb & 1).  On entry buffer 0 holds block
// (cid, 0) and pf the block after it, (pc, pv0), of the workgroup's run of
// chunks that ends before pend; car holds the state entering cid.  On exit car
// holds the state entering cid + 1 (its block 0 staged into buffer 0), and the
// same holds for the next chunk.  Results: a1 += dO S0, a2 += dR S0,
// a3 += U dS (tiles t = w + 8u, rows 16 (t / NJ), key channels 16 (t % NJ)),
// dPa += dO U^T, dTa += dU R^T (tile w < 4), hs[e] += S0 . dS over this
// thread's key channels 8 (tid / 32) + e (SC: only their sum counts, kept in
// hs[0..3] by channel pairs), and dv.  SC: scalar alpha (gamma, D); else channel alpha
// (Kx = K . exp(G), Kd = K . exp(G_C - G), no per-token factors).  The state
// moves on as S <- dec . S + U^T (D . K): dec = gamma_C, or exp(G_C) of this
// lane's key channels 16 (w % NJ) + 4 g4 + e; kdf = the X^T operand of D . K
// (Kd for channel alpha) for key channels 16 (w % NJ) ..
template <int DK, bool SC, int NQW, int NVB>
__device__ __forceinline__ void lean_value_blocks(
    const BwdParams& p, unsigned char* smem, int in_off, int lx_off, const bf16* Kx, const bf16* Kd,
    const bf16* Pt, const bf16* Tt, const bf16* Ttt, const float* gam, const float* Dd, int cid, int tid,
    LeanPf<DK>& pf, int& pc, int& pv0, int pend, LeanCarry<DK>& car, const Frag<bf16>& kdf,
    f32x4 dec, f32x4* a1, f32x4* a2, f32x4* a3, f32x4& dPa, f32x4& dTa, float* hs)
{
    using LV = LeanVB<DK>;
    constexpr int CK = 32, NJ = DK / 16, NKS = DK / 32, NW = 8, NQT = 2 * NJ;
    static_assert(NQT == NW * NQW, "every wave holds NQW of the C x d_k tiles");
    constexpr int LDK = LV::LDK, LB = LV::LB;
    const int l = tid & 63, g4 = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = cid % p.NC, valid = min(CK, p.L - n * CK);
    const size_t tok = (size_t)(cid / p.NC) * p.L + (size_t)n * CK;
    const unsigned char* kx = reinterpret_cast<const unsigned char*>(Kx);
    const unsigned char* kd = reinterpret_cast<const unsigned char*>(Kd);
    const unsigned char* pt = reinterpret_cast<const unsigned char*>(Pt);
    const unsigned char* tf = reinterpret_cast<const unsigned char*>(Tt);
    const unsigned char* tft = reinterpret_cast<const unsigned char*>(Ttt);
    unsigned char* xb = smem + lx_off;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
        const int v0 = 32 * vb;
        const unsigned char* ib = smem + in_off + (vb & 1) * LV::IN;
        // the next block's S0 into the free buffer (after the last block:
        // block 0 of the next chunk, whose step was taken in block 0)
        car.stage((vb + 1) % NVB, smem + in_off + ((vb + 1) & 1) * LV::IN, w, l);
        // ---- A: R = V - gamma . K S0^T (waves 0..3), dU = P^T dO + D . K dS^T
        // (waves 4..7); tile (tokens 16 tt .., value channels 16 cb ..)
        {
            const int q = w & 3, tt = q & 1, cb = q >> 1;
            const bool rw = w < 4;
            const unsigned char* ka = (rw ? kx : kd) + ((16 * tt + c16) * LDK + 8 * g4) * 2;
            const unsigned char* sa = ib + (rw ? LV::oS0 : LV::odS) + ((16 * cb + c16) * LDK + 8 * g4) * 2;
            f32x4 x = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) mma(x, rowf(ka + 64 * ks), rowf(sa + 64 * ks));
            f32x4 y;
            if (rw) {
                const f32x4 vv = trc<LB>(ib + LV::oV, 16 * tt, 16 * cb, l);
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = vv[e] - (SC ? gam[16 * tt + 4 * g4 + e] : 1.f) * x[e];
            } else {
                y = zero4();
                mma(y, rowf(pt + ((16 * tt + c16) * LB + 8 * g4) * 2), trn<LB>(ib + LV::odO, 0, 16 * cb, l));
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] += (SC ? Dd[16 * tt + 4 * g4 + e] : 1.f) * x[e];
            }
            st4bf(xb + (rw ? LV::oR : LV::odU) + ((16 * cb + c16) * LB + 16 * tt + 4 * g4) * 2, y);
        }
        __syncthreads();
        // ---- B: U = T~ R (waves 0..3), dR = T~^T dU (waves 4..7, = dv)
        {
            const int q = w & 3, tt = q & 1, cb = q >> 1;
            const bool up = w < 4;
            f32x4 z = zero4();
            mma(z, rowf((up ? tf : tft) + ((16 * tt + c16) * LB + 8 * g4) * 2),
                rowf(xb + (up ? LV::oR : LV::odU) + ((16 * cb + c16) * LB + 8 * g4) * 2));
            st4bf(xb + (up ? LV::oU : LV::odR) + ((16 * cb + c16) * LB + 16 * tt + 4 * g4) * 2, z);
            // waves 0..3: the next block into the free buffer (its reads were
            // issued a block ago), then read the one after it
            // (the block position advances on every wave: scalar arithmetic)
            if (pc < pend) {
                if (up) pf.store(smem + in_off + ((vb + 1) & 1) * LV::IN, tid);
                if (pv0 + 32 < p.DV) {
                    pv0 += 32;
                } else {
                    pv0 = 0;
                    ++pc;
                    pf.step(p);
                }
                if (up && pc < pend) pf.load(p, pc, pv0, tid);
            }
            if (!up) {
                // token 16 tt + 4 g4 + c16 % 4, value channels 16 cb + 4 (c16 / 4) ..
                // (a uniform base and a 32-bit lane offset)
                const f32x4 zt = quad_transpose(z);
                const int r = 16 * tt + 4 * g4 + (c16 & 3);
                bf16* dvb = reinterpret_cast<bf16*>(p.dv) + tok * p.DV + v0;
                if (r < valid)
                    st4(dvb + (uint32_t)(r * p.DV + 16 * cb + 4 * (c16 >> 2)), zt[0], zt[1], zt[2], zt[3]);
            }
        }
        __syncthreads();
        // ---- C: the carried state of this block over the chunk (S^T tiles:
        // key channels 16 (w % NJ) .., value rows 16 rt ..), then accumulate
        // over the block's value channels
#pragma unroll
        for (int u = 0; u < NQW; ++u) {
            const int rt = (w + NW * u) / NJ;
            f32x4 x = car.s[vb][u];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] *= dec[e];
            mma(x, kdf, rowf(xb + LV::oU + ((16 * rt + c16) * LB + 8 * g4) * 2));
            car.s[vb][u] = x;
        }
#pragma unroll
        for (int u = 0; u < NQW; ++u) {
            const int t = w + NW * u, rb = t / NJ, jb = t % NJ;   // (t < NQT: every wave has NQW tiles)
            const Frag<bf16> ado = rowf(ib + LV::odO + ((16 * rb + c16) * LB + 8 * g4) * 2);
            const Frag<bf16> adr = trn<LB>(xb + LV::odR, 0, 16 * rb, l);
            const Frag<bf16> au = trn<LB>(xb + LV::oU, 0, 16 * rb, l);
            const Frag<bf16> bs0 = trn<LDK>(ib + LV::oS0, 0, 16 * jb, l);
            const Frag<bf16> bds = trn<LDK>(ib + LV::odS, 0, 16 * jb, l);
            mma(a1[u], ado, bs0);
            mma(a2[u], adr, bs0);
            mma(a3[u], au, bds);
        }
        if (w < 4) {
            const int rb = w >> 1, sb = w & 1;
            mma(dPa, rowf(ib + LV::odO + ((16 * rb + c16) * LB + 8 * g4) * 2), trn<LB>(xb + LV::oU, 0, 16 * sb, l));
            mma(dTa, trn<LB>(xb + LV::odU, 0, 16 * rb, l), trn<LB>(xb + LV::oR, 0, 16 * sb, l));
        }
        if (tid < 32 * DK / 8) {
            const int i = tid & 31, j = 8 * (tid >> 5);
            const u32x4 sa = ld16(ib + LV::oS0 + (i * LDK + j) * 2), sb = ld16(ib + LV::odS + (i * LDK + j) * 2);
            if constexpr (SC) {
                // only the total is used: pairs of channels by bf16 dot products
                // (each bf16 product is exact in fp32)
                hs[0] = __builtin_amdgcn_fdot2_f32_bf16(bf2(sa.x), bf2(sb.x), hs[0], false);
                hs[1] = __builtin_amdgcn_fdot2_f32_bf16(bf2(sa.y), bf2(sb.y), hs[1], false);
                hs[2] = __builtin_amdgcn_fdot2_f32_bf16(bf2(sa.z), bf2(sb.z), hs[2], false);
                hs[3] = __builtin_amdgcn_fdot2_f32_bf16(bf2(sa.w), bf2(sb.w), hs[3], false);
            } else {
                // per channel: S0 with its other channel masked to zero
                const uint32_t av[4] = {sa.x, sa.y, sa.z, sa.w}, bv[4] = {sb.x, sb.y, sb.z, sb.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hs[2 * e] = __builtin_amdgcn_fdot2_f32_bf16(bf2(av[e] & 0xffffu), bf2(bv[e]), hs[2 * e], false);
                    hs[2 * e + 1] =
                        __builtin_amdgcn_fdot2_f32_bf16(bf2(av[e] & 0xffff0000u), bf2(bv[e]), hs[2 * e + 1], false);
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- grads
template <typename E, int DK, int CK>
struct GradLds : Strides<E, DK, CK> {
    using S = Strides<E, DK, CK>;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int FCC = CK * S::LF * 4, ECC = CK * S::LCK * ES;
    static constexpr int ECB = CK * S::LBV * ES, EBC = kBV * S::LCK * ES, FCB = CK * S::LBF * 4;
    // kept for the whole chunk
    static constexpr int off_K = 0;                            // [CK][LDK] E and [DK][LCK]
    static constexpr int off_Kt = off_K + CK * S::LDK * ES;
    static constexpr int off_Q = off_Kt + DK * S::LCK * ES;
    static constexpr int off_Qt = off_Q + CK * S::LDK * ES;
    static constexpr int off_Bm = off_Qt + DK * S::LCK * ES;   // [CK][LF] f32: K K^T . Gamma (strict)
    static constexpr int off_A = off_Bm + FCC;                 //   A
    static constexpr int off_T = off_A + FCC;                  //   T
    static constexpr int off_Tft = off_T + FCC;                //   T^T
    static constexpr int off_P = off_Tft + FCC;                //   P
    static constexpr int off_Tt = off_P + FCC;                 // [CK][LCK] E: T~, T~^T, P^T
    static constexpr int off_Ttt = off_Tt + ECC;
    static constexpr int off_Pt = off_Ttt + ECC;
    static constexpr int off_vec = off_Pt + ECC;               // g, gamma, D, beta, dg [CK]; parts
    static constexpr int NVEC = 5 * CK + 16 * CK + 8 + 6 * (CK / 16) * CK;
    // one block of value channels (reused by the last phase)
    static constexpr int off_blk = (off_vec + NVEC * 4 + 15) / 16 * 16;
    static constexpr int off_S0 = off_blk;                     // [kBV][LDK] E and [DK][LBV]
    static constexpr int off_S0t = off_S0 + kBV * S::LDK * ES;
    static constexpr int off_dS = off_S0t + DK * S::LBV * ES;
    static constexpr int off_dSt = off_dS + kBV * S::LDK * ES;
    static constexpr int off_dO = off_dSt + DK * S::LBV * ES;  // [CK][LBV] E
    static constexpr int off_gdO = off_dO + ECB;
    static constexpr int off_R = off_gdO + ECB;
    static constexpr int off_U = off_R + ECB;
    static constexpr int off_dU = off_U + ECB;
    static constexpr int off_dX = off_dU + ECB;
    static constexpr int off_dOt = off_dX + ECB;               // [kBV][LCK] E
    static constexpr int off_Rt = off_dOt + EBC;
    static constexpr int off_dUt = off_Rt + EBC;
    static constexpr int off_V = off_dUt + EBC;                // [CK][LBF] f32
    static constexpr int blk_end = off_V + FCB;
    // the last phase, over the block region
    // bf16, C = 32: double-buffered block inputs, then the tail region (whose
    // start also holds the block intermediates during the value loop)
    static constexpr bool LEAN = (ES == 2 && CK == 32);
    static constexpr int off_lean = off_blk;
    static constexpr int off_tail = LEAN ? off_blk + 2 * LeanVB<DK>::IN : off_blk;
    static constexpr int off_lx = off_tail;
    static constexpr int off_dTt = off_tail;                   // [CK][LF] f32
    static constexpr int off_dTb = off_dTt + FCC;
    static constexpr int off_Em = off_dTb + FCC;
    static constexpr int off_Y1t = off_Em + FCC;
    static constexpr int off_dA = off_Y1t + FCC;
    static constexpr int off_dPW = off_dA + FCC;               // [CK][LCK] E
    static constexpr int off_dPWt = off_dPW + ECC;
    static constexpr int off_dG = off_dPWt + ECC;
    static constexpr int off_dGt = off_dG + ECC;
    static constexpr int last_end = off_dGt + ECC;
    static constexpr int lx_end = off_lx + LeanVB<DK>::XB;
    static constexpr int m0 = LEAN ? (lx_end > last_end ? lx_end : last_end) : (blk_end > last_end ? blk_end : last_end);
    static constexpr int bytes = m0;
};

// NVB: value blocks of 32 channels (d_v / 32) for the lean form, whose
// value-block loop is unrolled; 0 for the other forms
template <typename E, int DK, int CK, int NVB>
__global__ __launch_bounds__(512) void chunk_bwd_grad_kernel(BwdParams p)
{
    using LY = GradLds<E, DK, CK>;
    static_assert(LY::LEAN ? (NVB == 2 || NVB == 4) : NVB == 0, "value blocks of the lean form");
    constexpr int NB = CK / 16, NJ = DK / 16, VE = Vec<E>::n;
    constexpr int LF = LY::LF, LDK = LY::LDK, LCK = LY::LCK, LBV = LY::LBV, LBF = LY::LBF;
    constexpr int NT = 512, NW = NT / kWave;     // 8 waves
    constexpr int NQT = NB * NJ;                 // C x DK tiles
    constexpr int NQW = (NQT + NW - 1) / NW;     // per wave
    constexpr bool FULLQ = NQT == NW * NQW;      // every wave holds NQW tiles (no test needed)
    constexpr int NCB = NB * (kBV / 16);         // C x kBV tiles (<= 4)
    constexpr int NCC = NB * NB;                 // C x C tiles (<= 4)
    extern __shared__ __align__(16) unsigned char smem[];
#define GL_E(name, off) E* name = reinterpret_cast<E*>(smem + LY::off)
#define GL_F(name, off) float* name = reinterpret_cast<float*>(smem + LY::off)
    GL_E(Ks, off_K); GL_E(Kt, off_Kt); GL_E(Qs, off_Q); GL_E(Qt, off_Qt);
    GL_F(Bm, off_Bm); GL_F(Af, off_A); GL_F(Tf, off_T); GL_F(Tft, off_Tft); GL_F(Pf, off_P);
    GL_E(Tt, off_Tt); GL_E(Ttt, off_Ttt); GL_E(Pt, off_Pt);
    GL_E(S0s, off_S0); GL_E(S0t, off_S0t); GL_E(dSs, off_dS); GL_E(dSt, off_dSt);
    GL_E(dOs, off_dO); GL_E(gdOs, off_gdO); GL_E(Rs, off_R); GL_E(Us, off_U);
    GL_E(dUs, off_dU); GL_E(dXs, off_dX); GL_E(dOt, off_dOt); GL_E(Rt, off_Rt); GL_E(dUt, off_dUt);
    GL_F(Vs, off_V);
    GL_F(dTt, off_dTt); GL_F(dTb, off_dTb); GL_F(Em, off_Em); GL_F(Y1t, off_Y1t); GL_F(dAf, off_dA);
    GL_E(dPW, off_dPW); GL_E(dPWt, off_dPWt); GL_E(dGf, off_dG); GL_E(dGt, off_dGt);
#undef GL_E
#undef GL_F
    float* gs = reinterpret_cast<float*>(smem + LY::off_vec);
    float* gam = gs + CK;
    float* Dd = gam + CK;
    float* bs = Dd + CK;
    float* dg = bs + CK;
    float* hgp = dg + CK;        // [8][CK] per-wave partial sums of the gamma terms
    float* frp = hgp + 8 * CK;   // [8][CK] per-wave partial sums of the D terms
    float* red = frp + 8 * CK;   // [8]: per-wave <dS_end, S0>
    // per-tile row ([tile column block][row]) and column ([tile row
    // block][column]) sums of the C x C terms: dP . P (eR, eC), dA . A (fR,
    // fC), T . dT~ (tC, columns) and dA . Bm (aR, rows)
    float* eR = red + 8;
    float* eC = eR + NB * CK;
    float* fR = eC + NB * CK;
    float* fC = fR + NB * CK;
    float* tC = fC + NB * CK;
    float* aR = tC + NB * CK;

    // Each workgroup walks chunks blockIdx.x, + gridDim.x, ...; the next
    // chunk's keys, queries, gates and first value block are read into
    // registers while the current chunk is worked on.
    RowStage<E, CK, DK, NT> ks, qs;
    float lav = 0.f, btv = 0.f;
    // (every read unconditional, from clamped indices: a read under a
    // condition, or a select on its value, would wait for it right here;
    // the entries past the chunk's end are zeroed where they are used)
    // and 16 bytes of the chunk's T (from the forward's prepass) per thread
    f32x4 tv;
    auto fetch_chunk = [&](int c, int tid) {
        const int n = c % p.NC, valid = min(CK, p.L - n * CK);
        const size_t tok = (size_t)(c / p.NC) * p.L + (size_t)n * CK;
        ks.prefetch(reinterpret_cast<const E*>(p.k) + tok * DK, DK, valid, tid);
        qs.prefetch(reinterpret_cast<const E*>(p.q) + tok * DK, DK, valid, tid);
        tv = *reinterpret_cast<const f32x4*>(p.Tck + (size_t)c * CK * CK + 4 * min(tid, CK * CK / 4 - 1));
        const size_t t = tok + min(tid, valid - 1);
        btv = p.beta[t];
        lav = p.log_alpha ? p.log_alpha[t] : 0.f;
    };
    // one block of value channels: S0 and dS_end rows, V and dO columns.
    // Thread x takes row x % kBV, so the transposed stores of a wave are
    // consecutive.
    constexpr int NSV = (kBV * DK / VE + NT - 1) / NT;   // 16-byte vectors per thread and state
    constexpr int PERV = kBV / VE, NVV = (CK * PERV + NT - 1) / NT;
    u32x4 sa[NSV], sb[NSV], va[NVV], da[NVV];
    auto fetch_block = [&](int c, int v0, int tid) {
        const int n = c % p.NC, valid = min(CK, p.L - n * CK);
        const size_t tok = (size_t)(c / p.NC) * p.L + (size_t)n * CK;
        const E* S0g = static_cast<const E*>(p.Sck) + (size_t)c * p.DV * DK;
        const E* dSg = static_cast<const E*>(p.dSck) + (size_t)c * p.DV * DK;
        const E* vg = reinterpret_cast<const E*>(p.v) + tok * p.DV;
        const E* dog = reinterpret_cast<const E*>(p.dO) + tok * p.DV;
#pragma unroll
        for (int u = 0; u < NSV; ++u) {
            const int xs = min(tid + NT * u, kBV * DK / VE - 1), i = xs % kBV, j = VE * (xs / kBV);
            sa[u] = ld16(S0g + (size_t)(v0 + i) * DK + j);
            sb[u] = ld16(dSg + (size_t)(v0 + i) * DK + j);
        }
#pragma unroll
        for (int u = 0; u < NVV; ++u) {
            const int x = min(tid + NT * u, CK * PERV - 1), r = min(x % CK, valid - 1), cc = (x / CK) * VE;
            va[u] = ld16(vg + (size_t)r * p.DV + v0 + cc);
            da[u] = ld16(dog + (size_t)r * p.DV + v0 + cc);
        }
    };
    // Chunks cid0, + cstep, ... below cend: the lean form (bf16, C = 32)
    // takes the run of p.span chunks from blockIdx.x * p.span in order and
    // carries the state across it; otherwise chunks blockIdx.x, + gridDim.x, ..
    const int cid0 = LY::LEAN ? (int)blockIdx.x * p.span : (int)blockIdx.x;
    const int cend = LY::LEAN ? min(cid0 + p.span, p.total) : p.total;
    const int cstep = LY::LEAN ? 1 : (int)gridDim.x;
    // (lean) the value blocks' staging: block 0 into buffer 0 (its S0 from
    // the carried state), the block after it into registers
    LeanPf<DK> lpf;
    LeanCarry<DK> car;
    int lpc = cid0, lpv0 = 0;
    if (cid0 < cend) {
        fetch_chunk(cid0, threadIdx.x);
        if constexpr (LY::LEAN) {
            lpf.at(p, lpc);
            if (threadIdx.x < 256) {
                lpf.load(p, lpc, 0, threadIdx.x);
                lpf.store(smem + LY::off_lean, threadIdx.x);
            }
            if (p.DV > 32) {
                lpv0 = 32;
            } else {
                ++lpc;
                lpf.step(p);
            }
            if (threadIdx.x < 256 && lpc < cend) lpf.load(p, lpc, lpv0, threadIdx.x);
        } else {
            fetch_block(cid0, 0, threadIdx.x);
        }
    }
    for (int cid = cid0; cid < cend; cid += cstep) {
    // lane-dependent values are re-derived per chunk (see opaque)
    const int tid = opaque(threadIdx.x), l = tid & (kWave - 1), g4 = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nxt = cid + cstep;
    const int bh = cid / p.NC, n = cid % p.NC;
    const int t0 = n * CK, valid = min(CK, p.L - t0);
    const size_t tok = (size_t)bh * p.L + t0;
    // (lean) a run's first chunk and a head's first chunk take the carried
    // state afresh (staged as block 0's S0 before the value blocks)
    const bool fresh = LY::LEAN && (cid == cid0 || n == 0);
    if constexpr (LY::LEAN) {
        if (fresh) car.load(p, cid, w, l);
    }

    // ---- the chunk's keys, queries and gates (zero past the end)
    ks.mask(valid, tid);
    qs.mask(valid, tid);
    ks.store(Ks, LDK, Kt, LCK, tid);
    qs.store(Qs, LDK, Qt, LCK, tid);
    for (int x = tid; x < 16 * CK; x += NT) hgp[x] = 0.f;   // hgp and frp
    if (w == 0) {
        const float g = scan32(l < valid ? lav : 0.f);
        const float gC = lane_value(g, CK - 1);
        if (l < CK) {
            gs[l] = g;
            gam[l] = __expf(g);
            Dd[l] = __expf(gC - g);
            bs[l] = l < valid ? btv : 0.f;
        }
    }
    __syncthreads();
    // ---- Gram and score tiles: Bm = strictly-lower(K K^T . Gamma),
    // A = diag(beta) Bm, P = Q K^T . Gamma (diagonal included)
    if (w < NCC) {
        const int rb = w / NB, ib = w % NB;
        f32x4 kk = zero4(), qk = zero4();
        if (ib <= rb) {
            tmma<E>(kk, Ks, LDK, 16 * rb, Ks, LDK, 16 * ib, DK, l);
            tmma<E>(qk, Qs, LDK, 16 * rb, Ks, LDK, 16 * ib, DK, l);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e, s = 16 * ib + c16;
            const float G = r >= s ? __expf(gs[r] - gs[s]) : 0.f;
            Bm[r * LF + s] = r > s ? kk[e] * G : 0.f;
            Af[r * LF + s] = r > s ? bs[r] * kk[e] * G : 0.f;
            Pf[r * LF + s] = qk[e] * G;
            Pt[s * LCK + r] = from_f32<E>(qk[e] * G);
        }
    }
    __syncthreads();
    if constexpr (LY::LEAN) {
        if (fresh) car.stage(0, smem + LY::off_lean, w, l);
    }
    // T, as the forward's prepass computed it (dense, zero above the diagonal)
    if (tid < CK * CK / 4) *reinterpret_cast<f32x4*>(Tf + (4 * tid / CK) * LF + 4 * tid % CK) = tv;
    __syncthreads();
    // T, T^T, T~, T~^T
    for (int x = tid; x < CK * CK; x += NT) {
        const int r = x % CK, s = x / CK;
        const float t = s <= r ? Tf[r * LF + s] : 0.f;
        Tf[r * LF + s] = t;
        Tft[s * LF + r] = t;
        Tt[r * LCK + s] = from_f32<E>(t * bs[s]);
        Ttt[s * LCK + r] = from_f32<E>(t * bs[s]);
    }

    // C x DK accumulators: dQa = (gamma dO) S0, dKa = dX S0, dKd = U dS_end
    f32x4 dQa[NQW], dKa[NQW], dKd[NQW];
#pragma unroll
    for (int u = 0; u < NQW; ++u) { dQa[u] = zero4(); dKa[u] = zero4(); dKd[u] = zero4(); }
    f32x4 dPa = zero4(), dTa = zero4();   // C x C tile w (w < NCC)
    float hS = 0.f;                       // this thread's part of <dS_end, S0>
    constexpr int NCB = NB * (kBV / 16);  // C x kBV tiles (<= 4)
    if constexpr (LY::LEAN) {
        float hs8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        // the carried state's step: D . K as an X^T operand, gamma_C
        Frag<bf16> kdf = trn<LDK>(reinterpret_cast<const unsigned char*>(Ks), 0, 16 * (w % NJ), l);
        {
            float kv[8];
            Pack<bf16>::unpack(__builtin_bit_cast(u32x4, kdf.v), kv);
#pragma unroll
            for (int j = 0; j < 8; ++j) kv[j] *= Dd[8 * g4 + j];
            kdf.v = __builtin_bit_cast(bf16x8, Pack<bf16>::pack(kv));
        }
        const float gC = gam[CK - 1];
        lean_value_blocks<DK, true, NQW, NVB>(p, smem, LY::off_lean, LY::off_lx, Ks, Ks, Pt, Tt, Ttt, gam, Dd, cid,
                                              tid, lpf, lpc, lpv0, cend, car, kdf, f32x4{gC, gC, gC, gC},
                                              dQa, dKa, dKd, dPa, dTa, hs8);
        // (gamma dO) S0 and dX S0 = -(gamma dR) S0 from the unscaled sums
#pragma unroll
        for (int u = 0; u < NQW; ++u) {
            const int t = w + NW * u;
            if (FULLQ || t < NQT) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float gr = gam[16 * (t / NJ) + 4 * g4 + e];
                    dQa[u][e] *= gr;
                    dKa[u][e] *= -gr;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) hS += hs8[e];
    } else {
    for (int v0 = 0; v0 < p.DV; v0 += kBV) {
            __syncthreads();   // the previous block's operands are consumed
    #pragma unroll
            for (int u = 0; u < NSV; ++u) {
                const int xs = tid + NT * u, i = xs % kBV, j = VE * (xs / kBV);
                if (xs >= kBV * DK / VE) continue;
                E a[VE], b[VE];
                __builtin_memcpy(a, &sa[u], 16);
                __builtin_memcpy(b, &sb[u], 16);
                st16(S0s + i * LDK + j, sa[u]);
                st16(dSs + i * LDK + j, sb[u]);
    #pragma unroll
                for (int e = 0; e < VE; ++e) {
                    S0t[(j + e) * LBV + i] = a[e];
                    dSt[(j + e) * LBV + i] = b[e];
                    hS += to_f32(a[e]) * to_f32(b[e]);
                }
            }
    #pragma unroll
            for (int u = 0; u < NVV; ++u) {
                const int x = tid + NT * u, r = x % CK, c = (x / CK) * VE;
                if (x < CK * PERV) {
                    float a[VE], d[VE];
                    Pack<E>::unpack(r < valid ? va[u] : u32x4{0u, 0u, 0u, 0u}, a);
                    Pack<E>::unpack(r < valid ? da[u] : u32x4{0u, 0u, 0u, 0u}, d);
    #pragma unroll
                    for (int j = 0; j < VE; ++j) {
                        Vs[r * LBF + c + j] = a[j];
                        dOs[r * LBV + c + j] = from_f32<E>(d[j]);
                        dOt[(c + j) * LCK + r] = from_f32<E>(d[j]);
                        gdOs[r * LBV + c + j] = from_f32<E>(gam[r] * d[j]);
                    }
                }
            }
            if (v0 + kBV < p.DV) fetch_block(cid, v0 + kBV, tid);
            else if (nxt < cend) fetch_block(nxt, 0, tid);
            __syncthreads();
            // ---- R = V - gamma K S0^T (waves 0..NCB-1); dU = P^T dO + D . K dS^T (waves 4..)
            if (w < NCB) {
                const int rb = w / 2, cb = w % 2;
                f32x4 x = zero4();
                tmma<E>(x, Ks, LDK, 16 * rb, S0s, LDK, 16 * cb, DK, l);
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * g4 + e, i = 16 * cb + c16;
                    const float rr = Vs[r * LBF + i] - gam[r] * x[e];
                    Rs[r * LBV + i] = from_f32<E>(rr);
                    Rt[i * LCK + r] = from_f32<E>(rr);
                }
            } else if (w >= 4 && w < 4 + NCB) {
                const int rb = (w - 4) / 2, cb = (w - 4) % 2;
                f32x4 kds = zero4(), du = zero4();
                tmma<E>(kds, Ks, LDK, 16 * rb, dSs, LDK, 16 * cb, DK, l);
                tmma<E>(du, Pt, LCK, 16 * rb, dOt + 16 * cb * LCK, LCK, 0, CK, l);
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * g4 + e, i = 16 * cb + c16;
                    const float dd = du[e] + Dd[r] * kds[e];
                    dUs[r * LBV + i] = from_f32<E>(dd);
                    dUt[i * LCK + r] = from_f32<E>(dd);
                }
            }
            __syncthreads();
            // ---- U = T~ R (waves 0..); dR = T~^T dU (= dV), dX = -gamma dR (waves 4..)
            if (w < NCB) {
                const int rb = w / 2, cb = w % 2;
                f32x4 u = zero4();
                tmma<E>(u, Tt, LCK, 16 * rb, Rt + 16 * cb * LCK, LCK, 0, CK, l);
    #pragma unroll
                for (int e = 0; e < 4; ++e) Us[(16 * rb + 4 * g4 + e) * LBV + 16 * cb + c16] = from_f32<E>(u[e]);
            } else if (w >= 4 && w < 4 + NCB) {
                const int rb = (w - 4) / 2, cb = (w - 4) % 2;
                f32x4 dr = zero4();
                tmma<E>(dr, Ttt, LCK, 16 * rb, dUt + 16 * cb * LCK, LCK, 0, CK, l);
                E* dvg = reinterpret_cast<E*>(p.dv) + tok * p.DV + v0;
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * g4 + e, i = 16 * cb + c16;
                    if (r < valid) dvg[(size_t)r * p.DV + i] = from_f32<E>(dr[e]);
                    dXs[r * LBV + i] = from_f32<E>(-gam[r] * dr[e]);
                }
            }
            __syncthreads();
            // ---- accumulate over the block's value channels
    #pragma unroll
            for (int u = 0; u < NQW; ++u) {
                const int t = w + NW * u;
                if (FULLQ || t < NQT) {
                    const int rb = t / NJ, jb = t % NJ;
                    tmma<E>(dQa[u], gdOs, LBV, 16 * rb, S0t, LBV, 16 * jb, kBV, l);
                    tmma<E>(dKa[u], dXs, LBV, 16 * rb, S0t, LBV, 16 * jb, kBV, l);
                    tmma<E>(dKd[u], Us, LBV, 16 * rb, dSt, LBV, 16 * jb, kBV, l);
                }
            }
            if (w < NCC) {
                const int rb = w / NB, sb = w % NB;
                tmma<E>(dPa, dOs, LBV, 16 * rb, Us, LBV, 16 * sb, kBV, l);
                tmma<E>(dTa, dUs, LBV, 16 * rb, Rs, LBV, 16 * sb, kBV, l);
            }
        }
    }
    __syncthreads();   // the block region is reused below
    // the next chunk's keys, queries and gates: issued here rather than at the
    // chunk's start, so that no wait at the value loop's entry covers them
    if (nxt < cend) fetch_chunk(nxt, tid);

    // ---- the dg terms that sum over key channels, from the accumulators
    // before the score terms join them, per row r:
    //   gamma dO (Q S0^T):  sum_j Q_rj (gamma dO S0)_rj
    //   -gamma dR . X:      sum_j K_rj (dX S0)_rj
    //   D . U . K dS^T:     sum_j K_rj D_r (U dS_end)_rj     (enters with -)
    // and dK = dX S0 + D . U dS_end.  The 16 lanes of a tile row are summed
    // side by side for all rows of the tile.
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        const int t = w + NW * u;
        if (FULLQ || t < NQT) {
            const int rb = t / NJ, jb = t % NJ;
            float h[4], f[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e, j = 16 * jb + c16;
                const float kq = to_f32(Ks[r * LDK + j]), qq = to_f32(Qs[r * LDK + j]);
                dKd[u][e] *= Dd[r];
                h[e] = qq * dQa[u][e] + kq * dKa[u][e];
                f[e] = kq * dKd[u][e];
                dKa[u][e] += dKd[u][e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h[e] = row16_sum(h[e]);
                f[e] = row16_sum(f[e]);
            }
            if (c16 == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hgp[w * CK + 16 * rb + 4 * g4 + e] += h[e];   // this wave's own slot
                    frp[w * CK + 16 * rb + 4 * g4 + e] += f[e];
                }
        }
    }
    // ---- C x C terms, with the row and column sums of dP . P and T . dT~
    if (w < NCC) {
        const int rb = w / NB, sb = w % NB;
        float ep[4], tp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e, s = 16 * sb + c16;
            const float W = r >= s ? __expf(gs[r] - gs[s]) : 0.f;
            dPW[r * LCK + s] = from_f32<E>(dPa[e] * W);
            dPWt[s * LCK + r] = from_f32<E>(dPa[e] * W);
            ep[e] = dPa[e] * Pf[r * LF + s];
            tp[e] = dTa[e] * Tf[r * LF + s];
            dTb[r * LF + s] = dTa[e] * bs[s];
        }
        tile_row_col_sums<true, true>(ep, eR + sb * CK + 16 * rb, eC + rb * CK + 16 * sb, g4, c16);
        tile_row_col_sums<false, true>(tp, nullptr, tC + rb * CK + 16 * sb, g4, c16);
    }
    {
        // <dS_end, S0> over the whole state
        float x = row16_sum(hS);
        x += __shfl_xor(x, 16, kWave);
        x += __shfl_xor(x, 32, kWave);
        if (l == 0) red[w] = x;
    }
    __syncthreads();
    // dQ += (dP . W) K, dK += (dP . W)^T Q; Y1 = dT~ diag(beta) T^T
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        const int t = w + NW * u;
        if (FULLQ || t < NQT) {
            const int rb = t / NJ, jb = t % NJ;
            tmma<E>(dQa[u], dPW, LCK, 16 * rb, Kt, LCK, 16 * jb, CK, l);
            tmma<E>(dKa[u], dPWt, LCK, 16 * rb, Qt, LCK, 16 * jb, CK, l);
        }
    }
    if (w < NCC) {
        const int rb = w / NB, sb = w % NB;
        f32x4 y = zero4();
        tmma<float>(y, dTb, LF, 16 * rb, Tf, LF, 16 * sb, CK, l);
#pragma unroll
        for (int e = 0; e < 4; ++e) Y1t[(16 * sb + c16) * LF + 16 * rb + 4 * g4 + e] = y[e];
    }
    __syncthreads();
    // dA = strictly-lower(-T^T Y1); dG = dA . diag(beta) Gamma; dA . A
    if (w < NCC) {
        const int rb = w / NB, sb = w % NB;
        f32x4 y = zero4();
        tmma<float>(y, Tft, LF, 16 * rb, Y1t, LF, 16 * sb, CK, l);
        float fp[4], ap[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e, s = 16 * sb + c16;
            const float da = r > s ? -y[e] : 0.f;
            const float dgv = r > s ? da * bs[r] * __expf(gs[r] - gs[s]) : 0.f;
            dGf[r * LCK + s] = from_f32<E>(dgv);
            dGt[s * LCK + r] = from_f32<E>(dgv);
            fp[e] = da * Af[r * LF + s];
            ap[e] = da * Bm[r * LF + s];
        }
        // row and column sums of dA . A; row sums of dA . Bm
        tile_row_col_sums<true, true>(fp, fR + sb * CK + 16 * rb, fC + rb * CK + 16 * sb, g4, c16);
        tile_row_col_sums<true, false>(ap, aR + sb * CK + 16 * rb, nullptr, g4, c16);
    }
    __syncthreads();
    // dK += dG K + dG^T K
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        const int t = w + NW * u;
        if (FULLQ || t < NQT) {
            const int rb = t / NJ, jb = t % NJ;
            tmma<E>(dKa[u], dGf, LCK, 16 * rb, Kt, LCK, 16 * jb, CK, l);
            tmma<E>(dKa[u], dGt, LCK, 16 * rb, Kt, LCK, 16 * jb, CK, l);
        }
    }
    // dbeta and dg per token, then d log alpha = suffix sums of dg
    if (w == 0) {
        float db = 0.f, dgl = 0.f, fr = 0.f;
        if (l < CK) {
            // dbeta_t = sum_u T_ut dT~_ut + sum_s dA_ts Bm_ts; the dg terms of
            // dP . P and dA . A (rows minus columns), the gamma and D terms
            float ea = 0.f, fa = 0.f, hg = 0.f;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                db += tC[b * CK + l] + aR[b * CK + l];
                ea += eR[b * CK + l] - eC[b * CK + l];
                fa += fR[b * CK + l] - fC[b * CK + l];
            }
#pragma unroll
            for (int x = 0; x < NW; ++x) {
                fr += frp[x * CK + l];
                hg += hgp[x * CK + l];
            }
            dgl = ea + fa + hg - fr;
        }
        // g_C enters gamma_C S0 and every D_r = e^{g_C - g_r}
        const float fsum = lane_value(scan32(fr), 31);   // fr is 0 past token CK - 1
        if (l == CK - 1) {
            float hs = 0.f;
            for (int x = 0; x < NW; ++x) hs += red[x];
            dgl += gam[CK - 1] * hs + fsum;
        }
        const float incl = scan32(dgl);
        const float total = lane_value(incl, CK - 1);
        if (l < valid) {
            p.dbeta[tok + l] = db;
            if (p.dlog_alpha) p.dlog_alpha[tok + l] = total - incl + dgl;
        }
    }
    // ---- dq, dk
    E* dqg = reinterpret_cast<E*>(p.dq) + tok * DK;
    E* dkg = reinterpret_cast<E*>(p.dk) + tok * DK;
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        const int t = w + NW * u;
        if (FULLQ || t < NQT) {
            const int rb = t / NJ, jb = t % NJ;
            // row 16 rb + 4 g4 + c16 % 4, columns 16 jb + 4 (c16 / 4) ..
            const f32x4 q4 = quad_transpose(dQa[u]), k4 = quad_transpose(dKa[u]);
            const int r = 16 * rb + 4 * g4 + (c16 & 3), j = 16 * jb + 4 * (c16 >> 2);
            if (r < valid) {
                st4(dqg + (size_t)r * DK + j, q4[0], q4[1], q4[2], q4[3]);
                st4(dkg + (size_t)r * DK + j, k4[0], k4[1], k4[2], k4[3]);
            }
        }
    }
    __syncthreads();   // the LDS is restaged for the next chunk
    }
}


// ------------------------------------------------------- grads, channel alpha
// Per-channel decay G (C x d_k, cumulative within the chunk).  With
// Kg = K . e^G, Qg = Q . e^G, Kd = K . e^{G_C - G} (from the forward's
// record) and the scores P_ri = sum_c q_rc k_ic e^{G_rc - G_ic}, A likewise
// from K, the gradients of one chunk are
//   dQ = (dO S0) . e^G + dQ_P,  dQ_P[r][c] = sum_i dPM_ri k_ic e^{G_rc - G_ic}
//   dK = (dX S0) . e^G + (U dS_end) . e^{G_C - G} + dK_A1 + dK_P2 + dK_A2
//        dK_A1[r][c] = sum_i dAb_ri k_ic e^{G_rc - G_ic}
//        dK_P2[i][c] = sum_r dPM_ri q_rc e^{G_rc - G_ic},  dK_A2 likewise with dAb, k
//   dG  = (dO S0) . Qg + (dX S0) . Kg - (U dS_end) . Kd + dQ_P . Q + (dK_A1 - dK_P2 - dK_A2) . K
//   dG_C += sum_r (U dS_end . Kd)_r + e^{G_C} <dS_end, S0> per channel,
// with dPM = dO U^T . M_incl and dAb = diag(beta) dA.  The four sums with the
// decay inside run per output tile of 16 tokens through a reference row m of
// the tile: e^{G_r - G_i} = e^{G_r - G_m} e^{G_m - G_i}.
constexpr int kBVC = 32;   // value channels per block (channel alpha)

template <typename E, int DK, int CK>
struct GradChLds : Strides<E, DK, CK> {
    using S = Strides<E, DK, CK>;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int LB = kBVC + S::PE;      // rows of kBVC elements
    static constexpr int LG = DK + 4;            // fp32 rows of d_k
    static constexpr int LBF = kBVC + 4;
    static constexpr int FCC = CK * S::LF * 4, ECC = CK * S::LCK * ES;
    static constexpr int ERD = CK * S::LDK * ES;
    // kept for the whole chunk
    static constexpr int off_K = 0;                            // raw K, Q; Kg, Kd [CK][LDK] E
    static constexpr int off_Q = off_K + ERD;
    static constexpr int off_Kg = off_Q + ERD;
    static constexpr int off_Kd = off_Kg + ERD;
    static constexpr int off_G = off_Kd + ERD;                 // [CK][LG] f32
    static constexpr int off_Bm = off_G + CK * LG * 4;         // [CK][LF] f32
    static constexpr int off_A = off_Bm + FCC;
    static constexpr int off_T = off_A + FCC;
    static constexpr int off_Tft = off_T + FCC;
    static constexpr int off_Tt = off_Tft + FCC;               // [CK][LCK] E
    static constexpr int off_Ttt = off_Tt + ECC;
    static constexpr int off_Pt = off_Ttt + ECC;
    static constexpr int off_vec = off_Pt + ECC;               // beta [CK], <dS, S0> per channel [DK],
    static constexpr int NVEC = CK + DK + 2 * (CK / 16) * CK;  //   tile sums for dbeta [2][NB][CK]
    static constexpr int off_fl = off_vec + NVEC * 4;          // [CK][DK] bytes: log alpha below the floor
    static constexpr int off_blk = (off_fl + CK * DK + 15) / 16 * 16;
    // one block of kBVC value channels
    static constexpr int off_S0 = off_blk;                     // [kBVC][LDK] E and [DK][LB]
    static constexpr int off_dS = off_S0 + kBVC * S::LDK * ES;
    static constexpr int off_S0t = off_dS + kBVC * S::LDK * ES;
    static constexpr int off_dSt = off_S0t + DK * LB * ES;
    static constexpr int off_dO = off_dSt + DK * LB * ES;      // [CK][LB] E
    static constexpr int off_R = off_dO + CK * LB * ES;
    static constexpr int off_U = off_R + CK * LB * ES;
    static constexpr int off_dU = off_U + CK * LB * ES;
    static constexpr int off_dX = off_dU + CK * LB * ES;
    static constexpr int off_dOt = off_dX + CK * LB * ES;      // [kBVC][LCK] E
    static constexpr int off_Rt = off_dOt + kBVC * S::LCK * ES;
    static constexpr int off_dUt = off_Rt + kBVC * S::LCK * ES;
    static constexpr int off_V = off_dUt + kBVC * S::LCK * ES; // [CK][LBF] f32
    static constexpr int blk_end = off_V + CK * LBF * 4;
    // last phases, over the block region
    // bf16, C = 32: double-buffered block inputs, then the last phases' region
    // (whose start also holds the block intermediates during the value loop)
    static constexpr bool LEAN = (ES == 2 && CK == 32);
    static constexpr int off_lean = off_blk;
    static constexpr int off_tail = LEAN ? off_blk + 2 * LeanVB<DK>::IN : off_blk;
    static constexpr int off_lx = off_tail;
    static constexpr int off_dTt = off_tail;                   // [CK][LF] f32 (triangular part)
    static constexpr int off_dTb = off_dTt + FCC;
    static constexpr int off_Y1t = off_dTb + FCC;
    static constexpr int off_dA = off_Y1t + FCC;
    static constexpr int off_dPM = off_dA + FCC;               // [CK][LCK] E
    static constexpr int off_dPMt = off_dPM + ECC;
    static constexpr int off_dAb = off_dPMt + ECC;
    static constexpr int off_dAbt = off_dAb + ECC;
    static constexpr int pair_end = off_dAbt + ECC;
    static constexpr int off_dGm = off_tail;                   // [CK][LG] f32 (after the pairs)
    static constexpr int off_Y3Kd = off_dGm + CK * LG * 4;
    static constexpr int last_end = off_Y3Kd + CK * LG * 4;
    static constexpr int lx_end = off_lx + LeanVB<DK>::XB;
    static constexpr int m1 = LEAN ? (lx_end > pair_end ? lx_end : pair_end) : (blk_end > pair_end ? blk_end : pair_end);
    static constexpr int bytes = m1 > last_end ? m1 : last_end;
};

template <typename E, int DK, int CK, int NVB>
__global__ __launch_bounds__(512) void chunk_bwd_grad_channel_kernel(BwdParams p)
{
    using LY = GradChLds<E, DK, CK>;
    static_assert(LY::LEAN ? (NVB == 2 || NVB == 4) : NVB == 0, "value blocks of the lean form");
    constexpr int NB = CK / 16, NJ = DK / 16, VE = Vec<E>::n;
    constexpr int LF = LY::LF, LDK = LY::LDK, LCK = LY::LCK, LB = LY::LB, LG = LY::LG, LBF = LY::LBF;
    constexpr int NT = 512, NW = NT / kWave;
    constexpr int NQT = NB * NJ, NQW = (NQT + NW - 1) / NW;
    constexpr bool FULLQ = NQT == NW * NQW;      // every wave holds NQW tiles (no test needed)
    constexpr int NCC = NB * NB, NPAIR = NB * (NB + 1) / 2, NKS = DK / 32;
    constexpr WsLayout WL = ws_layout((int)sizeof(E), DK, CK, kAlphaChannel);
    static_assert(NKS % 2 == 0 && 64 * NPAIR * 4 * 4 <= LY::FCC, "Bm halves");
    extern __shared__ __align__(16) unsigned char smem[];
#define GL_E(name, off) E* name = reinterpret_cast<E*>(smem + LY::off)
#define GL_F(name, off) float* name = reinterpret_cast<float*>(smem + LY::off)
    GL_E(Ks, off_K); GL_E(Qs, off_Q); GL_E(Kgs, off_Kg); GL_E(Kds, off_Kd); GL_F(Gs, off_G);
    GL_F(Bm, off_Bm); GL_F(Af, off_A); GL_F(Tf, off_T); GL_F(Tft, off_Tft);
    GL_E(Tt, off_Tt); GL_E(Ttt, off_Ttt); GL_E(Pt, off_Pt);
    GL_E(S0s, off_S0); GL_E(dSs, off_dS); GL_E(S0t, off_S0t); GL_E(dSt, off_dSt);
    GL_E(dOs, off_dO); GL_E(Rs, off_R); GL_E(Us, off_U); GL_E(dUs, off_dU); GL_E(dXs, off_dX);
    GL_E(dOt, off_dOt); GL_E(Rt, off_Rt); GL_E(dUt, off_dUt); GL_F(Vs, off_V);
    GL_F(dTt, off_dTt); GL_F(dTb, off_dTb); GL_F(Y1t, off_Y1t); GL_F(dAf, off_dA);
    GL_E(dPM, off_dPM); GL_E(dPMt, off_dPMt); GL_E(dAb, off_dAb); GL_E(dAbt, off_dAbt);
    GL_F(dGm, off_dGm); GL_F(Y3Kd, off_Y3Kd);
#undef GL_E
#undef GL_F
    float* bs = reinterpret_cast<float*>(smem + LY::off_vec);
    float* hC = bs + CK;                     // <dS_end, S0> per key channel
    float* tC = hC + DK;                     // column sums of T . dT~ per tile row block
    float* aR = tC + NB * CK;                // row sums of dA . Bm per tile column block
    unsigned char* fl = smem + LY::off_fl;   // 1 where log alpha is below the floor

    // Each workgroup walks chunks blockIdx.x, + gridDim.x, ...; the next
    // chunk's keys, queries, records, gates and first value block are read
    // into registers while the current chunk is worked on.
    constexpr int NLV = (CK * DK / 4 + NT - 1) / NT;
    constexpr int NPV = CK * CK / VE;
    RowStage<E, CK, DK, NT> ks, qs, kg, kd;
    f32x4 lv[NLV];
    u32x4 pv;
    float bv;
    f32x4 tv;   // 16 bytes of the chunk's T (from the forward's prepass) per thread
    auto fetch_chunk = [&](int c, int tid) {
        const int n = c % p.NC, valid = min(CK, p.L - n * CK);
        const size_t tok = (size_t)(c / p.NC) * p.L + (size_t)n * CK;
        const unsigned char* rec = p.ws + (size_t)c * WL.bytes;
        // (every read unconditional, from clamped indices: a read under a
        // condition, or a select on its value, would wait for it right here;
        // the entries past the chunk's end are zeroed where they are used)
        tv = *reinterpret_cast<const f32x4*>(p.Tck + (size_t)c * CK * CK + 4 * min(tid, CK * CK / 4 - 1));
        ks.prefetch(reinterpret_cast<const E*>(p.k) + tok * DK, DK, valid, tid);
        qs.prefetch(reinterpret_cast<const E*>(p.q) + tok * DK, DK, valid, tid);
        kg.prefetch(reinterpret_cast<const E*>(rec + WL.KG), DK, CK, tid);
        kd.prefetch(reinterpret_cast<const E*>(rec + WL.KD), DK, CK, tid);
#pragma unroll
        for (int j = 0; j < NLV; ++j) {
            const int x = min(tid + NT * j, CK * DK / 4 - 1), r = min((4 * x) / DK, valid - 1);
            lv[j] = *reinterpret_cast<const f32x4*>(p.log_alpha + (tok + r) * DK + (4 * x) % DK);
        }
        pv = ld16(rec + WL.M + 16 * min(tid, NPV - 1));
        bv = p.beta[tok + min(tid, valid - 1)];
    };
    // Thread x stages the 16-byte vector (value row x % kBVC, key channels
    // VE (x / kBVC) ..) of S0 and dS_end; its key channels are the same in
    // every block, so it also sums their products for <dS_end, S0>.
    constexpr int NSV = (kBVC * DK / VE + NT - 1) / NT;
    constexpr int PERV = kBVC / VE, NVV = (CK * PERV + NT - 1) / NT;
    constexpr int NCB = NB * (kBVC / 16);   // C x kBVC tiles (<= 4)
    u32x4 sa[NSV], sb[NSV], va[NVV], da[NVV];
    auto fetch_block = [&](int c, int v0, int tid) {
        const int n = c % p.NC, valid = min(CK, p.L - n * CK);
        const size_t tok = (size_t)(c / p.NC) * p.L + (size_t)n * CK;
        const E* S0g = static_cast<const E*>(p.Sck) + (size_t)c * p.DV * DK;
        const E* dSg = static_cast<const E*>(p.dSck) + (size_t)c * p.DV * DK;
        const E* vg = reinterpret_cast<const E*>(p.v) + tok * p.DV;
        const E* dog = reinterpret_cast<const E*>(p.dO) + tok * p.DV;
#pragma unroll
        for (int u = 0; u < NSV; ++u) {
            const int xs = min(tid + NT * u, kBVC * DK / VE - 1), i = xs % kBVC, j = VE * (xs / kBVC);
            sa[u] = ld16(S0g + (size_t)(v0 + i) * DK + j);
            sb[u] = ld16(dSg + (size_t)(v0 + i) * DK + j);
        }
#pragma unroll
        for (int u = 0; u < NVV; ++u) {
            const int x = min(tid + NT * u, CK * PERV - 1), r = min(x % CK, valid - 1), cc = (x / CK) * VE;
            va[u] = ld16(vg + (size_t)r * p.DV + v0 + cc);
            da[u] = ld16(dog + (size_t)r * p.DV + v0 + cc);
        }
    };
    // Chunks cid0, + cstep, ... below cend: the lean form (bf16, C = 32)
    // takes the run of p.span chunks from blockIdx.x * p.span in order and
    // carries the state across it; otherwise chunks blockIdx.x, + gridDim.x, ..
    const int cid0 = LY::LEAN ? (int)blockIdx.x * p.span : (int)blockIdx.x;
    const int cend = LY::LEAN ? min(cid0 + p.span, p.total) : p.total;
    const int cstep = LY::LEAN ? 1 : (int)gridDim.x;
    // (lean) the value blocks' staging: block 0 into buffer 0 (its S0 from
    // the carried state), the block after it into registers
    LeanPf<DK> lpf;
    LeanCarry<DK> car;
    int lpc = cid0, lpv0 = 0;
    if (cid0 < cend) {
        fetch_chunk(cid0, threadIdx.x);
        if constexpr (LY::LEAN) {
            lpf.at(p, lpc);
            if (threadIdx.x < 256) {
                lpf.load(p, lpc, 0, threadIdx.x);
                lpf.store(smem + LY::off_lean, threadIdx.x);
            }
            if (p.DV > 32) {
                lpv0 = 32;
            } else {
                ++lpc;
                lpf.step(p);
            }
            if (threadIdx.x < 256 && lpc < cend) lpf.load(p, lpc, lpv0, threadIdx.x);
        } else {
            fetch_block(cid0, 0, threadIdx.x);
        }
    }
    for (int cid = cid0; cid < cend; cid += cstep) {
    // lane-dependent values are re-derived per chunk (see vlane)
    const int tid = opaque(threadIdx.x), l = tid & (kWave - 1), g4 = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nxt = cid + cstep;
    const int bh = cid / p.NC, n = cid % p.NC;
    const int t0 = n * CK, valid = min(CK, p.L - t0);
    const size_t tok = (size_t)bh * p.L + t0;
    // (lean) a run's first chunk and a head's first chunk take the carried
    // state afresh (staged as block 0's S0 before the value blocks)
    const bool fresh = LY::LEAN && (cid == cid0 || n == 0);
    if constexpr (LY::LEAN) {
        if (fresh) car.load(p, cid, w, l);
    }

    // ---- keys, queries, the forward's decayed keys, log alpha (floored),
    // beta, and the score block P (masked; columns in tok_of_col order) transposed
    ks.mask(valid, tid);
    qs.mask(valid, tid);
    ks.store_plain(Ks, LDK, tid);
    qs.store_plain(Qs, LDK, tid);
    kg.store_plain(Kgs, LDK, tid);
    kd.store_plain(Kds, LDK, tid);
#pragma unroll
    for (int j = 0; j < NLV; ++j) {
        const int x = tid + NT * j, r = (4 * x) / DK, c = (4 * x) % DK;
        if (x < CK * DK / 4)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool in = r < valid;
                Gs[r * LG + c + e] = in ? fmaxf(lv[j][e], kChannelLogAlphaMin) : 0.f;
                fl[r * DK + c + e] = (in && lv[j][e] < kChannelLogAlphaMin) ? 1 : 0;
            }
    }
    if (tid < CK) bs[tid] = tid < valid ? bv : 0.f;
    if (tid < NPV) {
        const int r = (VE * tid) / CK, mc0 = (VE * tid) % CK;
        E pe[VE];
        __builtin_memcpy(pe, &pv, 16);
#pragma unroll
        for (int j = 0; j < VE; ++j) Pt[tok_of_col(CK, mc0 + j) * LCK + r] = pe[j];
    }
    __syncthreads();
    // cumulative sum down every key channel (the column is read whole first)
    if (tid < DK) {
        float col[CK];
#pragma unroll
        for (int r = 0; r < CK; ++r) col[r] = Gs[r * LG + tid];
#pragma unroll
        for (int r = 1; r < CK; ++r) col[r] += col[r - 1];
#pragma unroll
        for (int r = 0; r < CK; ++r) Gs[r * LG + tid] = col[r];
    }
    __syncthreads();
    // ---- Bm = strictly-lower(K K^T with the decay inside), A = diag(beta) Bm,
    // through the reference rows of each tile pair; waves w and w + 4 take
    // the two halves of the key channels (the second half via Tft)
    if (w < NPAIR || (w >= 4 && w < 4 + NPAIR)) {
        const int pw = w & 3, half = w >> 2;
        const int rb = (pw == 0) ? 0 : 1, ib = (pw == 2) ? 1 : 0;
        const int m = (rb == ib) ? 16 * rb + 7 : 16 * rb - 1;
        const int rl = 16 * rb + c16, rr = 16 * ib + c16;
        f32x4 acc = zero4();
        for (int ksx = half * (NKS / 2); ksx < (half + 1) * (NKS / 2); ++ksx) {
            const int c0 = 32 * ksx + 8 * g4;
            float fa[8], fb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float gm = Gs[m * LG + c0 + j];
                fa[j] = __expf(Gs[rl * LG + c0 + j] - gm);
                fb[j] = __expf(gm - Gs[rr * LG + c0 + j]);
            }
            Frag<E> kl, kr;
            load_scaled_frag(kl, Ks + rl * LDK + c0, fa);
            load_scaled_frag(kr, Ks + rr * LDK + c0, fb);
            mma(acc, kl, kr);
        }
        if (half) *reinterpret_cast<f32x4*>(Tft + 4 * (64 * pw + l)) = acc;
        else {
            // kept for after the barrier
            Bm[(16 * rb + 4 * g4) * LF + 16 * ib + c16] = acc[0];
            Bm[(16 * rb + 4 * g4 + 1) * LF + 16 * ib + c16] = acc[1];
            Bm[(16 * rb + 4 * g4 + 2) * LF + 16 * ib + c16] = acc[2];
            Bm[(16 * rb + 4 * g4 + 3) * LF + 16 * ib + c16] = acc[3];
        }
    }
    __syncthreads();
    if (w < NPAIR) {
        const int rb = (w == 0) ? 0 : 1, ib = (w == 2) ? 1 : 0;
        const f32x4 other = *reinterpret_cast<const f32x4*>(Tft + 4 * (64 * w + l));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e, i = 16 * ib + c16;
            const float b = Bm[r * LF + i] + other[e];
            Bm[r * LF + i] = r > i ? b : 0.f;
            Af[r * LF + i] = r > i ? bs[r] * b : 0.f;
        }
    }
    if constexpr (NB == 2) {
        if (w == 3) {   // the tile above the diagonal
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e, i = 16 + c16;
                Bm[r * LF + i] = 0.f;
                Af[r * LF + i] = 0.f;
            }
        }
    }
    __syncthreads();
    if constexpr (LY::LEAN) {
        if (fresh) car.stage(0, smem + LY::off_lean, w, l);
    }
    // T, as the forward's prepass computed it (dense, zero above the diagonal)
    if (tid < CK * CK / 4) *reinterpret_cast<f32x4*>(Tf + (4 * tid / CK) * LF + 4 * tid % CK) = tv;
    __syncthreads();
    for (int x = tid; x < CK * CK; x += NT) {
        const int r = x % CK, s2 = x / CK;
        const float t = s2 <= r ? Tf[r * LF + s2] : 0.f;
        Tf[r * LF + s2] = t;
        Tft[s2 * LF + r] = t;
        Tt[r * LCK + s2] = from_f32<E>(t * bs[s2]);
        Ttt[s2 * LCK + r] = from_f32<E>(t * bs[s2]);
    }

    // C x DK accumulators: Y1 = dO S0, Y2 = dX S0, Y3 = U dS_end
    f32x4 Y1[NQW], Y2[NQW], Y3[NQW];
#pragma unroll
    for (int u = 0; u < NQW; ++u) { Y1[u] = zero4(); Y2[u] = zero4(); Y3[u] = zero4(); }
    f32x4 dPa = zero4(), dTa = zero4();   // C x C tile w (w < NCC)
    float hacc[NSV][VE];
#pragma unroll
    for (int u = 0; u < NSV; ++u)
#pragma unroll
        for (int e = 0; e < VE; ++e) hacc[u][e] = 0.f;
    if constexpr (LY::LEAN) {
        float hs8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        // the carried state's step: K . exp(G_C - G) as an X^T operand, and
        // exp(G_C) of this lane's key channels
        const Frag<bf16> kdf = trn<LDK>(reinterpret_cast<const unsigned char*>(Kds), 0, 16 * (w % NJ), l);
        f32x4 dec;
#pragma unroll
        for (int e = 0; e < 4; ++e) dec[e] = __expf(Gs[(CK - 1) * LG + 16 * (w % NJ) + 4 * g4 + e]);
        lean_value_blocks<DK, false, NQW, NVB>(p, smem, LY::off_lean, LY::off_lx, Kgs, Kds, Pt, Tt, Ttt, nullptr,
                                               nullptr, cid, tid, lpf, lpc, lpv0, cend, car, kdf, dec,
                                               Y1, Y2, Y3, dPa, dTa, hs8);
        // dX S0 = -dR S0
#pragma unroll
        for (int u = 0; u < NQW; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) Y2[u][e] = -Y2[u][e];
        static_assert(NSV == 1 || !LY::LEAN, "one staged vector per thread");
#pragma unroll
        for (int e = 0; e < VE; ++e) hacc[0][e] = hs8[e];
    } else {
    for (int v0 = 0; v0 < p.DV; v0 += kBVC) {
            __syncthreads();   // the previous block's operands are consumed
    #pragma unroll
            for (int u = 0; u < NSV; ++u) {
                const int xs = tid + NT * u, i = xs % kBVC, j = VE * (xs / kBVC);
                if (xs >= kBVC * DK / VE) continue;
                E a[VE], b[VE];
                __builtin_memcpy(a, &sa[u], 16);
                __builtin_memcpy(b, &sb[u], 16);
                st16(S0s + i * LDK + j, sa[u]);
                st16(dSs + i * LDK + j, sb[u]);
    #pragma unroll
                for (int e = 0; e < VE; ++e) {
                    S0t[(j + e) * LB + i] = a[e];
                    dSt[(j + e) * LB + i] = b[e];
                    hacc[u][e] += to_f32(a[e]) * to_f32(b[e]);
                }
            }
    #pragma unroll
            for (int u = 0; u < NVV; ++u) {
                const int x = tid + NT * u, r = x % CK, c = (x / CK) * VE;
                if (x < CK * PERV) {
                    float a[VE];
                    E d[VE];
                    const u32x4 dz = r < valid ? da[u] : u32x4{0u, 0u, 0u, 0u};
                    Pack<E>::unpack(r < valid ? va[u] : u32x4{0u, 0u, 0u, 0u}, a);
                    __builtin_memcpy(d, &dz, 16);
    #pragma unroll
                    for (int j = 0; j < VE; ++j) {
                        Vs[r * LBF + c + j] = a[j];
                        dOs[r * LB + c + j] = d[j];
                        dOt[(c + j) * LCK + r] = d[j];
                    }
                }
            }
            if (v0 + kBVC < p.DV) fetch_block(cid, v0 + kBVC, tid);
            else if (nxt < cend) fetch_block(nxt, 0, tid);
            __syncthreads();
            // ---- R = V - Kg S0^T (waves 0..NCB-1); dU = P^T dO + Kd dS^T (waves 4..)
            if (w < NCB) {
                const int rb = w / 2, cb = w % 2;
                f32x4 x = zero4();
                tmma<E>(x, Kgs, LDK, 16 * rb, S0s, LDK, 16 * cb, DK, l);
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * g4 + e, i = 16 * cb + c16;
                    const float rr = Vs[r * LBF + i] - x[e];
                    Rs[r * LB + i] = from_f32<E>(rr);
                    Rt[i * LCK + r] = from_f32<E>(rr);
                }
            } else if (w >= 4 && w < 4 + NCB) {
                const int rb = (w - 4) / 2, cb = (w - 4) % 2;
                f32x4 du = zero4();
                tmma<E>(du, Kds, LDK, 16 * rb, dSs, LDK, 16 * cb, DK, l);
                tmma<E>(du, Pt, LCK, 16 * rb, dOt + 16 * cb * LCK, LCK, 0, CK, l);
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * g4 + e, i = 16 * cb + c16;
                    dUs[r * LB + i] = from_f32<E>(du[e]);
                    dUt[i * LCK + r] = from_f32<E>(du[e]);
                }
            }
            __syncthreads();
            // ---- U = T~ R (waves 0..); dR = T~^T dU (= dV), dX = -dR (waves 4..)
            if (w < NCB) {
                const int rb = w / 2, cb = w % 2;
                f32x4 u = zero4();
                tmma<E>(u, Tt, LCK, 16 * rb, Rt + 16 * cb * LCK, LCK, 0, CK, l);
    #pragma unroll
                for (int e = 0; e < 4; ++e) Us[(16 * rb + 4 * g4 + e) * LB + 16 * cb + c16] = from_f32<E>(u[e]);
            } else if (w >= 4 && w < 4 + NCB) {
                const int rb = (w - 4) / 2, cb = (w - 4) % 2;
                f32x4 dr = zero4();
                tmma<E>(dr, Ttt, LCK, 16 * rb, dUt + 16 * cb * LCK, LCK, 0, CK, l);
                E* dvg = reinterpret_cast<E*>(p.dv) + tok * p.DV + v0;
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * g4 + e, i = 16 * cb + c16;
                    if (r < valid) dvg[(size_t)r * p.DV + i] = from_f32<E>(dr[e]);
                    dXs[r * LB + i] = from_f32<E>(-dr[e]);
                }
            }
            __syncthreads();
            // ---- accumulate over the block's value channels
    #pragma unroll
            for (int u = 0; u < NQW; ++u) {
                const int t = w + NW * u;
                if (FULLQ || t < NQT) {
                    const int rb = t / NJ, jb = t % NJ;
                    tmma<E>(Y1[u], dOs, LB, 16 * rb, S0t, LB, 16 * jb, kBVC, l);
                    tmma<E>(Y2[u], dXs, LB, 16 * rb, S0t, LB, 16 * jb, kBVC, l);
                    tmma<E>(Y3[u], Us, LB, 16 * rb, dSt, LB, 16 * jb, kBVC, l);
                }
            }
            if (w < NCC) {
                const int rb = w / NB, sb = w % NB;
                tmma<E>(dPa, dOs, LB, 16 * rb, Us, LB, 16 * sb, kBVC, l);
                tmma<E>(dTa, dUs, LB, 16 * rb, Rs, LB, 16 * sb, kBVC, l);
            }
        }
    }
    // <dS_end, S0> per key channel: the kBVC threads that staged the same
    // key channels are the 32 lanes of one half wave (all sums reduced side
    // by side)
    static_assert(kBVC == 32, "a half wave: 16-lane rows, then across the two rows");
#pragma unroll
    for (int u = 0; u < NSV; ++u)
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            hacc[u][e] = row16_sum(hacc[u][e]);
            hacc[u][e] += __shfl_xor(hacc[u][e], 16, kWave);
        }
#pragma unroll
    for (int u = 0; u < NSV; ++u) {
        const int xs = tid + NT * u, j = VE * (xs / kBVC);
        if (xs % kBVC == 0 && xs < kBVC * DK / VE)
#pragma unroll
            for (int e = 0; e < VE; ++e) hC[j + e] = hacc[u][e];
    }
    __syncthreads();   // the block region is reused below
    // the next chunk's inputs: issued here rather than at the chunk's start,
    // so that no wait at the value loop's entry covers them
    if (nxt < cend) fetch_chunk(nxt, tid);
    // ---- triangular part: dPM, dT~; dA = strictly-lower(-T^T dT~ diag(beta) T^T)
    if (w < NCC) {
        const int rb = w / NB, sb = w % NB;
        float tp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e, s2 = 16 * sb + c16;
            const float dpm = r >= s2 ? dPa[e] : 0.f;
            dPM[r * LCK + s2] = from_f32<E>(dpm);
            dPMt[s2 * LCK + r] = from_f32<E>(dpm);
            dTb[r * LF + s2] = dTa[e] * bs[s2];
            tp[e] = dTa[e] * Tf[r * LF + s2];
        }
        tile_row_col_sums<false, true>(tp, nullptr, tC + rb * CK + 16 * sb, g4, c16);
    }
    __syncthreads();
    if (w < NCC) {
        const int rb = w / NB, sb = w % NB;
        f32x4 y = zero4();
        tmma<float>(y, dTb, LF, 16 * rb, Tf, LF, 16 * sb, CK, l);
#pragma unroll
        for (int e = 0; e < 4; ++e) Y1t[(16 * sb + c16) * LF + 16 * rb + 4 * g4 + e] = y[e];
    }
    __syncthreads();
    if (w < NCC) {
        const int rb = w / NB, sb = w % NB;
        f32x4 y = zero4();
        tmma<float>(y, Tft, LF, 16 * rb, Y1t, LF, 16 * sb, CK, l);
        float ap[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e, s2 = 16 * sb + c16;
            const float da = r > s2 ? -y[e] : 0.f;
            dAb[r * LCK + s2] = from_f32<E>(da * bs[r]);
            dAbt[s2 * LCK + r] = from_f32<E>(da * bs[r]);
            ap[e] = da * Bm[r * LF + s2];
        }
        tile_row_col_sums<true, false>(ap, aR + sb * CK + 16 * rb, nullptr, g4, c16);
    }
    __syncthreads();
    // dbeta_t = sum_u T_ut dT~_ut + sum_s dA_ts Bm_ts
    if (w == 0 && l < valid) {
        float db = 0.f;
#pragma unroll
        for (int b2 = 0; b2 < NB; ++b2) db += tC[b2 * CK + l] + aR[b2 * CK + l];
        p.dbeta[tok + l] = db;
    }

    // ---- the four sums with the decay inside the channel sum.  Output tile
    // ob (rows 16 ob ..) takes its reference row m = 16 ob + 7:
    // e^{G_r - G_i} = e^{G_r - G_m} e^{G_m - G_i}, neither factor above e^{80};
    // a factor that underflows belongs to a term below e^{-17} of the scale
    // (decays of at least e^{-10} per token).  The products keep fp32
    // accuracy: their terms of dG cancel in pairs in the suffix sums of
    // d log alpha, which bf16 operands would leave at a few percent of the
    // result.  For bf16 the fp32 operand is split into two bf16 parts
    // (hi + lo, about 16 bits) against the bf16 dPM and dAb.
    f32x4 QP[NQW], KP[NQW], KM[NQW];   // dQ_P, dK_A1, dK_P2 + dK_A2
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        QP[u] = zero4(); KP[u] = zero4(); KM[u] = zero4();
        const int t = w + NW * u;
        if (t >= NQT) continue;
        const int ob = t / NJ, c = 16 * (t % NJ) + c16, m = 16 * ob + 7;
        const float gm = Gs[m * LG + c];
        constexpr int KL = sizeof(E) == 2 ? 8 : 4;   // tokens per lane and MFMA
        // tokens k = KL g4 + j: i side (k < 16 (ob + 1)) and r side (16 ob <= k < CK)
        float sk[KL], sq[KL], sk2[KL];
#pragma unroll
        for (int j = 0; j < KL; ++j) {
            const int kt = KL * g4 + j;
            const bool in = kt < CK;
            const float g = in ? Gs[kt * LG + c] : 0.f;
            const float kx = in ? to_f32(Ks[kt * LDK + c]) : 0.f, qx = in ? to_f32(Qs[kt * LDK + c]) : 0.f;
            sk[j] = (kt < 16 * (ob + 1)) ? kx * __expf(gm - g) : 0.f;
            const float f = (kt >= 16 * ob && in) ? __expf(g - gm) : 0.f;
            sq[j] = qx * f;
            sk2[j] = kx * f;
        }
        const int arow = 16 * ob + c16;
        f32x4 a = zero4(), b = zero4(), km = zero4();
        if constexpr (sizeof(E) == 2) {
            Frag<bf16> skh, skl, sqh, sql, s2h, s2l;
            split_frag(sk, skh, skl);
            split_frag(sq, sqh, sql);
            split_frag(sk2, s2h, s2l);
            const Frag<bf16> apm = cfrag<bf16>(dPM, LCK, 16 * ob, 0, CK, l), aab = cfrag<bf16>(dAb, LCK, 16 * ob, 0, CK, l);
            const Frag<bf16> apt = cfrag<bf16>(dPMt, LCK, 16 * ob, 0, CK, l), aat = cfrag<bf16>(dAbt, LCK, 16 * ob, 0, CK, l);
            mma(a, apm, skh); mma(a, apm, skl);
            mma(b, aab, skh); mma(b, aab, skl);
            mma(km, apt, sqh); mma(km, apt, sql);
            mma(km, aat, s2h); mma(km, aat, s2l);
        } else {
            const f32x4 apm = load4f(dPM + arow * LCK + 4 * g4), aab = load4f(dAb + arow * LCK + 4 * g4);
            const f32x4 apt = load4f(dPMt + arow * LCK + 4 * g4), aat = load4f(dAbt + arow * LCK + 4 * g4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a = __builtin_amdgcn_mfma_f32_16x16x4f32(apm[j], sk[j], a, 0, 0, 0);
                b = __builtin_amdgcn_mfma_f32_16x16x4f32(aab[j], sk[j], b, 0, 0, 0);
                km = __builtin_amdgcn_mfma_f32_16x16x4f32(apt[j], sq[j], km, 0, 0, 0);
                km = __builtin_amdgcn_mfma_f32_16x16x4f32(aat[j], sk2[j], km, 0, 0, 0);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float d = Gs[(16 * ob + 4 * g4 + e) * LG + c] - gm;
            const float f = __expf(d), fi = __expf(-d);
            QP[u][e] = f * a[e];
            KP[u][e] = f * b[e];
            KM[u][e] = fi * km[e];
        }
    }
    __syncthreads();   // the pair operands give way to dG

    // ---- dq, dk, and dG per token and channel
    E* dqg = reinterpret_cast<E*>(p.dq) + tok * DK;
    E* dkg = reinterpret_cast<E*>(p.dk) + tok * DK;
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        const int t = w + NW * u;
        if (FULLQ || t < NQT) {
            const int rb = t / NJ, jb = t % NJ;
            f32x4 dq4, dk4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e, c = 16 * jb + c16;
                const float g = Gs[r * LG + c], gC = Gs[(CK - 1) * LG + c];
                const float eG = __expf(g), eD = __expf(gC - g);
                const float q = to_f32(Qs[r * LDK + c]), k = to_f32(Ks[r * LDK + c]);
                dq4[e] = Y1[u][e] * eG + QP[u][e];
                dk4[e] = Y2[u][e] * eG + Y3[u][e] * eD + KP[u][e] + KM[u][e];
                dGm[r * LG + c] = Y1[u][e] * q * eG + Y2[u][e] * k * eG - Y3[u][e] * k * eD + QP[u][e] * q +
                                  (KP[u][e] - KM[u][e]) * k;
                Y3Kd[r * LG + c] = Y3[u][e] * k * eD;
            }
            // row 16 rb + 4 g4 + c16 % 4, columns 16 jb + 4 (c16 / 4) ..
            dq4 = quad_transpose(dq4);
            dk4 = quad_transpose(dk4);
            const int r = 16 * rb + 4 * g4 + (c16 & 3), c = 16 * jb + 4 * (c16 >> 2);
            if (r < valid) {
                st4(dqg + (size_t)r * DK + c, dq4[0], dq4[1], dq4[2], dq4[3]);
                st4(dkg + (size_t)r * DK + c, dk4[0], dk4[1], dk4[2], dk4[3]);
            }
        }
    }
    __syncthreads();
    // d log alpha: suffix sums of dG down each channel, with the g_C terms
    // entering at the chunk's last token; zero where the floor was active
    // (the column is read whole first)
    if (tid < DK) {
        const int c = tid;
        float col[CK];
        float tail = __expf(Gs[(CK - 1) * LG + c]) * hC[c];
#pragma unroll
        for (int r = 0; r < CK; ++r) {
            col[r] = dGm[r * LG + c];
            tail += Y3Kd[r * LG + c];
        }
        float acc = tail;
#pragma unroll
        for (int r = CK - 1; r >= 0; --r) {
            acc += col[r];
            col[r] = fl[r * DK + c] ? 0.f : acc;
        }
        float* dla = p.dlog_alpha + tok * DK + c;
#pragma unroll
        for (int r = 0; r < CK; ++r)
            if (r < valid) dla[(size_t)r * DK] = col[r];
    }
    __syncthreads();   // the LDS is restaged for the next chunk
    }
}

template <typename K>
static hipError_t launch_lds(K* kern, int grid, int threads, int lds, hipStream_t stream, const BwdParams& bp)
{
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, stream, bp);
    return hipGetLastError();
}

template <typename E, int DK, int CK>
static hipError_t launch_bwd_t(const BwdParams& bp, int BH, bool channel, hipStream_t stream)
{
    using CL = ChainLds<E, DK, CK>;
    using GL = GradLds<E, DK, CK>;
    using GC = GradChLds<E, DK, CK>;
    static_assert(CL::bytes <= 160 * 1024 && GL::bytes <= 160 * 1024 && GC::bytes <= 160 * 1024, "LDS budget");
    // the lean form walks runs of chunks, every other form strides
    if ((sizeof(E) == 2 && CK == 32) != (bp.span > 0) || (bp.span > 0 && bp.DV != 64 && bp.DV != 128))
        return hipErrorInvalidValue;
    const int chains = BH * (bp.DV / kBV);
    // bf16 operands on 32-token steps take the pipelined chain (gdr_bwd_chain.hip)
    hipError_t err;
    if constexpr (sizeof(E) == 2 && CK == 32) err = launch_bwd_chain_pipe(bp, BH, DK, channel, stream);
    else err = channel ? launch_lds(chunk_bwd_chain_kernel<E, DK, CK, true>, chains, 384, CL::bytes, stream, bp)
                       : launch_lds(chunk_bwd_chain_kernel<E, DK, CK, false>, chains, 384, CL::bytes, stream, bp);
    if (err != hipSuccess) return err;
    // persistent, as many workgroups as fit the CUs (the next chunk's inputs
    // are read while the current one is worked on); with a span, one
    // workgroup per run of span chunks
    const int grid_ch = bp.span > 0 ? (bp.total + bp.span - 1) / bp.span
                                    : std::min(bp.total, (160 * 1024 / GC::bytes) * compute_units());
    const int grid_sc = bp.span > 0 ? (bp.total + bp.span - 1) / bp.span
                                    : std::min(bp.total, (160 * 1024 / GL::bytes) * compute_units());
    if constexpr (sizeof(E) == 2 && CK == 32) {
        if (bp.DV == 128)
            return channel ? launch_lds(chunk_bwd_grad_channel_kernel<E, DK, CK, 4>, grid_ch, 512, GC::bytes, stream, bp)
                           : launch_lds(chunk_bwd_grad_kernel<E, DK, CK, 4>, grid_sc, 512, GL::bytes, stream, bp);
        return channel ? launch_lds(chunk_bwd_grad_channel_kernel<E, DK, CK, 2>, grid_ch, 512, GC::bytes, stream, bp)
                       : launch_lds(chunk_bwd_grad_kernel<E, DK, CK, 2>, grid_sc, 512, GL::bytes, stream, bp);
    } else {
        return channel ? launch_lds(chunk_bwd_grad_channel_kernel<E, DK, CK, 0>, grid_ch, 512, GC::bytes, stream, bp)
                       : launch_lds(chunk_bwd_grad_kernel<E, DK, CK, 0>, grid_sc, 512, GL::bytes, stream, bp);
    }
}

}  // namespace

// Workspace of the backward: the forward's chunk records, the entry states
// the gradient kernel starts from, dS at every chunk's end and every chunk's
// T (fp32).
struct BwdWs {
    size_t off_Sck, off_dSck, off_T, bytes;
};

// Chunks per gradient workgroup for bf16 operands on 32-token steps: the
// chunks of all heads in about one contiguous run per CU, each walked in
// order with the state carried across it, so the recomputing scan keeps only
// the state entering every run.  0 otherwise (every chunk's state is kept).
// (A constant CU count, as for the forward's segment plan: the workspace
// size must not depend on the device.)
static int bwd_span(size_t total, int dtype, int CK)
{
    if (dtype != kBF16 || CK != 32 || total == 0) return 0;
    return (int)((total + kSegWorkgroups - 1) / kSegWorkgroups);
}

static BwdWs bwd_ws(int B, int H, int L, int dk, int dv, int C, int dtype, int mode)
{
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const int CK = chunk_step(C, dtype);
    const size_t BH = (size_t)B * H, NC = (size_t)((L + CK - 1) / CK);
    const int es = dtype == kBF16 ? 2 : 4;
    const int span = bwd_span(BH * NC, dtype, CK);
    const size_t nst = span > 0 ? (BH * NC + span - 1) / span : BH * NC;   // entry states kept
    BwdWs w{};
    size_t o = al(BH * NC * (size_t)ws_layout(es, dk, CK, mode).bytes);
    w.off_Sck = o; o = al(o + nst * dv * dk * es);
    w.off_dSck = o; o = al(o + BH * NC * dv * dk * es);
    w.off_T = o; o = al(o + BH * NC * CK * CK * 4);
    w.bytes = o;
    return w;
}

size_t bwd_workspace_bytes(int B, int H, int L, int dk, int dv, int C, int dtype, int mode)
{
    if ((size_t)B * H == 0 || L == 0) return 0;
    return bwd_ws(B, H, L, dk, dv, C, dtype, mode).bytes;
}

__global__ void copy_grad_state_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_bwd_chunked(const BwdArgs& b)
{
    const size_t BH = (size_t)b.B * b.H;
    if (BH == 0) return hipSuccess;
    if (b.part == kBwdKeep && b.L == 0) {
        // no tokens: the plain forward (the final state is the initial one)
        ChunkArgs a{b.B, b.H, 0, b.dk, b.dv, b.C, b.dtype, b.mode, b.q, b.k, b.v, b.beta, b.log_alpha, b.S0,
                    b.o, b.S_final, b.workspace, b.stream};
        return launch_fwd_chunked(a);
    }
    if (b.L == 0) {
        // no tokens: the gradient reaching S0 is the one given for S_final
        if (!b.dS0) return hipSuccess;
        const size_t n = BH * b.dv * b.dk;
        hipLaunchKernelGGL(copy_grad_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, b.stream,
                           b.dS_final, b.dS0, n);
        return hipGetLastError();
    }
    const int CK = chunk_step(b.C, b.dtype);
    const int NC = (b.L + CK - 1) / CK;
    const BwdWs w = bwd_ws(b.B, b.H, b.L, b.dk, b.dv, b.C, b.dtype, b.mode);
    unsigned char* ws = static_cast<unsigned char*>(b.workspace);
    // the forward (again, or for the first time with its outputs): the
    // prepass records, every chunk's T and the entry states the gradient
    // walk starts from
    const int span = bwd_span(BH * NC, b.dtype, CK);
    if (b.part != kBwdKept) {
        ChunkArgs a{b.B, b.H, b.L, b.dk, b.dv, b.C, b.dtype, b.mode, b.q, b.k, b.v, b.beta, b.log_alpha, b.S0,
                    b.part == kBwdKeep ? b.o : nullptr, b.part == kBwdKeep ? b.S_final : nullptr, ws, b.stream, 0u,
                    nullptr, 0, Varlen{}, ws + w.off_Sck, reinterpret_cast<float*>(ws + w.off_T), span};
        hipError_t err = launch_wy(a, CK);
        if (err != hipSuccess) return err;
        SegPlan one{1, NC, NC, 0, 0, 0, 0, 0};
        err = launch_scan(a, CK, one);
        if (err != hipSuccess || b.part == kBwdKeep) return err;
    }
    BwdParams bp{b.q, b.k, b.v, b.dO, b.beta, b.log_alpha, b.dS_final, ws,
                 ws + w.off_Sck, ws + w.off_dSck,
                 b.dq, b.dk_out, b.dv_out, b.dbeta, b.dlog_alpha, b.dS0, b.L, NC, b.dv, (int)(BH * NC),
                 reinterpret_cast<const float*>(ws + w.off_T), span, b.S0};
    const bool ch = b.mode == kAlphaChannel;
    if (b.dtype == kBF16) {
        if (b.dk == 128) return CK == 16 ? launch_bwd_t<bf16, 128, 16>(bp, (int)BH, ch, b.stream)
                                         : launch_bwd_t<bf16, 128, 32>(bp, (int)BH, ch, b.stream);
        return CK == 16 ? launch_bwd_t<bf16, 64, 16>(bp, (int)BH, ch, b.stream)
                        : launch_bwd_t<bf16, 64, 32>(bp, (int)BH, ch, b.stream);
    }
    return b.dk == 128 ? launch_bwd_t<float, 128, 16>(bp, (int)BH, ch, b.stream)
                       : launch_bwd_t<float, 64, 16>(bp, (int)BH, ch, b.stream);
}

}  // namespace gdr

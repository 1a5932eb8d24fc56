// gdr_segment.hip -- combining the segments of a segment-parallel chunk scan.
//
// The recurrence is affine in the state: over a run of tokens,
// S_end = S_entry P + Z, where Z is the end state reached from a zero entry
// state and P the product of the per-token maps S -> S Diag(alpha) (I - beta
// k k^T) (the erase factor of the delta rule, "Linear Attention & DeltaNet",
// "How it works", and the decay of "Gated DeltaNet" / "Kimi Delta
// Attention" in "linear attention and its gated descendants").  The output
// o_t = S_t q_t is then o_t(zero entry) + S_entry (P up to t) q_t.
//
// The scan has left, per head and segment g: Z_g (segment 0: its end state
// from the true initial state), P_g^T (g > 0), and for every token of a
// segment g > 0 the vector (P up to t) q_t.  Here:
//   seg_entry_kernel    E_1 = Z_0, E_{g+1} = E_g P_g + Z_g (in order), keeps
//                       E_g as bf16 for the next kernel and writes the final
//                       state E_SEG;
//   seg_correct_kernel  o_t += E_g (P up to t) q_t for every token of every
//                       segment g > 0.
// Both products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
#include "gdr_device.h"
#include "gdr_chunk.h"

namespace gdr {

namespace {

struct SegArgs {
    const float* Z;      // [BH][SEG][DV][DK]
    const float* Pt;     // [BH][SEG][DK][DK], P_g^T row-major
    bf16* Eb;            // [BH][SEG][DV][DK], entry states (g >= 1) as bf16
    const bf16* qt;      // [BH][L][DK]
    bf16* o;             // [BH][L][DV]
    float* S_final;      // [BH][DV][DK] or null
    int L, DV, SEG, TS;  // TS: tokens per later segment
    int T0;              // tokens of segment 0
};

// One workgroup per (head, 16 value rows), one wave per 16 key columns of E.
// The rows of E evolve independently: row r of E_{g+1} is row r of E_g times
// P_g plus row r of Z_g.  A wave reads its operands for the next segment (its
// 16 columns of P_g and its tile of Z_g) before the current product, so the
// sequential path holds only the product and the exchange of E_g's 16 rows
// through LDS.  That exchange alternates between two buffers with one barrier
// per segment: the compiler may schedule a wave's reads of the rows after a
// second barrier placed behind them (it did), so no barrier is relied on to
// order them before the rows are rewritten; a buffer is rewritten only two
// segments later, after the next barrier, which no wave passes before every
// wave has used its reads.
template <int DK>
__global__ __launch_bounds__(64 * (DK / 16)) void seg_entry_kernel(SegArgs p)
{
    constexpr int NKS = DK / 32;
    __shared__ __align__(16) float rows[2][16][DK + 4];
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15;
    const int j = wave_id();                 // key columns 16 j ..
    const int nrb = p.DV / 16;
    const int bh = blockIdx.x / nrb, r0 = 16 * (blockIdx.x % nrb);

    // segment g's operands, as read: P_g[k][16 j + c16] = P_g^T[16 j + c16][k]
    // for k = 32 ks + 8 g4 .. + 7, and the lane's four values of Z_g
    f32x4 plo[NKS], phi[NKS], z;
    auto load = [&](int g) {
        const size_t bs = (size_t)bh * p.SEG + g;
        const float* src = p.Pt + bs * DK * DK + (size_t)(16 * j + c16) * DK + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            plo[ks] = *reinterpret_cast<const f32x4*>(src + 32 * ks);
            phi[ks] = *reinterpret_cast<const f32x4*>(src + 32 * ks + 4);
        }
        const float* zg = p.Z + (bs * p.DV + r0) * DK + 16 * j + c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = zg[(size_t)(4 * g4 + i) * DK];
    };

    // e: lane holds E[r0 + 4 g4 + i][16 j + c16], i = 0..3; E_1 = Z_0
    load(0);
    f32x4 e = z;
    if (p.SEG > 1) load(1);
    for (int g = 1; g < p.SEG; ++g) {
        // keep E_g (bf16) and pass its rows to every wave
        bf16* eb = p.Eb + (((size_t)bh * p.SEG + g) * p.DV + r0) * DK + 16 * j + c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            eb[(size_t)(4 * g4 + i) * DK] = (bf16)e[i];
            rows[g & 1][4 * g4 + i][16 * j + c16] = e[i];
        }
        __syncthreads();
        Frag<bf16> a[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = rows[g & 1][c16][32 * ks + 8 * g4 + i];
            a[ks].v = __builtin_bit_cast(bf16x8, Pack<bf16>::pack(x));
        }
        // E_{g+1} = E_g P_g + Z_g
        Frag<bf16> b[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) { x[i] = plo[ks][i]; x[4 + i] = phi[ks][i]; }
            b[ks].v = __builtin_bit_cast(bf16x8, Pack<bf16>::pack(x));
        }
        f32x4 acc = z;
        if (g + 1 < p.SEG) load(g + 1);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) mma(acc, a[ks], b[ks]);
        e = acc;
    }
    if (p.S_final) {
        float* sf = p.S_final + ((size_t)bh * p.DV + r0) * DK + 16 * j + c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) sf[(size_t)(4 * g4 + i) * DK] = e[i];
    }
}

// One workgroup (four waves) per (head, segment g >= 1, kTokWG tokens), E_g
// (bf16) in LDS.  Each wave walks 32-token tiles.  The corrections
// E_g (P up to t) q_t of a 16-token half come out of the MFMA as
// [value][token] fragments and pass through the wave's own LDS tile to token
// rows, so that o is read and written as whole rows, 16 bytes a lane.  The
// next tile's q-transitions and o rows are read before the current tile's
// products.  A tile whose (P up to t) q_t are all exactly zero adds nothing
// (for a finite entry state),
// and its o rows are neither read nor written: with decaying gates a later
// segment's transition underflows to zero a few chunks in (GDN gates of
// log alpha about -2 per token: within two chunks), after which only the
// q-transitions are read.  Such a tile is seen once its q-transitions have
// arrived, so the next tile's o rows are read ahead only after a nonzero tile;
// otherwise they are read when needed.
constexpr int kTokWG = 512;

template <int DK, int DV>
__global__ __launch_bounds__(256) void seg_correct_kernel(SegArgs p, int tiles_per_seg)
{
    constexpr int NKS = DK / 32, NVT = DV / 16;
    constexpr int RS = DK + 8;      // E row stride (bf16 elements)
    constexpr int CS = DV + 4;      // correction tile row stride (floats)
    constexpr int LPR = DV / 8;     // lanes per o row, 16 bytes each
    constexpr int RPI = 64 / LPR;   // o rows per load or store instruction
    constexpr int NI = 32 / RPI;    // o instructions per 32-token tile
    extern __shared__ __align__(16) unsigned char smem[];
    bf16* es = reinterpret_cast<bf16*>(smem);
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15, w = wave_id();
    float* cs = reinterpret_cast<float*>(smem + DV * RS * 2) + w * 16 * CS;
    const int per_head = (p.SEG - 1) * tiles_per_seg;
    const int bh = blockIdx.x / per_head;
    const int rem = blockIdx.x % per_head;
    const int g = 1 + rem / tiles_per_seg, tile = rem % tiles_per_seg;
    const int t_seg = p.T0 + (g - 1) * p.TS, t_end = min(t_seg + p.TS, p.L);

    const bf16* eb = p.Eb + (((size_t)bh * p.SEG + g) * DV) * DK;
    for (int i = threadIdx.x; i < DV * DK / 8; i += 256) {
        const int r = i / (DK / 8), c = (i % (DK / 8)) * 8;
        st16(es + r * RS + c, ld16(eb + (size_t)r * DK + c));
    }
    __syncthreads();

    const bf16* qt = p.qt + (size_t)bh * p.L * DK;
    bf16* o = p.o + (size_t)bh * p.L * DV;
    const int tw0 = t_seg + kTokWG * tile;
    const int tw1 = min(tw0 + kTokWG, t_end);
    const int orow = l / LPR, ocol = (l % LPR) * 8;   // this lane's row in an o instruction, first column
    struct Tile {
        Frag<bf16> q[2][NKS];   // token 16 h + c16, key channels 32 ks + 8 g4 ..
        u32x4 o[NI];            // row RPI i + orow, columns ocol ..
    };
    auto load_q = [&](int t0, Tile& T) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int tc = min(t0 + 16 * h + c16, tw1 - 1);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                T.q[h][ks].v = *reinterpret_cast<const bf16x8*>(qt + (size_t)tc * DK + 32 * ks + 8 * g4);
        }
    };
    auto load_o = [&](int t0, Tile& T) {
#pragma unroll
        for (int i = 0; i < NI; ++i) T.o[i] = ld16(o + (size_t)min(t0 + RPI * i + orow, tw1 - 1) * DV + ocol);
    };
    Tile cur, nxt;
    int t0 = tw0 + 32 * w;   // wave-uniform
    bool cur_o = false;      // cur.o holds the tile's o rows
    if (t0 < tw1) {
        load_q(t0, cur);
        load_o(t0, cur);
        cur_o = true;
    }
    for (; t0 < tw1; t0 += 128) {
        // does any q-transition of this tile differ from zero (bits: -0 is zero too)
        unsigned bits = 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const u32x4 x = __builtin_bit_cast(u32x4, cur.q[h][ks].v);
                bits |= (x.x | x.y | x.z | x.w) & 0x7fff7fffu;
            }
        const bool live = __any(bits != 0u);   // wave-uniform
        bool nxt_o = false;
        if (t0 + 128 < tw1) {
            load_q(t0 + 128, nxt);
            if (live) {
                load_o(t0 + 128, nxt);
                nxt_o = true;
            }
        }
        if (!live) {
            cur = nxt;
            cur_o = nxt_o;
            continue;
        }
        if (!cur_o) load_o(t0, cur);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    Frag<bf16> a;
                    a.v = *reinterpret_cast<const bf16x8*>(es + (16 * vt + c16) * RS + 32 * ks + 8 * g4);
                    mma(acc, a, cur.q[h][ks]);
                }
                // acc[e]: value 16 vt + 4 g4 + e of token 16 h + c16
                *reinterpret_cast<f32x4*>(cs + c16 * CS + 16 * vt + 4 * g4) = acc;
            }
            wave_lds_fence();
#pragma unroll
            for (int i = h * (NI / 2); i < (h + 1) * (NI / 2); ++i) {
                const int r = RPI * i + orow;                 // row within the tile
                const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs + (r - 16 * h) * CS + ocol);
                const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + (r - 16 * h) * CS + ocol + 4);
                float x[8];
                Pack<bf16>::unpack(cur.o[i], x);
#pragma unroll
                for (int e = 0; e < 4; ++e) { x[e] += c0[e]; x[4 + e] += c1[e]; }
                if (t0 + r < tw1) st16(o + (size_t)(t0 + r) * DV + ocol, Pack<bf16>::pack(x));
            }
            wave_lds_fence();   // the next half rewrites the tile
        }
        cur = nxt;
        cur_o = nxt_o;
    }
}

template <int DK>
static hipError_t launch_combine_t(const ChunkArgs& a, int CK, const SegPlan& sp)
{
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    const int BH = a.B * a.H;
    SegArgs s{reinterpret_cast<const float*>(ws + sp.off_Z), reinterpret_cast<const float*>(ws + sp.off_P),
              reinterpret_cast<bf16*>(ws + sp.off_E), reinterpret_cast<const bf16*>(ws + sp.off_qt),
              static_cast<bf16*>(a.o), a.S_final, a.L, a.dv, sp.SEG, sp.NCS * CK, sp.N0 * CK};
    hipLaunchKernelGGL(seg_entry_kernel<DK>, dim3(BH * (a.dv / 16)), dim3(64 * (DK / 16)), 0, a.stream, s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int tiles = (s.TS + kTokWG - 1) / kTokWG;
    const dim3 grid(BH * (sp.SEG - 1) * tiles);
    // E_g, then one 16-token correction tile per wave (above the 64 KiB a
    // launch gets without asking, at d_k = d_v = 128)
    const int lds = a.dv * (DK + 8) * 2 + 4 * 16 * (a.dv + 4) * 4;
    auto* kern = a.dv == 128 ? seg_correct_kernel<DK, 128> : seg_correct_kernel<DK, 64>;
    err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, a.stream, s, tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_seg_combine(const ChunkArgs& a, int CK, const SegPlan& sp)
{
    // segmenting is planned for bf16 operands only
    if (a.dtype != kBF16) return hipErrorInvalidValue;
    return a.dk == 128 ? launch_combine_t<128>(a, CK, sp) : launch_combine_t<64>(a, CK, sp);
}

}  // namespace gdr

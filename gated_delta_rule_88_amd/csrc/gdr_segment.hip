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
    int L, DV, SEG, TS;  // TS: tokens per segment
};

// One wave per (head, 16 value rows).  The rows of E evolve independently:
// row r of E_{g+1} is row r of E_g times P_g plus row r of Z_g.
template <int DK>
__global__ __launch_bounds__(64) void seg_entry_kernel(SegArgs p)
{
    constexpr int NJ = DK / 16, NKS = DK / 32;
    __shared__ __align__(16) float rows[16][DK + 4];
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15;
    const int nrb = p.DV / 16;
    const int bh = blockIdx.x / nrb, r0 = 16 * (blockIdx.x % nrb);

    // e[j]: lane holds E[r0 + 4 g4 + i][16 j + c16], i = 0..3
    f32x4 e[NJ];
    const float* Z0 = p.Z + ((size_t)bh * p.SEG * p.DV + r0) * DK;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) e[j][i] = Z0[(size_t)(4 * g4 + i) * DK + 16 * j + c16];

    for (int g = 1; g < p.SEG; ++g) {
        const size_t bs = (size_t)bh * p.SEG + g;
        // keep E_g (bf16) and stage it row-major for the operand reads
        bf16* eb = p.Eb + (bs * p.DV + r0) * DK;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                eb[(size_t)(4 * g4 + i) * DK + 16 * j + c16] = (bf16)e[j][i];
                rows[4 * g4 + i][16 * j + c16] = e[j][i];
            }
        __syncthreads();
        Frag<bf16> a[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = rows[c16][32 * ks + 8 * g4 + i];
            a[ks].v = __builtin_bit_cast(bf16x8, Pack<bf16>::pack(x));
        }
        __syncthreads();
        // E_{g+1} = E_g P_g + Z_g; operand b[j][k] = P_g[k][j] = P_g^T[j][k]
        const float* Pt = p.Pt + bs * DK * DK;
        const float* Zg = p.Z + (bs * p.DV + r0) * DK;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = Zg[(size_t)(4 * g4 + i) * DK + 16 * j + c16];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const float* src = Pt + (size_t)(16 * j + c16) * DK + 32 * ks + 8 * g4;
                float x[8];
                const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) { x[i] = lo[i]; x[4 + i] = hi[i]; }
                Frag<bf16> b;
                b.v = __builtin_bit_cast(bf16x8, Pack<bf16>::pack(x));
                mma(acc, a[ks], b);
            }
            e[j] = acc;
        }
    }
    if (p.S_final) {
        float* sf = p.S_final + ((size_t)bh * p.DV + r0) * DK;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) sf[(size_t)(4 * g4 + i) * DK + 16 * j + c16] = e[j][i];
    }
}

// One workgroup per (head, segment g >= 1, kTokWG tokens): E_g (bf16) in LDS,
// each wave walks 16-token tiles and adds E_g (P up to t) q_t to o.  A tile's
// reads of o and q are all issued before its products, so one round trip to
// memory covers the whole tile.
constexpr int kTokWG = 512;

template <int DK>
__global__ __launch_bounds__(256) void seg_correct_kernel(SegArgs p, int tiles_per_seg)
{
    constexpr int NKS = DK / 32;
    constexpr int RS = DK + 8;                 // padded LDS row (elements)
    constexpr int MAXVT = 8;                   // d_v / 16 <= 8
    extern __shared__ __align__(16) unsigned char smem[];
    bf16* es = reinterpret_cast<bf16*>(smem);
    const int l = lane_id(), g4 = l >> 4, c16 = l & 15, w = wave_id();
    const int per_head = (p.SEG - 1) * tiles_per_seg;
    const int bh = blockIdx.x / per_head;
    const int rem = blockIdx.x % per_head;
    const int g = 1 + rem / tiles_per_seg, tile = rem % tiles_per_seg;
    const int t_seg = g * p.TS, t_end = min(t_seg + p.TS, p.L);
    const int nvt = p.DV / 16;

    const bf16* eb = p.Eb + (((size_t)bh * p.SEG + g) * p.DV) * DK;
    for (int i = threadIdx.x; i < p.DV * DK / 8; i += 256) {
        const int r = i / (DK / 8), c = (i % (DK / 8)) * 8;
        st16(es + r * RS + c, ld16(eb + (size_t)r * DK + c));
    }
    __syncthreads();

    const bf16* qt = p.qt + (size_t)bh * p.L * DK;
    bf16* o = p.o + (size_t)bh * p.L * p.DV;
    const int tw0 = t_seg + kTokWG * tile;
    const int tw1 = min(tw0 + kTokWG, t_end);
    for (int t0 = tw0 + 16 * w; t0 < tw1; t0 += 64) {   // wave-uniform
        const int t = t0 + c16;
        const bool live = t < tw1;
        const int tc = min(t, tw1 - 1);
        Frag<bf16> qf[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qf[ks].v = *reinterpret_cast<const bf16x8*>(qt + (size_t)tc * DK + 32 * ks + 8 * g4);
        // lane (g4, c16): o[t][16 vt + 4 g4 + i]
        bf16* orow = o + (size_t)tc * p.DV + 4 * g4;
        u32x2 cur[MAXVT];
#pragma unroll
        for (int vt = 0; vt < MAXVT; ++vt)
            if (vt < nvt) cur[vt] = ld8(orow + 16 * vt);
#pragma unroll
        for (int vt = 0; vt < MAXVT; ++vt) {
            if (vt < nvt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    Frag<bf16> a;
                    a.v = *reinterpret_cast<const bf16x8*>(es + (16 * vt + c16) * RS + 32 * ks + 8 * g4);
                    mma(acc, a, qf[ks]);
                }
                if (live)
                    st4(orow + 16 * vt, bf_lo(cur[vt].x) + acc[0], bf_hi(cur[vt].x) + acc[1],
                        bf_lo(cur[vt].y) + acc[2], bf_hi(cur[vt].y) + acc[3]);
            }
        }
    }
}

template <int DK>
static hipError_t launch_combine_t(const ChunkArgs& a, int CK, const SegPlan& sp)
{
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    const int BH = a.B * a.H;
    SegArgs s{reinterpret_cast<const float*>(ws + sp.off_Z), reinterpret_cast<const float*>(ws + sp.off_P),
              reinterpret_cast<bf16*>(ws + sp.off_E), reinterpret_cast<const bf16*>(ws + sp.off_qt),
              static_cast<bf16*>(a.o), a.S_final, a.L, a.dv, sp.SEG, sp.NCS * CK};
    hipLaunchKernelGGL(seg_entry_kernel<DK>, dim3(BH * (a.dv / 16)), dim3(64), 0, a.stream, s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int tiles = (s.TS + kTokWG - 1) / kTokWG;
    const int lds = a.dv * (DK + 8) * 2;
    hipLaunchKernelGGL(seg_correct_kernel<DK>, dim3(BH * (sp.SEG - 1) * tiles), dim3(256), lds, a.stream, s,
                       tiles);
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

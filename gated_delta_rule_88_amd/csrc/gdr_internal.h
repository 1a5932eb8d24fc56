// gdr_internal.h -- declarations shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdr {

constexpr int kAlphaNone = 0, kAlphaScalar = 1, kAlphaChannel = 2;
constexpr int kF32 = 0, kBF16 = 1;

// Channel-wise log-decay floor (see gdr.h): keeps every exponential of an
// 8-token partial sum of log alpha inside the fp32 range.
constexpr float kChannelLogAlphaMin = -10.0f;

// Input-side steps the library applies itself on request (gdr.h:
// GDR_PRO_L2NORM_QK, GDR_PRO_GATES).
constexpr unsigned kProNorm = 1u, kProGates = 2u;
constexpr float kNormEps = 1e-6f;   // x / max(||x||_2, eps)

struct DecodeArgs {
    int N, H, dk, dv, dtype, mode;
    const void *q, *k, *v;
    const float *beta, *log_alpha;
    float* S;
    void* o;
    hipStream_t stream;
    unsigned pro;
};

// Packed variable-length batch: NS sequences along one head row of L tokens
// (L = T, the packed length).  Per sequence, computed on the device from the
// caller's cumulative offsets (clamped into [0, T]): its first token, its
// length and its first chunk; choff[NS] is the number of chunks per head,
// at most NCmax = T / CK + NS.  Chunk records are [H][NCmax].
struct Varlen {
    const int *start, *len, *choff;   // start == NULL: fixed-length batch
    int NS, NCmax;
};

struct ChunkArgs {
    int B, H, L, dk, dv, C, dtype, mode;
    const void *q, *k, *v;
    const float *beta, *log_alpha, *S0;
    void* o;
    float* S_final;
    void* workspace;
    hipStream_t stream;
    unsigned pro;
    // packed variable-length batch (B = 1, L = T): cumulative offsets
    // [NS + 1] in device memory, or NULL; vl is filled in by the driver
    const int* cu_seqlens;
    int NS;
    Varlen vl;
    // backward's forward recompute: every chunk's entry state, or null
    void* Sck;
    // backward's forward recompute: every chunk's T = (I + A)^{-1} (fp32
    // [CK][CK], zero above the diagonal), or null
    float* Tout;
    // the entry state is kept for chunks 0, sck_every, 2 sck_every, ...
    // counted over all heads (0: every chunk)
    int sck_every;
};

struct BwdArgs {
    int B, H, L, dk, dv, C, dtype, mode;
    const void *q, *k, *v;
    const float *beta, *log_alpha, *S0;
    const void* dO;
    const float* dS_final;
    void *dq, *dk_out, *dv_out;
    float *dbeta, *dlog_alpha, *dS0;
    void* workspace;
    hipStream_t stream;
    // kBwdAll: recompute the forward's records and entry states, then the
    // gradients; kBwdKeep: the forward only, also writing o and S_final (a
    // training step's forward that keeps them); kBwdKept: the gradients only,
    // from a workspace a kBwdKeep call filled
    int part;
    void* o;
    float* S_final;
};
constexpr int kBwdAll = 0, kBwdKeep = 1, kBwdKept = 2;

// Bytes of device workspace the chunked forward needs.
size_t chunk_workspace_bytes(int B, int H, int L, int dk, int dv, int C, int dtype, int mode);
size_t varlen_workspace_bytes(int NS, int H, int T, int dk, int dv, int C, int dtype, int mode);

// The chunked forward's argument checks and launches (gdr_fwd_chunked_ex).
int fwd_chunked_checked(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                        const void* q, const void* k, const void* v,
                        const float* beta, int alpha_mode, const float* log_alpha,
                        const float* S0, void* o, float* S_final,
                        void* workspace, size_t workspace_bytes, hipStream_t stream,
                        unsigned prologue);
// Bytes of workspace the chunked forward plans for these sizes, or
// (size_t)-1 for sizes outside the domain.
size_t fwd_chunked_workspace_checked(int B, int H, int L, int dk, int dv, int C, int dtype, int mode);

hipError_t launch_decode_step(const DecodeArgs& a);
hipError_t launch_fwd_chunked(const ChunkArgs& a);
hipError_t launch_fwd_varlen(ChunkArgs a);
size_t bwd_workspace_bytes(int B, int H, int L, int dk, int dv, int C, int dtype, int mode);
hipError_t launch_bwd_chunked(const BwdArgs& b);

}  // namespace gdr

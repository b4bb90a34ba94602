// attn_kernels.h -- internal interface between the C ABI (attn_api.hip) and
// the kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>

namespace cattn {

struct RopeFreqs {
    double f[64];  // base^(-2i/D) / (2 pi), i < D/2: revolutions per position
};

// Element strides of a [B][H][T][D] tensor whose D elements are contiguous.
struct Strides {
    long long sb, sh;  // between batches, between heads
    int st;            // between tokens
};

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;   // forward: output; backward: input
    const void* dO;
    void* o_out;     // forward output (same buffer as o)
    void* dq;
    void* dk;
    void* dv;
    float* lse;      // forward: output; backward: input
    float* delta;    // backward workspace / output
    int B, H, T, D;
    float scale;
    int n_cu;        // compute units of the current device (work placement)
    int window;      // sliding window W (query q sees keys q-W < k <= q); 0 = plain causal.
                     // Only the bf16 D=64/128 kernels take it; the entry points with a
                     // window argument accept no other case.
    int dropout_p16;                  // attention dropout: round(p * 65536); 0 = none
    unsigned long long dropout_seed;  // Philox key
    // stored keep bits, [B*H][ceil(T/32)][T] words (bit t of word (bh, w, i): query i,
    // key 32w + t): the forward writes them when set, the backward reads them
    // instead of drawing; nullptr: the backward draws them again
    unsigned int* keep;
    // strides of q, k, v, o, dO, dq, dk, dv (contiguous unless a strided entry point set them)
    Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
    // RoPE / QK-norm prologue fused into the kernels (bf16, D = 64 / 128, no dropout).
    // Forward: q, k are the rows before the prologue; k_rot gets the keys after it (a
    // separate pass) and q_rot the queries (written by the forward).  Backward: q, k are
    // the rows after the prologue, xq, xk the rows before; dq, dk are taken with respect
    // to xq, xk.
    bool rope;
    const void* xq;
    const void* xk;
    void* q_rot;
    void* k_rot;
    Strides sxq, sxk, sqr, skr;
    int pos0, rope_flags;
    float q_gain, k_gain, rope_eps;
    RopeFreqs freqs;
};

// Decode (one query per sequence against a [B][T_max][H][D] KV cache).
struct DecodeArgs {
    const void* q;        // [B][H][D]
    const void* k_cache;  // [B][T_max][H][D]
    const void* v_cache;
    const int* lens;      // [B] cached positions per sequence (clamped to [0, T_max])
    void* o;              // [B][H][D]
    float* lse;           // [B][H]
    float* part;          // workspace: [B][H][decode_slices(T_max)][D + 4] fp32
    int B, H, T_max, D;
    int window;           // 0: every cached position
    float scale;
    int n_cu;             // compute units of the device (picks one launch or split-K)
};

int decode_slices(int T_max);
// true when launch_decode_bf16 takes the two-launch path (which needs a.part)
bool decode_two_launches(const DecodeArgs& a);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t st);
// launch_decode_bf16 with a.part pointing at the library's fixed scratch
// (CAUSAL_ATTN_DECODE_SCRATCH_BYTES per device); the caller has checked that
// the two-launch path's partials fit in it
hipError_t launch_decode_bf16_noalloc(DecodeArgs a, hipStream_t st);

// RoPE / QK norm on query and key rows (forward, or gradient when grad is set).

struct RopeArgs {
    const void* q;       // [B][H][T][D] views (strides sq, sk)
    const void* k;
    void* q_out;         // forward: results; gradient: dq, dk (strides sqo, sko)
    void* k_out;
    const void* dq_in;   // gradient only: d(loss)/d(forward result)
    const void* dk_in;
    Strides sq, sk, sqo, sko, sdq, sdk;
    RopeFreqs freqs;
    int B, H, T, D;
    int pos0;            // position of row t = pos0 + t
    int flags;           // bit 0: RoPE, bit 1: QK norm
    float q_gain, k_gain, eps;
    bool grad;
    bool k_only;  // forward on the keys alone (k -> k_out); q, q_out unused
};

hipError_t launch_rope_qknorm(const RopeArgs& a, hipStream_t st);

// LayerNorm and column sums over bf16 rows (the sublayer around the attention).
struct NormArgs {
    const void* x;     // [N][C] rows, `stride` elements apart
    const void* g;     // [C] gain (LayerNorm)
    const void* b;     // [C] bias (LayerNorm forward)
    const void* dy;    // gradient: d(loss)/d(LayerNorm output), rows like x
    const void* dres;  // gradient: residual term added to dx (nullptr: none)
    void* y;           // forward: output rows; colsum: the [C] sums
    void* dx;          // gradient: rows like x
    void* dg;          // gradient: [C]
    void* db;          // gradient: [C]
    void* workspace;   // fp32 column partials (layernorm_bwd_workgroups(N) x 2C, or
                       // colsum_row_blocks(N) x C)
    int N, C;
    long long stride;
    float eps;
    bool f32;          // colsum: fp32 rows (x), no workspace
};

int layernorm_bwd_workgroups(int N);
int colsum_row_blocks(int N);
hipError_t launch_layernorm_fwd(const NormArgs& a, hipStream_t st);
hipError_t launch_layernorm_bwd(const NormArgs& a, hipStream_t st);
hipError_t launch_colsum(const NormArgs& a, hipStream_t st);

// launch_dq_* computes delta (from o and dO) as well as dq.
hipError_t launch_fwd_bf16(const AttnArgs& a, hipStream_t st);
hipError_t launch_dq_bf16(const AttnArgs& a, hipStream_t st);
hipError_t launch_dkdv_bf16(const AttnArgs& a, hipStream_t st);
hipError_t launch_fwd_bf16_d64(const AttnArgs& a, hipStream_t st);
hipError_t launch_dq_bf16_d64(const AttnArgs& a, hipStream_t st);
hipError_t launch_dkdv_bf16_d64(const AttnArgs& a, hipStream_t st);
// the whole bf16 backward (Delta, dq, dk, dv)
hipError_t launch_bwd_bf16(const AttnArgs& a, hipStream_t st);
hipError_t launch_bwd_bf16_d64(const AttnArgs& a, hipStream_t st);
hipError_t launch_fwd_f32(const AttnArgs& a, hipStream_t st);
hipError_t launch_dq_f32(const AttnArgs& a, hipStream_t st);
hipError_t launch_dkdv_f32(const AttnArgs& a, hipStream_t st);

}  // namespace cattn

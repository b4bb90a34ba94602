// attn_device.h -- device-side types and helpers for the gfx950 attention
// kernels (MFMA wrappers, bf16 packing, LDS tile loaders).
//
// MFMA lane layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16):  lane l supplies A[l % 32][8 * (l / 32) + e], e = 0..7
//   B (16 x 32):  lane l supplies B[8 * (l / 32) + e][l % 32], e = 0..7
//   C (32 x 32):  lane l holds C[8 * (r / 4) + 4 * (l / 32) + (r % 4)][l % 32]
//                 in accumulator register r = 0..15.
// A C tile is turned into B operands for a following product whose
// contraction runs over the C tile's rows: K-step c (rows 16c .. 16c+15) takes
// registers 8 * (c % 2) .. 8 * (c % 2) + 7 of row-subtile c / 2.  Inside each
// 16-row chunk the lane then carries rows 8 * (e / 4) + 4 * (l / 32) + (e % 4),
// i.e. MFMA k-slot p holds row p with bits 2 and 3 swapped.  The matching A
// operand is read from an LDS tile whose rows were stored in that same order
// (see load_tile_transposed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS poisoning, for debug builds compiled with -DCATTN_LDS_POISON: every LDS
// array of a kernel is filled with all-ones words (a NaN as fp32 and as each
// bf16 half) before the kernel touches LDS, so that a read of LDS the kernel
// has not written shows up as NaN or as a changed result instead of reusing
// whatever an earlier workgroup left there.  Release builds compile it away.
template <typename T>
__device__ __forceinline__ void lds_poison_one(T& a)
{
    static_assert(sizeof(T) % 4 == 0, "LDS arrays are whole 32-bit words");
    uint32_t* w = (uint32_t*)&a;
    for (int i = threadIdx.x; i < (int)(sizeof(T) / 4); i += blockDim.x) w[i] = 0xFFFFFFFFu;
}

template <typename... Ts>
__device__ __forceinline__ void lds_poison(Ts&... a)
{
#ifdef CATTN_LDS_POISON
    (lds_poison_one(a), ...);
    __syncthreads();
#else
    ((void)a, ...);
#endif
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of x held by lane (l ^ 32).
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ bf16x8 zero_bf16x8()
{
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
    return z;
}

// 8 fp32 values -> 8 bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack_bf16x8(const f32x16& acc, int first)
{
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)acc[first + e];
    return r;
}

// Position of row `r` of a 16-row chunk inside a transposed LDS tile:
// bits 2 and 3 swapped (the k-slot order of an accumulator-derived B operand).
__device__ __forceinline__ int kslot_of_row(int r)
{
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Cooperative copy of rows [row0, row0 + ROWS) of a [T][HD] bf16 matrix into
// LDS, row-major with row stride LDS_STRIDE elements.  Rows >= T are zeroed.
template <int ROWS, int HD, int LDS_STRIDE, int NTHREADS>
__device__ __forceinline__ void load_tile_rows(bf16* __restrict__ lds, const bf16* __restrict__ src,
                                               int row0, int T, int tid)
{
    constexpr int CHUNKS = HD / 8;  // 16-byte chunks per row
#pragma unroll
    for (int c = tid; c < ROWS * CHUNKS; c += NTHREADS) {
        const int r = c / CHUNKS, cc = c % CHUNKS;
        bf16x8 val = zero_bf16x8();
        if (row0 + r < T) val = *(const bf16x8*)(src + (size_t)(row0 + r) * HD + cc * 8);
        *(bf16x8*)(lds + r * LDS_STRIDE + cc * 8) = val;
    }
}

// Cooperative transposed copy: rows [row0, row0 + ROWS) of a [T][HD] bf16
// matrix become columns of an [HD][ROWS] LDS tile (row stride LDS_STRIDE),
// with the rows of every 16-row chunk stored in k-slot order
// (kslot_of_row).  Rows >= T are zeroed.  Each work unit moves a 2-column x
// 8-row block: 8 dword loads, 4 packed 8-byte LDS stores.
template <int ROWS, int HD, int LDS_STRIDE, int NTHREADS>
__device__ __forceinline__ void load_tile_transposed(bf16* __restrict__ lds,
                                                     const bf16* __restrict__ src, int row0,
                                                     int T, int tid)
{
    static_assert(ROWS % 16 == 0, "transposed tiles hold whole 16-row chunks");
    constexpr int PAIRS = HD / 2;
    constexpr int OCTETS = ROWS / 8;
#pragma unroll
    for (int u = tid; u < PAIRS * OCTETS; u += NTHREADS) {
        const int dp = u % PAIRS, ko = u / PAIRS;
        uint32_t w[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int row = row0 + 8 * ko + r;
            w[r] = (row < T) ? *(const uint32_t*)(src + (size_t)row * HD + 2 * dp) : 0u;
        }
        // rows 8ko+0..3 go to slots 16*(ko/2) + 4*(ko%2) + 0..3,
        // rows 8ko+4..7 go to slots 16*(ko/2) + 8 + 4*(ko%2) + 0..3.
        const int s0 = 16 * (ko >> 1) + 4 * (ko & 1);
        const int s1 = s0 + 8;
        u32x2 lo0, lo1, hi0, hi1;
        lo0[0] = (w[0] & 0xffffu) | (w[1] << 16);
        lo0[1] = (w[2] & 0xffffu) | (w[3] << 16);
        lo1[0] = (w[4] & 0xffffu) | (w[5] << 16);
        lo1[1] = (w[6] & 0xffffu) | (w[7] << 16);
        hi0[0] = (w[0] >> 16) | (w[1] & 0xffff0000u);
        hi0[1] = (w[2] >> 16) | (w[3] & 0xffff0000u);
        hi1[0] = (w[4] >> 16) | (w[5] & 0xffff0000u);
        hi1[1] = (w[6] >> 16) | (w[7] & 0xffff0000u);
        bf16* even = lds + (2 * dp) * LDS_STRIDE;
        bf16* odd = even + LDS_STRIDE;
        *(u32x2*)(even + s0) = lo0;
        *(u32x2*)(even + s1) = lo1;
        *(u32x2*)(odd + s0) = hi0;
        *(u32x2*)(odd + s1) = hi1;
    }
}

// Store 4 consecutive fp32 values as bf16 (8 bytes).
__device__ __forceinline__ void store_bf16x4(bf16* dst, float a, float b, float c, float d)
{
    bf16x4 v;
    v[0] = (bf16)a;
    v[1] = (bf16)b;
    v[2] = (bf16)c;
    v[3] = (bf16)d;
    *(bf16x4*)dst = v;
}

}  // namespace cattn

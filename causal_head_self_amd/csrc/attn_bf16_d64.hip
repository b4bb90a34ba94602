// attn_bf16_d64.hip -- gfx950 kernels for causal multi-head self-attention
// at head dims 64 and 128 (tiles of 64-column panels), bf16 storage / fp32
// accumulation: forward, dQ and dK/dV, with optional sliding window and
// attention dropout, on strided [B][H][T][D] views.
//
// Same operation as attn_bf16.hip (CS336 from-scratch tutorial, lmnt.cn,
// section 5.1 CausalSelfAttention.forward; the tril mask keeps the diagonal,
// "Train Your Own LLM from Scratch", section 1; the backward is the exact
// gradient the pages train through, tutorial section 5.2).  The GPT-2-small,
// ~400M and long-context shapes run here:
//
//  * Streamed tiles (64 rows x 128 bytes) travel HBM -> LDS with the
//    asynchronous global_load_lds (16 bytes per lane; one wave instruction
//    fills 8 consecutive rows), double-buffered: the copy of tile j+1 is in
//    flight while tile j is multiplied, with one barrier per tile.
//  * LDS tiles are row-major with the 16-byte chunks of each row XOR-swizzled
//    (chunk ^ swz(row)), so that both the row reads of the MFMA A operand
//    (ds_read_b128, 16 rows per pass) and the transposing reads
//    (ds_read_b64_tr_b16, 4 rows x 64 bytes per pass) are bank-conflict free.
//  * Transposed operands (V^T, K^T, Q^T, dO^T) come straight from the
//    row-major tile through ds_read_b64_tr_b16: inside each 16-lane group,
//    lane i receives element i%4 of the 8-byte chunks fetched by lanes
//    4e + i/4 (e = 0..3), i.e. 4 consecutive rows of one column.
//  * Online softmax (forward): row max in-lane with v_max3 plus one
//    v_permlane32_swap; the running max is only raised when it grows by more
//    than 2^8 in the exponent (lazy rescale), so most tiles skip rescaling
//    the accumulators; the row sum is taken on the bf16 P that feeds the PV
//    product, two at a time with v_dot2_f32_bf16.
#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"

namespace cattn {
namespace d64 {

constexpr int HD = 64;           // columns per panel
constexpr int kThreads = 256;
constexpr int kRowsPerWG = 128;  // queries (forward, dQ) or keys (dK/dV) per workgroup
constexpr int kTile = 64;        // rows per streamed tile
constexpr int kTileBytes = kTile * HD * 2;  // one panel of a tile

// Head dim 64 * NP (NP = 1 or 2).  A streamed tile is NP panels of kTileBytes,
// panel p holding columns 64p .. 64p+63 of its 64 rows in the swizzled layout
// below, so that every copy and operand read works on one panel as it does at
// head dim 64.  Register-resident rows and accumulators grow with NP; at NP = 2
// the kernels run 2 waves per SIMD instead of 3.
template <int NP>
constexpr int kWavesPerEU = NP == 1 ? 3 : 2;
constexpr float kLazyRescale = 8.0f;  // log2 growth of the running max that forces a rescale

// Attention dropout (the softmax weights go through dropout before the product
// with V, CS336 tutorial section 5.1; inverted dropout in training mode).  The
// keep decision of weight (bh, query i, key j) is a Philox4x32-10 draw (Salmon
// et al., SC 2011): counter (j / 8, i, bh, 0) under the 64-bit seed as the key;
// key j takes the 16-bit half j % 2 of output word (j % 8) / 2 and is kept iff
// that value is >= p16.  Kept weights are scaled by 65536 / (65536 - p16),
// which the kernels apply once to their fp32 accumulators.
struct Dropout {
    uint32_t seed_lo, seed_hi;
    uint32_t p16;       // 0: no dropout
    float keep_scale;   // 65536 / (65536 - p16)
    // Stored keep bits (nullptr: none): word (bh, w, i) of [BH][ceil(T/32)][T] holds
    // bit t = keep decision of query i and key 32w + t.  The forward writes the
    // words it draws; the backward items then load them instead of drawing.
    uint32_t* keep;
};

// Word of the stored keep bits for query i and keys 32w .. 32w + 31.
__device__ __forceinline__ size_t keep_index(int bh, int w, int i, int T)
{
    return ((size_t)bh * ((T + 31) / 32) + w) * T + i;
}

// kWide: each 32 x 32 -> 64-bit product as one v_mad_u64_u32 (about the cost
// of a v_mul_hi_u32 alone), else as v_mul_hi_u32 + v_mul_lo_u32, which need no
// aligned register pair (the dK/dV items are at their register limit).
template <bool kWide>
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1, uint32_t (&r)[4])
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        uint32_t hi0, lo0, hi1, lo1;
        if constexpr (kWide) {
            const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
            hi0 = (uint32_t)(p0 >> 32);
            lo0 = (uint32_t)p0;
            hi1 = (uint32_t)(p1 >> 32);
            lo1 = (uint32_t)p1;
        } else {
            hi0 = __umulhi(0xD2511F53u, c0);
            lo0 = 0xD2511F53u * c0;
            hi1 = __umulhi(0xCD9E8D57u, c2);
            lo1 = 0xCD9E8D57u * c2;
        }
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    r[0] = c0;
    r[1] = c1;
    r[2] = c2;
    r[3] = c3;
}

// Draws of the 8-key block `blk` for query i: word w, half h is key 8 blk + 2w + h.
template <bool kWide>
__device__ __forceinline__ void drop_block(const Dropout& dr, int bh, int i, int blk, uint32_t (&r)[4])
{
    philox4x32_10<kWide>((uint32_t)blk, (uint32_t)i, (uint32_t)bh, 0u, dr.seed_lo, dr.seed_hi, r);
}

// Keep bits of the 8-key block `blk` for query i: bit t is key 8 blk + t.  Lanes
// draw only the blocks assigned to them and pass the bit words to the lanes
// whose accumulators hold those weights (one Philox call per 8 weights).
template <bool kWide = true>
__device__ __forceinline__ uint32_t drop_bits8(const Dropout& dr, int bh, int i, int blk)
{
    uint32_t r[4];
    drop_block<kWide>(dr, bh, i, blk, r);
    uint32_t b = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) b |= (uint32_t)(((r[t >> 1] >> (16 * (t & 1))) & 0xFFFFu) >= dr.p16) << t;
    return b;
}

// x through an empty asm statement: the compiler cannot treat values computed
// from the result as loop-invariant, so it recomputes them where they are used
// instead of hoisting them out of a loop (where they may be kept live across the
// tiles and spilled)
__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// The value of x held by lane l ^ 32 (v_permlane32_swap; which of the two
// results is the other lane's is told apart by comparing with x itself).
__device__ __forceinline__ uint32_t other_half_u32(uint32_t x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return r[0] == x ? r[1] : r[0];
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// XOR key of row r: a bijection of (r >> 1) & 7 whose value for the row pairs
// {4a, 4a+1} and {4a+2, 4a+3} differs in bit 2.
__device__ __forceinline__ int swz(int r)
{
    const int s = (r >> 1) & 7;
    return ((s & 1) << 2) | (s >> 1);
}

// Byte offset of 16-byte chunk `c` of row `r` in a swizzled tile.
__device__ __forceinline__ int chunk_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }

// Asynchronous copy of rows [row0, row0 + 64) of a [T][64] bf16 head into a
// swizzled LDS tile.  Each of the 4 waves moves 16 rows, 8 per instruction:
// lane l writes physical chunk l & 7 of row l >> 3 of its 1 KB block and so
// fetches that row's logical chunk (l & 7) ^ swz(row).  The per-lane byte
// offsets are constant; a full tile then needs only a scalar base per copy.
// Rows >= T (last tile only) read row T-1 instead (always valid memory); the
// kernels mask those rows.  Rows are `st` elements apart in memory (64 for a
// contiguous [B][H][T][64] tensor).
struct TileCopy {
    uint32_t cb[2];  // byte offset of this lane's 16 bytes inside its row, per instruction
    __device__ __forceinline__ TileCopy(int wave, int lane)
    {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int row = wave * 16 + it * 8 + (lane >> 3);
            cb[it] = (uint32_t)((lane & 7) ^ swz(row)) * 16u;
        }
    }
};

// All addresses are a wave-uniform base plus a 32-bit per-lane offset (the
// scalar-base form of global_load_lds), which keeps 64-bit address arithmetic
// out of the vector registers.
// kOpaque: take the lane index through an opaque copy, so that the per-lane
// offsets are recomputed at every copy instead of being kept live across the
// loops.  The kernels that run short of registers (dropout, head dim 128) use
// it: there the compiler otherwise spills those offsets, and reloading them
// makes each copy wait for the one issued before it.
template <bool kOpaque>
__device__ __forceinline__ void tile_load_async(char* tile, const bf16* __restrict__ head, int st,
                                                int row0, int T, int wave, const TileCopy& tc)
{
    const char* base = (const char*)head;
    const uint32_t sb = (uint32_t)st * 2u;
    int lane = __lane_id();
    if constexpr (kOpaque) asm volatile("" : "+v"(lane));
    if (row0 + kTile <= T) {  // wave-uniform: every row exists
        const char* b = base + (size_t)row0 * sb;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const uint32_t o = (uint32_t)(wave * 16 + it * 8 + (lane >> 3)) * sb + tc.cb[it];
            __builtin_amdgcn_global_load_lds((const void*)(b + o),
                                             (__attribute__((address_space(3))) void*)(tile + (wave * 16 + it * 8) * 128),
                                             16, 0, 0);
        }
    } else {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int row = wave * 16 + it * 8 + (lane >> 3);
            const uint32_t o = (uint32_t)min(row0 + row, T - 1) * sb + tc.cb[it];
            __builtin_amdgcn_global_load_lds((const void*)(base + o),
                                             (__attribute__((address_space(3))) void*)(tile + (wave * 16 + it * 8) * 128),
                                             16, 0, 0);
        }
    }
}

// The NP panels of a tile: columns 64p.. of the head go to panel p.
template <int NP, bool kOpaque = false>
__device__ __forceinline__ void tiles_load_async(char* tile, const bf16* __restrict__ head, int st,
                                                 int row0, int T, int wave, const TileCopy& tc)
{
    tile_load_async<kOpaque>(tile, head, st, row0, T, wave, tc);
    if constexpr (NP == 2) tile_load_async<kOpaque>(tile + kTileBytes, head + HD, st, row0, T, wave, tc);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima) as the builtin, which
// the compiler's wait-count pass sees, so that it does not wait again later for
// copies it cannot tell have landed
__device__ __forceinline__ void wait_async_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ bf16x8 lds_row_read(const char* tile, int off)
{
    return *(const bf16x8*)(tile + off);
}

// Two transposing reads -> the 8-element A operand of one k-step.
__device__ __forceinline__ bf16x8 lds_tr_read(const char* tile, int off0, int off1)
{
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tile + off0));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tile + off1));
    const v4s cat[2] = {lo, hi};
    return *(const bf16x8*)cat;
}

// Combined value over lanes l and l ^ 32 (max or sum).
__device__ __forceinline__ float halves_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float halves_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-lane LDS offsets of the operand reads (constant over the kernel).
struct Offsets {
    int nat[4];     // row read: row li, chunk 2*ks + hi   (add 4096 for rows 32..63)
    int tr[2][2];   // transposed read [half][dt]          (add 2048 per k-step)
    __device__ __forceinline__ Offsets(int lane)
    {
        const int li = lane & 31, hi = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) nat[ks] = chunk_off(li, 2 * ks + hi);
        const int j = lane & 15, g16 = lane >> 4;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                const int row = 8 * half + 4 * hi + (j >> 2);
                const int chunk = 2 * (2 * dt + (g16 & 1)) + ((j & 3) >> 1);
                tr[half][dt] = chunk_off(row, chunk) + 8 * (j & 1);
            }
    }
};

__device__ __forceinline__ bf16x8 pack8(const f32x16& acc, int first)
{
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)acc[first + e];
    return r;
}

// sum of 8 bf16 values in fp32, two per v_dot2_f32_bf16
__device__ __forceinline__ float sum8(bf16x8 v, float acc)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        bf16x2 p = {v[e], v[e + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(p, ones, acc, false);
    }
    return acc;
}

// S = A B over the 64 rows of an LDS tile: rows 0..31 -> s0, rows 32..63 -> s1.
// A is read from the tile (row reads, panel by panel), B comes from registers
// (k-steps 4p .. 4p+3 for panel p).
template <int NP>
__device__ __forceinline__ void tile_product(const char* tile, const Offsets& off,
                                             const bf16x8 (&breg)[4 * NP], f32x16& s0, f32x16& s1)
{
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const char* t = tile + p * kTileBytes;
        bf16x8 a[8];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            a[ks] = lds_row_read(t, off.nat[ks]);
            a[4 + ks] = lds_row_read(t, 4096 + off.nat[ks]);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            s0 = mfma32x32x16(a[ks], breg[4 * p + ks], s0);
            s1 = mfma32x32x16(a[4 + ks], breg[4 * p + ks], s1);
        }
    }
}

// Causal mask of a (key-subtile, query-lane) score tile: element r of s0
// holds row 8(r/4) + 4hi + r%4 of the tile (+32 in s1); it stays iff
// lo < that row offset <= lim (the causal window i - W < j <= i seen from the
// tile), otherwise it becomes -inf.
__device__ __forceinline__ void mask_band(f32x16& s0, f32x16& s1, int lim, int lo)
{
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + (r & 3);
        s0[r] = kk <= lim && kk > lo ? s0[r] : -INFINITY;
        s1[r] = kk + 32 <= lim && kk + 32 > lo ? s1[r] : -INFINITY;
    }
}

// Work placement.  Items are numbered heaviest first.  When a launch fits the
// machine in one pass, MI355X places workgroups x, x + n_cu, x + 2 n_cu, ... on
// one compute unit and workgroup x on XCD x % 8 (observed with per-workgroup
// hardware ids).  Every odd layer of n_cu workgroups takes its items in reverse,
// in blocks of 8 so that x % 8 and with it the XCD of each head's items does not
// change; each compute unit then holds a heavy, a middle and a light item
// instead of three of about the same weight.  A partial last layer keeps the
// plain order.  The map is a permutation of [0, n_items) for any n_cu.
__device__ __forceinline__ int item_of(int x, int n_items, int n_cu)
{
    if (n_cu <= 0 || (n_cu & 7)) return x;
    const int r = x / n_cu, p = x - r * n_cu;
    if (!(r & 1) || (r + 1) * n_cu > n_items) return x;
    return r * n_cu + 8 * ((n_cu >> 3) - 1 - (p >> 3)) + (p & 7);
}

// A [B][H][T][64] bf16 tensor with element strides: (b, h, t, d) sits at
// p + b*sb + h*sh + t*st + d.  Contiguous tensors have sb = H*T*64,
// sh = T*64, st = 64.
struct View {
    bf16* p;
    long long sb, sh;
    int st;
};

__device__ __forceinline__ bf16* head_of(const View& v, int bh, int H)
{
    const int b = bh / H, h = bh - b * H;
    return v.p + (long long)b * v.sb + (long long)h * v.sh;
}

// RoPE / QK-norm prologue fused into the kernels (nanochat, section 9 lists
// RoPE and QK norm among its attention's parts; standard forms, as in
// attn_rope.hip): the row at position p = pos0 + t becomes
//   y = gain * R(x) / sqrt(mean(x^2) + eps)   (R alone without the norm),
// R turning column pair (i, i + D/2) by p * base^(-2i/D).  The forward
// applies it to its register-resident query rows (and writes them out for the
// backward); the backward items apply the transposed Jacobian of the prologue
// to their dQ (dK) rows before storing them:
//   dx = R^T(gain/rms g - gain/rms^3 mean(g z) z),  z = R(x).
struct RopeP {
    View xq, xk;  // rows before the prologue (backward: where the gradient is taken)
    View yq;      // forward: the queries after the prologue, written for the backward
    int pos0, flags;  // flags: bit 0 RoPE, bit 1 QK norm
    float q_gain, k_gain, eps;
    RopeFreqs fr;  // revolutions per position of pair i, base^(-2i/D) / (2 pi)
    double step4, step8;  // base^(-8/D), base^(-16/D): pair i + 4 (+ 8) over pair i
};
struct NoRope {};
template <bool kRope>
using RopeArg = typename std::conditional<kRope, RopeP, NoRope>::type;

// Index 0, opaque to the compiler: table reads indexed from it are issued where
// the table is used, not hoisted to the kernel's start and held in scalar
// registers through the main loop.
__device__ __forceinline__ int here0()
{
    int z = 0;
    asm volatile("" : "+s"(z));
    return z;
}

// Position times this lane's frequency multiplier: a lane of the upper half
// (hi = 1) turns pair i + di where the lower half turns pair i, and
// base^(-2(i + di)/D) = base^(-2i/D) * step with step = base^(-2di/D), so one
// wave-uniform table entry serves both halves.
__device__ __forceinline__ double lane_pos(int p, int hi, double step)
{
    return (double)p * (hi ? step : 1.0);
}

// Cosine and sine of the angle pm * f revolutions (one fp64 multiply, the
// fraction to the hardware sine and cosine).
__device__ __forceinline__ void rope_angle(const RopeP& rp, double pm, double f, float& c, float& s)
{
    c = 1.f;
    s = 0.f;
    if (rp.flags & 1) {
        const double r = pm * f;
        const float turn = (float)(r - floor(r));
        s = __builtin_amdgcn_sinf(turn);
        c = __builtin_amdgcn_cosf(turn);
    }
}

// Forward prologue of one query row held as MFMA operands: x[ks] holds columns
// 16 ks + 8 hi .. + 7 (the other 32 of each 64 in lane l ^ 32), so pair
// (i, i + D/2) sits in x[ks] and x[ks + 2 NP] of the same lane.
template <int NP>
__device__ __forceinline__ void rope_rows(bf16x8 (&x)[4 * NP], const RopeP& rp, int p, int hi)
{
    constexpr int D = HD * NP, HALF = 2 * NP;
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4 * NP; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf((float)x[ks][e], (float)x[ks][e], ss);
    const bool norm = rp.flags & 2;
    const float f = norm ? rp.q_gain / sqrtf(halves_sum(ss) / (float)D + rp.eps) : 1.f;
    const int i0 = here0();
    const double pm = lane_pos(p, hi, rp.step8);
#pragma unroll
    for (int ks = 0; ks < HALF; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float c, s;
            rope_angle(rp, pm, rp.fr.f[i0 + 16 * ks + e], c, s);
            const float u = (float)x[ks][e], w = (float)x[ks + HALF][e];
            x[ks][e] = (bf16)(f * (u * c - w * s));
            x[ks + HALF][e] = (bf16)(f * (u * s + w * c));
        }
}

// Backward epilogue of one row: acc[dt][4g + e] times mult is the gradient with
// respect to the prologue's output at column 32 dt + 8 g + 4 hi + e (pair
// (i, i + D/2) in acc[dt] and acc[dt + NP] of the same lane); xr points at the
// row before the prologue, readable in every lane (for a row past T, valid
// false, it points at a row of the sequence and the lane's results are
// dropped; lanes l and l ^ 32 hold the same row).  Stores the gradient with
// respect to that row, in bf16, where valid.  The row's sum of squares and m = sum(g z) over the whole
// row are needed before any output, so the row is swept twice.  At head dim 64
// the row and its angles are kept in registers between the sweeps (the loads
// issued first, the angles computed while they are in flight); at 128 that
// would spill, so the second sweep loads and computes them again.
template <int NP>
__device__ __forceinline__ void rope_grad_store(const f32x16 (&acc)[2 * NP], float mult,
                                                const bf16* xr, bool valid, bf16* out,
                                                const RopeP& rp, float gain, int p, int hi)
{
    constexpr int D = HD * NP;
    constexpr bool kKeep = NP == 1;
    bf16x4 u[NP][4], w[NP][4];
    float c[NP][4][4], s[NP][4][4];
    auto load = [&](int dt, int g) {
        u[dt][g] = *(const bf16x4*)(xr + 32 * dt + 8 * g + 4 * hi);
        w[dt][g] = *(const bf16x4*)(xr + 32 * (dt + NP) + 8 * g + 4 * hi);
    };
    const int i0 = here0();
    const double pm = lane_pos(p, hi, rp.step4);
    auto angles = [&](int dt, int g) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            rope_angle(rp, pm, rp.fr.f[i0 + 32 * dt + 8 * g + e], c[dt][g][e], s[dt][g][e]);
    };
    // z = R(x) at (dt, g, e)
    auto rot = [&](int dt, int g, int e, float& zl, float& zh) {
        const float a = (float)u[dt][g][e], b = (float)w[dt][g][e];
        zl = a * c[dt][g][e] - b * s[dt][g][e];
        zh = a * s[dt][g][e] + b * c[dt][g][e];
    };
#pragma unroll
    for (int dt = 0; dt < NP; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) load(dt, g);
    float ss = 0.f, m = 0.f;
#pragma unroll
    for (int dt = 0; dt < NP; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            angles(dt, g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = (float)u[dt][g][e], b = (float)w[dt][g][e];
                float zl, zh;
                rot(dt, g, e, zl, zh);
                ss = fmaf(a, a, fmaf(b, b, ss));
                m = fmaf(mult * acc[dt][4 * g + e], zl, fmaf(mult * acc[dt + NP][4 * g + e], zh, m));
            }
        }
    float a1 = 1.f, a3 = 0.f;
    if (rp.flags & 2) {
        const float inv = 1.0f / sqrtf(halves_sum(ss) / (float)D + rp.eps);
        a1 = gain * inv;
        a3 = gain * inv * inv * inv * (halves_sum(m) / (float)D);
    }
    if (!valid) return;
    // dx = R^T(a1 g - a3 z)
#pragma unroll
    for (int dt = 0; dt < NP; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if constexpr (!kKeep) {
                load(dt, g);
                angles(dt, g);
            }
            float lo[4], hv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float zl, zh;
                rot(dt, g, e, zl, zh);
                const float cc = c[dt][g][e], sn = s[dt][g][e];
                const float dl = a1 * (mult * acc[dt][4 * g + e]) - a3 * zl;
                const float dh = a1 * (mult * acc[dt + NP][4 * g + e]) - a3 * zh;
                lo[e] = dl * cc + dh * sn;
                hv[e] = -dl * sn + dh * cc;
            }
            store_bf16x4(out + 32 * dt + 8 * g + 4 * hi, lo[0], lo[1], lo[2], lo[3]);
            store_bf16x4(out + 32 * (dt + NP) + 8 * g + 4 * hi, hv[0], hv[1], hv[2], hv[3]);
        }
}

// ---------------------------------------------------------------------------
// forward: 128 queries per workgroup (32 per wave), 64-key K and V tiles,
// double-buffered through LDS (the copy of tile j+1 is in flight while tile j
// is used).  On gfx950 a wave's MFMAs and VALU instructions largely serialise
// on its SIMD, so the kernel keeps the VALU count per tile low and lets the
// three waves that share a SIMD overlap each other's LDS latency.  Every wave
// needs tiles 0..last_w; only the last one crosses its diagonal and is masked.
// ---------------------------------------------------------------------------
template <int NP, bool kDrop, bool kKeep = false, bool kRope = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<NP>, kWavesPerEU<NP>))) void attn_fwd_d64_kernel(
    View Q, View K, View V, View O, float* __restrict__ LSE, int BH, int H, int T, int W,
    int n_qtiles, float scale, float scale_log2, int n_cu, Dropout dr, RopeArg<kRope> rp)
{
    // Separate arrays per buffer (not one indexed array): with the buffer of every
    // access known at compile time, the compiler can tell that an LDS read does not
    // touch the buffer an asynchronous copy is filling, and does not wait for it.
    __shared__ __attribute__((aligned(1024))) char sK0[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sK1[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sV0[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sV1[NP * kTileBytes];
    lds_poison(sK0, sK1, sV0, sV1);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, hi = lane >> 5;
    const int item = item_of(blockIdx.x, gridDim.x, n_cu);
    const int bh = item % BH;
    const int qt = n_qtiles - 1 - item / BH;  // heaviest tiles first
    const bf16* Kh = head_of(K, bh, H);
    const bf16* Vh = head_of(V, bh, H);
    const int q0w = qt * kRowsPerWG + wave * 32;  // wave-uniform
    const int qrow = q0w + li;
    const Offsets off(lane);
    const TileCopy tc(wave, lane);

    const int kv_end = min(T, qt * kRowsPerWG + kRowsPerWG);
    const int n_kv = (kv_end + kTile - 1) / kTile;
    const int last_w = min(n_kv - 1, (q0w + 31) / kTile);  // the wave's diagonal tile
    // window W (W >= T: the plain causal mask): query q sees keys q-W < k <= q
    const int lo = max(0, qt * kRowsPerWG - W + 1) / kTile;  // the workgroup's first tile
    const int first_w = max(0, q0w - W + 1) / kTile;        // the wave's first tile

    tiles_load_async<NP, kDrop || NP == 2>(sK0, Kh, K.st, lo * kTile, T, wave, tc);
    tiles_load_async<NP, kDrop || NP == 2>(sV0, Vh, V.st, lo * kTile, T, wave, tc);

    // rows past T read row T-1 (nothing of theirs is stored): unconditional loads
    // are all in flight at once, where loads under a divergent branch went out one
    // branch at a time
    bf16x8 qreg[4 * NP];
    const bf16* qr = head_of(Q, bh, H) + (size_t)min(qrow, T - 1) * Q.st + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 4 * NP; ++ks) qreg[ks] = *(const bf16x8*)(qr + 16 * ks);
    if constexpr (kRope) {  // the query rows after the prologue, also kept for the backward
        rope_rows<NP>(qreg, rp, rp.pos0 + qrow, hi);
        if (qrow < T) {
            bf16* yr = head_of(rp.yq, bh, H) + (size_t)qrow * rp.yq.st + 8 * hi;
#pragma unroll
            for (int ks = 0; ks < 4 * NP; ++ks) *(bf16x8*)(yr + 16 * ks) = qreg[ks];
        }
    }
    f32x16 oacc[2 * NP];
#pragma unroll
    for (int dt = 0; dt < 2 * NP; ++dt) oacc[dt] = f32x16{};
    // running max (raw dot-product units), shared by lanes l, l^32.  It starts
    // finite, so that a row none of whose keys is visible yet in a tile (a window's
    // lower edge) gives exp2(-inf) = 0 rather than inf - inf.
    float m = -1e30f;
    float l = 0.f;        // this lane's part of the normaliser

    // running max over the scores of a tile (two chains of v_max3); lazy rescale
    // of the accumulators
    auto update_max = [&](const f32x16& s0, const f32x16& s1) {
        float xa = fmaxf(s0[0], fmaxf(s0[1], s0[2]));
        float xb = fmaxf(s1[0], fmaxf(s1[1], s1[2]));
#pragma unroll
        for (int r = 3; r < 15; r += 2) {
            xa = fmaxf(xa, fmaxf(s0[r], s0[r + 1]));
            xb = fmaxf(xb, fmaxf(s1[r], s1[r + 1]));
        }
        const float mt = halves_max(fmaxf(fmaxf(xa, s0[15]), fmaxf(xb, s1[15])));
        const float m_new = fmaxf(m, mt);
        if (__builtin_expect(__any((m_new - m) * scale_log2 > kLazyRescale), 0)) {
            const float alpha = fast_exp2((m - m_new) * scale_log2);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < 2 * NP; ++dt) oacc[dt] *= alpha;
        }
    };

    // Tile j: S^T = K Q^T (all eight A operands read first), then all V^T
    // operands of the PV product are read while the softmax runs, so that none
    // of this wave's MFMAs waits on LDS; the other waves of the SIMD fill the
    // matrix core meanwhile.  On the wave's last tile (diag) the scores are masked.
    // One code path for both cases: two separately inlined variants of this body
    // made the register allocator spill.
    auto tile = [&](bool diag, int j, const char* kc, const char* vc) {
        // dropout keep bits of this tile for the lane's query: kw_lo for keys
        // 0..31, kw_hi for 32..63 (lane half hi draws keys 32hi .. 32hi+31).
        // Drawn before the S product: later, with S live, the draws spill.
        uint32_t kw_lo = 0, kw_hi = 0;
        if constexpr (kDrop) {
            uint32_t own = 0;
            if constexpr (kKeep && NP == 1) {
                // counters through opaque copies in the head-dim-64 kernel with
                // stored bits only: there the per-lane Philox terms the compiler
                // hoists out of the tile loop were spilled; elsewhere recomputing
                // them costs more than keeping them
                const int qo = opaque(qrow), bo = opaque(8 * j + 4 * hi);
#pragma unroll
                for (int m4 = 0; m4 < 4; ++m4) own |= drop_bits8(dr, bh, qo, bo + m4) << (8 * m4);
            } else {
#pragma unroll
                for (int m4 = 0; m4 < 4; ++m4) own |= drop_bits8(dr, bh, qrow, 8 * j + 4 * hi + m4) << (8 * m4);
            }
            const uint32_t oth = other_half_u32(own);
            kw_lo = hi ? oth : own;
            kw_hi = hi ? own : oth;
            // own: keys 64j + 32hi .. +31 of this lane's query (word 2j + hi); a
            // wave-uniform base and a 32-bit lane offset keep the address cheap
            if constexpr (kKeep) {
                uint32_t* const words = dr.keep + ((size_t)bh * ((T + 31) / 32) + 2 * j) * T;
                if (qrow < T && 64 * j + 32 * hi < T) words[(uint32_t)(hi * T + qrow)] = own;
            }
        }
        f32x16 s0, s1;
        tile_product<NP>(kc, off, qreg, s0, s1);
        bf16x8 tv[4][2 * NP];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int dt = 0; dt < 2; ++dt)
                    tv[c][2 * p + dt] = lds_tr_read(vc + p * kTileBytes, c * 2048 + off.tr[0][dt],
                                                    c * 2048 + off.tr[1][dt]);
        if (diag) {
            const int lim = qrow - j * kTile - 4 * hi;
            mask_band(s0, s1, lim, lim - W);
        }
        update_max(s0, s1);
        const float mc = m * scale_log2;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f32x16& sc = c < 2 ? s0 : s1;
            const int b = 8 * (c & 1);
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = (bf16)fast_exp2(fmaf(sc[b + e], scale_log2, -mc));
            l = sum8(pb, l);  // the normaliser is that of the undropped weights
            if constexpr (kDrop) {
                // element e of chunk c is key 32(c/2) + 16(c%2) + 4hi + e (+ 4 for e >= 4)
                const uint32_t w = (c >> 1) ? kw_hi : kw_lo;
                const int base = 16 * (c & 1) + 4 * hi;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (!((w >> (base + e + (e >> 2) * 4)) & 1u)) pb[e] = (bf16)0.0f;
            }
#pragma unroll
            for (int dt = 0; dt < 2 * NP; ++dt) oacc[dt] = mfma32x32x16(tv[c][dt], pb, oacc[dt]);
        }
    };

    // one step: after the barrier K(j), V(j) sit in kc, vc and every wave is done
    // with tile j-1 (in kl, vl), whose buffers are refilled with tile j+1.
    auto step = [&](int j, const char* kc, const char* vc, char* kl, char* vl) {
        wait_async_copies();
        __syncthreads();
        if (j + 1 < n_kv) {
            tiles_load_async<NP, kDrop || NP == 2>(kl, Kh, K.st, (j + 1) * kTile, T, wave, tc);
            tiles_load_async<NP, kDrop || NP == 2>(vl, Vh, V.st, (j + 1) * kTile, T, wave, tc);
        }
        // a tile needs the mask if it crosses the diagonal or the window's lower edge
        if (j >= first_w && j <= last_w)
            tile(j == last_w || j * kTile <= q0w + 31 - W, j, kc, vc);
    };

    for (int j = lo; j < n_kv; j += 2) {
        step(j, sK0, sV0, sK1, sV1);
        if (j + 1 < n_kv) step(j + 1, sK1, sV1, sK0, sV0);
    }

    l = halves_sum(l);
    if (qrow < T) {
        const float inv = (kDrop ? dr.keep_scale : 1.0f) / l;
        bf16* orow = head_of(O, bh, H) + (size_t)qrow * O.st;
#pragma unroll
        for (int dt = 0; dt < 2 * NP; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store_bf16x4(orow + 32 * dt + 8 * g + 4 * hi, oacc[dt][4 * g] * inv,
                             oacc[dt][4 * g + 1] * inv, oacc[dt][4 * g + 2] * inv,
                             oacc[dt][4 * g + 3] * inv);
        if (hi == 0) LSE[(size_t)bh * T + qrow] = m * scale + logf(l);
    }
}

// Arguments of the backward work items.
struct BwdParams {
    View Q, K, V, O, dO;
    const float* LSE;
    float* Delta;  // dQ items write it; dK/dV items read it unless they form it from O
    View dQ, dK, dV;
    int BH, H, T;
    int W;  // window: query q sees keys q-W < k <= q (W >= T: the plain causal mask)
    float scale, scale_log2;
    Dropout dr;
};

// ---------------------------------------------------------------------------
// dQ (and Delta) of one 128-query block: 64-key K/V tiles, double-buffered
// (the copy of tile j+1 is in flight while tile j is used).  Per tile: S^T and
// dP^T from row reads of K and V, dS^T = P^T (dP^T - Delta), then
// dQ^T += K^T dS^T with K^T from transposing reads.  Only the wave's last tile
// crosses its diagonal and is masked.
// Delta_i = sum_d dO_id O_id is formed from the rows the wave holds as MFMA
// operands and written out.
// ---------------------------------------------------------------------------
// kDeltaIn: Delta is read from memory (written by an earlier launch) instead of
// formed here from the item's O and dO rows and stored.
template <int NP, bool kDrop, bool kKeep = false, bool kRope = false, bool kDeltaIn = false>
__device__ __forceinline__ void dq_item(const BwdParams& a, int bh, int qt, char* sK0, char* sK1,
                                        char* sV0, char* sV1, float (*sW0)[kTile], float (*sW1)[kTile],
                                        const RopeArg<kRope>& rp = RopeArg<kRope>{})
{
    const int BH = a.BH, T = a.T;
    const float scale = a.scale, scale_log2 = a.scale_log2;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, hi = lane >> 5;
    (void)BH;
    const bf16* Kh = head_of(a.K, bh, a.H);
    const bf16* Vh = head_of(a.V, bh, a.H);
    const int q0w = qt * kRowsPerWG + wave * 32;
    const int qrow = q0w + li;
    const bool valid = qrow < T;
    const Offsets off(lane);
    const TileCopy tc(wave, lane);

    const int kv_end = min(T, qt * kRowsPerWG + kRowsPerWG);
    const int n_kv = (kv_end + kTile - 1) / kTile;
    const int last_w = min(n_kv - 1, (q0w + 31) / kTile);
    const int W = a.W;
    const int lo = max(0, qt * kRowsPerWG - W + 1) / kTile;  // the workgroup's first tile
    const int first_w = max(0, q0w - W + 1) / kTile;        // the wave's first tile

    // Stored keep bits travel with the tiles: for 64-key tile j each wave copies
    // the words of its 32 queries for key columns 2j (lanes 0-31) and 2j + 1
    // (lanes 32-63) into row `wave` of a keep buffer (sW0 / sW1), 4 bytes per
    // lane; a word read from memory right before its use would wait for every
    // copy in flight.  Rows past T and columns past the last read the last ones.
    auto keep_load_async = [&](int j, float (*wb)[kTile]) {
        if constexpr (kKeep) {
            const int wcol = min(2 * j + hi, (T + 31) / 32 - 1);
            __builtin_amdgcn_global_load_lds(
                (const void*)(a.dr.keep + keep_index(bh, wcol, min(q0w + li, T - 1), T)),
                (__attribute__((address_space(3))) void*)wb[wave], 4, 0, 0);
        }
    };
    tiles_load_async<NP, kDrop || NP == 2>(sK0, Kh, a.K.st, lo * kTile, T, wave, tc);
    tiles_load_async<NP, kDrop || NP == 2>(sV0, Vh, a.V.st, lo * kTile, T, wave, tc);
    keep_load_async(lo, sW0);

    bf16x8 qreg[4 * NP], greg[4 * NP];
    float dsum = 0.f;
    // rows past T read row T-1: their P is 0 (lse = -inf below) and nothing of
    // theirs is stored, and unconditional loads are all in flight at once
    const int qld = min(qrow, T - 1);
    const bf16* qr = head_of(a.Q, bh, a.H) + (size_t)qld * a.Q.st + 8 * hi;
    const bf16* gr = head_of(a.dO, bh, a.H) + (size_t)qld * a.dO.st + 8 * hi;
    const bf16* orr = head_of(a.O, bh, a.H) + (size_t)qld * a.O.st + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 4 * NP; ++ks) {
        qreg[ks] = *(const bf16x8*)(qr + 16 * ks);
        greg[ks] = *(const bf16x8*)(gr + 16 * ks);
        if constexpr (!kDeltaIn) {
            const bf16x8 orow = *(const bf16x8*)(orr + 16 * ks);
#pragma unroll
            for (int e = 0; e < 8; ++e) dsum = fmaf((float)greg[ks][e], (float)orow[e], dsum);
        }
    }
    float dlt;
    if constexpr (kDeltaIn) {
        dlt = valid ? a.Delta[(size_t)bh * T + qrow] : 0.f;
    } else {
        dlt = halves_sum(dsum);  // this lane's 32 columns + the other half's 32
        if (valid && hi == 0) a.Delta[(size_t)bh * T + qrow] = dlt;
    }
    // rows >= T: -lse = -inf makes P (and dS) exactly 0
    const float nlse2 = valid ? -a.LSE[(size_t)bh * T + qrow] * kLog2e : -INFINITY;
    // dP^T accumulators start from this block (-Delta of the lane's query in every
    // register), so that the MFMAs yield dP - Delta without a subtraction per element
    f32x16 ndl;
#pragma unroll
    for (int r = 0; r < 16; ++r) ndl[r] = -dlt;
    f32x16 dqacc[2 * NP];
#pragma unroll
    for (int dt = 0; dt < 2 * NP; ++dt) dqacc[dt] = f32x16{};

    // keys 32h .. 32h+31 of tile j: S^T, dP^T - Delta, dS^T, dQ^T += K^T dS^T
    auto half = [&](int h, bool diag, int k0, const char* kc, const char* vc,
                    const float (*wc)[kTile]) {
        // dP^T - Delta (without dropout), or dP^T alone, to be masked first
        f32x16 sv = f32x16{}, pv = kDrop ? f32x16{} : ndl;
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int o = p * kTileBytes + 4096 * h + off.nat[ks];
                sv = mfma32x32x16(lds_row_read(kc, o), qreg[4 * p + ks], sv);  // S^T
                pv = mfma32x32x16(lds_row_read(vc, o), greg[4 * p + ks], pv);  // dP^T - Delta
            }
        if (diag) {  // key row 32h + 8(r/4) + 4hi + r%4 is visible to query qrow iff
                     // qrow - W < key <= qrow
            const int lim = qrow - k0 - 4 * hi - 32 * h;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = 8 * (r >> 2) + (r & 3);
                sv[r] = kk <= lim && kk > lim - W ? sv[r] : -INFINITY;
            }
        }
        if constexpr (kDrop) {
            // dS = P (keep * keep_scale * dP - Delta).  Lane half hi draws keys
            // 16hi .. 16hi+15 of the half; w has bit b for key 32h + b.
            uint32_t w;
            if constexpr (kKeep) {  // stored by the forward, staged with the tile
                w = valid ? ((const uint32_t*)wc[wave])[32 * h + li] : 0u;
            } else {
                const int blk0 = (k0 + 32 * h) / 8 + 2 * hi;
                const uint32_t own = drop_bits8(a.dr, bh, qrow, blk0) |
                                     (drop_bits8(a.dr, bh, qrow, blk0 + 1) << 8);
                const uint32_t oth = other_half_u32(own);
                w = hi ? (oth | (own << 16)) : (own | (oth << 16));
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = fast_exp2(fmaf(sv[r], scale_log2, nlse2));
                const bool kept = (w >> (8 * (r >> 2) + 4 * hi + (r & 3))) & 1u;
                sv[r] = pr * (kept ? fmaf(pv[r], a.dr.keep_scale, -dlt) : -dlt);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) sv[r] = fast_exp2(fmaf(sv[r], scale_log2, nlse2)) * pv[r];  // dS^T
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int c = 2 * h + cc;
            const bf16x8 db = pack8(sv, 8 * cc);
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int dt = 0; dt < 2; ++dt) {
                    const int o = p * kTileBytes + c * 2048;
                    const bf16x8 av = lds_tr_read(kc, o + off.tr[0][dt], o + off.tr[1][dt]);
                    dqacc[2 * p + dt] = mfma32x32x16(av, db, dqacc[2 * p + dt]);
                }
        }
    };

    // after the barrier K(j), V(j) (and its keep words) sit in kc, vc (wc); every
    // wave is done with tile j-1 (in kl, vl, wl), whose buffers are refilled with
    // tile j+1.
    auto step = [&](int j, const char* kc, const char* vc, const float (*wc)[kTile], char* kl,
                    char* vl, float (*wl)[kTile]) {
        wait_async_copies();
        __syncthreads();
        if (j + 1 < n_kv) {
            tiles_load_async<NP, kDrop || NP == 2>(kl, Kh, a.K.st, (j + 1) * kTile, T, wave, tc);
            tiles_load_async<NP, kDrop || NP == 2>(vl, Vh, a.V.st, (j + 1) * kTile, T, wave, tc);
            keep_load_async(j + 1, wl);
        }
        if (j < first_w || j > last_w) return;
        const int k0 = j * kTile;
        // masked: the diagonal tile and tiles crossing the window's lower edge
        const bool diag = j == last_w || k0 <= q0w + 31 - W;
        half(0, diag, k0, kc, vc, wc);
        // keys 32..63 of the diagonal tile matter only if a query of the wave reaches them
        if (j < last_w || k0 + 32 <= q0w + 31) half(1, diag, k0, kc, vc, wc);
    };

    for (int j = lo; j < n_kv; j += 2) {
        step(j, sK0, sV0, sW0, sK1, sV1, sW1);
        if (j + 1 < n_kv) step(j + 1, sK1, sV1, sW1, sK0, sV0, sW0);
    }

    if constexpr (kRope) {  // through the prologue's transposed Jacobian (every lane takes part)
        const bf16* xr = head_of(rp.xq, bh, a.H) + (size_t)(valid ? qrow : 0) * rp.xq.st;
        rope_grad_store<NP>(dqacc, scale, xr, valid,
                            head_of(a.dQ, bh, a.H) + (size_t)qrow * a.dQ.st, rp, rp.q_gain,
                            rp.pos0 + qrow, hi);
    } else if (valid) {
        bf16* row = head_of(a.dQ, bh, a.H) + (size_t)qrow * a.dQ.st;
#pragma unroll
        for (int dt = 0; dt < 2 * NP; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store_bf16x4(row + 32 * dt + 8 * g + 4 * hi, dqacc[dt][4 * g] * scale,
                             dqacc[dt][4 * g + 1] * scale, dqacc[dt][4 * g + 2] * scale,
                             dqacc[dt][4 * g + 3] * scale);
    }
}

// ---------------------------------------------------------------------------
// dK, dV of one 128-key block (32 keys per wave): 64-query Q/dO tiles from T
// down to the diagonal, double-buffered.  Each tile is taken in two halves of 32
// queries so that only one S block and one dP block are live at a time (the
// kernel fits 3 waves per SIMD).  Per half: S and dP from row reads of Q and
// dO (one key column per lane), with the dP accumulator starting from -Delta
// of its row, so that it comes out as dP - Delta; P from lse; dS = P (dP -
// Delta); then dV^T += dO^T P and dK^T += Q^T dS with transposing reads.
// Only the last tile a wave visits crosses its diagonal and is masked; rows >= T
// carry -lse = -inf (P = 0) and Delta = 0.
// kDeltaFromO: Delta of each tile is formed here from the O tile, which is
// copied along with Q and dO: each wave, once its own copies of the next tile
// have landed, sums dO * O over the 16 rows it copied (4 lanes per row) and
// leaves -Delta in the row buffer, which the next step's barrier publishes.
// Otherwise Delta is read from memory (written by a dQ pass).
// ---------------------------------------------------------------------------
template <int NP, bool kDeltaFromO, bool kDrop, bool kKeep = false, bool kRope = false>
__device__ __forceinline__ void dkdv_item(const BwdParams& a, int bh, int kb, char* sQ0, char* sQ1,
                                          char* sG0, char* sG1, char* sO0, char* sO1,
                                          float (*sR0)[kTile], float (*sR1)[kTile],
                                          const RopeArg<kRope>& rp = RopeArg<kRope>{})
{
    static_assert(!(kRope && kDrop), "the fused prologue has no dropout variant");
    const int T = a.T;
    const float scale = a.scale, scale_log2 = a.scale_log2;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, hi = lane >> 5;
    const bf16* Qh = head_of(a.Q, bh, a.H);
    const bf16* Gh = head_of(a.dO, bh, a.H);
    const bf16* Oh = head_of(a.O, bh, a.H);
    const float* Lh = a.LSE + (size_t)bh * T;
    const float* Dh = kDeltaFromO ? nullptr : a.Delta + (size_t)bh * T;
    const int kv0 = kb * kRowsPerWG;
    const int k0w = kv0 + wave * 32;
    const int key = k0w + li;
    const bool valid = key < T;
    const Offsets off(lane);
    const TileCopy tc(wave, lane);

    const int n_q = (T + kTile - 1) / kTile;
    const int i0 = kv0 / kTile;
    const int first_w = k0w / kTile;  // first tile with a query >= a key of this wave
    // window: key k is seen by queries k <= q < k + W (W >= T: every later query)
    const int W = a.W;
    const int i_hi = min(n_q - 1, (kv0 + kRowsPerWG - 1 + W - 1) / kTile);  // the workgroup's last tile
    const int last_w = min(n_q - 1, (k0w + 31 + W - 1) / kTile);            // the wave's last tile

    // Per-row values of tile i (lse, and Delta when it is read from memory) travel
    // to LDS by the same asynchronous copy as the tiles, 4 bytes per lane of one
    // wave (rows >= T read row T-1).  Once a wave's own copies of a tile have
    // landed it turns them into the forms used below, in place: -lse*log2e (-inf
    // past T) and -Delta (0 past T); with kDeltaFromO every wave forms -Delta of
    // the 16 rows it copied from dO and O (4 lanes per row).  The next barrier
    // publishes them.
    // With stored keep bits, each wave also copies the words of its 32 keys for
    // the tile's 64 queries into row 2 + wave (a word read from memory right
    // before its use would wait for every copy in flight).
    auto rows_load_async = [&](int i, float (*rt)[kTile]) {
        const uint32_t o = (uint32_t)min(i * kTile + lane, T - 1) * 4u;
        if (wave == 0)
            __builtin_amdgcn_global_load_lds((const void*)((const char*)Lh + o),
                                             (__attribute__((address_space(3))) void*)rt[0], 4, 0, 0);
        if (!kDeltaFromO && wave == 1)
            __builtin_amdgcn_global_load_lds((const void*)((const char*)Dh + o),
                                             (__attribute__((address_space(3))) void*)rt[1], 4, 0, 0);
        if constexpr (kKeep) {
            // keys past T (a wave of the last block) read the last word column
            const int wcol = min(k0w / 32, (T + 31) / 32 - 1);
            __builtin_amdgcn_global_load_lds(
                (const void*)((const char*)(a.dr.keep + keep_index(bh, wcol, 0, T)) + o),
                (__attribute__((address_space(3))) void*)rt[2 + wave], 4, 0, 0);
        }
    };
    auto rows_finish = [&](int i, const char* gt, const char* ot, float (*rt)[kTile]) {
        // The lane-dependent addresses are recomputed here from an opaque copy of the
        // lane index rather than kept live across the loop (registers are the limit).
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const bool in = i * kTile + ln < T;
        if (wave == 0) rt[0][ln] = in ? -rt[0][ln] * kLog2e : -INFINITY;
        if (!kDeltaFromO && wave == 1) rt[1][ln] = in ? -rt[1][ln] : 0.f;
        if (kDeltaFromO) {
            const int row = wave * 16 + (ln >> 2), c0 = 2 * (ln & 3);
            float d = 0.f;
#pragma unroll
            for (int c = 0; c < 2 * NP; ++c) {
                const int o = (c >> 1) * kTileBytes + chunk_off(row, c0 + (c & 1));
                const bf16x8 gv = lds_row_read(gt, o), ov = lds_row_read(ot, o);
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
                for (int e = 0; e < 8; e += 2)
                    d = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{gv[e], gv[e + 1]},
                                                        bf16x2{ov[e], ov[e + 1]}, d, false);
            }
            // sum over the 4 lanes of the row (DPP quad permutations 1,0,3,2 and 2,3,0,1)
            d += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(d), 0xB1, 0xF, 0xF, false));
            d += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(d), 0x4E, 0xF, 0xF, false));
            if ((ln & 3) == 0) rt[1][row] = i * kTile + row < T ? -d : 0.f;
        }
    };

    // Tiles are visited from the last one down to the diagonal, so that every item
    // of a head streams the same tile at about the same time (they share it in L2).
    tiles_load_async<NP, kDrop || NP == 2>(sQ0, Qh, a.Q.st, i_hi * kTile, T, wave, tc);
    tiles_load_async<NP, kDrop || NP == 2>(sG0, Gh, a.dO.st, i_hi * kTile, T, wave, tc);
    if (kDeltaFromO) tiles_load_async<NP, kDrop || NP == 2>(sO0, Oh, a.O.st, i_hi * kTile, T, wave, tc);
    rows_load_async(i_hi, sR0);

    bf16x8 kreg[4 * NP], vreg[4 * NP];
    // keys past T read key T-1: they are masked on every query and their dK, dV
    // rows are not stored
    const int kld = min(key, T - 1);
    const bf16* kr = head_of(a.K, bh, a.H) + (size_t)kld * a.K.st + 8 * hi;
    const bf16* vr = head_of(a.V, bh, a.H) + (size_t)kld * a.V.st + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 4 * NP; ++ks) {
        kreg[ks] = *(const bf16x8*)(kr + 16 * ks);
        vreg[ks] = *(const bf16x8*)(vr + 16 * ks);
    }
    wait_async_copies();
    rows_finish(i_hi, sG0, sO0, sR0);
    f32x16 dkacc[2 * NP] = {}, dvacc[2 * NP] = {};

    // Drawn dropout bits: the keep bits of a half are drawn at the end of the half
    // before it (and those of the first half before the loop), when its S and dP
    // accumulators are dead: drawn later, with them live, the draws spilled.
    // Halves run in this order: tiles from min(i_hi, last_w) down to first_w,
    // in each tile half 0 (if some query of it reaches a key of the wave) and
    // then half 1.  This lane draws for query 32h + li of the half and the
    // keys 16hi .. 16hi+15 of the wave's 32 (bit t = key k0w + 16hi + t).
    auto runs_half0 = [&](int i) { return i > first_w || i * kTile + 31 >= k0w; };
    auto draw_half = [&](int i, int h) -> uint32_t {
        const int blk0 = k0w / 8 + 2 * hi, qd = i * kTile + 32 * h + li;
        if constexpr (NP == 2) {
            // head dim 128: the key block through an opaque copy.  Hoisted out of
            // the tile loop, the Philox terms of this lane's fixed block make the
            // compiler spill resident rows, reloaded (waiting for the copies in
            // flight) every half; at head dim 64 recomputing them costs more.
            const int bo = opaque(blk0);
            return drop_bits8<false>(a.dr, bh, qd, bo) | (drop_bits8<false>(a.dr, bh, qd, bo + 1) << 8);
        } else {
            return drop_bits8<false>(a.dr, bh, qd, blk0) | (drop_bits8<false>(a.dr, bh, qd, blk0 + 1) << 8);
        }
    };
    // Stored bits: this lane half's 16 keys of the word of query 32h + li of the
    // tile whose row buffer is rt (staged there by rows_load_async)
    // (lane-dependent addresses from an opaque copy of the lane index, recomputed
    // here rather than kept live across the loop, as in rows_finish)
    auto staged_half = [&](int i, int h, const float (*rt)[kTile]) -> uint32_t {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int l32 = ln & 31;
        const uint32_t w = ((const uint32_t*)rt[2 + wave])[32 * h + l32];
        return i * kTile + 32 * h + l32 < T ? (w >> (16 * (ln >> 5))) & 0xFFFFu : 0u;
    };
    uint32_t dbits = 0;  // keep bits of the half about to run
    if constexpr (kKeep) {  // the first tile's words are staged only by the step before it
        if (i_hi >= first_w && i_hi <= last_w) dbits = staged_half(i_hi, runs_half0(i_hi) ? 0 : 1, sR0);
    } else if constexpr (kDrop) {
        const int i_first = min(i_hi, last_w);
        if (i_first >= first_w) dbits = draw_half(i_first, runs_half0(i_first) ? 0 : 1);
    }

    // queries 32h .. 32h+31 of the tile in qc / gc / rc
    auto half = [&](int h, bool diag, int q0, const char* qc, const char* gc,
                    const float (*rc)[kTile]) {
        f32x16 sv = f32x16{}, dp;
        if constexpr (kDrop) {
            dp = f32x16{};  // dP alone: the keep mask applies before Delta is taken off
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {  // dP starts from -Delta of its row
                const f32x4 nd = *(const f32x4*)(rc[1] + 32 * h + 8 * g + 4 * hi);
#pragma unroll
                for (int e = 0; e < 4; ++e) dp[4 * g + e] = nd[e];
            }
        }
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int o = p * kTileBytes + 4096 * h + off.nat[ks];
                sv = mfma32x32x16(lds_row_read(qc, o), kreg[4 * p + ks], sv);   // S
                dp = mfma32x32x16(lds_row_read(gc, o), vreg[4 * p + ks], dp);   // dP - Delta
            }
        if (diag) {
            // element r holds query q0 + 32h + 8(r/4) + 4hi + r%4: kept iff
            // key <= query < key + W, i.e. lim <= 8(r/4) + r%4 < lim + W
            const int lim = key - q0 - 32 * h - 4 * hi;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qq = 8 * (r >> 2) + (r & 3);
                sv[r] = qq >= lim && qq < lim + W ? sv[r] : -INFINITY;
            }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 nl = *(const f32x4*)(rc[0] + 32 * h + 8 * g + 4 * hi);
            if constexpr (kDrop) {
                // register r is query 8g + 4hi + e of the half for this lane's key
                // li: bit li % 16 of the word drawn by lane (8g + 4hi + e) + 32 (li / 16)
                const f32x4 nd = *(const f32x4*)(rc[1] + 32 * h + 8 * g + 4 * hi);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    const float pr = fast_exp2(fmaf(sv[r], scale_log2, nl[e]));
                    const uint32_t wsrc = (uint32_t)__shfl((int)dbits, 8 * g + 4 * hi + e + 32 * (li >> 4), 64);
                    const bool kept = (wsrc >> (li & 15)) & 1u;
                    sv[r] = kept ? pr : 0.f;  // dropped weight (times keep_scale at the end)
                    dp[r] = pr * (kept ? fmaf(dp[r], a.dr.keep_scale, nd[e]) : nd[e]);  // dS
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    const float pr = fast_exp2(fmaf(sv[r], scale_log2, nl[e]));
                    sv[r] = pr;
                    dp[r] *= pr;  // dS
                }
            }
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int c = 2 * h + cc;  // 16-query chunk of the tile
            const bf16x8 pb = pack8(sv, 8 * cc);
            const bf16x8 sb = pack8(dp, 8 * cc);
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int dt = 0; dt < 2; ++dt) {
                    const int o0 = p * kTileBytes + c * 2048 + off.tr[0][dt];
                    const int o1 = p * kTileBytes + c * 2048 + off.tr[1][dt];
                    dvacc[2 * p + dt] = mfma32x32x16(lds_tr_read(gc, o0, o1), pb, dvacc[2 * p + dt]);
                    dkacc[2 * p + dt] = mfma32x32x16(lds_tr_read(qc, o0, o1), sb, dkacc[2 * p + dt]);
                }
        }
        if constexpr (kKeep) {  // the second half's words are in this tile's buffer
            if (h == 0) dbits = staged_half(q0 / kTile, 1, rc);
        } else if constexpr (kDrop) {  // the bits of the next half to run (if any)
            const int i = q0 / kTile;
            if (h == 0)
                dbits = draw_half(i, 1);
            else if (i - 1 >= first_w)
                dbits = draw_half(i - 1, runs_half0(i - 1) ? 0 : 1);
        }
    };

    // after the barrier tile i sits in qc, gc, (oc,) rc; every wave is done with tile
    // i+1 (in ql, gl, ol, rl), whose buffers are refilled with tile i-1.
    auto step = [&](int i, const char* qc, const char* gc, const float (*rc)[kTile], char* ql,
                    char* gl, char* ol, float (*rl)[kTile]) {
        wait_async_copies();
        __syncthreads();
        const bool more = i > i0;
        if (more) {
            tiles_load_async<NP, kDrop || NP == 2>(ql, Qh, a.Q.st, (i - 1) * kTile, T, wave, tc);
            tiles_load_async<NP, kDrop || NP == 2>(gl, Gh, a.dO.st, (i - 1) * kTile, T, wave, tc);
            if (kDeltaFromO) tiles_load_async<NP, kDrop || NP == 2>(ol, Oh, a.O.st, (i - 1) * kTile, T, wave, tc);
            rows_load_async(i - 1, rl);
        }
        if (i >= first_w && i <= last_w) {
            const int q0 = i * kTile;
            // masked: the diagonal tile and tiles reaching past the window of a key
            const bool diag = i == first_w || q0 + kTile - 1 >= k0w + W;
            // on the diagonal tile, queries 0..31 matter only if one of them is >= a key
            if (runs_half0(i)) half(0, diag, q0, qc, gc, rc);
            half(1, diag, q0, qc, gc, rc);
        }
        if (more) {
            wait_async_copies();
            rows_finish(i - 1, gl, ol, rl);
            if constexpr (kKeep)  // tile i-1's words have landed: its first half's bits
                if (i - 1 >= first_w && i - 1 <= last_w)
                    dbits = staged_half(i - 1, runs_half0(i - 1) ? 0 : 1, rl);
        }
    };

    for (int i = i_hi; i >= i0; i -= 2) {
        step(i, sQ0, sG0, sR0, sQ1, sG1, sO1, sR1);
        if (i - 1 >= i0) step(i - 1, sQ1, sG1, sR1, sQ0, sG0, sO0, sR0);
    }

    if constexpr (kRope) {
        // dV first (its accumulators are then free), then dK through the prologue's
        // transposed Jacobian (every lane takes part)
        if (valid) {
            bf16* vrow = head_of(a.dV, bh, a.H) + (size_t)key * a.dV.st;
#pragma unroll
            for (int dt = 0; dt < 2 * NP; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    store_bf16x4(vrow + 32 * dt + 8 * g + 4 * hi, dvacc[dt][4 * g],
                                 dvacc[dt][4 * g + 1], dvacc[dt][4 * g + 2], dvacc[dt][4 * g + 3]);
        }
        const bf16* xr = head_of(rp.xk, bh, a.H) + (size_t)(valid ? key : 0) * rp.xk.st;
        rope_grad_store<NP>(dkacc, scale, xr, valid,
                            head_of(a.dK, bh, a.H) + (size_t)key * a.dK.st, rp, rp.k_gain,
                            rp.pos0 + key, hi);
        return;
    }
    // with dropout the lane's key and half are recomputed here from an opaque copy
    // of the lane index (kept live across the loop, they were spilled)
    int key_e = key, hi_e = hi;
    if constexpr (kDrop) {
        const int le = opaque(lane);
        key_e = k0w + (le & 31);
        hi_e = le >> 5;
    }
    if (kDrop ? key_e < T : valid) {
        bf16* krow = head_of(a.dK, bh, a.H) + (size_t)key_e * a.dK.st;
        bf16* vrow = head_of(a.dV, bh, a.H) + (size_t)key_e * a.dV.st;
#pragma unroll
        for (int dt = 0; dt < 2 * NP; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hi_e;
                store_bf16x4(krow + d, dkacc[dt][4 * g] * scale, dkacc[dt][4 * g + 1] * scale,
                             dkacc[dt][4 * g + 2] * scale, dkacc[dt][4 * g + 3] * scale);
                const float vs = kDrop ? a.dr.keep_scale : 1.0f;
                store_bf16x4(vrow + d, dvacc[dt][4 * g] * vs, dvacc[dt][4 * g + 1] * vs,
                             dvacc[dt][4 * g + 2] * vs, dvacc[dt][4 * g + 3] * vs);
            }
    }
}

// dQ alone (also writes Delta).
template <int NP, bool kDrop, bool kKeep = false, bool kRope = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<NP>, kWavesPerEU<NP>))) void attn_bwd_dq_d64_kernel(
    BwdParams a, int n_qtiles, int n_cu, RopeArg<kRope> rp)
{
    // one array per buffer, so that reads are provably apart from in-flight copies
    __shared__ __attribute__((aligned(1024))) char sK0[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sK1[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sV0[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sV1[NP * kTileBytes];
    __shared__ __attribute__((aligned(16))) float sW0[kKeep ? 4 : 1][kTile];  // keep words per wave
    __shared__ __attribute__((aligned(16))) float sW1[kKeep ? 4 : 1][kTile];
    lds_poison(sK0, sK1, sV0, sV1, sW0, sW1);
    const int item = item_of(blockIdx.x, gridDim.x, n_cu);
    dq_item<NP, kDrop, kKeep, kRope>(a, item % a.BH, n_qtiles - 1 - item / a.BH, sK0, sK1, sV0, sV1,
                                     sW0, sW1, rp);
}

// dK, dV alone, from a Delta in memory.
template <int NP, bool kDrop, bool kKeep = false, bool kRope = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<NP>, kWavesPerEU<NP>))) void attn_bwd_dkdv_d64_kernel(
    BwdParams a, int n_cu, RopeArg<kRope> rp)
{
    __shared__ __attribute__((aligned(1024))) char sQ0[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sQ1[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sG0[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sG1[NP * kTileBytes];
    // [-lse*log2e, -Delta] per row, then (stored keep bits) each wave's keep words
    __shared__ __attribute__((aligned(16))) float sR0[kKeep ? 6 : 2][kTile];
    __shared__ __attribute__((aligned(16))) float sR1[kKeep ? 6 : 2][kTile];
    lds_poison(sQ0, sQ1, sG0, sG1, sR0, sR1);
    const int item = item_of(blockIdx.x, gridDim.x, n_cu);
    dkdv_item<NP, false, kDrop, kKeep, kRope>(a, item % a.BH, item / a.BH, sQ0, sQ1, sG0, sG1,
                                              nullptr, nullptr, sR0, sR1, rp);
}

// ---------------------------------------------------------------------------
// The whole backward in one launch: dK/dV items (forming Delta from O) and dQ
// items (writing Delta) are independent, so one grid holds both and each
// item's start (loading its resident rows from HBM) overlaps the others'
// compute instead of every item of a kernel loading at once.  Items run in
// order of decreasing tile count, a dK/dV item before a dQ item of the same
// count (a dK/dV tile costs more): level v holds the dK/dV items of key block v
// and the dQ items of query block n - 1 - v, BH of each.
// ---------------------------------------------------------------------------
template <bool kDrop, bool kKeep = false, bool kRope = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void attn_bwd_d64_kernel(
    BwdParams a, int n_blocks, int n_cu, RopeArg<kRope> rp)
{
    __shared__ __attribute__((aligned(1024))) char s0[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char s1[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char s2[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char s3[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char s4[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char s5[kTileBytes];
    // row values, then (stored keep bits) each wave's keep words: rows 2..5 serve
    // the dK/dV items and, as the keep buffers, the dQ items
    __shared__ __attribute__((aligned(16))) float sR0[kKeep ? 6 : 2][kTile];
    __shared__ __attribute__((aligned(16))) float sR1[kKeep ? 6 : 2][kTile];
    lds_poison(s0, s1, s2, s3, s4, s5, sR0, sR1);
    const int item = item_of(blockIdx.x, gridDim.x, n_cu);
    const int BH = a.BH;
    const int level = item / (2 * BH), r = item - level * 2 * BH;
    if (r < BH)
        dkdv_item<1, true, kDrop, kKeep, kRope>(a, r, level, s0, s1, s2, s3, s4, s5, sR0, sR1, rp);
    else
        dq_item<1, kDrop, kKeep, kRope>(a, r - BH, n_blocks - 1 - level, s0, s1, s2, s3, sR0 + 2,
                                        sR1 + 2, rp);
}

// ---------------------------------------------------------------------------
// Delta = rowsum(dO o O) of every row, as a dQ item forms it (same lanes, same
// order of the sums): 128 rows per workgroup, 32 per wave.  HBM-bound: reads
// 2 D bf16 per row, writes 4 bytes.
// ---------------------------------------------------------------------------
template <int NP>
__global__ __launch_bounds__(kThreads) void attn_delta_d64_kernel(BwdParams a, int n_blocks)
{
    const int T = a.T;
    const int bh = blockIdx.x / n_blocks, blk = blockIdx.x - bh * n_blocks;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 31, hi = lane >> 5;
    const int qrow = blk * kRowsPerWG + wave * 32 + li;
    const bool valid = qrow < T;
    const bf16* gr = head_of(a.dO, bh, a.H) + (size_t)(valid ? qrow : 0) * a.dO.st + 8 * hi;
    const bf16* orr = head_of(a.O, bh, a.H) + (size_t)(valid ? qrow : 0) * a.O.st + 8 * hi;
    bf16x8 g[4 * NP], o[4 * NP];
#pragma unroll
    for (int ks = 0; ks < 4 * NP; ++ks) {
        g[ks] = *(const bf16x8*)(gr + 16 * ks);
        o[ks] = *(const bf16x8*)(orr + 16 * ks);
    }
    float dsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4 * NP; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) dsum = fmaf((float)g[ks][e], (float)o[ks][e], dsum);
    const float dlt = halves_sum(dsum);
    if (valid && hi == 0) a.Delta[(size_t)bh * T + qrow] = dlt;
}

// ---------------------------------------------------------------------------
// Backward in one launch after the Delta pass (used at head dim 128): dK/dV
// items and dQ items as in the head-dim-64 kernel, both reading Delta from
// memory, so a dK/dV item needs no O tiles and the two kinds share 4 tile
// buffers (65 KB of LDS at NP = 2: two workgroups per CU, 2 waves per SIMD).
// Same item order: level v holds the dK/dV items of key block v and the dQ
// items of query block n - 1 - v.  Against a dQ launch followed by a dK/dV
// launch (384 workgroups each at B8 H6 T1024, for 512 slots, each launch
// waiting on its heaviest items) the step at that shape drops from 117 to
// 95 us.  At head dim 64 the kernel that forms Delta in its dK/dV items is as
// fast or faster (88 against 91 us), so it stays.
// ---------------------------------------------------------------------------
template <int NP, bool kDrop, bool kKeep = false, bool kRope = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<NP>, kWavesPerEU<NP>))) void attn_bwd_dpre_kernel(
    BwdParams a, int n_blocks, int n_cu, RopeArg<kRope> rp)
{
    __shared__ __attribute__((aligned(1024))) char s0[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char s1[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char s2[NP * kTileBytes];
    __shared__ __attribute__((aligned(1024))) char s3[NP * kTileBytes];
    __shared__ __attribute__((aligned(16))) float sR0[kKeep ? 6 : 2][kTile];
    __shared__ __attribute__((aligned(16))) float sR1[kKeep ? 6 : 2][kTile];
    lds_poison(s0, s1, s2, s3, sR0, sR1);
    const int item = item_of(blockIdx.x, gridDim.x, n_cu);
    const int BH = a.BH;
    const int level = item / (2 * BH), r = item - level * 2 * BH;
    if (r < BH)
        dkdv_item<NP, false, kDrop, kKeep, kRope>(a, r, level, s0, s1, s2, s3, nullptr, nullptr, sR0,
                                                  sR1, rp);
    else
        dq_item<NP, kDrop, kKeep, kRope, true>(a, r - BH, n_blocks - 1 - level, s0, s1, s2, s3,
                                               sR0 + 2, sR1 + 2, rp);
}

#ifndef CATTN_D64_KERNELS_ONLY
// The one-launch backward without dropout is instantiated in attn_bwd_plain.hip,
// which is compiled with its own instruction-scheduling strategy.
extern template __global__ void attn_bwd_d64_kernel<false, false, false>(BwdParams, int, int, NoRope);
#endif

}  // namespace d64

#ifndef CATTN_D64_KERNELS_ONLY
static d64::View view(const void* p, const Strides& s)
{
    return d64::View{(bf16*)p, s.sb, s.sh, s.st};
}

// the window the kernels use: W >= T (no lower edge) for the plain causal mask
static int window_of(const AttnArgs& a) { return a.window > 0 && a.window < a.T ? a.window : a.T; }

static d64::Dropout dropout_of(const AttnArgs& a)
{
    d64::Dropout d{};
    d.seed_lo = (uint32_t)a.dropout_seed;
    d.seed_hi = (uint32_t)(a.dropout_seed >> 32);
    d.p16 = (uint32_t)a.dropout_p16;
    d.keep_scale = (float)(65536.0 / (65536.0 - (double)a.dropout_p16));
    d.keep = a.keep;
    return d;
}

static d64::RopeP rope_p(const AttnArgs& a)
{
    d64::RopeP r;
    r.xq = view(a.xq, a.sxq);
    r.xk = view(a.xk, a.sxk);
    r.yq = view(a.q_rot, a.sqr);
    r.pos0 = a.pos0;
    r.flags = a.rope_flags;
    r.q_gain = a.q_gain;
    r.k_gain = a.k_gain;
    r.eps = a.rope_eps;
    r.fr = a.freqs;
    r.step4 = a.freqs.f[4] / a.freqs.f[0];
    r.step8 = a.freqs.f[8] / a.freqs.f[0];
    return r;
}

// Forward with the RoPE / QK-norm prologue: the keys through the prologue pass
// (k -> k_rot), then the forward on the raw queries (turned in registers and
// written to q_rot) and k_rot.
static hipError_t launch_fwd_rope_bf16_d64(const AttnArgs& a, hipStream_t st)
{
    RopeArgs r{};
    r.k = a.k;
    r.sk = a.sk;
    r.k_out = a.k_rot;
    r.sko = a.skr;
    r.dk_in = a.k;
    r.sdk = a.sk;
    r.B = a.B;
    r.H = a.H;
    r.T = a.T;
    r.D = a.D;
    r.pos0 = a.pos0;
    r.flags = a.rope_flags;
    r.q_gain = a.q_gain;
    r.k_gain = a.k_gain;
    r.eps = a.rope_eps;
    r.freqs = a.freqs;
    r.grad = false;
    r.k_only = true;
    const hipError_t e = launch_rope_qknorm(r, st);
    if (e != hipSuccess) return e;
    const int BH = a.B * a.H;
    const int nqt = (a.T + d64::kRowsPerWG - 1) / d64::kRowsPerWG;
    auto k = a.D == 128 ? d64::attn_fwd_d64_kernel<2, false, false, true>
                        : d64::attn_fwd_d64_kernel<1, false, false, true>;
    hipLaunchKernelGGL(k, dim3(nqt * BH), dim3(d64::kThreads), 0, st,
                       view(a.q, a.sq), view(a.k_rot, a.skr), view(a.v, a.sv), view(a.o_out, a.so),
                       a.lse, BH, a.H, a.T, window_of(a), nqt, a.scale, a.scale * kLog2e, a.n_cu,
                       dropout_of(a), rope_p(a));
    return hipGetLastError();
}

hipError_t launch_fwd_bf16_d64(const AttnArgs& a, hipStream_t st)
{
    if (a.rope) return launch_fwd_rope_bf16_d64(a, st);
    const int BH = a.B * a.H;
    const int nqt = (a.T + d64::kRowsPerWG - 1) / d64::kRowsPerWG;
    const bool drop = a.dropout_p16 > 0;
    const bool keep = drop && a.keep;  // also store the keep bits
    auto k = a.D == 128 ? (keep ? d64::attn_fwd_d64_kernel<2, true, true>
                                : drop ? d64::attn_fwd_d64_kernel<2, true> : d64::attn_fwd_d64_kernel<2, false>)
                        : (keep ? d64::attn_fwd_d64_kernel<1, true, true>
                                : drop ? d64::attn_fwd_d64_kernel<1, true> : d64::attn_fwd_d64_kernel<1, false>);
    hipLaunchKernelGGL(k, dim3(nqt * BH), dim3(d64::kThreads), 0, st,
                       view(a.q, a.sq), view(a.k, a.sk), view(a.v, a.sv), view(a.o_out, a.so),
                       a.lse, BH, a.H, a.T, window_of(a), nqt, a.scale, a.scale * kLog2e, a.n_cu,
                       dropout_of(a), d64::NoRope{});
    return hipGetLastError();
}

static d64::BwdParams bwd_params(const AttnArgs& a)
{
    d64::BwdParams p;
    p.Q = view(a.q, a.sq);
    p.K = view(a.k, a.sk);
    p.V = view(a.v, a.sv);
    p.O = view(a.o, a.so);
    p.dO = view(a.dO, a.sdo);
    p.LSE = a.lse;
    p.Delta = a.delta;
    p.dQ = view(a.dq, a.sdq);
    p.dK = view(a.dk, a.sdk);
    p.dV = view(a.dv, a.sdv);
    p.BH = a.B * a.H;
    p.H = a.H;
    p.T = a.T;
    p.W = window_of(a);
    p.scale = a.scale;
    p.scale_log2 = a.scale * kLog2e;
    p.dr = dropout_of(a);
    return p;
}

hipError_t launch_dq_bf16_d64(const AttnArgs& a, hipStream_t st)
{
    const int BH = a.B * a.H;
    const int nqt = (a.T + d64::kRowsPerWG - 1) / d64::kRowsPerWG;
    const bool drop = a.dropout_p16 > 0;
    const bool keep = drop && a.keep;  // load the stored keep bits
    auto k = a.D == 128 ? (keep ? d64::attn_bwd_dq_d64_kernel<2, true, true>
                                : drop ? d64::attn_bwd_dq_d64_kernel<2, true> : d64::attn_bwd_dq_d64_kernel<2, false>)
                        : (keep ? d64::attn_bwd_dq_d64_kernel<1, true, true>
                                : drop ? d64::attn_bwd_dq_d64_kernel<1, true> : d64::attn_bwd_dq_d64_kernel<1, false>);
    if (a.rope) {
        auto kr = a.D == 128 ? d64::attn_bwd_dq_d64_kernel<2, false, false, true>
                             : d64::attn_bwd_dq_d64_kernel<1, false, false, true>;
        hipLaunchKernelGGL(kr, dim3(nqt * BH), dim3(d64::kThreads), 0, st, bwd_params(a), nqt, a.n_cu,
                           rope_p(a));
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k, dim3(nqt * BH), dim3(d64::kThreads), 0, st, bwd_params(a), nqt, a.n_cu,
                       d64::NoRope{});
    return hipGetLastError();
}

hipError_t launch_dkdv_bf16_d64(const AttnArgs& a, hipStream_t st)
{
    const int BH = a.B * a.H;
    const int nkt = (a.T + d64::kRowsPerWG - 1) / d64::kRowsPerWG;
    const bool drop = a.dropout_p16 > 0;
    const bool keep = drop && a.keep;
    auto k = a.D == 128 ? (keep ? d64::attn_bwd_dkdv_d64_kernel<2, true, true>
                                : drop ? d64::attn_bwd_dkdv_d64_kernel<2, true> : d64::attn_bwd_dkdv_d64_kernel<2, false>)
                        : (keep ? d64::attn_bwd_dkdv_d64_kernel<1, true, true>
                                : drop ? d64::attn_bwd_dkdv_d64_kernel<1, true> : d64::attn_bwd_dkdv_d64_kernel<1, false>);
    if (a.rope) {
        auto kr = a.D == 128 ? d64::attn_bwd_dkdv_d64_kernel<2, false, false, true>
                             : d64::attn_bwd_dkdv_d64_kernel<1, false, false, true>;
        hipLaunchKernelGGL(kr, dim3(nkt * BH), dim3(d64::kThreads), 0, st, bwd_params(a), a.n_cu,
                           rope_p(a));
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k, dim3(nkt * BH), dim3(d64::kThreads), 0, st, bwd_params(a), a.n_cu,
                       d64::NoRope{});
    return hipGetLastError();
}

hipError_t launch_bwd_bf16_d64(const AttnArgs& a, hipStream_t st)
{
    const int BH = a.B * a.H;
    const int nb = (a.T + d64::kRowsPerWG - 1) / d64::kRowsPerWG;
    if (a.D == 128) {  // the Delta pass, then dK/dV and dQ items in one launch
        hipLaunchKernelGGL(d64::attn_delta_d64_kernel<2>, dim3(nb * BH), dim3(d64::kThreads), 0, st,
                           bwd_params(a), nb);
        if (a.rope) {
            hipLaunchKernelGGL((d64::attn_bwd_dpre_kernel<2, false, false, true>), dim3(2 * nb * BH),
                               dim3(d64::kThreads), 0, st, bwd_params(a), nb, a.n_cu, rope_p(a));
            return hipGetLastError();
        }
        auto k = a.dropout_p16 > 0 ? (a.keep ? d64::attn_bwd_dpre_kernel<2, true, true>
                                             : d64::attn_bwd_dpre_kernel<2, true>)
                                   : d64::attn_bwd_dpre_kernel<2, false>;
        hipLaunchKernelGGL(k, dim3(2 * nb * BH), dim3(d64::kThreads), 0, st, bwd_params(a), nb,
                           a.n_cu, d64::NoRope{});
        return hipGetLastError();
    }
    if (a.rope) {
        hipLaunchKernelGGL((d64::attn_bwd_d64_kernel<false, false, true>), dim3(2 * nb * BH),
                           dim3(d64::kThreads), 0, st, bwd_params(a), nb, a.n_cu, rope_p(a));
        return hipGetLastError();
    }
    auto k = a.dropout_p16 > 0 ? (a.keep ? d64::attn_bwd_d64_kernel<true, true> : d64::attn_bwd_d64_kernel<true>)
                               : d64::attn_bwd_d64_kernel<false>;
    hipLaunchKernelGGL(k, dim3(2 * nb * BH), dim3(d64::kThreads), 0, st, bwd_params(a), nb, a.n_cu,
                       d64::NoRope{});
    return hipGetLastError();
}

#endif  // CATTN_D64_KERNELS_ONLY

}  // namespace cattn

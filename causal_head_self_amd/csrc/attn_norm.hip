// attn_norm.hip -- the row passes of the pre-norm sublayer around the
// attention: LayerNorm forward, its gradient (with the residual branch's
// gradient added), and column sums (the gradient of a bias added to every
// row).  All three are HBM-bound: each reads its rows once and keeps them in
// registers.
//
// LayerNorm follows class LayerNorm of the CS336 from-scratch tutorial
// (section 3.4): mean and biased variance over the row, eps under the square
// root, then gain and bias:  y = (x - mean) / sqrt(var + eps) * g + b.
// Its gradient is the chain rule through that class: with xh = (x - mean) *
// rstd and e = dy * g,  dx = rstd * (e - mean(e) - xh * mean(e * xh)),
// dg = sum over rows of dy * xh, db = sum over rows of dy.  The backward
// recomputes mean and rstd from x instead of storing them.
//
// Layout: bf16 rows of C elements, row r at x + r * stride; g, b, dg, db bf16
// [C].  One wave per row, lane l holding 16-byte chunks l, l + 64, ... of it;
// fp32 arithmetic; wave sums by a fixed butterfly, so every result is
// deterministic.  Column partial sums go to a caller-owned fp32 workspace and
// are added up in a fixed order by a second launch.
#include "attn_device.h"
#include "attn_kernels.h"

namespace cattn {
namespace norm {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;  // rows in flight per workgroup
constexpr int kMaxC = 4096;            // LDS of the column partials: 2 * kMaxC floats
constexpr int kColThreads = 64;        // colsum: 8 columns per thread, one wave per block
constexpr int kColBlock = kColThreads * 8;

// Sum over the 64 lanes, the same value in every lane, in VALU cross-lane
// steps (no LDS round trips): quad swaps (DPP quad_perm 1,0,3,2 and 2,3,0,1),
// then the mirrored half row and the mirrored row, which leave each 16-lane row
// holding its sum, then v_permlane16_swap and v_permlane32_swap to add the
// rows.  Every step adds a pair of values in both of its lanes, so all lanes
// end with the same bits.
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v)
{
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF,
                                                          false));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v = dpp_add<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v = dpp_add<0x141>(v);  // row_half_mirror
    v = dpp_add<0x140>(v);  // row_mirror
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                      false, false);
    v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                      false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

__device__ __forceinline__ void load8(const bf16* p, float (&v)[8])
{
    const bf16x8 t = *(const bf16x8*)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)t[e];
}

__device__ __forceinline__ void store8(bf16* p, const float (&v)[8])
{
    bf16x8 t;
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = (bf16)v[e];
    *(bf16x8*)p = t;
}

// Row chunks are loaded for every lane, from clamped addresses (a lane whose
// chunk lies past C reloads the last one and counts it as zero), so the loads
// are not under divergent branches and the wait for them comes only where the
// values are used.
template <int NCH>
__device__ __forceinline__ void load_raw(const bf16* __restrict__ p, int lane, int nch,
                                         bf16x8 (&r)[NCH])
{
#pragma unroll
    for (int i = 0; i < NCH; ++i) r[i] = *(const bf16x8*)(p + 8 * min(lane + 64 * i, nch - 1));
}

// Element e of chunk i as fp32, 0 past C.
template <int NCH>
__device__ __forceinline__ float val(const bf16x8 (&r)[NCH], int i, int e, bool ok)
{
    return ok ? (float)r[i][e] : 0.f;
}

// NCH: chunks of 8 per lane, ceil(C / 512).
template <int NCH>
__global__ __launch_bounds__(kThreads) void layernorm_fwd_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ g, const bf16* __restrict__ b,
    bf16* __restrict__ y, int N, int C, long long stride, float eps)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= N) return;
    const int nch = C >> 3;
    bf16x8 xr[NCH], gr[NCH], br[NCH];
    load_raw<NCH>(x + (size_t)row * stride, lane, nch, xr);
    load_raw<NCH>(g, lane, nch, gr);
    load_raw<NCH>(b, lane, nch, br);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) s += val<NCH>(xr, i, e, lane + 64 * i < nch);
    const float inv_c = 1.0f / (float)C;
    const float mean = wave_sum(s) * inv_c;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
        if (lane + 64 * i < nch)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = (float)xr[i][e] - mean;
                q = fmaf(d, d, q);
            }
    const float rstd = 1.0f / sqrtf(wave_sum(q) * inv_c + eps);
    bf16* yr = y + (size_t)row * stride;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[e] = fmaf(((float)xr[i][e] - mean) * rstd, (float)gr[i][e], (float)br[i][e]);
            store8(yr + 8 * c, o);
        }
    }
}

// Gradient.  Workgroup w takes rows [w * rows_per_wg, (w + 1) * rows_per_wg),
// its wave j every kWaves-th of them from row j.  Each lane keeps the dg and db
// partial sums of its columns over the wave's rows; the four waves add theirs
// in LDS in wave order, and the workgroup writes [dg | db] (2C floats) to
// part[w].  A wave loads the next row's x and dy (the last row again when
// there is none) before it works on the current one, so that their latency
// overlaps that work.
template <int NCH>
__global__ __launch_bounds__(kThreads) void layernorm_bwd_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ g, const bf16* __restrict__ dy,
    const bf16* __restrict__ dres, bf16* __restrict__ dx, float* __restrict__ part, int N, int C,
    long long stride, float eps, int rows_per_wg)
{
    __shared__ __attribute__((aligned(16))) float s_part[2 * kMaxC];
    lds_poison(s_part);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nch = C >> 3;
    const float inv_c = 1.0f / (float)C;
    bf16x8 gr[NCH];
    load_raw<NCH>(g, lane, nch, gr);
    float ag[NCH][8], ab[NCH][8];
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) ag[i][e] = ab[i][e] = 0.f;
    const int r0 = blockIdx.x * rows_per_wg;
    const int r1 = min(N, r0 + rows_per_wg);
    // with 8 chunks per lane a second set of row registers would spill: each
    // row is then loaded as it comes
    constexpr bool kAhead = NCH <= 4;
    bf16x8 xr[NCH], dr[NCH], rr[NCH];
    int row = r0 + wave;
    if (kAhead && row < r1) {
        load_raw<NCH>(x + (size_t)row * stride, lane, nch, xr);
        load_raw<NCH>(dy + (size_t)row * stride, lane, nch, dr);
    }
    for (; row < r1; row += kWaves) {
        const size_t off = (size_t)row * stride;
        if (!kAhead) {
            load_raw<NCH>(x + off, lane, nch, xr);
            load_raw<NCH>(dy + off, lane, nch, dr);
        }
        // dres of this row is used last: loaded before the next row's x and dy,
        // it can be waited for while those are still in flight
        if (dres) load_raw<NCH>(dres + off, lane, nch, rr);
        const size_t nxt = (size_t)min(row + kWaves, r1 - 1) * stride;
        bf16x8 xn[NCH], dn[NCH];
        if (kAhead) {
            load_raw<NCH>(x + nxt, lane, nch, xn);
            load_raw<NCH>(dy + nxt, lane, nch, dn);
        }
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) s += val<NCH>(xr, i, e, lane + 64 * i < nch);
        const float mean = wave_sum(s) * inv_c;
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
            if (lane + 64 * i < nch)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float d = (float)xr[i][e] - mean;
                    q = fmaf(d, d, q);
                }
        const float rstd = 1.0f / sqrtf(wave_sum(q) * inv_c + eps);
        float s1 = 0.f, s2 = 0.f;
        float xh[NCH][8];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const bool ok = lane + 64 * i < nch;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xh[i][e] = ((float)xr[i][e] - mean) * rstd;
                const float d = val<NCH>(dr, i, e, ok);  // 0 past C: so is every term below
                const float ge = d * (float)gr[i][e];
                s1 += ge;
                s2 = fmaf(ge, xh[i][e], s2);
                ag[i][e] = fmaf(d, xh[i][e], ag[i][e]);
                ab[i][e] += d;
            }
        }
        const float m1 = wave_sum(s1) * inv_c;
        const float m2 = wave_sum(s2) * inv_c;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = lane + 64 * i;
            if (c < nch) {
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    o[e] = rstd * ((float)dr[i][e] * (float)gr[i][e] - m1 - xh[i][e] * m2);
                    if (dres) o[e] += (float)rr[i][e];
                }
                store8(dx + off + 8 * c, o);
            }
        }
        if (kAhead) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                xr[i] = xn[i];
                dr[i] = dn[i];
            }
        }
    }
    // the workgroup's column partials: waves 0..3 in turn
#pragma unroll 1
    for (int w = 0; w < kWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int c = lane + 64 * i;
                if (c < nch)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float* pg = &s_part[8 * c + e];
                        float* pb = &s_part[C + 8 * c + e];
                        *pg = w == 0 ? ag[i][e] : *pg + ag[i][e];
                        *pb = w == 0 ? ab[i][e] : *pb + ab[i][e];
                    }
            }
        }
        __syncthreads();
    }
    float* pw = part + (size_t)blockIdx.x * 2 * C;
    for (int j = threadIdx.x; j < 2 * C; j += kThreads) pw[j] = s_part[j];
}

// Column partial sums of a [N][M] bf16 matrix: workgroup (rb, cb) adds rows
// [rb * rows_per_blk, ...) of columns [cb * kColBlock, ...), 8 per thread, into
// part[rb][M].  Rows are read eight at a time (independent loads in flight),
// and added in row order.
__global__ __launch_bounds__(kColThreads) void colsum_part_kernel(
    const bf16* __restrict__ x, float* __restrict__ part, int N, int M, long long stride,
    int rows_per_blk)
{
    const int col = blockIdx.y * kColBlock + 8 * threadIdx.x;
    if (col >= M) return;
    const int r0 = blockIdx.x * rows_per_blk;
    const int r1 = min(N, r0 + rows_per_blk);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const bf16* xc = x + col;
    int r = r0;
    for (; r + 8 <= r1; r += 8) {
        bf16x8 t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = *(const bf16x8*)(xc + (size_t)(r + u) * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (float)t[u][e];
    }
    for (; r < r1; ++r) {
        const bf16x8 t = *(const bf16x8*)(xc + (size_t)r * stride);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (float)t[e];
    }
    float* pr = part + (size_t)blockIdx.x * M + col;
    *(f32x4*)pr = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)(pr + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// out[j] = sum over p < P of part[p][j], rounded once to bf16; out2 (if set)
// takes columns [M2, 2 * M2) when the partial rows hold two vectors side by
// side (LayerNorm: [dg | db]).  A workgroup takes 64 columns with 16 waves:
// wave w adds partials w, w + 16, ... (eight loads in flight per lane, eight
// running sums combined in a fixed tree), then the 16 wave sums are added in
// LDS in wave order.
constexpr int kRedWaves = 16;
__global__ __launch_bounds__(64 * kRedWaves) void colsum_reduce_kernel(
    const float* __restrict__ part, int P, int M, bf16* __restrict__ out, bf16* __restrict__ out2,
    int M2)
{
    __shared__ float s_sum[kRedWaves][64];
    lds_poison(s_sum);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int j = blockIdx.x * 64 + lane;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (j < M) {
        int p = w;
        for (; p + 7 * kRedWaves < P; p += 8 * kRedWaves) {
#pragma unroll
            for (int u = 0; u < 8; ++u) a[u] += part[(size_t)(p + u * kRedWaves) * M + j];
        }
        for (; p < P; p += kRedWaves) a[0] += part[(size_t)p * M + j];
    }
    s_sum[w][lane] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    __syncthreads();
    if (w == 0 && j < M) {
        float t = s_sum[0][lane];
#pragma unroll
        for (int v = 1; v < kRedWaves; ++v) t += s_sum[v][lane];
        if (out2 && j >= M2)
            out2[j - M2] = (bf16)t;
        else
            out[j] = (bf16)t;
    }
}

// Column sums of a few fp32 rows (the split-K partial products of a weight
// gradient), rounded once to bf16: thread t takes columns 4t .. 4t + 3 and
// adds rows 0, 1, ... in order.
__global__ __launch_bounds__(256) void sum_rows_f32_kernel(const float* __restrict__ x, int P,
                                                           int M, long long stride,
                                                           bf16* __restrict__ out)
{
    const long long col = 4LL * ((long long)blockIdx.x * 256 + threadIdx.x);
    if (col >= M) return;
    f32x4 acc = *(const f32x4*)(x + col);
    for (int p = 1; p < P; ++p) acc += *(const f32x4*)(x + (size_t)p * stride + col);
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (bf16)acc[e];
    *(bf16x4*)(out + col) = o;
}

int nch_of(int C) { return (C + 511) / 512; }

template <int NCH>
void fwd_launch(const NormArgs& a, hipStream_t st)
{
    hipLaunchKernelGGL(layernorm_fwd_kernel<NCH>, dim3((a.N + kWaves - 1) / kWaves),
                       dim3(kThreads), 0, st, (const bf16*)a.x, (const bf16*)a.g,
                       (const bf16*)a.b, (bf16*)a.y, a.N, a.C, a.stride, a.eps);
}

template <int NCH>
void bwd_launch(const NormArgs& a, int n_wg, int rows_per_wg, hipStream_t st)
{
    hipLaunchKernelGGL(layernorm_bwd_kernel<NCH>, dim3(n_wg), dim3(kThreads), 0, st,
                       (const bf16*)a.x, (const bf16*)a.g, (const bf16*)a.dy,
                       (const bf16*)a.dres, (bf16*)a.dx, (float*)a.workspace, a.N, a.C, a.stride,
                       a.eps, rows_per_wg);
}

}  // namespace norm

// Rows per workgroup of the LayerNorm gradient (16: four per wave) and of the
// column sums (32); the partial buffers follow from them.
int layernorm_bwd_workgroups(int N) { return (N + 15) / 16; }
// Column sums: at most 128 row blocks (of at least 8 rows), so that the
// reduction over them is one pass of independent loads.
int colsum_rows_per_block(int N) { return max(8, (N + 127) / 128); }
int colsum_row_blocks(int N) { return (N + colsum_rows_per_block(N) - 1) / colsum_rows_per_block(N); }

hipError_t launch_layernorm_fwd(const NormArgs& a, hipStream_t st)
{
    switch (norm::nch_of(a.C)) {
    case 1: norm::fwd_launch<1>(a, st); break;
    case 2: norm::fwd_launch<2>(a, st); break;
    case 3:
    case 4: norm::fwd_launch<4>(a, st); break;
    default: norm::fwd_launch<8>(a, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_layernorm_bwd(const NormArgs& a, hipStream_t st)
{
    const int n_wg = layernorm_bwd_workgroups(a.N);
    switch (norm::nch_of(a.C)) {
    case 1: norm::bwd_launch<1>(a, n_wg, 16, st); break;
    case 2: norm::bwd_launch<2>(a, n_wg, 16, st); break;
    case 3:
    case 4: norm::bwd_launch<4>(a, n_wg, 16, st); break;
    default: norm::bwd_launch<8>(a, n_wg, 16, st); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int M = 2 * a.C;
    hipLaunchKernelGGL(norm::colsum_reduce_kernel, dim3((M + 63) / 64), dim3(64 * norm::kRedWaves),
                       0, st, (const float*)a.workspace, n_wg, M, (bf16*)a.dg, (bf16*)a.db, a.C);
    return hipGetLastError();
}

hipError_t launch_colsum(const NormArgs& a, hipStream_t st)
{
    if (a.f32) {  // few rows: one pass, no partials
        const long long threads = (a.C + 3) / 4;
        hipLaunchKernelGGL(norm::sum_rows_f32_kernel, dim3((unsigned)((threads + 255) / 256)),
                           dim3(256), 0, st, (const float*)a.x, a.N, a.C, a.stride, (bf16*)a.y);
        return hipGetLastError();
    }
    const int P = colsum_row_blocks(a.N);
    hipLaunchKernelGGL(norm::colsum_part_kernel,
                       dim3(P, (a.C + norm::kColBlock - 1) / norm::kColBlock), dim3(norm::kColThreads),
                       0, st, (const bf16*)a.x, (float*)a.workspace, a.N, a.C, a.stride,
                       colsum_rows_per_block(a.N));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(norm::colsum_reduce_kernel, dim3((a.C + 63) / 64),
                       dim3(64 * norm::kRedWaves), 0, st, (const float*)a.workspace, P, a.C,
                       (bf16*)a.y, (bf16*)nullptr, a.C);
    return hipGetLastError();
}

}  // namespace cattn

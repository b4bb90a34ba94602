// attn_f32.hip -- fp32 kernels for causal multi-head self-attention (forward,
// Delta, dQ, dK/dV), same operation as attn_bf16.hip (CS336 from-scratch
// tutorial, lmnt.cn, section 5.1 CausalSelfAttention.forward, diagonal kept).
//
// gfx950 does have fp32 MFMA, but its dense fp32 rate (157 TFLOP/s) is that of
// the vector ALUs' packed FMA, so it would buy no throughput, and the fp32
// workloads here are small (the pages' tiny CPU config: T = 64, D = 32).  These
// kernels use plain fp32 FMA on the vector ALUs: one lane per query
// (forward, dQ) or per key (dK/dV), with 64-row K/V (or Q/dO) tiles shared
// through LDS.  Four waves hold the same 64 rows and each takes 16 rows of
// every tile; their partial results meet in LDS at the end, summed in wave
// order (the forward rescales its four softmax states to a common max first).
// With one wave per block the tiny configuration was bound by that one wave's
// chain of dependent LDS reads and FMAs (43 us for the forward).
#include "attn_device.h"
#include "attn_kernels.h"

namespace cattn {

constexpr int kRows = 64;             // rows per workgroup and per LDS tile
constexpr int kWaves = 4;             // waves per workgroup, all on the same 64 rows
constexpr int kSub = kRows / kWaves;  // rows of each tile that one wave takes
constexpr int kThreadsF32 = kRows * kWaves;

template <int HD>
__device__ __forceinline__ void load_rows_f32(float (*lds)[HD], const float* __restrict__ src,
                                              int row0, int T, int tid)
{
#pragma unroll 4
    for (int c = tid; c < kRows * HD / 4; c += kThreadsF32) {
        const int r = c / (HD / 4), cc = c % (HD / 4);
        f32x4 v = f32x4{};
        if (row0 + r < T) v = *(const f32x4*)(src + (size_t)(row0 + r) * HD + 4 * cc);
        *(f32x4*)(&lds[r][4 * cc]) = v;
    }
}

template <int HD>
__global__ __launch_bounds__(kThreadsF32) void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int T, int n_qtiles,
    float scale_log2)
{
    __shared__ __attribute__((aligned(16))) float sK[kRows][HD];
    __shared__ __attribute__((aligned(16))) float sV[kRows][HD];
    __shared__ float sO[kWaves - 1][kRows][HD];  // waves 1.. hand their state to wave 0
    __shared__ float sM[kWaves - 1][kRows], sL[kWaves - 1][kRows];
    lds_poison(sK, sV, sO, sM, sL);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x % BH;
    const int qt = n_qtiles - 1 - blockIdx.x / BH;
    const size_t head = (size_t)bh * T * HD;
    const int qrow = qt * kRows + lane;
    const bool valid = qrow < T;

    float q[HD], o[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) {
        q[d] = valid ? Q[head + (size_t)qrow * HD + d] : 0.f;
        o[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;  // base-2 scaled running max, normaliser

    const int kv_end = min(T, qt * kRows + kRows);
    const int n_kv = (kv_end + kRows - 1) / kRows;
    const int c0 = kSub * wave;  // this wave's keys of each tile
    for (int j = 0; j < n_kv; ++j) {
        const int k0 = j * kRows;
        __syncthreads();
        load_rows_f32<HD>(sK, K + head, k0, T, tid);
        load_rows_f32<HD>(sV, V + head, k0, T, tid);
        __syncthreads();
        const int last = min(c0 + kSub - 1, qrow - k0);  // last visible key of the wave's rows
        if (last < c0) continue;
        float s[kSub];
        float mc = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < kSub; ++kk) {
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < HD; ++d) dot = fmaf(q[d], sK[c0 + kk][d], dot);
            s[kk] = (c0 + kk <= last) ? dot * scale_log2 : -INFINITY;
            mc = fmaxf(mc, s[kk]);
        }
        const float m_new = fmaxf(m, mc);
        const float alpha = fast_exp2(m - m_new);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < HD; ++d) o[d] *= alpha;
#pragma unroll
        for (int kk = 0; kk < kSub; ++kk) {
            const float p = fast_exp2(s[kk] - m_new);
            l += p;
#pragma unroll
            for (int d = 0; d < HD; ++d) o[d] = fmaf(p, sV[c0 + kk][d], o[d]);
        }
        m = m_new;
    }
    // wave 0 merges the four states: M = max m_w, o = sum_w o_w 2^(m_w - M), likewise l
    if (wave > 0) {
        sM[wave - 1][lane] = m;
        sL[wave - 1][lane] = l;
#pragma unroll
        for (int d = 0; d < HD; ++d) sO[wave - 1][lane][d] = o[d];
    }
    __syncthreads();
    if (wave > 0 || !valid) return;
    float M = m;
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w) M = fmaxf(M, sM[w][lane]);
    // every valid query sees key 0, so M is finite; a wave with no visible key has
    // m = -inf and weight 0
    const float a0 = fast_exp2(m - M);
    float lt = l * a0;
#pragma unroll
    for (int d = 0; d < HD; ++d) o[d] *= a0;
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w) {
        const float aw = fast_exp2(sM[w][lane] - M);
        lt = fmaf(sL[w][lane], aw, lt);
#pragma unroll
        for (int d = 0; d < HD; ++d) o[d] = fmaf(sO[w][lane][d], aw, o[d]);
    }
    const float inv = 1.0f / lt;
#pragma unroll
    for (int d = 0; d < HD; ++d) O[head + (size_t)qrow * HD + d] = o[d] * inv;
    LSE[(size_t)bh * T + qrow] = M * kLn2 + logf(lt);
}

template <int HD>
__global__ __launch_bounds__(256) void attn_delta_f32_kernel(const float* __restrict__ O,
                                                             const float* __restrict__ dO,
                                                             float* __restrict__ Delta,
                                                             long long rows)
{
    constexpr int LPR = HD / 4;
    const long long row = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
    const int sub = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const f32x4 o = *(const f32x4*)(O + row * HD + 4 * sub);
        const f32x4 g = *(const f32x4*)(dO + row * HD + 4 * sub);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(o[e], g[e], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && sub == 0) Delta[row] = acc;
}

// Rows of the partial sums a wave hands to wave 0 (waves 1..kWaves-1).
template <int HD>
using PartF32 = float[kWaves - 1][kRows][HD];

// Sum of the four waves' values of x (wave 0's x plus waves 1.. from part, in
// wave order) into x of wave 0; every wave calls it.
template <int HD>
__device__ __forceinline__ void merge_sum(float (&x)[HD], PartF32<HD>& part, int wave, int lane)
{
    __syncthreads();  // part is free (an earlier merge has been read)
    if (wave > 0) {
#pragma unroll
        for (int d = 0; d < HD; ++d) part[wave - 1][lane][d] = x[d];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
            for (int d = 0; d < HD; ++d) x[d] += part[w][lane][d];
    }
}

template <int HD>
__global__ __launch_bounds__(kThreadsF32) void attn_bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    float* __restrict__ dQ, int BH, int T, int n_qtiles, float scale, float scale_log2)
{
    __shared__ __attribute__((aligned(16))) float sK[kRows][HD];
    __shared__ __attribute__((aligned(16))) float sV[kRows][HD];
    __shared__ PartF32<HD> part;
    lds_poison(sK, sV, part);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x % BH;
    const int qt = n_qtiles - 1 - blockIdx.x / BH;
    const size_t head = (size_t)bh * T * HD;
    const int qrow = qt * kRows + lane;
    const bool valid = qrow < T;

    float q[HD], g[HD], dq[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) {
        q[d] = valid ? Q[head + (size_t)qrow * HD + d] : 0.f;
        g[d] = valid ? dO[head + (size_t)qrow * HD + d] : 0.f;
        dq[d] = 0.f;
    }
    const float lse2 = valid ? LSE[(size_t)bh * T + qrow] * kLog2e : 0.f;
    const float dlt = valid ? Delta[(size_t)bh * T + qrow] : 0.f;

    const int kv_end = min(T, qt * kRows + kRows);
    const int n_kv = (kv_end + kRows - 1) / kRows;
    const int c0 = kSub * wave;  // this wave's keys of each tile
    for (int j = 0; j < n_kv; ++j) {
        const int k0 = j * kRows;
        __syncthreads();
        load_rows_f32<HD>(sK, K + head, k0, T, tid);
        load_rows_f32<HD>(sV, V + head, k0, T, tid);
        __syncthreads();
        const int last = valid ? min(c0 + kSub - 1, qrow - k0) : -1;
        for (int kk = c0; kk <= last; ++kk) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int d = 0; d < HD; ++d) {
                s = fmaf(q[d], sK[kk][d], s);
                dp = fmaf(g[d], sV[kk][d], dp);
            }
            const float p = fast_exp2(fmaf(s, scale_log2, -lse2));
            const float ds = p * (dp - dlt);
#pragma unroll
            for (int d = 0; d < HD; ++d) dq[d] = fmaf(ds, sK[kk][d], dq[d]);
        }
    }
    merge_sum<HD>(dq, part, wave, lane);
    if (wave == 0 && valid) {
#pragma unroll
        for (int d = 0; d < HD; ++d) dQ[head + (size_t)qrow * HD + d] = dq[d] * scale;
    }
}

template <int HD>
__global__ __launch_bounds__(kThreadsF32) void attn_bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    float* __restrict__ dK, float* __restrict__ dV, int BH, int T, float scale, float scale_log2)
{
    __shared__ __attribute__((aligned(16))) float sQ[kRows][HD];
    __shared__ __attribute__((aligned(16))) float sG[kRows][HD];
    __shared__ float sL[kRows], sD[kRows];
    __shared__ PartF32<HD> part;
    lds_poison(sQ, sG, sL, sD, part);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x % BH;
    const int kt = blockIdx.x / BH;
    const size_t head = (size_t)bh * T * HD;
    const int key = kt * kRows + lane;
    const bool valid = key < T;

    float k[HD], v[HD], dk[HD], dv[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) {
        k[d] = valid ? K[head + (size_t)key * HD + d] : 0.f;
        v[d] = valid ? V[head + (size_t)key * HD + d] : 0.f;
        dk[d] = 0.f;
        dv[d] = 0.f;
    }
    const int n_q = (T + kRows - 1) / kRows;
    const int c0 = kSub * wave;  // this wave's queries of each tile
    for (int i = kt; i < n_q; ++i) {
        const int q0 = i * kRows;
        __syncthreads();
        load_rows_f32<HD>(sQ, Q + head, q0, T, tid);
        load_rows_f32<HD>(sG, dO + head, q0, T, tid);
        if (tid < kRows) {
            sL[tid] = (q0 + tid < T) ? LSE[(size_t)bh * T + q0 + tid] * kLog2e : 0.f;
            sD[tid] = (q0 + tid < T) ? Delta[(size_t)bh * T + q0 + tid] : 0.f;
        }
        __syncthreads();
        const int first = valid ? max(c0, key - q0) : kRows;  // first query >= key
        const int end = min(c0 + kSub, T - q0);
        for (int qq = first; qq < end; ++qq) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int d = 0; d < HD; ++d) {
                s = fmaf(sQ[qq][d], k[d], s);
                dp = fmaf(sG[qq][d], v[d], dp);
            }
            const float p = fast_exp2(fmaf(s, scale_log2, -sL[qq]));
            const float ds = p * (dp - sD[qq]);
#pragma unroll
            for (int d = 0; d < HD; ++d) {
                dk[d] = fmaf(ds, sQ[qq][d], dk[d]);
                dv[d] = fmaf(p, sG[qq][d], dv[d]);
            }
        }
    }
    merge_sum<HD>(dk, part, wave, lane);
    merge_sum<HD>(dv, part, wave, lane);
    if (wave == 0 && valid) {
#pragma unroll
        for (int d = 0; d < HD; ++d) {
            dK[head + (size_t)key * HD + d] = dk[d] * scale;
            dV[head + (size_t)key * HD + d] = dv[d];
        }
    }
}

template <int HD>
static hipError_t fwd(const AttnArgs& a, hipStream_t st)
{
    const int BH = a.B * a.H;
    const int nqt = (a.T + kRows - 1) / kRows;
    hipLaunchKernelGGL(attn_fwd_f32_kernel<HD>, dim3(nqt * BH), dim3(kThreadsF32), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (float*)a.o_out, a.lse, BH, a.T, nqt, a.scale * kLog2e);
    return hipGetLastError();
}

template <int HD>
static hipError_t delta(const AttnArgs& a, hipStream_t st)
{
    const long long rows = (long long)a.B * a.H * a.T;
    constexpr int rpb = 256 / (HD / 4);
    hipLaunchKernelGGL(attn_delta_f32_kernel<HD>, dim3((unsigned)((rows + rpb - 1) / rpb)),
                       dim3(256), 0, st, (const float*)a.o, (const float*)a.dO, a.delta, rows);
    return hipGetLastError();
}

template <int HD>
static hipError_t dq(const AttnArgs& a, hipStream_t st)
{
    const int BH = a.B * a.H;
    const int nt = (a.T + kRows - 1) / kRows;
    hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<HD>, dim3(nt * BH), dim3(kThreadsF32), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (const float*)a.dO, (const float*)a.lse, (const float*)a.delta,
                       (float*)a.dq, BH, a.T, nt, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

template <int HD>
static hipError_t dkdv(const AttnArgs& a, hipStream_t st)
{
    const int BH = a.B * a.H;
    const int nt = (a.T + kRows - 1) / kRows;
    hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<HD>, dim3(nt * BH), dim3(kThreadsF32), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (const float*)a.dO, (const float*)a.lse, (const float*)a.delta,
                       (float*)a.dk, (float*)a.dv, BH, a.T, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

hipError_t launch_fwd_f32(const AttnArgs& a, hipStream_t st)
{
    return a.D == 64 ? fwd<64>(a, st) : fwd<32>(a, st);
}

hipError_t launch_dq_f32(const AttnArgs& a, hipStream_t st)
{
    const hipError_t e = a.D == 64 ? delta<64>(a, st) : delta<32>(a, st);
    if (e != hipSuccess) return e;
    return a.D == 64 ? dq<64>(a, st) : dq<32>(a, st);
}

hipError_t launch_dkdv_f32(const AttnArgs& a, hipStream_t st)
{
    return a.D == 64 ? dkdv<64>(a, st) : dkdv<32>(a, st);
}

}  // namespace cattn

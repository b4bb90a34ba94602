// attn_bf16.hip -- gfx950 MFMA kernels for causal multi-head self-attention
// with bf16 storage and fp32 accumulation: forward, Delta, dQ and dK/dV.
//
// Operation: causal scaled dot-product attention per (batch, head), as in the
// CS336 from-scratch tutorial (lmnt.cn), section 5.1 model.py,
// CausalSelfAttention.forward, with the diagonal kept (tril mask, "Train Your
// Own LLM from Scratch", section 1).  The backward is the exact gradient of
// that function (the pages train through it with loss.backward(), tutorial
// section 5.2):
//   dP = dO V^T, Delta_i = sum_d dO_id O_id, dS = P * (dP - Delta),
//   dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
//
// Design (one workgroup = 4 wave64s, one wave per SIMD):
//   forward / dQ: a workgroup owns 128 queries (32 per wave, kept in
//     registers as MFMA B operands) and streams 64-key K/V tiles through LDS.
//     Scores are computed transposed, S^T = K Q^T, so that each lane owns one
//     query column: the online-softmax row max and row sum are in-lane
//     reductions plus one exchange with lane ^ 32.  P^T (or dS^T) leaves the
//     accumulators directly as the B operand of O^T = V^T P^T
//     (dQ^T = K^T dS^T); V^T / K^T come from LDS tiles stored transposed.
//   dK/dV: a workgroup owns 128 keys (32 per wave, in registers) and streams
//     64-query Q/dO tiles (row-major and transposed copies) through LDS;
//     S = Q K^T leaves each lane owning one key column, and P / dS become the
//     B operands of dV^T = dO^T P and dK^T = Q^T dS.
//   Fully masked tiles are skipped (per wave), the diagonal tiles are masked
//   per element (key > query -> -inf), and rows >= T are zero-filled on load.
//   Work-groups are ordered longest-first, and all tiles of one (batch, head)
//   share blockIdx % 8 (one XCD, one L2) whenever B*H is a multiple of 8.
//   No atomics: every output element is written once by one lane.
#include "attn_device.h"
#include "attn_kernels.h"

namespace cattn {

constexpr int kThreads = 256;
constexpr int kBlockQ = 128;  // queries per workgroup (forward, dQ)
constexpr int kBlockK = 128;  // keys per workgroup (dK/dV)
constexpr int kTileN = 64;    // keys per streamed tile (forward, dQ)
constexpr int kTileM = 64;    // queries per streamed tile (dK/dV)

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int BH, int T, int n_qtiles, float scale,
    float scale_log2)
{
    constexpr int KS = HD / 16;        // MFMA k-steps over the head dim
    constexpr int DT = HD / 32;        // 32-row output subtiles over the head dim
    constexpr int KST = HD + 8;        // padded LDS row stride (row-major K)
    constexpr int VST = kTileN + 8;    // padded LDS row stride (V^T)
    __shared__ __attribute__((aligned(16))) bf16 sK[kTileN * KST];
    __shared__ __attribute__((aligned(16))) bf16 sVt[HD * VST];
    lds_poison(sK, sVt);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, hi = lane >> 5;
    const int bh = blockIdx.x % BH;
    const int qt = n_qtiles - 1 - blockIdx.x / BH;  // heaviest tiles first
    const size_t head = (size_t)bh * T * HD;
    const bf16* Qh = Q + head;
    const bf16* Kh = K + head;
    const bf16* Vh = V + head;

    const int q0w = qt * kBlockQ + wave * 32;  // first query of this wave
    const int qrow = q0w + li;                 // query of this lane

    bf16x8 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qreg[ks] = (qrow < T) ? *(const bf16x8*)(Qh + (size_t)qrow * HD + 16 * ks + 8 * hi)
                              : zero_bf16x8();

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
    float m = -INFINITY;  // running max of the raw dot products of this row
    float l = 0.f;        // this lane's share of the running normaliser

    const int kv_end = min(T, qt * kBlockQ + kBlockQ);
    const int n_kv = (kv_end + kTileN - 1) / kTileN;
    for (int j = 0; j < n_kv; ++j) {
        const int k0 = j * kTileN;
        __syncthreads();
        load_tile_rows<kTileN, HD, KST, kThreads>(sK, Kh, k0, T, tid);
        load_tile_transposed<kTileN, HD, VST, kThreads>(sVt, Vh, k0, T, tid);
        __syncthreads();
        if (k0 > q0w + 31) continue;  // every key of the tile follows every query of the wave

        // S^T = K Q^T : two 32-key subtiles
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s[kt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = *(const bf16x8*)(sK + (32 * kt + li) * KST + 16 * ks + 8 * hi);
                s[kt] = mfma32x32x16(a, qreg[ks], s[kt]);
            }
        }
        if (k0 + kTileN - 1 > q0w) {  // the tile crosses this wave's diagonal
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * kt + 8 * (r >> 2) + 4 * hi + (r & 3);
                    if (key > qrow) s[kt][r] = -INFINITY;
                }
        }
        float mt = s[0][0];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kt][r]);
        mt = fmaxf(mt, other_half(mt));
        const float m_new = fmaxf(m, mt);
        const float alpha = fast_exp2((m - m_new) * scale_log2);
        const float mc = m_new * scale_log2;
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[kt][r], scale_log2, -mc));
                s[kt][r] = p;
                rs += p;
            }
        l = fmaf(l, alpha, rs);
        m = m_new;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;

        // O^T += V^T P^T : contraction over the 64 keys in 4 k-steps
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x8 pb = pack_bf16x8(s[c >> 1], 8 * (c & 1));
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 a = *(const bf16x8*)(sVt + (32 * dt + li) * VST + 16 * c + 8 * hi);
                oacc[dt] = mfma32x32x16(a, pb, oacc[dt]);
            }
        }
    }

    l += other_half(l);
    if (qrow < T) {
        const float inv = 1.0f / l;
        bf16* orow = O + head + (size_t)qrow * HD;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store_bf16x4(orow + 32 * dt + 8 * g + 4 * hi, oacc[dt][4 * g] * inv,
                             oacc[dt][4 * g + 1] * inv, oacc[dt][4 * g + 2] * inv,
                             oacc[dt][4 * g + 3] * inv);
        if (hi == 0) LSE[(size_t)bh * T + qrow] = m * scale + logf(l);
    }
}

// ---------------------------------------------------------------------------
// Delta_i = sum_d dO_id * O_id (fp32), one row per HD/8 lanes
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(kThreads) void attn_delta_bf16_kernel(
    const bf16* __restrict__ O, const bf16* __restrict__ dO, float* __restrict__ Delta,
    long long rows)
{
    constexpr int LPR = HD / 8;  // lanes per row
    const long long row = (long long)blockIdx.x * (kThreads / LPR) + threadIdx.x / LPR;
    const int sub = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const bf16x8 o = *(const bf16x8*)(O + row * HD + 8 * sub);
        const bf16x8 g = *(const bf16x8*)(dO + row * HD + 8 * sub);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && sub == 0) Delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dQ: per 128 queries, stream 64-key tiles
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(kThreads, 2) void attn_bwd_dq_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    bf16* __restrict__ dQ, int BH, int T, int n_qtiles, float scale, float scale_log2)
{
    constexpr int KS = HD / 16;
    constexpr int DT = HD / 32;
    constexpr int KST = HD + 8;
    constexpr int TST = kTileN + 8;
    __shared__ __attribute__((aligned(16))) bf16 sK[kTileN * KST];
    __shared__ __attribute__((aligned(16))) bf16 sV[kTileN * KST];
    __shared__ __attribute__((aligned(16))) bf16 sKt[HD * TST];
    lds_poison(sK, sV, sKt);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, hi = lane >> 5;
    const int bh = blockIdx.x % BH;
    const int qt = n_qtiles - 1 - blockIdx.x / BH;
    const size_t head = (size_t)bh * T * HD;
    const bf16* Kh = K + head;
    const bf16* Vh = V + head;

    const int q0w = qt * kBlockQ + wave * 32;
    const int qrow = q0w + li;
    const bool valid = qrow < T;

    bf16x8 qreg[KS], greg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const size_t off = head + (size_t)qrow * HD + 16 * ks + 8 * hi;
        qreg[ks] = valid ? *(const bf16x8*)(Q + off) : zero_bf16x8();
        greg[ks] = valid ? *(const bf16x8*)(dO + off) : zero_bf16x8();
    }
    // rows >= T get lse = +inf, so their P (and dS) is exactly 0
    const float lse2 = valid ? LSE[(size_t)bh * T + qrow] * kLog2e : INFINITY;
    const float dlt = valid ? Delta[(size_t)bh * T + qrow] : 0.f;

    f32x16 dqacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dqacc[dt] = f32x16{};

    const int kv_end = min(T, qt * kBlockQ + kBlockQ);
    const int n_kv = (kv_end + kTileN - 1) / kTileN;
    for (int j = 0; j < n_kv; ++j) {
        const int k0 = j * kTileN;
        __syncthreads();
        load_tile_rows<kTileN, HD, KST, kThreads>(sK, Kh, k0, T, tid);
        load_tile_rows<kTileN, HD, KST, kThreads>(sV, Vh, k0, T, tid);
        load_tile_transposed<kTileN, HD, TST, kThreads>(sKt, Kh, k0, T, tid);
        __syncthreads();
        if (k0 > q0w + 31) continue;

        f32x16 s[2], dp[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s[kt] = f32x16{};
            dp[kt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int off = (32 * kt + li) * KST + 16 * ks + 8 * hi;
                s[kt] = mfma32x32x16(*(const bf16x8*)(sK + off), qreg[ks], s[kt]);
                dp[kt] = mfma32x32x16(*(const bf16x8*)(sV + off), greg[ks], dp[kt]);
            }
        }
        const bool diag = k0 + kTileN - 1 > q0w;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(fmaf(s[kt][r], scale_log2, -lse2));
                if (diag) {
                    const int key = k0 + 32 * kt + 8 * (r >> 2) + 4 * hi + (r & 3);
                    if (key > qrow) p = 0.f;
                }
                s[kt][r] = p * (dp[kt][r] - dlt);  // dS^T
            }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x8 db = pack_bf16x8(s[c >> 1], 8 * (c & 1));
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 a = *(const bf16x8*)(sKt + (32 * dt + li) * TST + 16 * c + 8 * hi);
                dqacc[dt] = mfma32x32x16(a, db, dqacc[dt]);
            }
        }
    }

    if (valid) {
        bf16* row = dQ + head + (size_t)qrow * HD;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store_bf16x4(row + 32 * dt + 8 * g + 4 * hi, dqacc[dt][4 * g] * scale,
                             dqacc[dt][4 * g + 1] * scale, dqacc[dt][4 * g + 2] * scale,
                             dqacc[dt][4 * g + 3] * scale);
    }
}

// ---------------------------------------------------------------------------
// dK, dV: per 128 keys, stream 64-query tiles from the diagonal to T
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(kThreads, 2) void attn_bwd_dkdv_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int BH, int T, float scale, float scale_log2)
{
    constexpr int KS = HD / 16;
    constexpr int DT = HD / 32;
    constexpr int RST = HD + 8;       // row-major tiles
    constexpr int TST = kTileM + 8;   // transposed tiles
    __shared__ __attribute__((aligned(16))) bf16 sQ[kTileM * RST];
    __shared__ __attribute__((aligned(16))) bf16 sG[kTileM * RST];
    __shared__ __attribute__((aligned(16))) bf16 sQt[HD * TST];
    __shared__ __attribute__((aligned(16))) bf16 sGt[HD * TST];
    __shared__ __attribute__((aligned(16))) float sL[kTileM];
    __shared__ __attribute__((aligned(16))) float sD[kTileM];
    lds_poison(sQ, sG, sQt, sGt, sL, sD);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, hi = lane >> 5;
    const int bh = blockIdx.x % BH;
    const int kt_blk = blockIdx.x / BH;  // ascending: the first keys see the most queries
    const size_t head = (size_t)bh * T * HD;
    const bf16* Qh = Q + head;
    const bf16* Gh = dO + head;
    const float* Lh = LSE + (size_t)bh * T;
    const float* Dh = Delta + (size_t)bh * T;

    const int kv0 = kt_blk * kBlockK;
    const int k0w = kv0 + wave * 32;
    const int key = k0w + li;
    const bool valid = key < T;

    bf16x8 kreg[KS], vreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const size_t off = head + (size_t)key * HD + 16 * ks + 8 * hi;
        kreg[ks] = valid ? *(const bf16x8*)(K + off) : zero_bf16x8();
        vreg[ks] = valid ? *(const bf16x8*)(V + off) : zero_bf16x8();
    }
    f32x16 dkacc[DT], dvacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        dkacc[dt] = f32x16{};
        dvacc[dt] = f32x16{};
    }

    const int n_q = (T + kTileM - 1) / kTileM;
    for (int i = kv0 / kTileM; i < n_q; ++i) {
        const int q0 = i * kTileM;
        __syncthreads();
        load_tile_rows<kTileM, HD, RST, kThreads>(sQ, Qh, q0, T, tid);
        load_tile_rows<kTileM, HD, RST, kThreads>(sG, Gh, q0, T, tid);
        load_tile_transposed<kTileM, HD, TST, kThreads>(sQt, Qh, q0, T, tid);
        load_tile_transposed<kTileM, HD, TST, kThreads>(sGt, Gh, q0, T, tid);
        if (tid < kTileM) {
            const bool ok = q0 + tid < T;
            sL[tid] = ok ? Lh[q0 + tid] * kLog2e : INFINITY;
            sD[tid] = ok ? Dh[q0 + tid] : 0.f;
        }
        __syncthreads();
        if (q0 + kTileM - 1 < k0w) continue;  // every query of the tile precedes every key of the wave

        // S = Q K^T, dP = dO V^T : two 32-query subtiles; lane owns one key column
        f32x16 s[2], dp[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            s[qt] = f32x16{};
            dp[qt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int off = (32 * qt + li) * RST + 16 * ks + 8 * hi;
                s[qt] = mfma32x32x16(*(const bf16x8*)(sQ + off), kreg[ks], s[qt]);
                dp[qt] = mfma32x32x16(*(const bf16x8*)(sG + off), vreg[ks], dp[qt]);
            }
        }
        const bool diag = q0 < k0w + 31;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int qr = 32 * qt + 8 * g + 4 * hi;  // first of 4 consecutive queries
                const f32x4 l4 = *(const f32x4*)(sL + qr);
                const f32x4 d4 = *(const f32x4*)(sD + qr);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    float p = fast_exp2(fmaf(s[qt][r], scale_log2, -l4[e]));
                    if (diag && key > q0 + qr + e) p = 0.f;
                    s[qt][r] = p;
                    dp[qt][r] = p * (dp[qt][r] - d4[e]);  // dS
                }
            }
        // dV^T += dO^T P, dK^T += Q^T dS : contraction over the 64 queries
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x8 pb = pack_bf16x8(s[c >> 1], 8 * (c & 1));
            const bf16x8 db = pack_bf16x8(dp[c >> 1], 8 * (c & 1));
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int off = (32 * dt + li) * TST + 16 * c + 8 * hi;
                dvacc[dt] = mfma32x32x16(*(const bf16x8*)(sGt + off), pb, dvacc[dt]);
                dkacc[dt] = mfma32x32x16(*(const bf16x8*)(sQt + off), db, dkacc[dt]);
            }
        }
    }

    if (valid) {
        bf16* krow = dK + head + (size_t)key * HD;
        bf16* vrow = dV + head + (size_t)key * HD;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hi;
                store_bf16x4(krow + d, dkacc[dt][4 * g] * scale, dkacc[dt][4 * g + 1] * scale,
                             dkacc[dt][4 * g + 2] * scale, dkacc[dt][4 * g + 3] * scale);
                store_bf16x4(vrow + d, dvacc[dt][4 * g], dvacc[dt][4 * g + 1],
                             dvacc[dt][4 * g + 2], dvacc[dt][4 * g + 3]);
            }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int HD>
static hipError_t launch_fwd(const AttnArgs& a, hipStream_t st)
{
    const int BH = a.B * a.H;
    const int nqt = (a.T + kBlockQ - 1) / kBlockQ;
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<HD>, dim3(nqt * BH), dim3(kThreads), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o_out, a.lse,
                       BH, a.T, nqt, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

template <int HD>
static hipError_t launch_delta(const AttnArgs& a, hipStream_t st)
{
    const long long rows = (long long)a.B * a.H * a.T;
    constexpr int rows_per_block = kThreads / (HD / 8);
    hipLaunchKernelGGL(attn_delta_bf16_kernel<HD>,
                       dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                       dim3(kThreads), 0, st, (const bf16*)a.o, (const bf16*)a.dO, a.delta, rows);
    return hipGetLastError();
}

template <int HD>
static hipError_t launch_dq(const AttnArgs& a, hipStream_t st)
{
    const int BH = a.B * a.H;
    const int nqt = (a.T + kBlockQ - 1) / kBlockQ;
    hipLaunchKernelGGL(attn_bwd_dq_bf16_kernel<HD>, dim3(nqt * BH), dim3(kThreads), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.dO,
                       (const float*)a.lse, (const float*)a.delta, (bf16*)a.dq, BH, a.T, nqt,
                       a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

template <int HD>
static hipError_t launch_dkdv(const AttnArgs& a, hipStream_t st)
{
    const int BH = a.B * a.H;
    const int nkt = (a.T + kBlockK - 1) / kBlockK;
    hipLaunchKernelGGL(attn_bwd_dkdv_bf16_kernel<HD>, dim3(nkt * BH), dim3(kThreads), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.dO,
                       (const float*)a.lse, (const float*)a.delta, (bf16*)a.dk, (bf16*)a.dv, BH,
                       a.T, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const AttnArgs& a, hipStream_t st)
{
    return a.D == 32 ? launch_fwd<32>(a, st) : launch_fwd_bf16_d64(a, st);  // D = 64 or 128
}

hipError_t launch_dq_bf16(const AttnArgs& a, hipStream_t st)
{
    if (a.D != 32) return launch_dq_bf16_d64(a, st);  // Delta fused into the dQ kernel
    const hipError_t e = launch_delta<32>(a, st);
    return e == hipSuccess ? launch_dq<32>(a, st) : e;
}

hipError_t launch_dkdv_bf16(const AttnArgs& a, hipStream_t st)
{
    return a.D == 32 ? launch_dkdv<32>(a, st) : launch_dkdv_bf16_d64(a, st);
}

hipError_t launch_bwd_bf16(const AttnArgs& a, hipStream_t st)
{
    if (a.D != 32) return launch_bwd_bf16_d64(a, st);  // D = 64: dQ and dK/dV items in one grid
    const hipError_t e = launch_dq_bf16(a, st);
    return e == hipSuccess ? launch_dkdv_bf16(a, st) : e;
}

}  // namespace cattn

// attn_decode.hip -- decode attention on gfx950: one new token per sequence
// against its key/value cache, bf16 storage, fp32 arithmetic.
//
// nanochat, section 8 (inference engine): the KV cache is kept in FA3's
// native (B, T, H, D) layout; after the prompt is prefilled, tokens are
// produced one at a time, and each attends to every cached position up to and
// including its own (with a sliding window, the W most recent).  Per cached
// position the work is two length-D dot products against 4D bytes of K and V,
// so the op is bound by HBM bandwidth, not by the matrix cores; it runs on the
// vector ALUs and is built to stream the cache once at full width.
//
// Two paths.  One launch (decode_fused_kernel, below): a workgroup per (b, h)
// whose waves split the cache and merge through LDS.  Split-K in two launches,
// for few heads with long caches:
//   decode_partial_kernel: one wave per (sequence, slice of 64 cached
//     positions, head).  Workgroups are numbered (b, slice, h), h fastest, so
//     neighbouring waves stream neighbouring bytes of the same cache rows.
//     A group of 8 lanes takes one position (8 positions per step, all 64
//     positions' K and V loads issued before any arithmetic); each lane holds
//     D/8 columns, 16 bytes per 64 columns, so each load instruction moves
//     eight fully used 128-byte segments.  Scores are summed inside the group
//     (DPP), the slice's softmax runs in base 2 on fp32, and the slice's
//     partial (running max m, normaliser l, unnormalised o) goes to the
//     workspace.
//   decode_combine_kernel: four waves per (b, h) merge the slices' partials:
//     M = max m_s, L = sum 2^(m_s - M) l_s, o = sum 2^(m_s - M) o_s / L,
//     lse = (M + log2 L) ln 2.
#include <atomic>

#include "../../include/causal_attn.h"
#include "attn_device.h"
#include "attn_kernels.h"

namespace cattn {
namespace dec {

constexpr int kPos = 64;         // cached positions per wave
constexpr int kSteps = kPos / 8;  // positions per lane group

// Sum over the 8 lanes of an aligned group (quad swaps, then the mirrored
// half-row, which pairs lane i of one quad with lane 3 - i of the other).
__device__ __forceinline__ float group8_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    return x;
}

// Partial of one (b, slice, h).  NL = D / 64 (16-byte loads per lane per row).
// part row layout (D + 4 floats): o[0..D), m (base-2 units), l, 2 unused.
template <int NL>
__global__ __launch_bounds__(64) void decode_partial_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int* __restrict__ lens, float* __restrict__ part, int H, int Tmax, int n_slice,
    int window, float scale_log2)
{
    constexpr int D = 64 * NL;
    const int lane = threadIdx.x;
    const int g = lane >> 3, sub = lane & 7;
    const int h = blockIdx.x % H;
    const int r = blockIdx.x / H;
    const int slice = r % n_slice, b = r / n_slice;
    const int len = min(max(lens[b], 0), Tmax);
    const int first = window > 0 ? max(0, len - window) : 0;
    const int p0 = slice * kPos;
    const int lo = max(first, p0), hi = min(len, p0 + kPos);

    const size_t row = (size_t)H * D;  // elements between consecutive positions
    const bf16* kb = kc + (size_t)b * Tmax * row + (size_t)h * D + 8 * sub;
    const bf16* vb = vc + (size_t)b * Tmax * row + (size_t)h * D + 8 * sub;

    // every load of the slice first
    bf16x8 kr[kSteps][NL], vr[kSteps][NL];
#pragma unroll
    for (int it = 0; it < kSteps; ++it) {
        const int p = p0 + 8 * it + g;
        const bool in = p >= lo && p < hi;
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            kr[it][n] = in ? *(const bf16x8*)(kb + (size_t)p * row + 64 * n) : zero_bf16x8();
            vr[it][n] = in ? *(const bf16x8*)(vb + (size_t)p * row + 64 * n) : zero_bf16x8();
        }
    }
    float qf[NL][8];
    const bf16* qr = q + ((size_t)b * H + h) * D + 8 * sub;
#pragma unroll
    for (int n = 0; n < NL; ++n) {
        const bf16x8 qv = *(const bf16x8*)(qr + 64 * n);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[n][e] = (float)qv[e] * scale_log2;
    }

    // scores of the group's 8 positions (base-2 units), masked outside [lo, hi)
    float s[kSteps];
    float m = -INFINITY;
#pragma unroll
    for (int it = 0; it < kSteps; ++it) {
        float acc = 0.f;
#pragma unroll
        for (int n = 0; n < NL; ++n)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(qf[n][e], (float)kr[it][n][e], acc);
        acc = group8_sum(acc);
        const int p = p0 + 8 * it + g;
        s[it] = (p >= lo && p < hi) ? acc : -INFINITY;
        m = fmaxf(m, s[it]);
    }
    float l = 0.f;
    float o[NL][8];
#pragma unroll
    for (int n = 0; n < NL; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[n][e] = 0.f;
    if (m != -INFINITY) {
#pragma unroll
        for (int it = 0; it < kSteps; ++it) {
            const float pr = fast_exp2(s[it] - m);  // 0 for a masked position
            l += pr;
#pragma unroll
            for (int n = 0; n < NL; ++n)
#pragma unroll
                for (int e = 0; e < 8; ++e) o[n][e] = fmaf(pr, (float)vr[it][n][e], o[n][e]);
        }
    }

    // merge the 8 groups (lanes l, l ^ 8, l ^ 16, l ^ 32 hold the same columns)
    float M = m;
#pragma unroll
    for (int k = 8; k < 64; k <<= 1) M = fmaxf(M, __shfl_xor(M, k, 64));
    const float f = m == -INFINITY ? 0.f : fast_exp2(m - M);
    l *= f;
#pragma unroll
    for (int k = 8; k < 64; k <<= 1) l += __shfl_xor(l, k, 64);
#pragma unroll
    for (int n = 0; n < NL; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = o[n][e] * f;
#pragma unroll
            for (int k = 8; k < 64; k <<= 1) x += __shfl_xor(x, k, 64);
            o[n][e] = x;
        }

    float* out = part + (((size_t)b * H + h) * n_slice + slice) * (D + 4);
    if (g == 0) {
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            *(f32x4*)(out + 64 * n + 8 * sub) = f32x4{o[n][0], o[n][1], o[n][2], o[n][3]};
            *(f32x4*)(out + 64 * n + 8 * sub + 4) = f32x4{o[n][4], o[n][5], o[n][6], o[n][7]};
        }
    }
    if (lane == 0) {
        out[D] = M;  // -inf for a slice with no visible position
        out[D + 1] = l;
    }
}

// Merge of the slices of one (b, h) into o (bf16) and lse (natural log).
// kCW waves per (b, h): wave w merges a contiguous share of the slices, then
// wave 0 adds the waves' sums in LDS.  Within a wave, slices are taken 64 at
// a time, one per lane: their m and l load in one round, the weights
// 2^(m_s - M) are formed in the lanes, and each weight is broadcast
// (readlane) to the sum over the slices' o rows, whose loads are independent
// of one another.  Every wave forms the global M itself.
constexpr int kCW = 4;

template <int NL>
__global__ __launch_bounds__(64 * kCW) void decode_combine_kernel(const float* __restrict__ part,
                                                                  bf16* __restrict__ o,
                                                                  float* __restrict__ lse,
                                                                  int n_slice)
{
    constexpr int D = 64 * NL;
    constexpr int P = D + 4;
    __shared__ float s_acc[kCW][D];
    __shared__ float s_L[kCW];
    lds_poison(s_acc, s_L);
    const int bh = blockIdx.x, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float* pb = part + (size_t)bh * n_slice * P;
    float M = -INFINITY;
    for (int s = lane; s < n_slice; s += 64) M = fmaxf(M, pb[(size_t)s * P + D]);
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) M = fmaxf(M, __shfl_xor(M, k, 64));
    const int per = (n_slice + kCW - 1) / kCW;
    const int sb = wave * per, se = min(n_slice, sb + per);
    float L = 0.f;
    float acc[NL];
#pragma unroll
    for (int n = 0; n < NL; ++n) acc[n] = 0.f;
    if (M != -INFINITY) {
        for (int s0 = sb; s0 < se; s0 += 64) {
            const int s = s0 + lane;
            const float* ps = pb + (size_t)s * P;
            // 0 for a lane past the wave's last slice and for an empty slice (m = -inf)
            const float w = s < se ? fast_exp2(ps[D] - M) : 0.f;
            L = s < se ? fmaf(w, ps[D + 1], L) : L;
            const int cnt = min(64, se - s0);
            const float* row = pb + (size_t)s0 * P + lane;
            // blocks of 8 slices, loads first (readlane is convergent, so the
            // compiler does not unroll a loop with a remainder around it)
            int j = 0;
            for (; j + 8 <= cnt; j += 8) {
                float r[8][NL];
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int n = 0; n < NL; ++n) r[u][n] = row[(size_t)(j + u) * P + 64 * n];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j + u));
#pragma unroll
                    for (int n = 0; n < NL; ++n) acc[n] = fmaf(wj, r[u][n], acc[n]);
                }
            }
            for (; j < cnt; ++j) {
                const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
#pragma unroll
                for (int n = 0; n < NL; ++n) acc[n] = fmaf(wj, row[(size_t)j * P + 64 * n], acc[n]);
            }
        }
#pragma unroll
        for (int k = 1; k < 64; k <<= 1) L += __shfl_xor(L, k, 64);
    }
#pragma unroll
    for (int n = 0; n < NL; ++n) s_acc[wave][lane + 64 * n] = acc[n];
    if (lane == 0) s_L[wave] = L;
    __syncthreads();
    if (wave != 0) return;
    float Lt = 0.f;
#pragma unroll
    for (int w = 0; w < kCW; ++w) Lt += s_L[w];
    const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;
#pragma unroll
    for (int n = 0; n < NL; ++n) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < kCW; ++w) a += s_acc[w][lane + 64 * n];
        o[(size_t)bh * D + lane + 64 * n] = (bf16)(a * inv);
    }
    if (lane == 0) lse[bh] = M == -INFINITY ? -INFINITY : (M + log2f(Lt)) * kLn2;
}

// Whole decode of one (b, h) in one workgroup of NW waves: wave w takes the
// slices w, w + NW, ... of 64 cached positions with the loads and scores of
// decode_partial_kernel, and keeps a running max, normaliser and output across
// its slices (online softmax, base 2).  The waves then meet in LDS, where wave
// 0 merges their states as decode_combine_kernel merges slices.  No workspace
// and no second launch.
template <int NL, int NW>
__global__ __launch_bounds__(64 * NW) void decode_fused_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int* __restrict__ lens, bf16* __restrict__ o, float* __restrict__ lse, int H, int Tmax,
    int n_slice, int window, float scale_log2)
{
    constexpr int D = 64 * NL;
    __shared__ float s_o[NW][D];
    __shared__ float s_m[NW], s_l[NW];
    lds_poison(s_o, s_m, s_l);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int g = lane >> 3, sub = lane & 7;
    const int bh = blockIdx.x;
    const int h = bh % H, b = bh / H;
    const int len = min(max(lens[b], 0), Tmax);
    const int first = window > 0 ? max(0, len - window) : 0;

    const size_t row = (size_t)H * D;
    const bf16* kb = kc + (size_t)b * Tmax * row + (size_t)h * D + 8 * sub;
    const bf16* vb = vc + (size_t)b * Tmax * row + (size_t)h * D + 8 * sub;
    float qf[NL][8];
    const bf16* qr = q + (size_t)bh * D + 8 * sub;
#pragma unroll
    for (int n = 0; n < NL; ++n) {
        const bf16x8 qv = *(const bf16x8*)(qr + 64 * n);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[n][e] = (float)qv[e] * scale_log2;
    }

    float m = -INFINITY, l = 0.f;  // running state of this lane group
    float acc[NL][8];
#pragma unroll
    for (int n = 0; n < NL; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[n][e] = 0.f;

    for (int slice = wave; slice < n_slice; slice += nw) {
        const int p0 = slice * kPos;
        const int lo = max(first, p0), hi = min(len, p0 + kPos);
        if (lo >= hi) continue;  // wave-uniform
        bf16x8 kr[kSteps][NL], vr[kSteps][NL];
#pragma unroll
        for (int it = 0; it < kSteps; ++it) {
            const int p = p0 + 8 * it + g;
            const bool in = p >= lo && p < hi;
#pragma unroll
            for (int n = 0; n < NL; ++n) {
                kr[it][n] = in ? *(const bf16x8*)(kb + (size_t)p * row + 64 * n) : zero_bf16x8();
                vr[it][n] = in ? *(const bf16x8*)(vb + (size_t)p * row + 64 * n) : zero_bf16x8();
            }
        }
        float sc[kSteps];
        float mx = m;
#pragma unroll
        for (int it = 0; it < kSteps; ++it) {
            float d = 0.f;
#pragma unroll
            for (int n = 0; n < NL; ++n)
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(qf[n][e], (float)kr[it][n][e], d);
            d = group8_sum(d);
            const int p = p0 + 8 * it + g;
            sc[it] = (p >= lo && p < hi) ? d : -INFINITY;
            mx = fmaxf(mx, sc[it]);
        }
        if (mx == -INFINITY) continue;  // no visible position for this group yet
        const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mx);
        l *= alpha;
#pragma unroll
        for (int n = 0; n < NL; ++n)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[n][e] *= alpha;
#pragma unroll
        for (int it = 0; it < kSteps; ++it) {
            const float pr = fast_exp2(sc[it] - mx);  // 0 for a masked position
            l += pr;
#pragma unroll
            for (int n = 0; n < NL; ++n)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[n][e] = fmaf(pr, (float)vr[it][n][e], acc[n][e]);
        }
        m = mx;
    }

    // the wave's 8 groups (lanes l, l ^ 8, l ^ 16, l ^ 32 hold the same columns)
    float M = m;
#pragma unroll
    for (int k = 8; k < 64; k <<= 1) M = fmaxf(M, __shfl_xor(M, k, 64));
    const float f = m == -INFINITY ? 0.f : fast_exp2(m - M);
    l *= f;
#pragma unroll
    for (int k = 8; k < 64; k <<= 1) l += __shfl_xor(l, k, 64);
#pragma unroll
    for (int n = 0; n < NL; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = acc[n][e] * f;
#pragma unroll
            for (int k = 8; k < 64; k <<= 1) x += __shfl_xor(x, k, 64);
            acc[n][e] = x;
        }
    if (g == 0) {
#pragma unroll
        for (int n = 0; n < NL; ++n)
#pragma unroll
            for (int e = 0; e < 8; ++e) s_o[wave][64 * n + 8 * sub + e] = acc[n][e];
    }
    if (lane == 0) {
        s_m[wave] = M;
        s_l[wave] = l;
    }
    __syncthreads();
    if (wave != 0) return;

    // wave 0: lane c owns columns c + 64 n
    float Mx = -INFINITY;
    for (int w = 0; w < nw; ++w) Mx = fmaxf(Mx, s_m[w]);
    float L = 0.f, out[NL];
#pragma unroll
    for (int n = 0; n < NL; ++n) out[n] = 0.f;
    if (Mx != -INFINITY) {
        for (int w = 0; w < nw; ++w) {
            const float mw = s_m[w];
            const float ww = mw == -INFINITY ? 0.f : fast_exp2(mw - Mx);
            L = fmaf(ww, s_l[w], L);
#pragma unroll
            for (int n = 0; n < NL; ++n) out[n] = fmaf(ww, s_o[w][lane + 64 * n], out[n]);
        }
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
    for (int n = 0; n < NL; ++n) o[(size_t)bh * D + lane + 64 * n] = (bf16)(out[n] * inv);
    if (lane == 0) lse[bh] = Mx == -INFINITY ? -INFINITY : (Mx + log2f(L)) * kLn2;
}

}  // namespace dec

int decode_slices(int T_max) { return (T_max + dec::kPos - 1) / dec::kPos; }

// One launch when every wave has at most one slice, or when the heads alone
// spread over half the compute units or more.  Otherwise (few heads, long
// caches) one workgroup per head would leave most compute units idle and each
// streaming its whole cache; the split path spreads the slices over the
// machine and pays a second launch for the merge.
bool decode_two_launches(const DecodeArgs& a)
{
    const int nw = a.D == 128 ? 8 : 16;  // waves of a one-launch workgroup
    return !(decode_slices(a.T_max) <= nw || (long long)a.B * a.H * 2 >= a.n_cu);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t st)
{
    const int n_slice = decode_slices(a.T_max);
    const float sl2 = a.scale * kLog2e;
    const long long heads = (long long)a.B * a.H;
    if (!decode_two_launches(a)) {
        const dim3 grid((unsigned)heads);
        if (a.D == 128)
            hipLaunchKernelGGL((dec::decode_fused_kernel<2, 8>), grid, dim3(64 * min(8, n_slice)), 0, st,
                               (const bf16*)a.q, (const bf16*)a.k_cache, (const bf16*)a.v_cache, a.lens,
                               (bf16*)a.o, a.lse, a.H, a.T_max, n_slice, a.window, sl2);
        else
            hipLaunchKernelGGL((dec::decode_fused_kernel<1, 16>), grid, dim3(64 * min(16, n_slice)), 0, st,
                               (const bf16*)a.q, (const bf16*)a.k_cache, (const bf16*)a.v_cache, a.lens,
                               (bf16*)a.o, a.lse, a.H, a.T_max, n_slice, a.window, sl2);
        return hipGetLastError();
    }
    const dim3 grid_p((unsigned)(a.B * n_slice * a.H)), grid_c((unsigned)(a.B * a.H));
    if (a.D == 128) {
        hipLaunchKernelGGL(dec::decode_partial_kernel<2>, grid_p, dim3(64), 0, st, (const bf16*)a.q,
                           (const bf16*)a.k_cache, (const bf16*)a.v_cache, a.lens, a.part, a.H,
                           a.T_max, n_slice, a.window, sl2);
    } else {
        hipLaunchKernelGGL(dec::decode_partial_kernel<1>, grid_p, dim3(64), 0, st, (const bf16*)a.q,
                           (const bf16*)a.k_cache, (const bf16*)a.v_cache, a.lens, a.part, a.H,
                           a.T_max, n_slice, a.window, sl2);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.D == 128)
        hipLaunchKernelGGL(dec::decode_combine_kernel<2>, grid_c, dim3(64 * dec::kCW), 0, st, a.part,
                           (bf16*)a.o, a.lse, n_slice);
    else
        hipLaunchKernelGGL(dec::decode_combine_kernel<1>, grid_c, dim3(64 * dec::kCW), 0, st, a.part,
                           (bf16*)a.o, a.lse, n_slice);
    return hipGetLastError();
}

// The partials of attn_decode_noalloc, for callers that cannot allocate:
// [B][H][slices][D + 4] fp32 of the call, at most
// CAUSAL_ATTN_DECODE_SCRATCH_BYTES.  The name is a host-side stand-in for the
// array; kernels get the device address that hipGetSymbolAddress returns for
// the current device (each device holds its own copy).
static __device__ __align__(256) float scratch[CAUSAL_ATTN_DECODE_SCRATCH_BYTES / sizeof(float)];

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept; concurrent first calls store the same
// value.
static hipError_t scratch_address(float** out)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<float*> addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    float* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void* v = nullptr;
        e = hipGetSymbolAddress(&v, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (v == nullptr) return hipErrorInvalidSymbol;
        p = (float*)v;
        addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_decode_bf16_noalloc(DecodeArgs a, hipStream_t st)
{
    float* p = nullptr;
    const hipError_t e = scratch_address(&p);
    if (e != hipSuccess) return e;
    a.part = p;
    return launch_decode_bf16(a, st);
}

}  // namespace cattn

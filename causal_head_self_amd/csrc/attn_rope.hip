// attn_rope.hip -- RoPE and QK norm on the query and key rows of every head
// (forward and gradient), bf16 storage, fp32 arithmetic, gfx950.
//
// nanochat, section 9, lists RoPE position encoding and QK norm (x1.2) among
// the parts of its attention.  The forms used (the standard ones; the pages
// print no formulas):
//   RoPE: the column pair (i, i + D/2) of the row at position p = pos0 + t is
//         turned by the angle p * base^(-2i/D):
//           y_i = x_i cos - x_{i+D/2} sin,  y_{i+D/2} = x_i sin + x_{i+D/2} cos
//   QK norm: y = gain * y / sqrt(mean(x^2) + eps), no learned weight.
// Rotation keeps the root mean square, so the order of the two does not matter.
//
// Both passes read each row once and write it once, so they are bound by HBM
// bandwidth.  A group of 8 lanes owns one row; lane s holds columns
// [s*NE, s*NE + NE) and their partners [D/2 + s*NE, ...), NE = D/16, so each
// rotation pair sits in one lane and the row's sum of squares is one group sum
// (DPP).  Angles are kept in revolutions: position times base^(-2i/D) / (2 pi)
// is one fp64 multiply (the frequencies come from the host in fp64), its
// fractional part goes to fp32 and to the hardware sine and cosine, which take
// revolutions (v_sin_f32 / v_cos_f32).  The angle is then exact to about
// 1e-7 of a turn at any position below 2^24, at the cost of a few fp64 and
// two transcendental instructions per pair.
#include "attn_device.h"
#include "attn_kernels.h"

namespace cattn {
namespace rope {

constexpr int kThreads = 256;
constexpr int kRowsPerWG = kThreads / 8;

__device__ __forceinline__ float group8_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    return x;
}

template <int NE>
struct Vec;
template <>
struct Vec<4> {
    typedef bf16x4 T;
};
template <>
struct Vec<8> {
    typedef bf16x8 T;
};

struct RowView {
    bf16* p;
    long long sb, sh;
    int st;
};

__device__ __forceinline__ bf16* row_ptr(const RowView& v, int b, int h, int t)
{
    return v.p + (long long)b * v.sb + (long long)h * v.sh + (long long)t * v.st;
}

struct Pair {  // the two tensors of a launch (blockIdx.y = 0: queries, 1: keys)
    RowView x[2], y[2], g[2];
    float gain[2];
};

// y = gain * R(x) / rms(x)   (forward; y = R(x) without the norm), or
// dx = R^T (gain/rms dy - z gain/rms^3 mean(dy z)), z = R(x)   (gradient;
// dx = R^T dy without the norm).  R is the identity without RoPE.
template <int NE, bool kGrad>
__global__ __launch_bounds__(kThreads) void rope_qknorm_kernel(Pair a, RopeFreqs fr, int B, int H,
                                                               int T, int pos0, int flags,
                                                               float eps)
{
    typedef typename Vec<NE>::T V;
    constexpr int D = 16 * NE, HALF = D / 2;
    const int which = blockIdx.y;
    const int lane = threadIdx.x & 7;
    const long long row = (long long)blockIdx.x * kRowsPerWG + (threadIdx.x >> 3);
    if (row >= (long long)B * H * T) return;  // whole 8-lane groups leave together
    // rows in (b, t, h) order: neighbouring groups take the heads of one token,
    // which lie side by side in the fused [B][T][3][H][D] layout
    const int h = (int)(row % H);
    const long long bt = row / H;
    const int t = (int)(bt % T), b = (int)(bt / T);
    const bool use_rope = flags & 1, use_norm = flags & 2;
    const float gain = a.gain[which];

    const bf16* xr = row_ptr(a.x[which], b, h, t) + lane * NE;
    const V xlo = *(const V*)xr, xhi = *(const V*)(xr + HALF);
    float c[NE], s[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        c[e] = 1.f;
        s[e] = 0.f;
        if (use_rope) {
            const double r = (double)(pos0 + t) * fr.f[lane * NE + e];
            const float turn = (float)(r - floor(r));  // [0, 1)
            s[e] = __builtin_amdgcn_sinf(turn);
            c[e] = __builtin_amdgcn_cosf(turn);
        }
    }
    // z = R(x); the sum of squares of x (= that of z up to rounding) from x
    float zl[NE], zh[NE], ss = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const float u = (float)xlo[e], w = (float)xhi[e];
        zl[e] = u * c[e] - w * s[e];
        zh[e] = u * s[e] + w * c[e];
        ss = fmaf(u, u, fmaf(w, w, ss));
    }
    float inv = 1.f;  // 1 / rms
    if (use_norm) inv = 1.0f / sqrtf(group8_sum(ss) / (float)D + eps);

    if (!kGrad) {
        const float f = use_norm ? gain * inv : 1.f;  // the gain belongs to the norm
        V ylo, yhi;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            ylo[e] = (bf16)(f * zl[e]);
            yhi[e] = (bf16)(f * zh[e]);
        }
        bf16* yr = row_ptr(a.y[which], b, h, t) + lane * NE;
        *(V*)yr = ylo;
        *(V*)(yr + HALF) = yhi;
        return;
    }

    const bf16* gr = row_ptr(a.g[which], b, h, t) + lane * NE;
    const V glo = *(const V*)gr, ghi = *(const V*)(gr + HALF);
    float dl[NE], dh[NE];
    if (use_norm) {
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) m = fmaf((float)glo[e], zl[e], fmaf((float)ghi[e], zh[e], m));
        m = group8_sum(m) / (float)D;
        const float a1 = gain * inv, a3 = gain * inv * inv * inv * m;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            dl[e] = a1 * (float)glo[e] - a3 * zl[e];
            dh[e] = a1 * (float)ghi[e] - a3 * zh[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            dl[e] = (float)glo[e];
            dh[e] = (float)ghi[e];
        }
    }
    V olo, ohi;
#pragma unroll
    for (int e = 0; e < NE; ++e) {  // R^T
        olo[e] = (bf16)(dl[e] * c[e] + dh[e] * s[e]);
        ohi[e] = (bf16)(-dl[e] * s[e] + dh[e] * c[e]);
    }
    bf16* orow = row_ptr(a.y[which], b, h, t) + lane * NE;
    *(V*)orow = olo;
    *(V*)(orow + HALF) = ohi;
}

}  // namespace rope

static rope::RowView rview(const void* p, const Strides& s)
{
    return rope::RowView{(bf16*)p, s.sb, s.sh, s.st};
}

hipError_t launch_rope_qknorm(const RopeArgs& a, hipStream_t st)
{
    rope::Pair p{};
    p.x[0] = rview(a.q, a.sq);
    p.x[1] = rview(a.k, a.sk);
    p.y[0] = rview(a.q_out, a.sqo);
    p.y[1] = rview(a.k_out, a.sko);
    p.g[0] = rview(a.dq_in, a.sdq);
    p.g[1] = rview(a.dk_in, a.sdk);
    p.gain[0] = a.q_gain;
    p.gain[1] = a.k_gain;
    if (a.k_only) {  // the keys in slot 0, one launch row of workgroups
        p.x[0] = p.x[1];
        p.y[0] = p.y[1];
        p.g[0] = p.g[1];
        p.gain[0] = p.gain[1];
    }
    const long long rows = (long long)a.B * a.H * a.T;
    const dim3 grid((unsigned)((rows + rope::kRowsPerWG - 1) / rope::kRowsPerWG), a.k_only ? 1 : 2);
    const dim3 block(rope::kThreads);
    if (a.D == 128) {
        if (a.grad)
            hipLaunchKernelGGL((rope::rope_qknorm_kernel<8, true>), grid, block, 0, st, p, a.freqs,
                               a.B, a.H, a.T, a.pos0, a.flags, a.eps);
        else
            hipLaunchKernelGGL((rope::rope_qknorm_kernel<8, false>), grid, block, 0, st, p, a.freqs,
                               a.B, a.H, a.T, a.pos0, a.flags, a.eps);
    } else {
        if (a.grad)
            hipLaunchKernelGGL((rope::rope_qknorm_kernel<4, true>), grid, block, 0, st, p, a.freqs,
                               a.B, a.H, a.T, a.pos0, a.flags, a.eps);
        else
            hipLaunchKernelGGL((rope::rope_qknorm_kernel<4, false>), grid, block, 0, st, p, a.freqs,
                               a.B, a.H, a.T, a.pos0, a.flags, a.eps);
    }
    return hipGetLastError();
}

}  // namespace cattn

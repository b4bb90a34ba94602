// attn_api.hip -- the C ABI declared in include/causal_attn.h: argument
// validation (all of it before any HIP call) and dispatch to the kernels.
#include <atomic>
#include <math.h>
#include <stdint.h>

#include "../../include/causal_attn.h"
#include "attn_kernels.h"

namespace {

struct Buf {
    const void* p;
    bool row_tensor;  // [B][H][T] fp32 (lse, delta) instead of [B][H][T][D]
};

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

// Head dims with kernels: 32 and 64 in both dtypes, 128 in bf16.
bool head_dim_ok(int D, int dtype) { return D == 32 || D == 64 || (D == 128 && dtype == ATTN_BF16); }

// Checks shared by every entry point, in the documented order:
// NULL, shape, dtype, D, scale, overflow, alignment, aliasing.
template <int NI, int NO>
int validate(const Buf (&in)[NI], const Buf (&out)[NO], int B, int H, int T, int D, float scale,
             int dtype)
{
    for (const Buf& b : in)
        if (!b.p) return ATTN_ERR_NULL;
    for (const Buf& b : out)
        if (!b.p) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || T < 1) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (!head_dim_ok(D, dtype)) return ATTN_ERR_UNSUPPORTED_D;
    if (!isfinite(scale) || !(scale > 0.0f)) return ATTN_ERR_SCALE;
    const long long BH = (long long)B * H;
    const long long tiles = (T + 63) / 64;  // the finest row tiling any kernel launches
    if ((long long)T * D > 0x7fffffffLL || BH * tiles > 0x7fffffffLL ||
        BH * (long long)T > (1LL << 35))
        return ATTN_ERR_OVERFLOW;
    for (const Buf& b : in)
        if ((uintptr_t)b.p % (b.row_tensor ? 4 : 16)) return ATTN_ERR_ALIGN;
    for (const Buf& b : out)
        if ((uintptr_t)b.p % (b.row_tensor ? 4 : 16)) return ATTN_ERR_ALIGN;
    const size_t rows = (size_t)BH * T;
    const size_t tensor_bytes = rows * D * (dtype == ATTN_BF16 ? 2 : 4);
    auto span = [&](const Buf& b) {
        const uintptr_t lo = (uintptr_t)b.p;
        return Span{lo, lo + (b.row_tensor ? rows * sizeof(float) : tensor_bytes)};
    };
    for (int i = 0; i < NO; ++i) {
        for (int j = 0; j < NI; ++j)
            if (overlaps(span(out[i]), span(in[j]))) return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < NO; ++j)
            if (overlaps(span(out[i]), span(out[j]))) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

// Compute units of the current device, queried once per device (callers on
// several threads may race to fill the cache; they store the same value).
int cu_count()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int c = cached[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
        c = n > 0 ? n : -1;
        cached[dev].store(c, std::memory_order_relaxed);
    }
    return c > 0 ? c : 0;
}

cattn::AttnArgs make_args(int B, int H, int T, int D, float scale)
{
    cattn::AttnArgs a{};
    a.n_cu = cu_count();
    a.window = 0;
    const cattn::Strides c{(long long)H * T * D, (long long)T * D, D};
    a.sq = a.sk = a.sv = a.so = a.sdo = a.sdq = a.sdk = a.sdv = c;
    a.B = B;
    a.H = H;
    a.T = T;
    a.D = D;
    a.scale = scale;
    return a;
}

int status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// ---- strided views ----------------------------------------------------------

struct VSpan {
    const attn_view_t* v;
    bool output;
};

// Elements a view can touch: [lo, hi) relative to its data pointer.
long long view_extent(const attn_view_t& v, int B, int H, int T, int D)
{
    return (long long)(B - 1) * v.stride_b + (long long)(H - 1) * v.stride_h +
           (long long)(T - 1) * v.stride_t + D;
}

// Conservative disjointness test of two views of one element size (bytes es).
bool views_disjoint(const attn_view_t& a, const attn_view_t& b, int B, int H, int T, int D, int es)
{
    const uintptr_t alo = (uintptr_t)a.data, ahi = alo + (uintptr_t)view_extent(a, B, H, T, D) * es;
    const uintptr_t blo = (uintptr_t)b.data, bhi = blo + (uintptr_t)view_extent(b, B, H, T, D) * es;
    if (ahi <= blo || bhi <= alo) return true;
    // intersecting ranges: accept translates of one lattice whose token footprints
    // do not meet modulo stride_t
    if (a.stride_b != b.stride_b || a.stride_h != b.stride_h || a.stride_t != b.stride_t)
        return false;
    const long long st = a.stride_t;
    if (st <= 0 || a.stride_b % st != 0) return false;
    const long long w = (long long)(H - 1) * a.stride_h + D;  // footprint of one token
    const long long diff = (long long)((intptr_t)blo - (intptr_t)alo);
    if (diff % es != 0) return false;
    const long long r = (((diff / es) % st) + st) % st;
    return r >= w && st - r >= w;
}

// True when the (b, h, t, d) elements of a view address distinct memory: taken
// in order of increasing stride (the D columns have stride 1; dimensions of
// size 1 do not count), every stride must exceed the span of the dimensions
// before it.  An output that fails this would have several lanes write one
// element.
bool view_is_injective(const attn_view_t& v, int B, int H, int T, int D)
{
    long long st[3] = {v.stride_t, v.stride_h, v.stride_b};
    long long sz[3] = {T, H, B};
    for (int i = 0; i < 3; ++i)  // sort by stride (three elements)
        for (int j = i + 1; j < 3; ++j)
            if (st[j] < st[i]) {
                const long long a = st[i], b = sz[i];
                st[i] = st[j];
                sz[i] = sz[j];
                st[j] = a;
                sz[j] = b;
            }
    long long span = D;  // elements spanned by the dimensions taken so far
    for (int i = 0; i < 3; ++i) {
        if (sz[i] <= 1) continue;
        if (st[i] < span) return false;
        span = st[i] * (sz[i] - 1) + span;
    }
    return true;
}

int validate_views(const VSpan* vs, int n, const float* const* rows, int nrows, int B, int H,
                   int T, int D, float scale, int dtype)
{
    for (int i = 0; i < n; ++i)
        if (!vs[i].v->data) return ATTN_ERR_NULL;
    for (int i = 0; i < nrows; ++i)
        if (!rows[i]) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || T < 1) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (!head_dim_ok(D, dtype)) return ATTN_ERR_UNSUPPORTED_D;
    if (!isfinite(scale) || !(scale > 0.0f)) return ATTN_ERR_SCALE;
    if (dtype != ATTN_BF16 || (D != 64 && D != 128)) return ATTN_ERR_LAYOUT;
    const long long BH = (long long)B * H;
    if ((long long)T * D > 0x7fffffffLL || BH * ((T + 63) / 64) > 0x7fffffffLL ||
        BH * (long long)T > (1LL << 35))
        return ATTN_ERR_OVERFLOW;
    for (int i = 0; i < n; ++i) {
        const attn_view_t& v = *vs[i].v;
        if (v.stride_b < 0 || v.stride_h < 0 || v.stride_t < D || v.stride_b % 8 ||
            v.stride_h % 8 || v.stride_t % 8 || (long long)T * v.stride_t * 2 >= (1LL << 32))
            return ATTN_ERR_LAYOUT;
    }
    for (int i = 0; i < n; ++i)
        if ((uintptr_t)vs[i].v->data % 16) return ATTN_ERR_ALIGN;
    for (int i = 0; i < nrows; ++i)
        if ((uintptr_t)rows[i] % 4) return ATTN_ERR_ALIGN;
    // aliasing: outputs against themselves and against everything (views and row tensors)
    const size_t row_bytes = (size_t)BH * T * sizeof(float);
    for (int i = 0; i < n; ++i) {
        if (!vs[i].output) continue;
        if (!view_is_injective(*vs[i].v, B, H, T, D)) return ATTN_ERR_ALIAS;
        for (int j = 0; j < n; ++j)
            if (j != i && !(vs[j].output && j < i) &&
                !views_disjoint(*vs[i].v, *vs[j].v, B, H, T, D, 2))
                return ATTN_ERR_ALIAS;
        const uintptr_t lo = (uintptr_t)vs[i].v->data;
        const uintptr_t hi = lo + (uintptr_t)view_extent(*vs[i].v, B, H, T, D) * 2;
        for (int j = 0; j < nrows; ++j) {
            const uintptr_t rlo = (uintptr_t)rows[j], rhi = rlo + row_bytes;
            if (lo < rhi && rlo < hi) return ATTN_ERR_ALIAS;
        }
    }
    return ATTN_OK;
}

// round(p * 65536) for a dropout probability 0 <= p < 1, capped at 65535;
// -1 for anything else.
int dropout_threshold(float p)
{
    if (!isfinite(p) || p < 0.0f || !(p < 1.0f)) return -1;
    const double t = floor((double)p * 65536.0 + 0.5);
    return t > 65535.0 ? 65535 : (int)t;
}

cattn::Strides strides_of(const attn_view_t& v)
{
    return cattn::Strides{v.stride_b, v.stride_h, (int)v.stride_t};
}

}  // namespace

namespace {

int rope_params_ok(int T, int pos0, float base, float q_gain, float k_gain, float eps, int flags)
{
    if (flags < 0 || flags > 3 || pos0 < 0 || (long long)pos0 + T > (1LL << 24)) return 0;
    if ((flags & ATTN_ROPE) && (!isfinite(base) || !(base > 0.0f))) return 0;
    if (!isfinite(q_gain) || !isfinite(k_gain) || !isfinite(eps) || eps < 0.0f) return 0;
    return 1;
}

cattn::RopeArgs rope_args(int B, int H, int T, int D, int pos0, float base, float q_gain,
                          float k_gain, float eps, int flags, bool grad)
{
    cattn::RopeArgs a{};
    a.B = B;
    a.H = H;
    a.T = T;
    a.D = D;
    a.pos0 = pos0;
    a.flags = flags;
    a.q_gain = q_gain;
    a.k_gain = k_gain;
    a.eps = eps;
    a.grad = grad;
    for (int i = 0; i < D / 2; ++i)  // revolutions per position, base^(-2i/D) / (2 pi)
        a.freqs.f[i] = pow((double)base, -2.0 * (double)i / (double)D) / 6.283185307179586;
    return a;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return CAUSAL_ATTN_ABI_VERSION; }

const char* attn_status_str(int st)
{
    switch (st) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE:
        return "B, H and T must be >= 1 (LayerNorm / column sums: N >= 1, 8 <= C <= 4096 and "
               "M >= 8, multiples of 8)";
    case ATTN_ERR_UNSUPPORTED_D: return "head dim D must be 32 or 64 (or 128 with bf16)";
    case ATTN_ERR_DTYPE: return "dtype must be ATTN_F32 or ATTN_BF16";
    case ATTN_ERR_ALIGN: return "tensors must be 16-byte aligned (lse/delta 4-byte)";
    case ATTN_ERR_OVERFLOW: return "T*D or the launch grid exceeds 2^31 - 1";
    case ATTN_ERR_SCALE: return "scale must be finite and > 0";
    case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
    case ATTN_ERR_HIP: return "HIP kernel launch failed";
    case ATTN_ERR_LAYOUT:
        return "strided views need bf16, D = 64 or 128, strides that are non-negative multiples of 8 "
               "with stride_t >= D, and T * stride_t * 2 < 2^32 (row passes: stride >= C, a "
               "multiple of 8)";
    case ATTN_ERR_WORKSPACE:
        return "workspace smaller than the entry point's *_workspace_bytes() (attn_decode, "
               "attn_layernorm_bwd, attn_colsum)";
    case ATTN_ERR_PARAM:
        return "RoPE / QK norm: flags must be 0..3, 0 <= pos0 and pos0 + T <= 2^24, rope_base "
               "finite and > 0, gains finite, eps finite and >= 0; dropout_p must be in [0, 1); "
               "LayerNorm eps finite and >= 0";
    case ATTN_ERR_SCRATCH:
        return "attn_decode_noalloc: the two-launch path would need more than the library's "
               "fixed scratch (CAUSAL_ATTN_DECODE_SCRATCH_BYTES); use attn_decode with a workspace";
    default: return "unknown status";
    }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int T, int D, float scale, int dtype, void* stream)
{
    const Buf in[3] = {{q, false}, {k, false}, {v, false}};
    const Buf out[2] = {{o, false}, {lse, true}};
    const int st = validate(in, out, B, H, T, D, scale, dtype);
    if (st != ATTN_OK) return st;
    cattn::AttnArgs a = make_args(B, H, T, D, scale);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.o_out = o;
    a.lse = lse;
    hipStream_t s = (hipStream_t)stream;
    return status(dtype == ATTN_BF16 ? cattn::launch_fwd_bf16(a, s) : cattn::launch_fwd_f32(a, s));
}

int attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                const float* lse, float* delta, void* dq, int B, int H, int T, int D, float scale,
                int dtype, void* stream)
{
    const Buf in[6] = {{q, false}, {k, false}, {v, false}, {o, false}, {dO, false}, {lse, true}};
    const Buf out[2] = {{delta, true}, {dq, false}};
    const int st = validate(in, out, B, H, T, D, scale, dtype);
    if (st != ATTN_OK) return st;
    cattn::AttnArgs a = make_args(B, H, T, D, scale);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dO = dO;
    a.lse = const_cast<float*>(lse);
    a.delta = delta;
    a.dq = dq;
    hipStream_t s = (hipStream_t)stream;
    return status(dtype == ATTN_BF16 ? cattn::launch_dq_bf16(a, s) : cattn::launch_dq_f32(a, s));
}

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                  const float* delta, void* dk, void* dv, int B, int H, int T, int D,
                  float scale, int dtype, void* stream)
{
    const Buf in[6] = {{q, false}, {k, false}, {v, false}, {dO, false}, {lse, true},
                       {delta, true}};
    const Buf out[2] = {{dk, false}, {dv, false}};
    const int st = validate(in, out, B, H, T, D, scale, dtype);
    if (st != ATTN_OK) return st;
    cattn::AttnArgs a = make_args(B, H, T, D, scale);
    a.q = q;
    a.k = k;
    a.v = v;
    a.dO = dO;
    a.lse = const_cast<float*>(lse);
    a.delta = const_cast<float*>(delta);
    a.dk = dk;
    a.dv = dv;
    hipStream_t s = (hipStream_t)stream;
    return status(dtype == ATTN_BF16 ? cattn::launch_dkdv_bf16(a, s)
                                     : cattn::launch_dkdv_f32(a, s));
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dO, void* dq, void* dk, void* dv, float* delta, int B, int H, int T,
             int D, float scale, int dtype, void* stream)
{
    const Buf in[6] = {{q, false}, {k, false}, {v, false}, {o, false}, {dO, false}, {lse, true}};
    const Buf out[4] = {{dq, false}, {dk, false}, {dv, false}, {delta, true}};
    const int st = validate(in, out, B, H, T, D, scale, dtype);
    if (st != ATTN_OK) return st;
    cattn::AttnArgs a = make_args(B, H, T, D, scale);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dO = dO;
    a.lse = const_cast<float*>(lse);
    a.delta = delta;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == ATTN_BF16) return status(cattn::launch_bwd_bf16(a, s));
    hipError_t e = cattn::launch_dq_f32(a, s);
    if (e == hipSuccess) e = cattn::launch_dkdv_f32(a, s);
    return status(e);
}

// Argument checks of the strided forward (in the documented order).
static int fwd_strided_check(const attn_view_t& q, const attn_view_t& k, const attn_view_t& v,
                             const attn_view_t& o, const float* lse, int B, int H, int T, int D,
                             int window, float dropout_p, float scale, int dtype)
{
    const VSpan vs[4] = {{&q, false}, {&k, false}, {&v, false}, {&o, true}};
    const float* rows[1] = {lse};
    int st = validate_views(vs, 4, rows, 1, B, H, T, D, scale, dtype);
    if (st != ATTN_OK) return st;
    if (window < 0) return ATTN_ERR_SHAPE;
    if (dropout_threshold(dropout_p) < 0) return ATTN_ERR_PARAM;
    // lse (an output) must not overlap an input view either
    const uintptr_t rlo = (uintptr_t)lse, rhi = rlo + (size_t)B * H * T * sizeof(float);
    for (int i = 0; i < 3; ++i) {
        const uintptr_t lo = (uintptr_t)vs[i].v->data;
        const uintptr_t hi = lo + (uintptr_t)view_extent(*vs[i].v, B, H, T, D) * 2;
        if (lo < rhi && rlo < hi) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

static int fwd_strided(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o, float* lse,
                       int B, int H, int T, int D, int window, float dropout_p,
                       unsigned long long seed, float scale, int dtype, unsigned int* keep,
                       void* stream)
{
    const int st = fwd_strided_check(q, k, v, o, lse, B, H, T, D, window, dropout_p, scale, dtype);
    if (st != ATTN_OK) return st;
    const int p16 = dropout_threshold(dropout_p);
    cattn::AttnArgs a = make_args(B, H, T, D, scale);
    a.q = q.data;
    a.k = k.data;
    a.v = v.data;
    a.o = o.data;
    a.o_out = o.data;
    a.lse = lse;
    a.sq = strides_of(q);
    a.sk = strides_of(k);
    a.sv = strides_of(v);
    a.so = strides_of(o);
    a.window = window;
    a.dropout_p16 = p16;
    a.dropout_seed = seed;
    a.keep = keep;
    return status(cattn::launch_fwd_bf16(a, (hipStream_t)stream));
}

// Argument checks of the strided backward (in the documented order).
static int bwd_strided_check(const attn_view_t& q, const attn_view_t& k, const attn_view_t& v,
                             const attn_view_t& o, const float* lse, const attn_view_t& dO,
                             const attn_view_t& dq, const attn_view_t& dk, const attn_view_t& dv,
                             const float* delta, int B, int H, int T, int D, int window,
                             float dropout_p, float scale, int dtype)
{
    const VSpan vs[8] = {{&q, false}, {&k, false}, {&v, false}, {&o, false},
                         {&dO, false}, {&dq, true}, {&dk, true}, {&dv, true}};
    const float* rows[2] = {lse, delta};
    int st = validate_views(vs, 8, rows, 2, B, H, T, D, scale, dtype);
    if (st != ATTN_OK) return st;
    if (window < 0) return ATTN_ERR_SHAPE;
    if (dropout_threshold(dropout_p) < 0) return ATTN_ERR_PARAM;
    // delta (an output) must not overlap lse or an input view
    const size_t rb = (size_t)B * H * T * sizeof(float);
    const uintptr_t dlo = (uintptr_t)delta, dhi = dlo + rb;
    if (dlo < (uintptr_t)lse + rb && (uintptr_t)lse < dhi) return ATTN_ERR_ALIAS;
    for (int i = 0; i < 5; ++i) {
        const uintptr_t lo = (uintptr_t)vs[i].v->data;
        const uintptr_t hi = lo + (uintptr_t)view_extent(*vs[i].v, B, H, T, D) * 2;
        if (lo < dhi && dlo < hi) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

static int bwd_strided(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o,
                       const float* lse, attn_view_t dO, attn_view_t dq, attn_view_t dk,
                       attn_view_t dv, float* delta, int B, int H, int T, int D, int window,
                       float dropout_p, unsigned long long seed, float scale, int dtype,
                       const unsigned int* keep, void* stream)
{
    const int st = bwd_strided_check(q, k, v, o, lse, dO, dq, dk, dv, delta, B, H, T, D, window,
                                     dropout_p, scale, dtype);
    if (st != ATTN_OK) return st;
    const int p16 = dropout_threshold(dropout_p);
    cattn::AttnArgs a = make_args(B, H, T, D, scale);
    a.q = q.data;
    a.k = k.data;
    a.v = v.data;
    a.o = o.data;
    a.dO = dO.data;
    a.lse = const_cast<float*>(lse);
    a.delta = delta;
    a.dq = dq.data;
    a.dk = dk.data;
    a.dv = dv.data;
    a.sq = strides_of(q);
    a.sk = strides_of(k);
    a.sv = strides_of(v);
    a.so = strides_of(o);
    a.sdo = strides_of(dO);
    a.sdq = strides_of(dq);
    a.sdk = strides_of(dk);
    a.sdv = strides_of(dv);
    a.window = window;
    a.dropout_p16 = p16;
    a.dropout_seed = seed;
    a.keep = const_cast<unsigned int*>(keep);
    return status(cattn::launch_bwd_bf16(a, (hipStream_t)stream));
}

int attn_fwd_strided(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o, float* lse,
                     int B, int H, int T, int D, int window, float dropout_p,
                     unsigned long long seed, float scale, int dtype, void* stream)
{
    return fwd_strided(q, k, v, o, lse, B, H, T, D, window, dropout_p, seed, scale, dtype, nullptr,
                       stream);
}

int attn_bwd_strided(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o,
                     const float* lse, attn_view_t dO, attn_view_t dq, attn_view_t dk,
                     attn_view_t dv, float* delta, int B, int H, int T, int D, int window,
                     float dropout_p, unsigned long long seed, float scale, int dtype,
                     void* stream)
{
    return bwd_strided(q, k, v, o, lse, dO, dq, dk, dv, delta, B, H, T, D, window, dropout_p, seed,
                       scale, dtype, nullptr, stream);
}

size_t attn_dropout_keep_bytes(int B, int H, int T)
{
    if (B < 1 || H < 1 || T < 1) return 0;
    return (size_t)B * H * (size_t)((T + 31) / 32) * T * sizeof(unsigned int);
}

// The keep-bit buffer: present, aligned, large enough, and apart from every
// other buffer of the call (views given with their element extents).
static int check_keep(const void* keep, size_t keep_bytes, int B, int H, int T, int D,
                      const attn_view_t* const* views, int n_views, const float* const* rows,
                      int n_rows)
{
    if (!keep) return ATTN_ERR_NULL;
    if ((uintptr_t)keep % 4) return ATTN_ERR_ALIGN;
    const size_t need = attn_dropout_keep_bytes(B, H, T);
    if (keep_bytes < need) return ATTN_ERR_WORKSPACE;
    const uintptr_t klo = (uintptr_t)keep, khi = klo + need;
    for (int i = 0; i < n_views; ++i) {
        const uintptr_t lo = (uintptr_t)views[i]->data;
        const uintptr_t hi = lo + (uintptr_t)view_extent(*views[i], B, H, T, D) * 2;
        if (lo < khi && klo < hi) return ATTN_ERR_ALIAS;
    }
    const size_t rb = (size_t)B * H * T * sizeof(float);
    for (int i = 0; i < n_rows; ++i)
        if ((uintptr_t)rows[i] < khi && klo < (uintptr_t)rows[i] + rb) return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

int attn_fwd_strided_keep(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o, float* lse,
                          int B, int H, int T, int D, int window, float dropout_p,
                          unsigned long long seed, float scale, int dtype, unsigned int* keep,
                          size_t keep_bytes, void* stream)
{
    // the checks of attn_fwd_strided first, then those of the keep buffer
    const int st = fwd_strided_check(q, k, v, o, lse, B, H, T, D, window, dropout_p, scale, dtype);
    if (st != ATTN_OK) return st;
    const attn_view_t* views[4] = {&q, &k, &v, &o};
    const float* rows[1] = {lse};
    const int ks = check_keep(keep, keep_bytes, B, H, T, D, views, 4, rows, 1);
    if (ks != ATTN_OK) return ks;
    return fwd_strided(q, k, v, o, lse, B, H, T, D, window, dropout_p, seed, scale, dtype, keep,
                       stream);
}

int attn_bwd_strided_keep(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o,
                          const float* lse, attn_view_t dO, attn_view_t dq, attn_view_t dk,
                          attn_view_t dv, float* delta, int B, int H, int T, int D, int window,
                          float dropout_p, float scale, int dtype, const unsigned int* keep,
                          size_t keep_bytes, void* stream)
{
    const int st = bwd_strided_check(q, k, v, o, lse, dO, dq, dk, dv, delta, B, H, T, D, window,
                                     dropout_p, scale, dtype);
    if (st != ATTN_OK) return st;
    const attn_view_t* views[8] = {&q, &k, &v, &o, &dO, &dq, &dk, &dv};
    const float* rows[2] = {lse, delta};
    const int ks = check_keep(keep, keep_bytes, B, H, T, D, views, 8, rows, 2);
    if (ks != ATTN_OK) return ks;
    return bwd_strided(q, k, v, o, lse, dO, dq, dk, dv, delta, B, H, T, D, window, dropout_p, 0,
                       scale, dtype, keep, stream);
}

// The prologue parameters of the fused entry points, as for attn_rope_qknorm_*.
static void set_rope(cattn::AttnArgs& a, int pos0, float base, float q_gain, float k_gain,
                     float eps, int flags)
{
    const cattn::RopeArgs r = rope_args(a.B, a.H, a.T, a.D, pos0, base, q_gain, k_gain, eps, flags,
                                        false);
    a.rope = true;
    a.pos0 = pos0;
    a.rope_flags = flags;
    a.q_gain = q_gain;
    a.k_gain = k_gain;
    a.rope_eps = eps;
    a.freqs = r.freqs;
}

int attn_fwd_strided_rope(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o, float* lse,
                          attn_view_t q_rot, attn_view_t k_rot, int B, int H, int T, int D,
                          int window, float scale, int pos0, float rope_base, float q_gain,
                          float k_gain, float eps, int flags, int dtype, void* stream)
{
    const VSpan vs[6] = {{&q, false}, {&k, false}, {&v, false},
                         {&o, true},  {&q_rot, true}, {&k_rot, true}};
    const float* rows[1] = {lse};
    int st = validate_views(vs, 6, rows, 1, B, H, T, D, scale, dtype);
    if (st != ATTN_OK) return st;
    if (window < 0) return ATTN_ERR_SHAPE;
    if (!rope_params_ok(T, pos0, rope_base, q_gain, k_gain, eps, flags)) return ATTN_ERR_PARAM;
    const uintptr_t rlo = (uintptr_t)lse, rhi = rlo + (size_t)B * H * T * sizeof(float);
    for (int i = 0; i < 3; ++i) {  // lse (an output) apart from the inputs
        const uintptr_t lo = (uintptr_t)vs[i].v->data;
        const uintptr_t hi = lo + (uintptr_t)view_extent(*vs[i].v, B, H, T, D) * 2;
        if (lo < rhi && rlo < hi) return ATTN_ERR_ALIAS;
    }
    cattn::AttnArgs a = make_args(B, H, T, D, scale);
    a.q = q.data;
    a.k = k.data;
    a.v = v.data;
    a.o = o.data;
    a.o_out = o.data;
    a.lse = lse;
    a.sq = strides_of(q);
    a.sk = strides_of(k);
    a.sv = strides_of(v);
    a.so = strides_of(o);
    a.q_rot = q_rot.data;
    a.k_rot = k_rot.data;
    a.sqr = strides_of(q_rot);
    a.skr = strides_of(k_rot);
    a.window = window;
    set_rope(a, pos0, rope_base, q_gain, k_gain, eps, flags);
    return status(cattn::launch_fwd_bf16(a, (hipStream_t)stream));
}

int attn_bwd_strided_rope(attn_view_t q, attn_view_t k, attn_view_t q_rot, attn_view_t k_rot,
                          attn_view_t v, attn_view_t o, const float* lse, attn_view_t dO,
                          attn_view_t dq, attn_view_t dk, attn_view_t dv, float* delta, int B,
                          int H, int T, int D, int window, float scale, int pos0, float rope_base,
                          float q_gain, float k_gain, float eps, int flags, int dtype, void* stream)
{
    const VSpan vs[10] = {{&q, false},  {&k, false},  {&q_rot, false}, {&k_rot, false},
                          {&v, false},  {&o, false},  {&dO, false},    {&dq, true},
                          {&dk, true},  {&dv, true}};
    const float* rows[2] = {lse, delta};
    int st = validate_views(vs, 10, rows, 2, B, H, T, D, scale, dtype);
    if (st != ATTN_OK) return st;
    if (window < 0) return ATTN_ERR_SHAPE;
    if (!rope_params_ok(T, pos0, rope_base, q_gain, k_gain, eps, flags)) return ATTN_ERR_PARAM;
    const size_t rb = (size_t)B * H * T * sizeof(float);
    const uintptr_t dlo = (uintptr_t)delta, dhi = dlo + rb;  // delta (an output) apart from inputs
    if (dlo < (uintptr_t)lse + rb && (uintptr_t)lse < dhi) return ATTN_ERR_ALIAS;
    for (int i = 0; i < 7; ++i) {
        const uintptr_t lo = (uintptr_t)vs[i].v->data;
        const uintptr_t hi = lo + (uintptr_t)view_extent(*vs[i].v, B, H, T, D) * 2;
        if (lo < dhi && dlo < hi) return ATTN_ERR_ALIAS;
    }
    cattn::AttnArgs a = make_args(B, H, T, D, scale);
    a.q = q_rot.data;  // the attention runs on the rows after the prologue
    a.k = k_rot.data;
    a.v = v.data;
    a.o = o.data;
    a.dO = dO.data;
    a.lse = const_cast<float*>(lse);
    a.delta = delta;
    a.dq = dq.data;
    a.dk = dk.data;
    a.dv = dv.data;
    a.sq = strides_of(q_rot);
    a.sk = strides_of(k_rot);
    a.sv = strides_of(v);
    a.so = strides_of(o);
    a.sdo = strides_of(dO);
    a.sdq = strides_of(dq);
    a.sdk = strides_of(dk);
    a.sdv = strides_of(dv);
    a.xq = q.data;
    a.xk = k.data;
    a.sxq = strides_of(q);
    a.sxk = strides_of(k);
    a.window = window;
    set_rope(a, pos0, rope_base, q_gain, k_gain, eps, flags);
    return status(cattn::launch_bwd_bf16(a, (hipStream_t)stream));
}

size_t attn_decode_workspace_bytes(int B, int H, int T_max, int D)
{
    if (B < 1 || H < 1 || T_max < 1 || D < 1) return 0;
    return (size_t)B * H * cattn::decode_slices(T_max) * (size_t)(D + 4) * sizeof(float);
}

// Argument checks of attn_decode (in the documented order); workspace == nullptr
// with check_workspace false: those of attn_decode_noalloc.
static int decode_check(const void* q, const void* k_cache, const void* v_cache,
                        const int* cache_lens, const void* o, const float* lse,
                        const void* workspace, size_t workspace_bytes, bool check_workspace,
                        int B, int H, int T_max, int D, int window, float scale, int dtype)
{
    if (!q || !k_cache || !v_cache || !cache_lens || !o || !lse || (check_workspace && !workspace))
        return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || T_max < 1 || window < 0) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED_D;
    if (!isfinite(scale) || !(scale > 0.0f)) return ATTN_ERR_SCALE;
    const long long slices = cattn::decode_slices(T_max);
    if ((long long)B * H * slices > 0x7fffffffLL || (long long)B * T_max * H * D > (1LL << 40))
        return ATTN_ERR_OVERFLOW;
    for (const void* p : {q, k_cache, v_cache, o})
        if ((uintptr_t)p % 16) return ATTN_ERR_ALIGN;
    if (check_workspace && (uintptr_t)workspace % 16) return ATTN_ERR_ALIGN;
    if ((uintptr_t)lse % 4 || (uintptr_t)cache_lens % 4) return ATTN_ERR_ALIGN;
    const size_t need = attn_decode_workspace_bytes(B, H, T_max, D);
    if (check_workspace && workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    const size_t bh = (size_t)B * H;
    const size_t cache = (size_t)B * T_max * H * D * 2;
    auto span = [](const void* p, size_t n) {
        return Span{(uintptr_t)p, (uintptr_t)p + n};
    };
    const Span in[4] = {span(q, bh * D * 2), span(k_cache, cache), span(v_cache, cache),
                        span(cache_lens, (size_t)B * 4)};
    const Span out[3] = {span(o, bh * D * 2), span(lse, bh * 4), span(workspace, need)};
    const int n_out = check_workspace ? 3 : 2;
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < 4; ++j)
            if (overlaps(out[i], in[j])) return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(out[i], out[j])) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

static cattn::DecodeArgs decode_args(const void* q, const void* k_cache, const void* v_cache,
                                     const int* cache_lens, void* o, float* lse, int B, int H,
                                     int T_max, int D, int window, float scale)
{
    cattn::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.lens = cache_lens;
    a.o = o;
    a.lse = lse;
    a.part = nullptr;
    a.B = B;
    a.H = H;
    a.T_max = T_max;
    a.D = D;
    a.window = window;
    a.scale = scale;
    a.n_cu = cu_count();
    return a;
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int* cache_lens,
                void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int H,
                int T_max, int D, int window, float scale, int dtype, void* stream)
{
    const int st = decode_check(q, k_cache, v_cache, cache_lens, o, lse, workspace,
                                workspace_bytes, true, B, H, T_max, D, window, scale, dtype);
    if (st != ATTN_OK) return st;
    cattn::DecodeArgs a =
        decode_args(q, k_cache, v_cache, cache_lens, o, lse, B, H, T_max, D, window, scale);
    a.part = (float*)workspace;
    return status(cattn::launch_decode_bf16(a, (hipStream_t)stream));
}

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int* cache_lens, void* o, float* lse, int B, int H, int T_max,
                        int D, int window, float scale, int dtype, void* stream)
{
    const int st = decode_check(q, k_cache, v_cache, cache_lens, o, lse, nullptr, 0, false, B, H,
                                T_max, D, window, scale, dtype);
    if (st != ATTN_OK) return st;
    const cattn::DecodeArgs a =
        decode_args(q, k_cache, v_cache, cache_lens, o, lse, B, H, T_max, D, window, scale);
    if (cattn::decode_two_launches(a) &&
        attn_decode_workspace_bytes(B, H, T_max, D) > CAUSAL_ATTN_DECODE_SCRATCH_BYTES)
        return ATTN_ERR_SCRATCH;
    return status(cattn::launch_decode_bf16_noalloc(a, (hipStream_t)stream));
}

int attn_rope_qknorm_fwd(attn_view_t q, attn_view_t k, attn_view_t q_out, attn_view_t k_out,
                         int B, int H, int T, int D, int pos0, float rope_base, float q_gain,
                         float k_gain, float eps, int flags, int dtype, void* stream)
{
    const VSpan vs[4] = {{&q, false}, {&k, false}, {&q_out, true}, {&k_out, true}};
    int st = validate_views(vs, 4, nullptr, 0, B, H, T, D, 1.0f, dtype);
    if (st != ATTN_OK) return st;
    if (!rope_params_ok(T, pos0, rope_base, q_gain, k_gain, eps, flags)) return ATTN_ERR_PARAM;
    cattn::RopeArgs a = rope_args(B, H, T, D, pos0, rope_base, q_gain, k_gain, eps, flags, false);
    a.q = q.data;
    a.k = k.data;
    a.q_out = q_out.data;
    a.k_out = k_out.data;
    a.dq_in = q.data;  // unused by the forward
    a.dk_in = k.data;
    a.sq = strides_of(q);
    a.sk = strides_of(k);
    a.sqo = strides_of(q_out);
    a.sko = strides_of(k_out);
    a.sdq = a.sq;
    a.sdk = a.sk;
    return status(cattn::launch_rope_qknorm(a, (hipStream_t)stream));
}

int attn_rope_qknorm_bwd(attn_view_t q, attn_view_t k, attn_view_t dq_out, attn_view_t dk_out,
                         attn_view_t dq, attn_view_t dk, int B, int H, int T, int D, int pos0,
                         float rope_base, float q_gain, float k_gain, float eps, int flags,
                         int dtype, void* stream)
{
    const VSpan vs[6] = {{&q, false}, {&k, false}, {&dq_out, false}, {&dk_out, false},
                         {&dq, true}, {&dk, true}};
    int st = validate_views(vs, 6, nullptr, 0, B, H, T, D, 1.0f, dtype);
    if (st != ATTN_OK) return st;
    if (!rope_params_ok(T, pos0, rope_base, q_gain, k_gain, eps, flags)) return ATTN_ERR_PARAM;
    cattn::RopeArgs a = rope_args(B, H, T, D, pos0, rope_base, q_gain, k_gain, eps, flags, true);
    a.q = q.data;
    a.k = k.data;
    a.q_out = dq.data;
    a.k_out = dk.data;
    a.dq_in = dq_out.data;
    a.dk_in = dk_out.data;
    a.sq = strides_of(q);
    a.sk = strides_of(k);
    a.sqo = strides_of(dq);
    a.sko = strides_of(dk);
    a.sdq = strides_of(dq_out);
    a.sdk = strides_of(dk_out);
    return status(cattn::launch_rope_qknorm(a, (hipStream_t)stream));
}

}  // extern "C"

// ---- row passes of the sublayer (LayerNorm, column sums) ----------------------

namespace {

// Bytes of N rows of C bf16 elements `stride` apart.
size_t rows_bytes(int N, int C, long long stride) { return ((size_t)(N - 1) * stride + C) * 2; }

int rows_check(int N, int C, long long stride, int dtype, int c_max, bool f32_ok = false)
{
    if (N < 1 || C < 8 || C % 8 || C > c_max) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 && !(f32_ok && dtype == ATTN_F32)) return ATTN_ERR_DTYPE;
    if (stride < C || stride % 8) return ATTN_ERR_LAYOUT;
    if ((long long)(N - 1) * stride > (1LL << 40)) return ATTN_ERR_OVERFLOW;
    return ATTN_OK;
}

bool aligned16(const void* p) { return (uintptr_t)p % 16 == 0; }

Span span_of(const void* p, size_t bytes)
{
    return Span{(uintptr_t)p, (uintptr_t)p + bytes};
}

// Outputs (first n_out) must not overlap any span after them or each other.
bool spans_alias(const Span* s, int n_out, int n)
{
    for (int i = 0; i < n_out; ++i)
        for (int j = i + 1; j < n; ++j)
            if (overlaps(s[i], s[j])) return true;
    return false;
}

}  // namespace

extern "C" {

size_t attn_layernorm_workspace_bytes(int N, int C)
{
    if (N < 1 || C < 1) return 0;
    return (size_t)cattn::layernorm_bwd_workgroups(N) * 2 * C * sizeof(float);
}

size_t attn_colsum_workspace_bytes(int N, int M)
{
    if (N < 1 || M < 1) return 0;
    return (size_t)cattn::colsum_row_blocks(N) * M * sizeof(float);
}

int attn_layernorm_fwd(const void* x, const void* g, const void* b, void* y, int N, int C,
                       long long stride, float eps, int dtype, void* stream)
{
    if (!x || !g || !b || !y) return ATTN_ERR_NULL;
    int st = rows_check(N, C, stride, dtype, 4096);
    if (st != ATTN_OK) return st;
    if (!isfinite(eps) || eps < 0.0f) return ATTN_ERR_PARAM;
    if (!aligned16(x) || !aligned16(g) || !aligned16(b) || !aligned16(y)) return ATTN_ERR_ALIGN;
    const size_t rb = rows_bytes(N, C, stride);
    const Span sp[4] = {span_of(y, rb), span_of(x, rb), span_of(g, 2 * (size_t)C),
                        span_of(b, 2 * (size_t)C)};
    if (spans_alias(sp, 1, 4)) return ATTN_ERR_ALIAS;
    cattn::NormArgs a{};
    a.x = x;
    a.g = g;
    a.b = b;
    a.y = y;
    a.N = N;
    a.C = C;
    a.stride = stride;
    a.eps = eps;
    return status(cattn::launch_layernorm_fwd(a, (hipStream_t)stream));
}

int attn_layernorm_bwd(const void* x, const void* g, const void* dy, const void* dres, void* dx,
                       void* dg, void* db, void* workspace, size_t workspace_bytes, int N, int C,
                       long long stride, float eps, int dtype, void* stream)
{
    if (!x || !g || !dy || !dx || !dg || !db || !workspace) return ATTN_ERR_NULL;
    int st = rows_check(N, C, stride, dtype, 4096);
    if (st != ATTN_OK) return st;
    if (!isfinite(eps) || eps < 0.0f) return ATTN_ERR_PARAM;
    if (!aligned16(x) || !aligned16(g) || !aligned16(dy) || (dres && !aligned16(dres)) ||
        !aligned16(dx) || !aligned16(dg) || !aligned16(db) || !aligned16(workspace))
        return ATTN_ERR_ALIGN;
    const size_t need = attn_layernorm_workspace_bytes(N, C);
    if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    const size_t rb = rows_bytes(N, C, stride), cb = 2 * (size_t)C;
    const Span sp[8] = {span_of(dx, rb), span_of(dg, cb), span_of(db, cb), span_of(workspace, need),
                        span_of(x, rb), span_of(g, cb), span_of(dy, rb),
                        span_of(dres ? dres : x, rb)};
    if (spans_alias(sp, 4, 8)) return ATTN_ERR_ALIAS;
    cattn::NormArgs a{};
    a.x = x;
    a.g = g;
    a.dy = dy;
    a.dres = dres;
    a.dx = dx;
    a.dg = dg;
    a.db = db;
    a.workspace = workspace;
    a.N = N;
    a.C = C;
    a.stride = stride;
    a.eps = eps;
    return status(cattn::launch_layernorm_bwd(a, (hipStream_t)stream));
}

int attn_colsum(const void* x, void* out, void* workspace, size_t workspace_bytes, int N, int M,
                long long stride, int dtype, void* stream)
{
    const bool f32 = dtype == ATTN_F32;
    if (!x || !out || (!workspace && !f32)) return ATTN_ERR_NULL;
    int st = rows_check(N, M, stride, dtype, 1 << 30, true);
    if (st != ATTN_OK) return st;
    if (!aligned16(x) || !aligned16(out) || (!f32 && !aligned16(workspace))) return ATTN_ERR_ALIGN;
    const size_t need = f32 ? 0 : attn_colsum_workspace_bytes(N, M);
    if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    const size_t in_bytes = ((size_t)(N - 1) * stride + M) * (f32 ? 4 : 2);
    const Span sp[3] = {span_of(out, 2 * (size_t)M), span_of(workspace, need), span_of(x, in_bytes)};
    if (spans_alias(sp, 2, 3)) return ATTN_ERR_ALIAS;
    cattn::NormArgs a{};
    a.x = x;
    a.y = out;
    a.workspace = workspace;
    a.N = N;
    a.C = M;
    a.stride = stride;
    a.f32 = f32;
    return status(cattn::launch_colsum(a, (hipStream_t)stream));
}

}  // extern "C"

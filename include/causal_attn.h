/*
 * causal_attn.h -- C ABI of the MI355X (gfx950) causal multi-head
 * self-attention library, libcausal_attn.so.
 *
 * The operation (forward) is the causal scaled dot-product attention of one
 * head, applied independently to every (batch, head) pair:
 *
 *     S = scale * Q K^T,  S[i][j] = -inf for j > i  (keys after the query),
 *     P = softmax over j of S[i][:],  O = P V,
 *     lse[i] = log(sum_{j<=i} exp(S[i][j]))   (natural log),
 *
 * as defined by the CS336 from-scratch tutorial (lmnt.cn), section 5.1
 * model.py, CausalSelfAttention.forward (scores times 1/sqrt(head dim), the
 * tril mask filled with -inf, softmax over keys, weights times v), with the
 * diagonal kept: the mask is tril(ones(T, T)) ("Train Your Own LLM from
 * Scratch", section 1).  Section 3.3 of the tutorial states the mask's
 * purpose: -inf above the diagonal, weight 0 after the softmax.  The backward
 * is the exact gradient of that function; the pages train through it with
 * loss.backward() (tutorial section 5.2, train.py).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers on the current HIP device.
 *   - q, k, v, o, dO, dq, dk, dv: contiguous row-major [B][H][T][D] of the
 *     element type `dtype` (D fastest).  Their addresses must be 16-byte
 *     aligned.
 *   - lse and delta: contiguous fp32 [B][H][T], 4-byte aligned.
 *   - dtype: ATTN_F32 (float) or ATTN_BF16 (bfloat16 storage; every product
 *     is accumulated in fp32).
 *   - D must be 32 or 64, or 128 with ATTN_BF16.  B, H, T >= 1, any T (the
 *     last tile is ragged).
 *   - scale must be finite and > 0 (the pages use 1/sqrt(D)).
 *   - stream is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it and the call returns without synchronising: buffers must stay
 *     alive until the stream has run the work.
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     allocates no memory.  Its only mutable global state is a per-device
 *     cache of the device's compute-unit count (which picks the work
 *     placement), filled on first use with atomic stores of the same value
 *     by any racing threads, and the per-device address of the fixed scratch
 *     of attn_decode_noalloc (below).  Calls on different streams with
 *     disjoint buffers may run concurrently, except attn_decode_noalloc calls
 *     on one device, which share that device's scratch.
 *   - Outputs are fully overwritten, never accumulated into.  No output may
 *     overlap an input or another output.
 *   - Errors: every argument check runs before any HIP call; on a non-zero
 *     return no work was enqueued and no output was touched, except
 *     ATTN_ERR_HIP, which reports a failed kernel launch (outputs undefined).
 *     Results are deterministic: no atomics, fixed summation order.
 */
#ifndef CAUSAL_ATTN_H
#define CAUSAL_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_F32 = 0,
    ATTN_BF16 = 1
} attn_dtype_t;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,          /* a required pointer is NULL              */
    ATTN_ERR_SHAPE = 2,         /* B, H or T < 1 (row passes: N, C, M)      */
    ATTN_ERR_UNSUPPORTED_D = 3, /* D not in {32, 64} (bf16: {32, 64, 128})  */
    ATTN_ERR_DTYPE = 4,         /* dtype not ATTN_F32 / ATTN_BF16           */
    ATTN_ERR_ALIGN = 5,         /* tensor not 16-byte (lse/delta 4-byte) aligned */
    ATTN_ERR_OVERFLOW = 6,      /* T*D or the launch grid exceeds 2^31 - 1  */
    ATTN_ERR_SCALE = 7,         /* scale not finite or not > 0              */
    ATTN_ERR_ALIAS = 8,         /* an output overlaps an input or output    */
    ATTN_ERR_HIP = 9,           /* a kernel launch failed                   */
    ATTN_ERR_LAYOUT = 10,       /* strided views: unsupported dtype/D or strides */
    ATTN_ERR_WORKSPACE = 11,    /* a workspace smaller than required        */
    ATTN_ERR_PARAM = 12,        /* RoPE / QK norm / LayerNorm parameters, or dropout_p */
    ATTN_ERR_SCRATCH = 13       /* attn_decode_noalloc: beyond its fixed scratch */
} attn_status_t;

/* Forward.  Reads q, k, v; writes o ([B][H][T][D], dtype) and lse
 * ([B][H][T], fp32, natural log of the row's softmax normaliser over the
 * scaled scores).  lse is what attn_bwd needs to recompute P. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int T, int D, float scale, int dtype, void* stream);

/* Backward of L = sum(dO * O) for the forward above.  Reads q, k, v, o, lse
 * (as written by attn_fwd with the same arguments) and dO; writes dq, dk, dv
 * ([B][H][T][D], dtype).  delta is caller-owned fp32 [B][H][T] workspace; on
 * return it holds Delta[i] = sum_d dO[i][d] * o[i][d], the softmax-backward
 * row term.  For bf16 at D = 64 this is one kernel launch on `stream` whose
 * dK/dV work forms Delta itself from o and dO; for bf16 at D = 128, a launch
 * that writes Delta and then one launch of dQ and dK/dV work that reads it;
 * otherwise it enqueues the two stages below (dQ with Delta, then dK/dV).
 * Either way the results equal those of the two stages up to the fp32
 * summation order. */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dO, void* dq, void* dk, void* dv,
             float* delta, int B, int H, int T, int D, float scale, int dtype,
             void* stream);

/* The backward as two stages, callable one by one with the same argument
 * conventions, in this order on one stream (or with an event between them):
 * attn_bwd_dkdv reads the delta that attn_bwd_dq writes.
 *
 * attn_bwd_dq:   delta[i] = sum_d dO[i][d] * o[i][d] (fp32 accumulation) and
 *                dq = scale * dS k, with P recomputed from lse and
 *                dS = P * (dO v^T - delta).
 * attn_bwd_dkdv: dk = scale * dS^T q and dv = P^T dO, same P and dS. */
int attn_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                const void* dO, const float* lse, float* delta, void* dq, int B,
                int H, int T, int D, float scale, int dtype, void* stream);
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                  const float* lse, const float* delta, void* dk, void* dv, int B,
                  int H, int T, int D, float scale, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Strided views.  The pages' tensors are per-head views of the c_attn output,
 * q, k, v = split(x W_attn + b) viewed as [B][T][H][D] and transposed to
 * [B][H][T][D] (CS336 tutorial, section 5.1, CausalSelfAttention.forward), and
 * the attention output goes back through the inverse transpose into [B][T][C].
 * These entry points take such views directly, so no layout copy is needed.
 *
 * attn_view_t describes a [B][H][T][D] tensor whose D elements are contiguous:
 * element (b, h, t, d) is at data + b*stride_b + h*stride_h + t*stride_t + d,
 * strides counted in elements of the call's dtype.  Examples (C = H*D):
 *   contiguous [B][H][T][D]:        stride_b = H*T*D, stride_h = T*D, stride_t = D
 *   [B][T][H][D] (= [B][T][C]):      stride_b = T*C,   stride_h = D,   stride_t = C
 *   q of a [B][T][3][H][D] qkv:      stride_b = 3*T*C, stride_h = D,   stride_t = 3*C
 *                                    (k at data + C, v at data + 2*C)
 *
 * Supported for dtype ATTN_BF16 with D = 64 or 128 (else ATTN_ERR_LAYOUT).  Each view
 * needs a 16-byte-aligned data pointer, non-negative strides that are
 * multiples of 8, stride_t >= D, and T * stride_t * 2 bytes below 2^32
 * (ATTN_ERR_LAYOUT otherwise).  lse and delta stay contiguous fp32 [B][H][T].
 * Aliasing: inputs may share memory with each other.  An output must not share
 * an element with an input or another output, nor address one element twice
 * (taken in order of increasing stride, each stride of a dimension of size > 1
 * must reach past the elements the smaller ones span).  The check (ATTN_ERR_ALIAS) is
 * conservative: two views whose address ranges intersect are accepted only if
 * they have equal strides, stride_b is a multiple of stride_t, and their
 * per-token footprints of (H-1)*stride_h + D elements do not meet modulo
 * stride_t (as for q, k, v or dq, dk, dv in one [B][T][3][H][D] buffer).
 * Results equal those of attn_fwd / attn_bwd on contiguous copies of the same
 * values, bit for bit. */
typedef struct {
    void* data;
    long long stride_b;
    long long stride_h;
    long long stride_t;
} attn_view_t;

/* Sliding window (window >= 1): query i sees only the `window` most recent
 * keys, i - window < j <= i, the band of the causal mask (the nanochat page,
 * section 9, lists sliding-window attention; its SSSL pattern mixes short
 * windows with full-context layers).  window = 0 (or >= T) is the plain causal
 * mask.  window < 0 is rejected with ATTN_ERR_SHAPE.  lse is then the
 * log-sum-exp over the window. */

/* Attention dropout (dropout_p > 0).  The CS336 tutorial (section 5.1)
 * passes the softmax weights through nn.Dropout before the product with v;
 * every configuration on the pages uses p = 0.  In training mode that is
 * inverted dropout: each weight P[i][j] is kept with probability 1 - p and
 * scaled by 1 / (1 - p), or zeroed; lse stays that of the undropped weights.
 * The decisions are reproducible: weight (b, h, i, j) is kept iff the 16-bit
 * half (j % 2) of word (j % 8) / 2 of Philox4x32-10(counter = (j / 8, i,
 * b * H + h, 0), key = (seed mod 2^32, seed / 2^32)) is >= p16, with
 * p16 = round(p * 65536) (p is quantised to 1/65536) and kept weights scaled by
 * 65536 / (65536 - p16).  The backward must get the same dropout_p and seed
 * as the forward.  dropout_p must be finite with 0 <= p < 1
 * (ATTN_ERR_PARAM otherwise); p = 0 runs the kernels without dropout. */

/* attn_fwd on strided views (q, k, v read; o written), with a window and
 * dropout. */
int attn_fwd_strided(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o, float* lse,
                     int B, int H, int T, int D, int window, float dropout_p,
                     unsigned long long seed, float scale, int dtype, void* stream);

/* attn_bwd on strided views (q, k, v, o, dO read; dq, dk, dv written); delta as
 * in attn_bwd; window, dropout_p and seed as in the forward call.  One kernel
 * launch at D = 64, two at D = 128. */
int attn_bwd_strided(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o,
                     const float* lse, attn_view_t dO, attn_view_t dq, attn_view_t dk,
                     attn_view_t dv, float* delta, int B, int H, int T, int D, int window,
                     float dropout_p, unsigned long long seed, float scale, int dtype,
                     void* stream);

/* Stored keep bits: the dropout forward's keep decisions kept for its backward.
 * With dropout the forward and both backward stages each draw the keep bits of
 * the weights they touch (Philox, as above).  These two entry points let the
 * forward store its draws in a caller-owned buffer and the backward load them
 * instead of drawing again; the results are bit for bit those of
 * attn_fwd_strided / attn_bwd_strided with the same dropout_p and seed.
 *
 *   keep:       uint32 words, [B*H][ceil(T/32)][T]: bit t of word (b*H + h, w, i)
 *               is the keep decision of query i and key 32 w + t (1 = kept).  The
 *               forward writes the words of the (query, 32-key block) pairs it
 *               visits and never writes the rest.  The backward may read words
 *               the forward did not write (in a tile that crosses the diagonal,
 *               or with a window), but only for pairs the mask removes, whose
 *               weight is zero whatever the bit says, so the results do not
 *               depend on them.  The caller owns the
 *               buffer; 4-byte aligned; it must not overlap any other buffer of
 *               the call (ATTN_ERR_ALIAS).
 *   keep_bytes: its size, at least attn_dropout_keep_bytes(B, H, T)
 *               (ATTN_ERR_WORKSPACE otherwise; 0 for a non-positive size).
 *
 * The backward takes the forward's dropout_p (the keep scale) but no seed.
 * With dropout_p = 0 the buffer is neither written nor read.  Errors: those of
 * the strided call first, then ATTN_ERR_NULL, ATTN_ERR_ALIGN,
 * ATTN_ERR_WORKSPACE and ATTN_ERR_ALIAS for the keep buffer. */
size_t attn_dropout_keep_bytes(int B, int H, int T);
int attn_fwd_strided_keep(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o, float* lse,
                          int B, int H, int T, int D, int window, float dropout_p,
                          unsigned long long seed, float scale, int dtype, unsigned int* keep,
                          size_t keep_bytes, void* stream);
int attn_bwd_strided_keep(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o,
                          const float* lse, attn_view_t dO, attn_view_t dq, attn_view_t dk,
                          attn_view_t dv, float* delta, int B, int H, int T, int D, int window,
                          float dropout_p, float scale, int dtype, const unsigned int* keep,
                          size_t keep_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Decode against a KV cache.  nanochat, section 8 (inference engine): the
 * cache is kept in FA3's native (B, T, H, D) layout, a prompt is prefilled
 * into it, then tokens are produced one at a time, each attending to every
 * cached position up to and including its own.  One call computes, for every
 * sequence b and head h, the attention of the new token's query over
 * positions 0 .. len_b - 1 of the cache (the token's own key and value are
 * already stored at position len_b - 1): row len_b - 1 of the causal forward
 * above.  With window W > 0 only the W most recent positions,
 * max(0, len_b - W) .. len_b - 1, take part.
 *
 *   q:        [B][H][D] dtype (the new token of each sequence), 16-byte aligned
 *   k_cache:  [B][T_max][H][D] dtype, contiguous, 16-byte aligned
 *   v_cache:  [B][T_max][H][D] dtype, contiguous, 16-byte aligned
 *   cache_lens: int32 [B] device array, len_b cached positions of sequence b;
 *             values are clamped to [0, T_max]; len_b = 0 gives o = 0 and
 *             lse = -inf for that sequence
 *   o:        [B][H][D] dtype, written
 *   lse:      fp32 [B][H], written (natural log, as for attn_fwd)
 *   workspace: device memory of at least attn_decode_workspace_bytes(B, H,
 *             T_max, D) bytes, 16-byte aligned, owned by the caller; its
 *             content on entry does not matter, and it may be overwritten
 *             (the one-launch path below leaves it untouched)
 *   dtype:    ATTN_BF16 only (else ATTN_ERR_DTYPE); D = 64 or 128 (else
 *             ATTN_ERR_UNSUPPORTED_D); window >= 0 (else ATTN_ERR_SHAPE)
 *
 * All arithmetic after the bf16 loads is fp32.  One kernel launch on `stream`
 * (a workgroup per head, merging its waves' partial softmaxes in LDS) when
 * T_max <= 1024 at D = 64 (512 at D = 128) or when B*H is at least half the
 * device's compute units; otherwise two (per-slice partial softmax into the
 * workspace, then their merge).  No synchronisation.
 * Errors: as for attn_fwd, checked before any HIP call, plus
 * ATTN_ERR_WORKSPACE for a workspace below the required size; outputs and the
 * workspace must not overlap each other or any input (ATTN_ERR_ALIAS). */
size_t attn_decode_workspace_bytes(int B, int H, int T_max, int D);
int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int* cache_lens,
                void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int H,
                int T_max, int D, int window, float scale, int dtype, void* stream);

/* attn_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same operation, arguments (less the workspace),
 * layouts, checks and kernels as attn_decode; the per-slice partials of the
 * two-launch path go to a scratch array of CAUSAL_ATTN_DECODE_SCRATCH_BYTES
 * that the library holds in device memory.  Each GPU the library runs on
 * holds its own copy of that array until the process ends; its address is
 * looked up (hipGetSymbolAddress) on the first call on each device.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   - The argument checks of attn_decode run first (without the workspace
 *     ones), then the device's compute-unit count is queried, which picks the
 *     path; a call whose two-launch path would need more scratch than the
 *     maximum (attn_decode_workspace_bytes(B, H, T_max, D) bytes) returns
 *     ATTN_ERR_SCRATCH with nothing enqueued.  The one-launch path uses no
 *     scratch.
 *   - Every call on one device shares that device's scratch, which keeps the
 *     last call's partials.  Calls that overlap in time on one device (other
 *     streams, other host threads) race on it: the caller serialises them.
 *     Nothing in it needs clearing; each call writes every slot it reads.
 *   - A failed address lookup returns ATTN_ERR_HIP. */
#define CAUSAL_ATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int* cache_lens, void* o, float* lse, int B, int H, int T_max,
                        int D, int window, float scale, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * RoPE and QK norm on the query and key rows.  nanochat, section 9, lists
 * RoPE position encoding and QK norm (x1.2) among its attention's parts; the
 * pages print no formulas, so these are the standard forms:
 *   RoPE (flags & ATTN_ROPE): the column pair (i, i + D/2), i < D/2, of the
 *     row at position p = pos0 + t is turned by p * rope_base^(-2i/D):
 *       y_i = x_i cos - x_{i+D/2} sin,   y_{i+D/2} = x_i sin + x_{i+D/2} cos
 *   QK norm (flags & ATTN_QK_NORM): the row is divided by
 *     sqrt(mean_d x_d^2 + eps) (no learned weight) and multiplied by q_gain
 *     for queries, k_gain for keys (the pages quote 1.2).
 * The two commute (rotation keeps the root mean square).  Queries and keys go
 * through one launch; attention then runs on the results (q_out, k_out).
 *
 * Views as for the strided entry points (bf16, D = 64 or 128).  fwd reads q, k
 * and writes q_out, k_out; bwd reads q, k (the forward's inputs) and dq_out,
 * dk_out (gradients with respect to q_out, k_out) and writes dq, dk.  Outputs
 * must not overlap inputs or each other (ATTN_ERR_ALIAS).  ATTN_ERR_PARAM:
 * flags outside 0..3, pos0 < 0 or pos0 + T > 2^24, rope_base not finite or
 * <= 0 (with ATTN_ROPE), gains not finite, eps not finite or < 0.  fp32
 * arithmetic; one kernel launch each; no synchronisation. */
#define ATTN_ROPE 1
#define ATTN_QK_NORM 2
int attn_rope_qknorm_fwd(attn_view_t q, attn_view_t k, attn_view_t q_out, attn_view_t k_out,
                         int B, int H, int T, int D, int pos0, float rope_base, float q_gain,
                         float k_gain, float eps, int flags, int dtype, void* stream);
int attn_rope_qknorm_bwd(attn_view_t q, attn_view_t k, attn_view_t dq_out, attn_view_t dk_out,
                         attn_view_t dq, attn_view_t dk, int B, int H, int T, int D, int pos0,
                         float rope_base, float q_gain, float k_gain, float eps, int flags,
                         int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Attention with the RoPE / QK-norm prologue above fused into its kernels
 * (nanochat, section 9: RoPE and QK norm on the queries and keys of its
 * attention).  The result is that of attn_rope_qknorm_fwd followed by
 * attn_fwd_strided on its outputs, and for the backward attn_bwd_strided
 * followed by attn_rope_qknorm_bwd, with fewer passes over memory:
 *   fwd: the keys go through the prologue pass (k -> k_rot); the forward
 *        kernel reads the raw queries, applies the prologue to them in
 *        registers and writes them to q_rot.  q_rot and k_rot are outputs
 *        that the backward needs.
 *   bwd: the kernels run on q_rot and k_rot and apply the prologue's
 *        transposed Jacobian to each dQ and dK row in registers, so dq and dk
 *        come out with respect to the raw q and k (no intermediate gradient
 *        of q_rot or k_rot is stored).
 * Views, window and scale as for the strided entry points (bf16, D = 64 or
 * 128); prologue parameters as for attn_rope_qknorm_fwd (ATTN_ERR_PARAM).
 * No dropout.  Outputs (o, lse, q_rot, k_rot; dq, dk, dv, delta) must not
 * overlap any input or each other (ATTN_ERR_ALIAS).  Errors as for the
 * strided calls, checked before any HIP call; two launches each way (the key
 * pass and the forward; the backward launches as attn_bwd_strided). */
int attn_fwd_strided_rope(attn_view_t q, attn_view_t k, attn_view_t v, attn_view_t o, float* lse,
                          attn_view_t q_rot, attn_view_t k_rot, int B, int H, int T, int D,
                          int window, float scale, int pos0, float rope_base, float q_gain,
                          float k_gain, float eps, int flags, int dtype, void* stream);
int attn_bwd_strided_rope(attn_view_t q, attn_view_t k, attn_view_t q_rot, attn_view_t k_rot,
                          attn_view_t v, attn_view_t o, const float* lse, attn_view_t dO,
                          attn_view_t dq, attn_view_t dk, attn_view_t dv, float* delta, int B,
                          int H, int T, int D, int window, float scale, int pos0, float rope_base,
                          float q_gain, float k_gain, float eps, int flags, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * The row passes of the pre-norm sublayer around the attention (CS336
 * tutorial, section 5.1: Block.forward adds attn(ln_1(x)) to x; section 3.4,
 * class LayerNorm: mean and biased variance over the row, eps added under the
 * square root, then gain and bias), and the gradient of its biases.
 *
 * attn_layernorm_fwd:  y[r][c] = (x[r][c] - mean_r) / sqrt(var_r + eps) * g[c] + b[c]
 *   over N rows of C elements.  x, y: bf16 rows `stride` elements apart
 *   (stride >= C, a multiple of 8; y uses the same stride); g, b: bf16 [C].
 *   Requirements: N >= 1 and 8 <= C <= 4096 with C % 8 == 0 (else
 *   ATTN_ERR_SHAPE); stride as stated (ATTN_ERR_LAYOUT); dtype ATTN_BF16
 *   (ATTN_ERR_DTYPE); eps finite and >= 0 (ATTN_ERR_PARAM); x, y, g, b 16-byte
 *   aligned (ATTN_ERR_ALIGN); y overlapping an input is ATTN_ERR_ALIAS.
 *
 * attn_layernorm_bwd:  the gradient of sum(dy * y) + sum(dres * x):
 *   dx = rstd * (e - mean_c(e) - xh * mean_c(e * xh)) + dres,
 *   with xh = (x - mean) * rstd, e = dy * g, rstd = 1 / sqrt(var + eps);
 *   dg[c] = sum_r dy[r][c] * xh[r][c], db[c] = sum_r dy[r][c].
 *   The row statistics are recomputed from x.  dres (the residual branch's
 *   gradient) may be NULL.  x, dy, dres, dx: rows as in the forward; g, dg,
 *   db: bf16 [C].  workspace: fp32 partial column sums, at least
 *   attn_layernorm_workspace_bytes(N, C) bytes, 16-byte aligned (contents on
 *   entry do not matter; undefined on return).  Checks as the forward, plus
 *   ATTN_ERR_WORKSPACE; outputs and workspace may not overlap inputs or each
 *   other (ATTN_ERR_ALIAS).
 *
 * attn_colsum:  out[j] = sum_r x[r][j] (the gradient of a bias added to every
 *   row), for N rows of M elements `stride` apart; out bf16 [M], each sum
 *   rounded once.  8 <= M <= 2^30, M % 8 == 0, stride >= M and a multiple of 8.
 *   dtype ATTN_BF16: workspace of at least attn_colsum_workspace_bytes(N, M)
 *   bytes; fixed summation order: blocks of max(8, ceil(N / 128)) rows, then
 *   the blocks in a fixed order.  dtype ATTN_F32 (a few rows, such as the
 *   partial products of a weight gradient split over row blocks): the rows
 *   are added in order, no workspace (it may be NULL).
 */
size_t attn_layernorm_workspace_bytes(int N, int C);
int attn_layernorm_fwd(const void* x, const void* g, const void* b, void* y, int N, int C,
                       long long stride, float eps, int dtype, void* stream);
int attn_layernorm_bwd(const void* x, const void* g, const void* dy, const void* dres, void* dx,
                       void* dg, void* db, void* workspace, size_t workspace_bytes, int N, int C,
                       long long stride, float eps, int dtype, void* stream);
size_t attn_colsum_workspace_bytes(int N, int M);
int attn_colsum(const void* x, void* out, void* workspace, size_t workspace_bytes, int N, int M,
                long long stride, int dtype, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* attn_status_str(int status);

/* ABI version of this header: (major << 16) | minor. */
int attn_abi_version(void);

#define CAUSAL_ATTN_ABI_VERSION ((1 << 16) | 8)

#ifdef __cplusplus
}
#endif

#endif /* CAUSAL_ATTN_H */

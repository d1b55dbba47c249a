/*
 * kvq_oracle.c -- CPU oracle for quantized-KV attention.  TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the package's smoke() check and bench.py's cpu_baseline leg may
 * call into this file.  The GPU library never links, loads or calls it, and it
 * shares no source with the GPU library: no headers, helpers or tables.
 *
 * What it computes is read from the pages of the @mlx-bun/inference
 * 0.0.0-stage -> 1.0.0 diff (my.diffend.io, pages 78, 80 and 81).  Citations
 * below name the page and the file/symbol shown on it:
 *   [p80 model.ts header]        Gemma 4 parity notes: SDPA scale 1.0, full layers
 *                                have head_dim 512 and a single KV head; sliding
 *                                layers use a rotating cache whose reads own the window.
 *   [p80 model.ts attentionTraining]
 *                                keys/values transposed to [B, H, L, D], appended to
 *                                the layer's cache, then read.attend(q, 1.0).
 *   [p78 gemma4-e4b.ts Gemma4Layer / LAYERS]
 *                                each cache carries an affine width (4 or 8 bits) and
 *                                a group size (64).
 * The pages name the affine scheme but give no formula; the plainest reading
 * is taken and written out below (min/max affine quantizer, bias rounded down
 * and scale rounded up to bf16, round-half-even codes).
 *
 * Precision: the quantizer runs in IEEE fp32 with round-to-nearest-even and no
 * fused multiply-add (build with -ffp-contract=off); dequantization and
 * attention run in fp64.
 *
 * A layer's cache may instead hold bf16 values, unquantized: the pages keep
 * the sliding layers' caches in bf16 under the other KV scheme they compose
 *   [p80 model.ts cacheLayers note]  sliding layers compose a ring of the window
 *                                and stay bf16; the full layers' read is deferred.
 * Such a cache stores each fp32 key or value rounded to the nearest bf16 (ties
 * to even), and its read uses those values exactly.
 *
 * Status codes: 0 ok, 1 invalid argument (bad bits/shape, non-finite or
 * out-of-domain input), 2 capacity (the cache cannot hold every key a query
 * must see).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KVQO_GROUP 64
/* Inputs with |x| above this are rejected: beyond it the bf16 bias or the
 * scale could round to infinity. */
#define KVQO_MAX_ABS 1e38f

static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Largest bf16 value <= x (x finite).  A bf16 value is an fp32 value whose low
 * 16 bits are zero.  Dropping the low bits moves x toward zero; for a negative
 * x that is upward, so one bf16 step away from zero is taken instead. */
static float bf16_round_down(float x)
{
    uint32_t u = bits_of(x);
    if ((u & 0xFFFFu) == 0) return x;
    uint32_t toward_zero = u & 0xFFFF0000u;
    if (u & 0x80000000u) return float_of(toward_zero + 0x10000u);
    return float_of(toward_zero);
}

/* Smallest bf16 value >= x (x finite). */
static float bf16_round_up(float x)
{
    uint32_t u = bits_of(x);
    if ((u & 0xFFFFu) == 0) return x;
    uint32_t toward_zero = u & 0xFFFF0000u;
    if (u & 0x80000000u) return float_of(toward_zero);
    return float_of(toward_zero + 0x10000u);
}

static double bf16_to_double(uint16_t h) { return (double)float_of((uint32_t)h << 16); }

/* Affine quantization of one group of n fp32 values to `bits`-bit codes
 * [p78 gemma4-e4b.ts Gemma4Layer.kv {bits, groupSize}]:
 *   mn, mx  = min and max of the group (-0 read as +0)
 *   bias    = mn rounded down to bf16           (so bias <= every value)
 *   scale   = ((mx - bias) / (2^bits - 1)) rounded up to bf16
 *   code_i  = clamp(rint((x_i - bias) / scale), 0, 2^bits - 1), or 0 when scale == 0
 * Every step is one fp32 operation rounded to nearest even.  Returns 1 if any
 * value is non-finite or above KVQO_MAX_ABS in magnitude. */
int kvqo_quantize_group(const float *x, int n_el, int bits,
                        uint8_t *codes, uint16_t *scale_bits, uint16_t *bias_bits)
{
    if (bits != 4 && bits != 8) return 1;
    if (n_el <= 0) return 1;
    const int top = (1 << bits) - 1;
    for (int i = 0; i < n_el; ++i)
        if (!(fabsf(x[i]) <= KVQO_MAX_ABS)) return 1;

    float mn = x[0], mx = x[0];
    for (int i = 1; i < n_el; ++i) {
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    mn = mn + 0.0f;   /* -0 + +0 = +0 under round-to-nearest */
    mx = mx + 0.0f;

    const float bias = bf16_round_down(mn);
    const float step = (mx - bias) / (float)top;
    const float scale = bf16_round_up(step);

    for (int i = 0; i < n_el; ++i) {
        if (scale == 0.0f) { codes[i] = 0; continue; }
        const float ratio = (x[i] - bias) / scale;
        float r = rintf(ratio);
        if (r < 0.0f) r = 0.0f;
        if (r > (float)top) r = (float)top;
        codes[i] = (uint8_t)r;
    }
    *scale_bits = (uint16_t)(bits_of(scale) >> 16);
    *bias_bits = (uint16_t)(bits_of(bias) >> 16);
    return 0;
}

/* Append T new tokens per sequence to a cache of R slots, plain layout:
 *   x       fp32 [B][H][T][D]   keys (already normed and roped) or values,
 *           in the [B, H, L, D] layout the pages transpose to
 *           [p80 model.ts attentionTraining]
 *   pos0    [B] absolute position of each sequence's first new token
 *   codes   uint8 [B][H][R][D]   one code per byte (unpacked)
 *   scales, biases  bf16 bits [B][H][R][D/64]
 * Token t of sequence b lands in slot (pos0[b] + t) mod R: a ring for sliding
 * layers [p80 model.ts header: rotating cache], a plain array for full layers
 * (R = capacity).  When T > R only the last R tokens are written, since the
 * earlier ones would be overwritten within the same append.  Everything is
 * validated before anything is written. */
int kvqo_append(const float *x, int B, int H, int T, int D, int bits, int R,
                const int32_t *pos0, uint8_t *codes, uint16_t *scales, uint16_t *biases)
{
    if (B < 0 || H <= 0 || T < 0 || D <= 0 || D % KVQO_GROUP != 0 || R <= 0) return 1;
    if (bits != 4 && bits != 8) return 1;
    const int G = D / KVQO_GROUP;
    for (int b = 0; b < B; ++b) if (pos0[b] < 0) return 1;
    const int64_t total = (int64_t)B * H * T * D;
    for (int64_t i = 0; i < total; ++i)
        if (!(fabsf(x[i]) <= KVQO_MAX_ABS)) return 1;

    const int first = T > R ? T - R : 0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int t = first; t < T; ++t) {
                const int64_t pos = (int64_t)pos0[b] + t;
                const int64_t slot = pos % R;
                const float *src = x + (((int64_t)b * H + h) * T + t) * D;
                const int64_t row = ((int64_t)b * H + h) * R + slot;
                for (int g = 0; g < G; ++g) {
                    int st = kvqo_quantize_group(src + g * KVQO_GROUP, KVQO_GROUP, bits,
                                                 codes + row * D + g * KVQO_GROUP,
                                                 scales + row * G + g, biases + row * G + g);
                    if (st) return st;
                }
            }
    return 0;
}

/* The bf16 value nearest to x (finite, |x| <= KVQO_MAX_ABS), ties to the one
 * whose last mantissa bit is 0.  The two candidates are x with its low 16 bits
 * dropped (toward zero) and the next bf16 value away from zero; their distances
 * to x are exact in fp64. */
static uint16_t bf16_nearest_even(float x)
{
    const uint32_t u = bits_of(x);
    const uint32_t toward = u & 0xFFFF0000u;
    if (toward == u) return (uint16_t)(u >> 16);
    const uint32_t away = toward + 0x10000u;
    const double d_toward = fabs((double)x - (double)float_of(toward));
    const double d_away = fabs((double)float_of(away) - (double)x);
    uint32_t r;
    if (d_toward < d_away) r = toward;
    else if (d_away < d_toward) r = away;
    else r = ((toward >> 16) & 1u) ? away : toward;
    return (uint16_t)(r >> 16);
}

/* One fp32 value rounded to bf16 as above (bit pattern); 0xFFFF flags an input
 * outside the domain (non-finite or |x| > KVQO_MAX_ABS). */
uint16_t kvqo_bf16(float x)
{
    if (!(fabsf(x) <= KVQO_MAX_ABS)) return 0xFFFFu;
    return bf16_nearest_even(x);
}

/* Append T new tokens per sequence to an unquantized bf16 cache of R slots
 * [p80 model.ts cacheLayers note: sliding layers stay bf16]:
 *   x     fp32 [B][H][T][D]
 *   vals  bf16 bits [B][H][R][D]
 * with the slots, the ring and the T > R rule of kvqo_append. */
int kvqo_append_bf16(const float *x, int B, int H, int T, int D, int R,
                     const int32_t *pos0, uint16_t *vals)
{
    if (B < 0 || H <= 0 || T < 0 || D <= 0 || R <= 0) return 1;
    for (int b = 0; b < B; ++b) if (pos0[b] < 0) return 1;
    const int64_t total = (int64_t)B * H * T * D;
    for (int64_t i = 0; i < total; ++i)
        if (!(fabsf(x[i]) <= KVQO_MAX_ABS)) return 1;
    const int first = T > R ? T - R : 0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int t = first; t < T; ++t) {
                const int64_t slot = ((int64_t)pos0[b] + t) % R;
                const float *src = x + (((int64_t)b * H + h) * T + t) * D;
                uint16_t *dst = vals + (((int64_t)b * H + h) * R + slot) * D;
                for (int d = 0; d < D; ++d) dst[d] = bf16_nearest_even(src[d]);
            }
    return 0;
}

/* Pack unpacked codes row by row into little-endian uint32 words: word w of a
 * row holds elements [w*k, (w+1)*k) with k = 32/bits, element e at bits
 * [bits*(e mod k), bits*(e mod k + 1)). */
void kvqo_pack_words(const uint8_t *codes, int64_t n_rows, int D, int bits, uint32_t *words)
{
    const int per = 32 / bits;
    const int wpr = D / per;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int w = 0; w < wpr; ++w) {
            uint32_t acc = 0;
            for (int e = 0; e < per; ++e)
                acc |= (uint32_t)codes[r * D + (int64_t)w * per + e] << (bits * e);
            words[r * wpr + w] = acc;
        }
}

/* Dequantize a plain-layout cache to fp64: x = code * scale + bias.  With a
 * bf16 scale and bias and an 8-bit code the product and sum are exact in fp64. */
void kvqo_dequant(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                  int64_t n_rows, int D, double *out)
{
    const int G = D / KVQO_GROUP;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int d = 0; d < D; ++d) {
            const double s = bf16_to_double(scales[r * G + d / KVQO_GROUP]);
            const double b = bf16_to_double(biases[r * G + d / KVQO_GROUP]);
            out[r * D + d] = (double)codes[r * D + d] * s + b;
        }
}

/* One side (K or V) of a cache as the attention reads it: affine codes with a
 * bf16 scale and bias per group, or (bf16 != NULL) bf16 values. */
typedef struct {
    const uint8_t *codes;
    const uint16_t *scales, *biases;
    const uint16_t *bf16;
} kvqo_side;

/* Element d of cache row `row`, in fp64: code * scale + bias (exact), or the
 * stored bf16 value. */
static double side_value(const kvqo_side *s, int64_t row, int D, int d)
{
    if (s->bf16) return bf16_to_double(s->bf16[row * D + d]);
    const int G = D / KVQO_GROUP;
    return (double)s->codes[row * D + d] * bf16_to_double(s->scales[row * G + d / KVQO_GROUP])
         + bf16_to_double(s->biases[row * G + d / KVQO_GROUP]);
}

/* Scaled-dot-product attention over a cache, in fp64
 * [p80 model.ts attentionTraining: read.attend(q, 1.0); header: SDPA scale 1.0].
 *   q    bf16 bits [B][Hq][C][D]; query i of sequence b sits at absolute
 *        position p = len[b] - C + i (the C new tokens were appended first)
 *   len  [B] tokens appended so far, including the C new ones
 *   W    0 for a full layer, else the sliding window
 *   out  fp64 [B][Hq][C][D]
 * Query head hq reads KV head hq / (Hq/Hkv) (contiguous GQA groups).  Query p
 * sees key positions j with lo <= j <= p, lo = max(0, p - W + 1) for a window
 * layer and 0 for a full one (causal in both cases); key j sits in slot j mod R
 * and is still there only if j >= len - R.  If a visible key was overwritten
 * the call fails with 2.
 *   z_j = scale * sum_d q_d * khat_{j,d};  w_j = exp(z_j - max z);
 *   out_d = sum_j w_j * vhat_{j,d} / sum_j w_j. */
static int attend(const kvqo_side *ks, const kvqo_side *vs,
                  int B, int Hkv, int D, int R, int W,
                  const uint16_t *q, int Hq, int C, const int32_t *len,
                  double scale, double *out, int nthreads)
{
    if (B < 0 || Hkv <= 0 || D <= 0 || D % KVQO_GROUP != 0 || R <= 0 || W < 0) return 1;
    if (Hq <= 0 || Hq % Hkv != 0 || C <= 0) return 1;
    const int per_kv = Hq / Hkv;
    for (int b = 0; b < B; ++b) {
        if (len[b] < C) return 1;
        const int64_t oldest = (int64_t)len[b] - R;          /* oldest position still held */
        const int64_t p_first = (int64_t)len[b] - C;
        const int64_t need = W > 0 ? (p_first - W + 1 > 0 ? p_first - W + 1 : 0) : 0;
        if (need < oldest) return 2;
    }

    const int64_t rows = (int64_t)B * Hq * C;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t row = 0; row < rows; ++row) {
        const int i = (int)(row % C);
        const int hq = (int)((row / C) % Hq);
        const int b = (int)(row / ((int64_t)C * Hq));
        const int hkv = hq / per_kv;
        const int64_t p = (int64_t)len[b] - C + i;
        const int64_t lo = W > 0 ? (p - W + 1 > 0 ? p - W + 1 : 0) : 0;
        const int64_t n = p - lo + 1;
        const uint16_t *qrow = q + row * D;
        double *o = out + row * D;
        double *z = (double *)malloc((size_t)n * sizeof(double));
        if (!z) { status = 1; continue; }

        double zmax = -INFINITY;
        for (int64_t j = lo; j <= p; ++j) {
            const int64_t kr = ((int64_t)b * Hkv + hkv) * R + j % R;
            double acc = 0.0;
            for (int d = 0; d < D; ++d) acc += bf16_to_double(qrow[d]) * side_value(ks, kr, D, d);
            z[j - lo] = scale * acc;
            if (z[j - lo] > zmax) zmax = z[j - lo];
        }
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        double wsum = 0.0;
        for (int64_t j = lo; j <= p; ++j) {
            const double w = exp(z[j - lo] - zmax);
            wsum += w;
            const int64_t vr = ((int64_t)b * Hkv + hkv) * R + j % R;
            for (int d = 0; d < D; ++d) o[d] += w * side_value(vs, vr, D, d);
        }
        for (int d = 0; d < D; ++d) o[d] /= wsum;
        free(z);
    }
    return status;
}

/* Attention over an affine-quantized cache (plain layouts of kvqo_append). */
int kvqo_attend(const uint8_t *k_codes, const uint16_t *k_scales, const uint16_t *k_biases,
                const uint8_t *v_codes, const uint16_t *v_scales, const uint16_t *v_biases,
                int B, int Hkv, int D, int R, int W,
                const uint16_t *q, int Hq, int C, const int32_t *len,
                double scale, double *out, int nthreads)
{
    const kvqo_side ks = {k_codes, k_scales, k_biases, NULL};
    const kvqo_side vs = {v_codes, v_scales, v_biases, NULL};
    return attend(&ks, &vs, B, Hkv, D, R, W, q, Hq, C, len, scale, out, nthreads);
}

/* The same over any mix of sides: a side whose *_bf16 pointer is not NULL is
 * read as bf16 values [B][H][R][D] (kvqo_append_bf16), the other as codes. */
int kvqo_attend_any(const uint8_t *k_codes, const uint16_t *k_scales, const uint16_t *k_biases,
                    const uint16_t *k_bf16,
                    const uint8_t *v_codes, const uint16_t *v_scales, const uint16_t *v_biases,
                    const uint16_t *v_bf16,
                    int B, int Hkv, int D, int R, int W,
                    const uint16_t *q, int Hq, int C, const int32_t *len,
                    double scale, double *out, int nthreads)
{
    const kvqo_side ks = {k_codes, k_scales, k_biases, k_bf16};
    const kvqo_side vs = {v_codes, v_scales, v_biases, v_bf16};
    return attend(&ks, &vs, B, Hkv, D, R, W, q, Hq, C, len, scale, out, nthreads);
}

/* ---------------------------------------------------------------------------
 * Norm and rotation before the append [p80 model.ts attentionTraining: keys go
 * through kNorm, then the cache's position rotation (RoPE), then appendWindow;
 * values go through vNorm; p80 model.ts header: the value norm is an RMS norm
 * without a learned scale].  The pages give neither the reduction order of the
 * norm nor the rotation's frequencies (ProportionalRoPE is not on them), so
 * this library fixes, for one row x[0..D) of one (token, head):
 *   ss = sum of x_d^2 in fp64 over a complete binary tree: leaves in index
 *        order, zero-padded to the next power of 2, each level adding pairs
 *        (2i, 2i+1)
 *   r  = fp32(1 / sqrt(ss / D + eps)), computed in fp64 and rounded once
 *   y_d = fp32(x_d * r), then for keys fp32(y_d * w_d) with the norm's weight w
 *   rotation (keys, when rope_dims > 0): with h = rope_dims / 2 and the caller's
 *        table c = cos[pos][j], s = sin[pos][j] at the token's absolute position,
 *        for j < h:  y_j' = fp32(fp32(y_j c) - fp32(y_{j+h} s)),
 *                    y_{j+h}' = fp32(fp32(y_{j+h} c) + fp32(y_j s));
 *        columns at and past rope_dims pass unchanged.
 * Every fp32 step is one IEEE operation rounded to nearest even (no FMA). */
static double tree_sumsq(const float *x, int n)
{
    double buf[512];
    int P = 1;
    while (P < n) P <<= 1;
    for (int i = 0; i < P; ++i) buf[i] = i < n ? (double)x[i] * (double)x[i] : 0.0;
    for (int w = P; w > 1; w >>= 1)
        for (int i = 0; i < w / 2; ++i) buf[i] = buf[2 * i] + buf[2 * i + 1];
    return buf[0];
}

/* The RMS factor r of one row (see above). */
float kvqo_rms_factor(const float *x, int n, float eps)
{
    return (float)(1.0 / sqrt(tree_sumsq(x, n) / (double)n + (double)eps));
}

/* Normalize (and, with rope_dims > 0, rotate) `rows` rows of D values:
 *   x, y   fp32 [rows][D] (may not alias)
 *   w      fp32 [D] norm weight, or NULL for the un-scaled norm
 *   pos    int32 [rows] absolute position of each row's token (used only by the
 *          rotation); cos_tab, sin_tab fp32 [rope_positions][rope_dims / 2]
 * Returns 1 for invalid arguments (D not in 1..512, rope_dims odd or > D, eps
 * negative or not finite, a position outside the table, a non-finite input or
 * a result above 1e38 in magnitude), else 0. */
int kvqo_norm_rows(const float *x, int64_t rows, int D, const float *w, float eps,
                   const float *cos_tab, const float *sin_tab, int rope_dims, int rope_positions,
                   const int32_t *pos, float *y)
{
    if (D < 1 || D > 512 || rope_dims < 0 || rope_dims % 2 || rope_dims > D) return 1;
    if (!(eps >= 0.0f) || !isfinite(eps)) return 1;
    if (rope_dims > 0 && (!cos_tab || !sin_tab || !pos)) return 1;
    const int h = rope_dims / 2;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * D;
        float *yr = y + r * D;
        for (int d = 0; d < D; ++d)
            if (!(fabsf(xr[d]) <= KVQO_MAX_ABS)) return 1;
        const float f = kvqo_rms_factor(xr, D, eps);
        for (int d = 0; d < D; ++d) {
            const float t = xr[d] * f;
            yr[d] = w ? t * w[d] : t;
        }
        if (h > 0) {
            if (pos[r] < 0 || pos[r] >= rope_positions) return 1;
            const float *c = cos_tab + (int64_t)pos[r] * h;
            const float *s = sin_tab + (int64_t)pos[r] * h;
            for (int j = 0; j < h; ++j) {
                const float a = yr[j], b = yr[j + h];
                const float ac = a * c[j], bs = b * s[j], bc = b * c[j], as = a * s[j];
                yr[j] = ac - bs;
                yr[j + h] = bc + as;
            }
        }
        for (int d = 0; d < D; ++d)
            if (!(fabsf(yr[d]) <= KVQO_MAX_ABS)) return 1;
    }
    return 0;
}

/* Threads an OpenMP region would use (1 without OpenMP). */
int kvqo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

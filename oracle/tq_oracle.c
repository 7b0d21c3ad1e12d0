/*
 * tq_oracle.c -- plain, slow CPU reference for TurboQuant speculative-decode
 * verification attention over a 3-/4-/8-bit-key, 4-bit-value KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or generator with
 * the HIP library; the two meet only in the documented byte layout of the
 * cache and in seeded input arrays.
 *
 * Sources (the pages are cited by title and section):
 *  - "Speculative decoding on Intel Arc: TurboQuant KV + a fused N_spec
 *    kernel" (turboquant-xpu blog, 2026-04-14), Context: keys are rotated by
 *    a Walsh-Hadamard transform and coded with a precomputed Lloyd-Max
 *    codebook, values get uniform scalar quantisation; the k3v4_nc preset is
 *    3-bit MSE keys + 4-bit values + norm correction, and the method spans
 *    3-4 bits per coordinate (TL;DR and Context: 3-8x capacity).  The
 *    k4v4_nc preset is the same key coder with a 16-level codebook [R23].
 *    Part 3: the decode
 *    loop does "bit-unpack + centroid gather + norm correction" per key tile,
 *    Q arrives already rotated, online softmax over N_spec queries.  Part 4:
 *    query n of the speculative window attends to cached_len + n + 1 tokens.
 *    Part 6: the k8v4 dequant is an FP8 bitcast.  Part 2 (Roofline): the
 *    k8v4 slot is 196 B per token and KV head.
 *  - "Three SYCL attempts on Arc B70" (turboquant-xpu blog, 2026-04-15),
 *    TL;DR: the PoC shape N_spec=8, B=4, Hq=32, Hk=4, D=128, seqlen=8192.
 *
 * Where the pages leave a step open, this file takes one explicit reading;
 * every reading is tagged [Rn] where it is taken.  Arithmetic:
 *  - store: IEEE binary32, round-to-nearest-even, no FMA contraction
 *    (compile with -ffp-contract=off), correctly rounded sqrtf and '/'.
 *    Codes are integers decided in binary32, so they are exact by definition.
 *  - verify: binary64 throughout (the plain definition of softmax attention).
 *
 * D is fixed at 128 (the only head size the pages use).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TQO_D 128
#define TQO_BLOCK 16

enum { TQO_K8V4 = 1, TQO_K3V4_NC = 2, TQO_K4V4_NC = 3 };

/* Levels of the Lloyd-Max key codebook: 8 (3-bit codes) or 16 (4-bit codes);
 * 0 for the FP8-key preset. */
static int lm_levels(int preset)
{
    return preset == TQO_K3V4_NC ? 8 : (preset == TQO_K4V4_NC ? 16 : 0);
}

/* ------------------------------------------------------------------------ */
/* binary16 <-> binary32 (IEEE 754), written out bit by bit.                 */
/* ------------------------------------------------------------------------ */

float tqo_half_to_float(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15);
    uint32_t e = (h >> 10) & 0x1F;
    uint32_t m = h & 0x3FF;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24); /* subnormal (or zero): m * 2^-24, exact */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(m | 0x400), (int)e - 25); /* (1024+m) * 2^(e-25) */
    return sign ? -v : v;
}

/* Round-to-nearest-even; overflow goes to infinity; every NaN becomes the
 * canonical quiet NaN 0x7E00 (sign dropped). */
uint16_t tqo_float_to_half(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7FFFFFFFu;
    if (ax > 0x7F800000u)
        return 0x7E00;
    if (ax == 0x7F800000u)
        return sign | 0x7C00;
    int e = (int)(ax >> 23) - 127;
    if (e >= -14) {
        if (e > 15)
            return sign | 0x7C00;
        uint32_t mant = ax & 0x7FFFFFu;
        uint32_t h = ((uint32_t)(e + 15) << 10) | (mant >> 13);
        uint32_t rem = mant & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u)))
            h += 1; /* a carry into the exponent is the correct result */
        if (h >= 0x7C00u)
            return sign | 0x7C00;
        return sign | (uint16_t)h;
    }
    /* below the binary16 normal range: multiple of 2^-24, RNE via rintf */
    float a;
    memcpy(&a, &ax, 4);
    float q = rintf(a * 16777216.0f); /* exact scaling by 2^24 */
    return sign | (uint16_t)q;          /* q == 1024 is the smallest normal */
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3 ("e4m3fn"): bias 7, no infinities, 0x7F/0xFF are NaN,        */
/* largest finite 448.  Decoding is the format's definition; encoding is     */
/* round-to-nearest-even with saturation to +-448 [R8].                      */
/* ------------------------------------------------------------------------ */

float tqo_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    float v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexpf((float)m, -9);
    else
        v = ldexpf((float)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

uint8_t tqo_e4m3_encode(float x)
{
    if (isnan(x))
        return 0x7F;
    uint8_t s = signbit(x) ? 0x80 : 0x00;
    float a = fabsf(x);
    if (a >= 448.0f)
        return s | 0x7E; /* saturate (this includes +-inf) */
    if (a < 0.015625f) { /* below 2^-6: subnormal grid of step 2^-9 */
        float q = rintf(a * 512.0f);   /* exact scaling, RNE */
        return s | (uint8_t)q;         /* q == 8 is the smallest normal 0x08 */
    }
    int E;
    frexpf(a, &E);             /* a = f * 2^E, f in [0.5, 1): exponent E-1 */
    int e = E - 1;
    float frac = ldexpf(a, -e) - 1.0f; /* in [0, 1), exact */
    float q = rintf(frac * 8.0f);      /* mantissa, RNE */
    int mi = (int)q;
    if (mi == 8) {
        mi = 0;
        e += 1;
    }
    int code = ((e + 7) << 3) | mi;
    if (code > 0x7E)
        code = 0x7E;
    return s | (uint8_t)code;
}

/* ------------------------------------------------------------------------ */
/* Lloyd-Max codebook for N(0, 1/D) [R4], 8 levels (3 bits).                */
/* Lloyd's two optimality conditions are iterated in binary64: each level is */
/* the conditional mean of its cell, each threshold the midpoint of its two  */
/* neighbours.  The unit-variance levels u_j are computed and then divided   */
/* by sqrt(128); the tables are the binary32 roundings of                    */
/*   c_j   = u_j / sqrt(128)                                                 */
/*   tau_j = ((u_{j-1} + u_j) / 2) / sqrt(128)          (j = 1..7)           */
/* ------------------------------------------------------------------------ */

static double std_pdf(double z) { return exp(-0.5 * z * z) * 0.39894228040143267794; }

/* P(a < Z < b) for a standard normal Z, evaluated on the side of zero where
 * erfc does not cancel. */
static double std_mass(double a, double b)
{
    const double r2 = 0.70710678118654752440;
    if (a >= 0.0)
        return 0.5 * (erfc(a * r2) - erfc(b * r2));
    if (b <= 0.0)
        return 0.5 * (erfc(-b * r2) - erfc(-a * r2));
    return 1.0 - 0.5 * erfc(-a * r2) - 0.5 * erfc(b * r2);
}

/* E[Z | a < Z < b] = (pdf(a) - pdf(b)) / P(a < Z < b). */
static double std_cond_mean(double a, double b)
{
    double pa = isinf(a) ? 0.0 : std_pdf(a);
    double pb = isinf(b) ? 0.0 : std_pdf(b);
    return (pa - pb) / std_mass(a, b);
}

/* Unit-variance Lloyd-Max levels u[0..nl-1] and thresholds t[0..nl-2]
 * (fp64): Lloyd's iteration (each threshold the midpoint of its two levels,
 * each level the mean of its cell) from evenly spaced levels 0.5 apart. */
void tqo_lloyd_max_unit_n(int nl, double *u, double *t, int iters)
{
    for (int j = 0; j < nl; ++j)
        u[j] = -0.25 * (nl - 1) + 0.5 * j; /* any ordered start converges for N(0,1) */
    for (int it = 0; it < iters; ++it) {
        for (int j = 1; j < nl; ++j)
            t[j - 1] = 0.5 * (u[j - 1] + u[j]);
        for (int j = 0; j < nl; ++j) {
            double lo = (j == 0) ? -INFINITY : t[j - 1];
            double hi = (j == nl - 1) ? INFINITY : t[j];
            u[j] = std_cond_mean(lo, hi);
        }
    }
    for (int j = 1; j < nl; ++j)
        t[j - 1] = 0.5 * (u[j - 1] + u[j]);
}

void tqo_lloyd_max_unit(double *u, double *t, int iters) { tqo_lloyd_max_unit_n(8, u, t, iters); }

/* The N(0, 1/128) codebook of nl levels (8 or 16) as binary32: levels
 * u_j / sqrt(128), thresholds t_j / sqrt(128) [R4]. */
void tqo_codebook_n(int nl, float *centroids, float *thresholds)
{
    double u[16], t[15];
    tqo_lloyd_max_unit_n(nl, u, t, 2000);
    const double s = sqrt(128.0);
    for (int j = 0; j < nl; ++j)
        centroids[j] = (float)(u[j] / s);
    for (int j = 0; j < nl - 1; ++j)
        thresholds[j] = (float)(t[j] / s);
}

void tqo_codebook(float *centroids8, float *thresholds7) { tqo_codebook_n(8, centroids8, thresholds7); }

/* ------------------------------------------------------------------------ */
/* Walsh-Hadamard transform (Sylvester order) and the fixed summation tree.  */
/* ------------------------------------------------------------------------ */

/* Unnormalised in-place WHT [R1]: butterflies (a, b) -> (a + b, a - b) on
 * index pairs (j, j + h) with bit h of j clear, for h = 1, 2, 4, ..., 64 in
 * that order.  The result is H128 x with H_ij = (-1)^popcount(i & j). */
void tqo_wht128_f32(float *a)
{
    for (int h = 1; h < TQO_D; h <<= 1)
        for (int j = 0; j < TQO_D; ++j)
            if (!(j & h)) {
                float x = a[j], y = a[j + h];
                a[j] = x + y;
                a[j + h] = x - y;
            }
}

/* Sum of squares by the stride-halving tree [R3]: a[i] = x[i]*x[i], then for
 * s = 64, 32, ..., 1: a[i] = a[i] + a[i + s] for i < s.  Returns a[0]. */
float tqo_tree_sumsq_f32(const float *x)
{
    float a[TQO_D];
    for (int i = 0; i < TQO_D; ++i)
        a[i] = x[i] * x[i];
    for (int s = TQO_D / 2; s >= 1; s >>= 1)
        for (int i = 0; i < s; ++i)
            a[i] = a[i] + a[i + s];
    return a[0];
}

/* ------------------------------------------------------------------------ */
/* Quantisers (one token-head vector of D = 128 binary16 values).            */
/* ------------------------------------------------------------------------ */

/* The Lloyd-Max cell of y: #{ j : y >= tau_j } over the nl - 1 thresholds,
 * so a value on a threshold goes to the upper cell and NaN to cell 0 [R5]. */
int tqo_lloyd_code(int nl, const float *th, float y)
{
    int c = 0;
    for (int j = 0; j < nl - 1; ++j)
        if (y >= th[j])
            c++;
    return c;
}

/* Lloyd-Max keys (k3v4_nc: nl = 8, k4v4_nc: nl = 16): norm, rotation,
 * codes against the nl-level codebook, norm correction.
 *   n     = sqrtf(tree sum of x^2)
 *   y_i   = WHT(x)_i * r,  r = 1 / (sqrt(128) * n)          (rotated unit vector)
 *   code  = #{ j : y >= tau_j }  (0 .. nl-1)                [R5]
 *   gamma = 1 / sqrtf(tree sum of c[code]^2)                [R6]
 *   stored: codes, n_h = half(n), g_h = half(gamma)
 * so that the dequantised rotated key c[code] * n * gamma has norm n. */
void tqo_quant_key_lm(int nl, const uint16_t *kh, const float *cb, const float *th,
                      uint8_t *codes, uint16_t *n_h, uint16_t *g_h)
{
    float x[TQO_D], z[TQO_D], chat[TQO_D];
    for (int i = 0; i < TQO_D; ++i)
        x[i] = tqo_half_to_float(kh[i]);
    float n = sqrtf(tqo_tree_sumsq_f32(x));
    memcpy(z, x, sizeof z);
    tqo_wht128_f32(z);
    float r = 1.0f / (sqrtf(128.0f) * n);
    for (int i = 0; i < TQO_D; ++i) {
        int c = tqo_lloyd_code(nl, th, z[i] * r);
        codes[i] = (uint8_t)c;
        chat[i] = cb[c];
    }
    float g = 1.0f / sqrtf(tqo_tree_sumsq_f32(chat));
    *n_h = tqo_float_to_half(n);
    *g_h = tqo_float_to_half(g);
}

void tqo_quant_key_k3(const uint16_t *kh, const float *cb, const float *th,
                      uint8_t *codes, uint16_t *n_h, uint16_t *g_h)
{
    tqo_quant_key_lm(8, kh, cb, th, codes, n_h, g_h);
}

/* k8v4 keys [R8]: per-token scale s = half(amax / 448), codes e4m3(x / s);
 * all codes are 0 when s rounds to 0.  No rotation. */
void tqo_quant_key_k8(const uint16_t *kh, uint8_t *codes, uint16_t *s_h)
{
    float x[TQO_D], amax = 0.0f;
    for (int i = 0; i < TQO_D; ++i) {
        x[i] = tqo_half_to_float(kh[i]);
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    uint16_t sh = tqo_float_to_half(amax / 448.0f);
    float s = tqo_half_to_float(sh);
    for (int i = 0; i < TQO_D; ++i)
        codes[i] = (s == 0.0f) ? 0 : tqo_e4m3_encode(x[i] / s);
    *s_h = sh;
}

/* Values [R9]: asymmetric min-max 4-bit codes.
 *   zero = half(vmin + 0) (exact; -0 -> +0), scale = half((vmax - vmin) / 15)
 *   q = rintf((v - zero) / scale); code = 0 unless q > 0, 15 if q >= 15
 * (so NaN gives 0); all codes are 0 when scale rounds to 0. */
void tqo_quant_val(const uint16_t *vh, uint8_t *codes, uint16_t *scale_h, uint16_t *zero_h)
{
    float v[TQO_D];
    float vmin = INFINITY, vmax = -INFINITY; /* NaN elements never win a compare */
    for (int i = 0; i < TQO_D; ++i) {
        v[i] = tqo_half_to_float(vh[i]);
        if (v[i] < vmin)
            vmin = v[i];
        if (v[i] > vmax)
            vmax = v[i];
    }
    uint16_t zh = tqo_float_to_half(vmin + 0.0f); /* exact; -0 becomes +0 */
    float zero = tqo_half_to_float(zh);
    uint16_t sc = tqo_float_to_half((vmax - vmin) / 15.0f);
    float s = tqo_half_to_float(sc);
    for (int i = 0; i < TQO_D; ++i) {
        int c = 0;
        if (s != 0.0f) {
            float q = rintf((v[i] - zero) / s);
            if (q > 0.0f)
                c = (q >= 15.0f) ? 15 : (int)q;
        }
        codes[i] = (uint8_t)c;
    }
    *scale_h = sc;
    *zero_h = zh;
}

/* ------------------------------------------------------------------------ */
/* Physical cache layout [R7], [R10], [R11].                                 */
/*                                                                           */
/* Per (b, hk) the sequence is cut into 16-token blocks; block blk of (b,hk) */
/* starts at base + ((b*Hk + hk)*nblk + blk) * block_bytes, nblk =           */
/* ceil(max_seq/16).  Token tb = pos % 16 of a block.                        */
/*                                                                           */
/* k3v4_nc block (1920 B = 16 x 120):                                        */
/*   [0, 768)     key codes, 48 B per token at tb*48 (see pack_k3_codes)     */
/*   [768, 1792)  value nibbles (see val_byte_offset)                        */
/*   [1792,1824)  n_h[16]   [1824,1856) gamma_h[16]                           */
/*   [1856,1888)  vscale_h[16]  [1888,1920) vzero_h[16]                      */
/* k4v4_nc block (2176 B = 16 x 136):                                        */
/*   [0, 1024)    key nibbles, 64 B per token at tb*64 (see pack_k4_codes)   */
/*   [1024,2048)  value nibbles                                              */
/*   [2048,2080)  n_h[16]   [2080,2112) gamma_h[16]                           */
/*   [2112,2144)  vscale_h[16]  [2144,2176) vzero_h[16]                      */
/* k8v4 block (3168 B = 16 x 198):                                           */
/*   [0, 2048)    e4m3 key codes, 128 B per token at tb*128, byte d = coord d*/
/*   [2048,3072)  value nibbles                                              */
/*   [3072,3104)  kscale_h[16]  [3104,3136) vscale_h[16]  [3136,3168) vzero_h */
/* binary16 fields and dwords are little-endian.                             */
/* ------------------------------------------------------------------------ */

size_t tqo_slot_bytes(int preset)
{
    return preset == TQO_K3V4_NC ? 120 : (preset == TQO_K4V4_NC ? 136 : 198);
}
size_t tqo_block_bytes(int preset) { return TQO_BLOCK * tqo_slot_bytes(preset); }

/* Offsets inside a block: value nibbles, then the four binary16 fields
 * (Lloyd-Max presets: n_h, gamma_h, vscale_h, vzero_h; k8v4: kscale_h,
 * vscale_h, vzero_h), 32 B each. */
static size_t val_region(int preset)
{
    return preset == TQO_K3V4_NC ? 768 : (preset == TQO_K4V4_NC ? 1024 : 2048);
}
static size_t meta_region(int preset) { return val_region(preset) + 1024; }

/* Value nibbles: byte p (0..63) of a token holds coordinate 2p in its low
 * and 2p+1 in its high nibble.  Byte p = 2i + e of token tb lives in dword
 * ((i*2 + h)*2 + e)*2 + q  (h = tb/8, q = (tb/4)%2) at byte position
 * {0, 2, 1, 3}[tb % 4]. */
static size_t val_byte_offset(int tb, int p)
{
    static const int posmap[4] = {0, 2, 1, 3};
    int i = p / 2, e = p % 2, h = tb / 8, q = (tb / 4) % 2;
    size_t dw = (size_t)(((i * 2 + h) * 2 + e) * 2 + q);
    return dw * 4 + (size_t)posmap[tb % 4];
}

/* k3 key codes of one token (128 codes of 3 bits) -> 48 bytes.
 * Coordinate d = 64h + 32g + 8k + e (h, g in {0,1}; k in 0..3; e in 0..7)
 * goes to the dword triple W0,W1,W2 = dwords 6h+3g+{0,1,2}, byte lane
 * b = e % 4, slot sl = 2k + e/4, with these bit positions inside the lane:
 *   sl 0: W0 bits 0-2   sl 1: W0 bits 3-5   sl 2: W1 bits 0-2
 *   sl 3: W1 bits 3-5   sl 4: W2 bits 0-2   sl 5: W2 bits 3-5
 *   sl 6: code bits 0,1 -> W0 bits 6,7, code bit 2 -> W2 bit 6
 *   sl 7: code bits 0,1 -> W1 bits 6,7, code bit 2 -> W2 bit 7          */
static void pack_k3_codes(const uint8_t *codes, uint8_t *out48)
{
    uint32_t w[12];
    memset(w, 0, sizeof w);
    for (int d = 0; d < TQO_D; ++d) {
        int h = d / 64, g = (d / 32) % 2, k = (d / 8) % 4, e = d % 8;
        int b = e % 4, sl = 2 * k + e / 4;
        uint32_t c = codes[d] & 7u;
        uint32_t *W = &w[6 * h + 3 * g];
        int sh = 8 * b;
        switch (sl) {
        case 0: W[0] |= c << sh; break;
        case 1: W[0] |= c << (sh + 3); break;
        case 2: W[1] |= c << sh; break;
        case 3: W[1] |= c << (sh + 3); break;
        case 4: W[2] |= c << sh; break;
        case 5: W[2] |= c << (sh + 3); break;
        case 6:
            W[0] |= (c & 3u) << (sh + 6);
            W[2] |= (c >> 2) << (sh + 6);
            break;
        default:
            W[1] |= (c & 3u) << (sh + 6);
            W[2] |= (c >> 2) << (sh + 7);
            break;
        }
    }
    for (int j = 0; j < 12; ++j)
        for (int by = 0; by < 4; ++by)
            out48[4 * j + by] = (uint8_t)(w[j] >> (8 * by));
}

static void unpack_k3_codes(const uint8_t *in48, uint8_t *codes)
{
    uint32_t w[12];
    for (int j = 0; j < 12; ++j)
        w[j] = (uint32_t)in48[4 * j] | ((uint32_t)in48[4 * j + 1] << 8) |
               ((uint32_t)in48[4 * j + 2] << 16) | ((uint32_t)in48[4 * j + 3] << 24);
    for (int d = 0; d < TQO_D; ++d) {
        int h = d / 64, g = (d / 32) % 2, k = (d / 8) % 4, e = d % 8;
        int b = e % 4, sl = 2 * k + e / 4;
        const uint32_t *W = &w[6 * h + 3 * g];
        int sh = 8 * b;
        uint32_t c;
        switch (sl) {
        case 0: c = W[0] >> sh; break;
        case 1: c = W[0] >> (sh + 3); break;
        case 2: c = W[1] >> sh; break;
        case 3: c = W[1] >> (sh + 3); break;
        case 4: c = W[2] >> sh; break;
        case 5: c = W[2] >> (sh + 3); break;
        case 6: c = ((W[0] >> (sh + 6)) & 3u) | (((W[2] >> (sh + 6)) & 1u) << 2); break;
        default: c = ((W[1] >> (sh + 6)) & 3u) | (((W[2] >> (sh + 7)) & 1u) << 2); break;
        }
        codes[d] = (uint8_t)(c & 7u);
    }
}

/* k4 key codes of one token (128 codes of 4 bits) -> 64 bytes [R23].  The
 * stored nibble of code c (0..15, levels ascending; the codebook is
 * symmetric, c_(15-j) = -c_j) is sign-magnitude: bit 3 set for the
 * negative levels (c < 8), bits 0-2 the rank of |c_c| counted from zero,
 * i.e. nibble = c - 8 for c >= 8 and 8 + (7 - c) for c < 8.  Coordinate
 * d = 8j + e (j in 0..15, e in 0..7) goes to byte 4j + e % 4, low nibble
 * for e < 4 and high nibble for e >= 4. */
static uint8_t k4_nibble(uint8_t c) { return (uint8_t)(c >= 8 ? c - 8 : 8 + (7 - c)); }
static uint8_t k4_code(uint8_t nib) { return (uint8_t)(nib >= 8 ? 7 - (nib - 8) : nib + 8); }

static void pack_k4_codes(const uint8_t *codes, uint8_t *out64)
{
    memset(out64, 0, 64);
    for (int d = 0; d < TQO_D; ++d) {
        int j = d / 8, e = d % 8;
        out64[4 * j + e % 4] |= (uint8_t)((k4_nibble(codes[d] & 15u)) << (e < 4 ? 0 : 4));
    }
}

static void unpack_k4_codes(const uint8_t *in64, uint8_t *codes)
{
    for (int d = 0; d < TQO_D; ++d) {
        int j = d / 8, e = d % 8;
        codes[d] = k4_code((uint8_t)((in64[4 * j + e % 4] >> (e < 4 ? 0 : 4)) & 15u));
    }
}

static void put_u16(uint8_t *p, uint16_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
}
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Logical record of one token-head, unpacked. */
typedef struct {
    uint8_t kcode[TQO_D];
    uint8_t vcode[TQO_D];
    uint16_t kmeta0, kmeta1; /* k3/k4: n_h, gamma_h; k8: kscale_h, unused */
    uint16_t vscale, vzero;
} tqo_record;

void tqo_write_record(int preset, uint8_t *block, int tb, const uint8_t *kcode,
                      const uint8_t *vcode, uint16_t kmeta0, uint16_t kmeta1,
                      uint16_t vscale, uint16_t vzero)
{
    size_t voff = val_region(preset), mo = meta_region(preset);
    if (preset == TQO_K8V4) {
        memcpy(block + (size_t)tb * 128, kcode, TQO_D);
        put_u16(block + mo + 2 * tb, kmeta0);
        put_u16(block + mo + 32 + 2 * tb, vscale);
        put_u16(block + mo + 64 + 2 * tb, vzero);
    } else {
        if (preset == TQO_K3V4_NC)
            pack_k3_codes(kcode, block + (size_t)tb * 48);
        else
            pack_k4_codes(kcode, block + (size_t)tb * 64);
        put_u16(block + mo + 2 * tb, kmeta0);
        put_u16(block + mo + 32 + 2 * tb, kmeta1);
        put_u16(block + mo + 64 + 2 * tb, vscale);
        put_u16(block + mo + 96 + 2 * tb, vzero);
    }
    for (int p = 0; p < TQO_D / 2; ++p)
        block[voff + val_byte_offset(tb, p)] =
            (uint8_t)((vcode[2 * p] & 15u) | ((vcode[2 * p + 1] & 15u) << 4));
}

void tqo_read_record(int preset, const uint8_t *block, int tb, uint8_t *kcode,
                     uint8_t *vcode, uint16_t *kmeta0, uint16_t *kmeta1,
                     uint16_t *vscale, uint16_t *vzero)
{
    size_t voff = val_region(preset), mo = meta_region(preset);
    if (preset == TQO_K8V4) {
        memcpy(kcode, block + (size_t)tb * 128, TQO_D);
        *kmeta0 = get_u16(block + mo + 2 * tb);
        *kmeta1 = 0;
        *vscale = get_u16(block + mo + 32 + 2 * tb);
        *vzero = get_u16(block + mo + 64 + 2 * tb);
    } else {
        if (preset == TQO_K3V4_NC)
            unpack_k3_codes(block + (size_t)tb * 48, kcode);
        else
            unpack_k4_codes(block + (size_t)tb * 64, kcode);
        *kmeta0 = get_u16(block + mo + 2 * tb);
        *kmeta1 = get_u16(block + mo + 32 + 2 * tb);
        *vscale = get_u16(block + mo + 64 + 2 * tb);
        *vzero = get_u16(block + mo + 96 + 2 * tb);
    }
    for (int p = 0; p < TQO_D / 2; ++p) {
        uint8_t by = block[voff + val_byte_offset(tb, p)];
        vcode[2 * p] = by & 15u;
        vcode[2 * p + 1] = by >> 4;
    }
}

static uint8_t *block_ptr(int preset, uint8_t *base, int Hk, int max_seq, int b, int hk, int pos)
{
    size_t nblk = (size_t)((max_seq + TQO_BLOCK - 1) / TQO_BLOCK);
    size_t idx = ((size_t)b * (size_t)Hk + (size_t)hk) * nblk + (size_t)(pos / TQO_BLOCK);
    return base + idx * tqo_block_bytes(preset);
}

/* ------------------------------------------------------------------------ */
/* store: quantise T new tokens (all Hk heads) into the cache.               */
/* K, V: binary16 [T, Hk, 128]; token t goes to (seq_idx[t], pos[t]).        */
/* Returns 0, or -1 on an out-of-range index (nothing written for it).       */
/* ------------------------------------------------------------------------ */

int tqo_store(int preset, int B, int Hk, int max_seq, uint8_t *cache, const uint16_t *K,
              const uint16_t *V, const int32_t *seq_idx, const int32_t *pos, int T)
{
    float cb[16], th[15];
    const int nl = lm_levels(preset);
    if (nl)
        tqo_codebook_n(nl, cb, th);
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (long th_i = 0; th_i < (long)T * Hk; ++th_i) {
        int t = (int)(th_i / Hk), hk = (int)(th_i % Hk);
        int b = seq_idx[t], p = pos[t];
        if (b < 0 || b >= B || p < 0 || p >= max_seq) {
            bad = 1;
            continue;
        }
        const uint16_t *kh = K + ((size_t)t * Hk + hk) * TQO_D;
        const uint16_t *vh = V + ((size_t)t * Hk + hk) * TQO_D;
        uint8_t kc[TQO_D], vc[TQO_D];
        uint16_t m0 = 0, m1 = 0, vs, vz;
        if (nl)
            tqo_quant_key_lm(nl, kh, cb, th, kc, &m0, &m1);
        else
            tqo_quant_key_k8(kh, kc, &m0);
        tqo_quant_val(vh, vc, &vs, &vz);
        tqo_write_record(preset, block_ptr(preset, cache, Hk, max_seq, b, hk, p), p % TQO_BLOCK,
                         kc, vc, m0, m1, vs, vz);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* store into a paged pool: page p holds the 16-token blocks of every KV     */
/* head, head hk's at pool + (p * Hk + hk) * block bytes (the pages' cache   */
/* is counted as blocks of 16 tokens x Hk heads: "Speculative decoding on    */
/* Intel Arc", Part 2, Roofline).  Token t goes to slot slots[t] =            */
/* page * 16 + position in the page; a negative slot is padding (skipped).   */
/* Returns 0, or -1 when a page is outside the pool (nothing written for it).*/
/* ------------------------------------------------------------------------ */

int tqo_store_paged(int preset, int Hk, int num_pages, uint8_t *pool, const uint16_t *K,
                    const uint16_t *V, const int32_t *slots, int T)
{
    float cb[16], th[15];
    const int nl = lm_levels(preset);
    if (nl)
        tqo_codebook_n(nl, cb, th);
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (long th_i = 0; th_i < (long)T * Hk; ++th_i) {
        int t = (int)(th_i / Hk), hk = (int)(th_i % Hk);
        int sl = slots[t];
        if (sl < 0)
            continue;
        int page = sl / TQO_BLOCK, tb = sl % TQO_BLOCK;
        if (page >= num_pages) {
            bad = 1;
            continue;
        }
        const uint16_t *kh = K + ((size_t)t * Hk + hk) * TQO_D;
        const uint16_t *vh = V + ((size_t)t * Hk + hk) * TQO_D;
        uint8_t kc[TQO_D], vc[TQO_D];
        uint16_t m0 = 0, m1 = 0, vs, vz;
        if (nl)
            tqo_quant_key_lm(nl, kh, cb, th, kc, &m0, &m1);
        else
            tqo_quant_key_k8(kh, kc, &m0);
        tqo_quant_val(vh, vc, &vs, &vz);
        uint8_t *blk = pool + ((size_t)page * (size_t)Hk + (size_t)hk) * tqo_block_bytes(preset);
        tqo_write_record(preset, blk, tb, kc, vc, m0, m1, vs, vz);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantisation of one token-head (binary64).                              */
/*   k3v4_nc, k4v4_nc: khat_rot[d] = c[code] * n_h * gamma_h (rotated space) */
/*   k8v4:    khat[d]     = e4m3(code) * kscale_h                            */
/*   values:  vhat[d]     = code * vscale_h + vzero_h                        */
/* ------------------------------------------------------------------------ */

void tqo_dequant(int preset, int Hk, int max_seq, const uint8_t *cache, int b, int hk, int t,
                 const float *cb, double *khat, double *vhat)
{
    uint8_t kc[TQO_D], vc[TQO_D];
    uint16_t m0, m1, vs, vz;
    const uint8_t *blk = block_ptr(preset, (uint8_t *)cache, Hk, max_seq, b, hk, t);
    tqo_read_record(preset, blk, t % TQO_BLOCK, kc, vc, &m0, &m1, &vs, &vz);
    double vscale = tqo_half_to_float(vs), vzero = tqo_half_to_float(vz);
    if (preset != TQO_K8V4) {
        double f = (double)tqo_half_to_float(m0) * (double)tqo_half_to_float(m1);
        for (int d = 0; d < TQO_D; ++d)
            khat[d] = (double)cb[kc[d]] * f;
    } else {
        double s = tqo_half_to_float(m0);
        for (int d = 0; d < TQO_D; ++d)
            khat[d] = (double)tqo_e4m3_decode(kc[d]) * s;
    }
    for (int d = 0; d < TQO_D; ++d)
        vhat[d] = (double)vc[d] * vscale + vzero;
}

/* Normalised Hadamard applied to a query (binary64, dense closed form):
 * q'_i = sum_j (-1)^popcount(i & j) q_j / sqrt(128). */
static void hadamard_f64(const double *q, double *out)
{
    const double s = 1.0 / sqrt(128.0);
    for (int i = 0; i < TQO_D; ++i) {
        double acc = 0.0;
        for (int j = 0; j < TQO_D; ++j)
            acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -q[j] : q[j];
        out[i] = acc * s;
    }
}

/* ------------------------------------------------------------------------ */
/* verify: N_spec-query attention over the quantised cache (binary64).       */
/*   Q: [N, B, Hq, 128] binary32 (q_dtype 0) or binary16 (q_dtype 1)         */
/*   seq_lens[b]: tokens in the cache for sequence b, the N new ones         */
/*   included; cached = seq_lens[b] - N                              [R13]  */
/*   hk = hq / (Hq/Hk)                                               [R12]  */
/*   E(n) = causal ? min(cached + n + 1, seq_len) : seq_len                  */
/*   s_t  = sm_scale * <q', khat_t>  for t < E (k3/k4: q' = H q, k8: q' = q) */
/*   out  = sum_t softmax(s)_t vhat_t          (two passes, no splits)       */
/* sm_scale == 0 selects 1/sqrt(128) [R14].  out: binary64 [N, B, Hq, 128].  */
/* ------------------------------------------------------------------------ */

int tqo_verify(int preset, int B, int Hk, int max_seq, const uint8_t *cache, const void *Q,
               int q_dtype, const int32_t *seq_lens, int N, int Hq, int causal, double sm_scale,
               double *out)
{
    if (Hq % Hk != 0 || N < 1)
        return -1;
    int G = Hq / Hk;
    float cb[16], th[15];
    const int nl = lm_levels(preset);
    if (nl)
        tqo_codebook_n(nl, cb, th);
    if (sm_scale == 0.0)
        sm_scale = 1.0 / sqrt((double)TQO_D);
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > max_seq)
            return -1;

#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < (long)B * Hk; ++u) {
        int b = (int)(u / Hk), hk = (int)(u % Hk);
        int L = seq_lens[b], cached = L - N;
        double *kh = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * TQO_D);
        double *vh = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * TQO_D);
        double *s = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        for (int t = 0; t < L; ++t)
            tqo_dequant(preset, Hk, max_seq, cache, b, hk, t, cb, kh + (size_t)t * TQO_D,
                        vh + (size_t)t * TQO_D);
        for (int g = 0; g < G; ++g) {
            int hq = hk * G + g;
            for (int n = 0; n < N; ++n) {
                double q[TQO_D], qp[TQO_D];
                size_t qoff = (((size_t)n * B + b) * Hq + hq) * TQO_D;
                for (int d = 0; d < TQO_D; ++d)
                    q[d] = q_dtype == 0 ? (double)((const float *)Q)[qoff + d]
                                        : (double)tqo_half_to_float(((const uint16_t *)Q)[qoff + d]);
                if (preset != TQO_K8V4)
                    hadamard_f64(q, qp);
                else
                    memcpy(qp, q, sizeof q);
                int E = causal ? cached + n + 1 : L;
                if (E > L)
                    E = L;
                double *o = out + qoff;
                if (E <= 0) {
                    for (int d = 0; d < TQO_D; ++d)
                        o[d] = NAN;
                    continue;
                }
                double m = -INFINITY;
                for (int t = 0; t < E; ++t) {
                    double acc = 0.0;
                    for (int d = 0; d < TQO_D; ++d)
                        acc += qp[d] * kh[(size_t)t * TQO_D + d];
                    s[t] = sm_scale * acc;
                    if (s[t] > m) /* a NaN score still reaches the output via exp */
                        m = s[t];
                }
                double l = 0.0;
                for (int d = 0; d < TQO_D; ++d)
                    o[d] = 0.0;
                for (int t = 0; t < E; ++t) {
                    double p = exp(s[t] - m);
                    l += p;
                    for (int d = 0; d < TQO_D; ++d)
                        o[d] += p * vh[(size_t)t * TQO_D + d];
                }
                for (int d = 0; d < TQO_D; ++d)
                    o[d] /= l;
            }
        }
        free(kh);
        free(vh);
        free(s);
    }
    return 0;
}

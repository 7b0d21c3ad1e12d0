/*
 * Sanitizer driver for the oracle (test infrastructure): the oracle's C
 * source compiled into one program with AddressSanitizer and
 * UndefinedBehaviorSanitizer, run over small stores, paged stores,
 * dequantisations and verifies of every preset, including the edge inputs
 * the tests use (zero, huge and NaN tokens, empty and clamped lengths,
 * out-of-range indices, padding slots).  Any sanitizer report aborts with a
 * non-zero status; the test that builds this program checks the status.
 */
#include "../../oracle/tq_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 88172645463325252ull;

static double urand(void) /* xorshift64, [0, 1) */
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) / 9007199254740992.0;
}

static double nrand(void) /* Box-Muller */
{
    double u = urand(), v = urand();
    if (u < 1e-300)
        u = 1e-300;
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}

static void fill_half(uint16_t *h, size_t n, double scale)
{
    for (size_t i = 0; i < n; ++i)
        h[i] = tqo_float_to_half((float)(nrand() * scale));
}

static int run_preset(int preset)
{
    const int B = 2, Hk = 2, Hq = 6, N = 3, S = 37, T = B * S;
    const size_t cb = (size_t)B * Hk * ((S + 15) / 16) * tqo_block_bytes(preset);
    uint8_t *cache = calloc(cb, 1);
    uint16_t *K = malloc(sizeof(uint16_t) * T * Hk * TQO_D);
    uint16_t *V = malloc(sizeof(uint16_t) * T * Hk * TQO_D);
    int32_t *si = malloc(sizeof(int32_t) * T), *po = malloc(sizeof(int32_t) * T);
    fill_half(K, (size_t)T * Hk * TQO_D, 1.0);
    fill_half(V, (size_t)T * Hk * TQO_D, 3.0);
    /* edge tokens: zero key, huge value, NaN key */
    memset(K, 0, sizeof(uint16_t) * TQO_D);
    for (int d = 0; d < TQO_D; ++d)
        V[TQO_D * Hk + d] = (d & 1) ? 0x7BFF : 0xFBFF;
    K[2 * TQO_D * Hk + 5] = 0x7E00;
    for (int t = 0; t < T; ++t) {
        si[t] = t / S;
        po[t] = t % S;
    }
    if (tqo_store(preset, B, Hk, S, cache, K, V, si, po, T) != 0)
        return 1;
    /* out-of-range indices are reported and skipped */
    si[0] = B;
    po[1] = S;
    if (tqo_store(preset, B, Hk, S, cache, K, V, si, po, 2) != -1)
        return 2;

    float c[16], t[15];
    const int nl = preset == TQO_K3V4_NC ? 8 : (preset == TQO_K4V4_NC ? 16 : 0);
    if (nl)
        tqo_codebook_n(nl, c, t);
    double kh[TQO_D], vh[TQO_D];
    for (int tt = 0; tt < S; tt += 7)
        tqo_dequant(preset, Hk, S, cache, 1, 1, tt, c, kh, vh);

    float *Q = malloc(sizeof(float) * N * B * Hq * TQO_D);
    for (int i = 0; i < N * B * Hq * TQO_D; ++i)
        Q[i] = (float)nrand();
    double *out = malloc(sizeof(double) * N * B * Hq * TQO_D);
    int32_t lens[2] = {S, 0}; /* a sequence with no token: NaN rows */
    for (int causal = 0; causal < 2; ++causal)
        if (tqo_verify(preset, B, Hk, S, cache, Q, 0, lens, N, Hq, causal, 0.0, out) != 0)
            return 3;
    lens[1] = S + 1; /* longer than the cache: refused */
    if (tqo_verify(preset, B, Hk, S, cache, Q, 0, lens, N, Hq, 1, 0.0, out) != -1)
        return 4;

    /* paged pool: 8 pages, padding and out-of-pool slots */
    const int pages = 8;
    uint8_t *pool = calloc((size_t)pages * Hk * tqo_block_bytes(preset), 1);
    int32_t slots[6] = {0, 17, -1, 8 * 16, 127, 33};
    if (tqo_store_paged(preset, Hk, pages, pool, K, V, slots, 6) != -1)
        return 5;

    free(pool);
    free(out);
    free(Q);
    free(po);
    free(si);
    free(V);
    free(K);
    free(cache);
    return 0;
}

int main(void)
{
    for (int p = 1; p <= 3; ++p) {
        int rc = run_preset(p);
        if (rc != 0) {
            printf("preset %d: check %d failed\n", p, rc);
            return 10 + rc;
        }
    }
    /* conversions over every binary16 pattern */
    for (uint32_t h = 0; h < 65536; ++h) {
        float f = tqo_half_to_float((uint16_t)h);
        (void)tqo_float_to_half(f);
        (void)tqo_e4m3_encode(f);
    }
    for (int cc = 0; cc < 256; ++cc)
        (void)tqo_e4m3_decode((uint8_t)cc);
    printf("oracle driver ok\n");
    return 0;
}

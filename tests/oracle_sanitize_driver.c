/*
 * Driver for the sanitizer build of the CPU oracle (test infrastructure, not part of the GPU
 * path): calls every function of oracle/msa_oracle.h on small inputs that reach its edge cases
 * (zero, tiny, subnormal-scale and saturating groups; ragged contexts; empty, short and tied
 * selection rows; ids that are -1, past the context or past the query position), so that an
 * AddressSanitizer / UndefinedBehaviorSanitizer build reports any out-of-bounds access, use of
 * uninitialized heap memory caught by ASan, or undefined behaviour. Test data come from a small
 * linear congruential generator; nothing here computes a step of the method.
 * Exit status 0 and the line "oracle sanitize run ok" on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/msa_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {  /* in [0, 1) */
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}
static float normalish(void) { return (float)(uniform() + uniform() + uniform() - 1.5) * 2.0f; }

static uint16_t bf16_bits_of(float x) {  /* truncation: any bit pattern is a valid input */
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

static void *xmalloc(size_t n) {
    void *p = malloc(n);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

int main(void) {
    enum { D = 128, G = 4 };
    double acc = 0.0;  /* results are summed so that no call is optimized away */

    /* scalar codecs: every byte, every nibble, a sweep of floats including edge values */
    for (int b = 0; b < 256; b++) acc += isnan(orc_e4m3_value((uint8_t)b)) ? 0.0 : orc_e4m3_value((uint8_t)b);
    for (int n = 0; n < 16; n++) acc += orc_e2m1_value((uint8_t)n);
    const float edges[] = {0.0f, -0.0f, 1e-30f, 1e-9f, 0.001953125f, 0.5f, 1.0f, 447.9f, 448.0f,
                           464.0f, 1e6f, 3.4e38f, INFINITY};
    for (size_t i = 0; i < sizeof edges / sizeof edges[0]; i++) {
        acc += orc_e4m3_encode(edges[i]) + orc_e2m1_encode_magnitude(edges[i]);
    }
    for (int i = 0; i < 4096; i++) {
        const float x = (float)(uniform() * 500.0);
        acc += orc_e4m3_encode(x) + orc_e2m1_encode_magnitude((float)(uniform() * 8.0));
    }
    for (int i = 0; i < 65536; i += 97) acc += isnan(orc_bf16_value((uint16_t)i)) ? 0.0 : 1.0;

    /* quantize / dequantize: 40 vectors, some of them all zero, tiny, huge or mixed */
    const int n_vec = 40;
    float *x = xmalloc(sizeof(float) * n_vec * D);
    for (int v = 0; v < n_vec; v++)
        for (int e = 0; e < D; e++) {
            float val = normalish();
            if (v == 0) val = 0.0f;
            if (v == 1) val *= 1e-12f;
            if (v == 2) val *= 1e6f;
            if (v == 3 && e % 16 == 3) val = 1e5f;
            if (v == 4 && e % 16 == 0) val = -0.0f;
            x[v * D + e] = val;
        }
    uint8_t *codes = xmalloc((size_t)n_vec * 64), *scales = xmalloc((size_t)n_vec * 8);
    orc_nvfp4_quantize(x, n_vec, codes, scales);
    double *deq = xmalloc(sizeof(double) * n_vec * D);
    orc_nvfp4_dequantize(codes, scales, n_vec, deq);
    for (int i = 0; i < n_vec * D; i++) acc += deq[i];
    uint8_t nib[16], sb;
    orc_nvfp4_quantize_group(x + 5 * D, nib, &sb);
    acc += sb;

    /* index scores over a ragged context (T not a multiple of 128), q = 3 rows per group */
    const int T = 300, q = 3, nb_out = 5;
    float *ik = xmalloc(sizeof(float) * T * D);
    for (int i = 0; i < T * D; i++) ik[i] = normalish();
    uint8_t *ikc = xmalloc((size_t)T * 64), *iks = xmalloc((size_t)T * 8);
    orc_nvfp4_quantize(ik, T, ikc, iks);
    uint16_t *qi = xmalloc(sizeof(uint16_t) * q * G * D);
    for (int i = 0; i < q * G * D; i++) qi[i] = bf16_bits_of(normalish());
    double *sc = xmalloc(sizeof(double) * q * G * nb_out);
    orc_index_scores(qi, ikc, iks, T, q, nb_out, sc);
    for (int i = 0; i < q * G * nb_out; i++) acc += isinf(sc[i]) ? 0.0 : sc[i];
    orc_index_scores_lse(qi, ikc, iks, T, q, nb_out, sc);
    for (int i = 0; i < q * G * nb_out; i++) acc += isinf(sc[i]) ? 0.0 : sc[i];
    orc_index_scores(qi, ikc, iks, 1, 1, 1, sc);  /* one token, one row */
    acc += sc[0];

    /* selection: empty, short, exactly 16, 17 and long rows, ties and -inf */
    const int lens[] = {0, 1, 15, 16, 17, 40, 300};
    double *row = xmalloc(sizeof(double) * 300);
    int32_t ids[64];
    for (size_t li = 0; li < sizeof lens / sizeof lens[0]; li++) {
        const int n = lens[li];
        for (int i = 0; i < n; i++) row[i] = (i % 7 == 0) ? 1.0 : (i % 11 == 0 ? -INFINITY : floor(uniform() * 4.0));
        for (int topk = 1; topk <= 64; topk *= 4) {
            double margin = 0.0;
            acc += orc_block_topk(row, n, topk, ids, &margin);
            for (int i = 0; i < topk; i++) acc += ids[i];
            acc += isfinite(margin) ? margin : 0.0;
        }
    }

    /* attention of one token over ids that include -1, a block past the context and a block
       past the query position */
    float *kv = xmalloc(sizeof(float) * T * G * D);
    uint8_t *kc = xmalloc((size_t)T * G * 64), *ks = xmalloc((size_t)T * G * 8);
    uint8_t *vc = xmalloc((size_t)T * G * 64), *vs = xmalloc((size_t)T * G * 8);
    for (int i = 0; i < T * G * D; i++) kv[i] = normalish();
    orc_nvfp4_quantize(kv, (int64_t)T * G, kc, ks);
    for (int i = 0; i < T * G * D; i++) kv[i] = normalish();
    orc_nvfp4_quantize(kv, (int64_t)T * G, vc, vs);
    uint16_t *qq = xmalloc(sizeof(uint16_t) * 64 * D);
    for (int i = 0; i < 64 * D; i++) qq[i] = bf16_bits_of(normalish());
    int32_t sel[G * 16];
    for (int g = 0; g < G; g++)
        for (int k = 0; k < 16; k++) sel[g * 16 + k] = k < 3 ? k : (k == 3 ? 7 : -1);
    double *out = xmalloc(sizeof(double) * 64 * D);
    const int64_t positions[] = {T - 1, 130, 0};
    for (int i = 0; i < 3; i++) {
        orc_sparse_attention_token(qq, kc, ks, vc, vs, T, sel, 16, positions[i], 0.0883883476, out);
        for (int j = 0; j < 64 * D; j++) acc += out[j];
    }
    orc_sparse_attention_token(qq, kc, ks, vc, vs, T, sel, 16, T - 1, -0.05, out);
    for (int j = 0; j < 64 * D; j++) acc += out[j];

    free(x); free(codes); free(scales); free(deq); free(ik); free(ikc); free(iks); free(qi);
    free(sc); free(row); free(kv); free(kc); free(ks); free(vc); free(vs); free(qq); free(out);
    printf("oracle sanitize run ok (checksum %.6g)\n", acc);
    return 0;
}

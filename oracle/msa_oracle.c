/*
 * Plain CPU oracle for the MiniMax Sparse Attention (MSA) decode path with NVFP4 caches.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. It shares no code, header, table or constant with the HIP path.
 *
 * Every routine is written for clarity, single-threaded, in fp64 wherever the method does
 * floating point, except where the method itself fixes fp32 (the quantizer's two fp32
 * divisions, see orc_nvfp4_quantize_group). Data are in plain logical layouts:
 *   NVFP4 vector of 128 elements = 64 code bytes (element 2i in the low nibble of byte i,
 *   element 2i+1 in the high nibble) + 8 scale bytes (scale g covers elements 16g..16g+15).
 *   Index keys:  codes [T][64],     scales [T][8]      (one shared head per token)
 *   K and V:     codes [T][4][64],  scales [T][4][8]   (4 KV heads per token)
 *   bf16 values are passed as their raw 16-bit patterns.
 *
 * Sources (web pages; cited by title and section):
 *   [M31]  "vLLM day-0 support for MiniMax-M3.1-Flash" (the vLLM post, read in its Spanish and
 *          Korean renderings): sections "MSA primer", "NVFP4 MSA kernel", "Indexer NVFP4 DCP",
 *          "NVIDIA Rubin optimized MSA".
 *   [M3]   "MiniMax M3 on vLLM" (Chinese rendering of the vLLM M3 post): sections
 *          "MSA mechanism", "MiniMax sparse attention backend", "Prefill execution",
 *          "Decode execution", "Speculative decoding in the decode kernels".
 *   [NOTES] "MiniMax-M3.1-Flash serving notes": sections "How MSA reads memory",
 *          "The capacity numbers".
 * Readings taken where the pages are silent are marked READING.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "msa_oracle.h"

/* ---------------------------------------------------------------- codec ---------------- */

/* E4M3 scale byte -> value. The pages name E4M3 for the NVFP4 block scale ([NOTES] "The
 * capacity numbers": one FP8 scale per 16 values; [M31] "NVFP4 MSA kernel": 256 possible
 * E4M3 scales). READING: the OCP FP8 E4M3 "FN" encoding: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, exponent 15 with mantissa 7 is NaN, largest
 * finite value 448, subnormals (exponent field 0) are (m/8) * 2^-6. */
double orc_e4m3_value(uint8_t b) {
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* E2M1 nibble -> value: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
 * subnormal (m * 0.5). This is the standard FP4 E2M1 element whose eight magnitudes the pages
 * count ([M31] "NVFP4 MSA kernel": eight E2M1 magnitudes). */
double orc_e2m1_value(uint8_t nibble) {
    int sign = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 3;
    int m = nibble & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

/* Non-negative fp32 -> E4M3 byte, nearest representable finite value, ties to the even
 * code, values beyond 448 saturate to 448 (READING: "satfinite"). Brute force over the 127
 * non-negative finite codes, so no rounding trick can be wrong. */
uint8_t orc_e4m3_encode(float x) {
    if (x > 448.0f) x = 448.0f; /* saturate first: far above 448 every distance would tie */
    uint8_t best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs(orc_e4m3_value((uint8_t)c) - (double)x);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = (uint8_t)c;
            best_d = d;
        }
    }
    return best;
}

/* Non-negative fp32 ratio -> E2M1 magnitude code 0..7: nearest of the eight magnitudes, ties
 * to the even code, saturating at 6 (READING: round-to-nearest-even on the E2M1 grid). */
uint8_t orc_e2m1_encode_magnitude(float r) {
    if (r > 6.0f) r = 6.0f; /* saturate first: far above 6 every distance would tie */
    uint8_t best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 8; c++) {
        double d = fabs(orc_e2m1_value((uint8_t)c) - (double)r);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = (uint8_t)c;
            best_d = d;
        }
    }
    return best;
}

/* NVFP4 quantization of one group of 16 contiguous elements ([NOTES] "The capacity numbers":
 * 4-bit values plus one FP8 scale per 16 values; scale = amax/6 per 16 contiguous elements,
 * as the workload recipe states).
 * READING (the pages give no rounding rule):
 *   s32 = amax / 6 in IEEE fp32 (round to nearest);  scale byte = E4M3 nearest-even of s32,
 *   saturating;  s = its value;  if s == 0 every magnitude is 0;  otherwise each element's
 *   magnitude code is the E2M1 nearest-even of the fp32 quotient |x| / s.  The sign bit is the
 *   sign bit of x, also when the magnitude rounds to 0.  No second, per-tensor scale.
 * nibbles[i] receives sign<<3 | magnitude for element i. */
void orc_nvfp4_quantize_group(const float *x, uint8_t *nibbles, uint8_t *scale_byte) {
    float amax = 0.0f;
    for (int i = 0; i < 16; i++) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    volatile float six = 6.0f;            /* keep the division an fp32 division */
    float s32 = amax / six;
    uint8_t sc = orc_e4m3_encode(s32);
    float s = (float)orc_e4m3_value(sc);  /* exact: every E4M3 value is an fp32 value */
    for (int i = 0; i < 16; i++) {
        uint8_t sign = signbit(x[i]) ? 8 : 0;
        uint8_t mag = 0;
        if (s > 0.0f) {
            volatile float r = fabsf(x[i]) / s;
            mag = orc_e2m1_encode_magnitude(r);
        }
        nibbles[i] = (uint8_t)(sign | mag);
    }
    *scale_byte = sc;
}

/* Quantize n_vec vectors of 128 fp32 elements into logical NVFP4 storage (72 B per vector:
 * 64 code bytes + 8 scale bytes). */
void orc_nvfp4_quantize(const float *x, int64_t n_vec, uint8_t *codes, uint8_t *scales) {
    uint8_t nib[16];
    for (int64_t v = 0; v < n_vec; v++) {
        for (int g = 0; g < 8; g++) {
            orc_nvfp4_quantize_group(x + v * 128 + g * 16, nib, scales + v * 8 + g);
            for (int i = 0; i < 8; i++)
                codes[v * 64 + g * 8 + i] = (uint8_t)(nib[2 * i] | (nib[2 * i + 1] << 4));
        }
    }
}

/* Exact dequantization: value = E2M1(code) * E4M3(scale) ([M31] "NVFP4 MSA kernel": a scaled
 * value is the E2M1 magnitude times the E4M3 scale with the sign applied). READING: the product
 * is kept exact (fp64 here); the pages' AMD table re-rounds it to FP8, their Rubin path keeps
 * scores exact ([M31] "NVIDIA Rubin optimized MSA"); the exact form is the definition. */
void orc_nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t n_vec, double *out) {
    for (int64_t v = 0; v < n_vec; v++)
        for (int e = 0; e < 128; e++) {
            uint8_t byte = codes[v * 64 + e / 2];
            uint8_t nib = (e & 1) ? (byte >> 4) : (byte & 15);
            out[v * 128 + e] = orc_e2m1_value(nib) * orc_e4m3_value(scales[v * 8 + e / 16]);
        }
}

double orc_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ---------------------------------------------------------------- indexer --------------- */

/* Index scores and per-block max-pool for one sequence ([M31] "MSA primer": one index query
 * per GQA group is scored against every key of the single shared index-key head, and the
 * token scores are max-pooled into one score per 128-token block; [M3] "MSA mechanism":
 * the partial last block is masked and the causal boundary inside a block is respected).
 *   q_idx  : [q][4][128] bf16 index queries of this sequence's q query tokens
 *   ik_*   : the sequence's index keys in logical token order, T tokens
 *   out    : [q][4][nb_out]; out = max over valid tokens of the block, -inf if none.
 * Query token j sits at position p = T - q + j (READING: the context length T counts the
 * query tokens, which are already in the cache). A token t is valid for j iff t <= p.
 * READING: the score is the plain dot product, no 1/sqrt(d), activation or weight. */
void orc_index_scores(const uint16_t *q_idx, const uint8_t *ik_codes, const uint8_t *ik_scales,
                      int32_t T, int32_t q, int32_t nb_out, double *out) {
    double *key = (double *)malloc(sizeof(double) * 128 * (size_t)(T > 0 ? T : 1));
    orc_nvfp4_dequantize(ik_codes, ik_scales, T, key);
    double qv[128];
    for (int j = 0; j < q; j++) {
        int64_t p = (int64_t)T - q + j;
        for (int g = 0; g < 4; g++) {
            for (int d = 0; d < 128; d++) qv[d] = orc_bf16_value(q_idx[((size_t)j * 4 + g) * 128 + d]);
            for (int blk = 0; blk < nb_out; blk++) {
                double best = -INFINITY;
                for (int64_t t = (int64_t)blk * 128; t < (int64_t)blk * 128 + 128; t++) {
                    if (t > p || t >= T) break;
                    double s = 0.0;
                    for (int d = 0; d < 128; d++) s += qv[d] * key[t * 128 + d];
                    if (s > best) best = s;
                }
                out[((size_t)j * 4 + g) * nb_out + blk] = best;
            }
        }
    }
    free(key);
}

/* The same scores with the block's log-sum-exp in place of its max ([M3] "Prefill execution":
 * the block-level reduction may be max or log-sum-exp depending on the model config).
 * READING: natural logarithm of the sum of exp of the plain token scores of the block's valid
 * tokens (no temperature), -inf if none; computed as m + log(sum exp(s - m)), m the max. */
void orc_index_scores_lse(const uint16_t *q_idx, const uint8_t *ik_codes, const uint8_t *ik_scales,
                          int32_t T, int32_t q, int32_t nb_out, double *out) {
    double *key = (double *)malloc(sizeof(double) * 128 * (size_t)(T > 0 ? T : 1));
    orc_nvfp4_dequantize(ik_codes, ik_scales, T, key);
    double qv[128], sc[128];
    for (int j = 0; j < q; j++) {
        int64_t p = (int64_t)T - q + j;
        for (int g = 0; g < 4; g++) {
            for (int d = 0; d < 128; d++) qv[d] = orc_bf16_value(q_idx[((size_t)j * 4 + g) * 128 + d]);
            for (int blk = 0; blk < nb_out; blk++) {
                int cnt = 0;
                double m = -INFINITY;
                for (int64_t t = (int64_t)blk * 128; t < (int64_t)blk * 128 + 128; t++) {
                    if (t > p || t >= T) break;
                    double s = 0.0;
                    for (int d = 0; d < 128; d++) s += qv[d] * key[t * 128 + d];
                    sc[cnt++] = s;
                    if (s > m) m = s;
                }
                double r = -INFINITY;
                if (cnt > 0) {
                    double sum = 0.0;
                    for (int i = 0; i < cnt; i++) sum += exp(sc[i] - m);
                    r = m + log(sum);
                }
                out[((size_t)j * 4 + g) * nb_out + blk] = r;
            }
        }
    }
    free(key);
}

/* ---------------------------------------------------------------- selection ------------- */

/* Block selection for one (sequence, query token, group) row ([M31] "MSA primer": keep the 16
 * best blocks with the most recent block always kept, at most 2,048 keys; [M3] "MSA
 * mechanism": local_blocks = 1, init_blocks = 0, the local block must not be counted twice).
 *   scores: the row's block scores for the n eligible blocks 0..n-1 (n = floor(p/128) + 1);
 *   forced block f = n - 1 (the block holding the query token, READING per token position).
 * READING: the forced block is one of the topk (cap topk*128 keys): if n <= topk all n blocks
 * are kept; otherwise f plus the best topk-1 of blocks 0..n-2 by (score descending, block
 * index ascending). ids_out[topk] is ascending, padded with -1.
 * margin: (lowest kept non-forced score - highest dropped score) / |lowest kept score|, or
 * +inf when nothing is dropped. Returns the number of ids written. */
int orc_block_topk(const double *scores, int32_t n, int32_t topk, int32_t *ids_out, double *margin) {
    for (int i = 0; i < topk; i++) ids_out[i] = -1;
    *margin = INFINITY;
    if (n <= 0) return 0;
    if (n <= topk) {
        for (int i = 0; i < n; i++) ids_out[i] = i;
        return n;
    }
    char *taken = (char *)calloc((size_t)n, 1);
    int count = 0;
    double low_kept = INFINITY;
    for (int k = 0; k < topk - 1; k++) {
        int arg = -1;
        for (int i = 0; i < n - 1; i++) {
            if (taken[i]) continue;
            if (arg < 0 || scores[i] > scores[arg]) arg = i; /* strict: earlier index wins ties */
        }
        taken[arg] = 1;
        if (scores[arg] < low_kept) low_kept = scores[arg];
    }
    taken[n - 1] = 1;
    double high_dropped = -INFINITY;
    for (int i = 0; i < n - 1; i++)
        if (!taken[i] && scores[i] > high_dropped) high_dropped = scores[i];
    for (int i = 0; i < n; i++)
        if (taken[i]) ids_out[count++] = i;
    *margin = (low_kept - high_dropped) / fabs(low_kept);
    free(taken);
    return count;
}

/* ---------------------------------------------------------------- attention ------------- */

/* Exact GQA attention of one query token over a given block list ([M31] "MSA primer" and its
 * Figure 1: every query head of a GQA group attends exactly to the blocks its group's indexer
 * selected; [M3] "Prefill execution": the result equals dense attention restricted to the
 * selected set, with an online-softmax-equivalent result).
 *   q       : [64][128] bf16 query heads of this token
 *   k_*,v_* : the sequence's K and V in logical order (T tokens, 4 heads)
 *   ids     : [4][n_ids] selected logical block ids per group (-1 entries are skipped)
 *   p       : the token's position; keys t <= p and t < T in the selected blocks are used
 *   scale   : softmax scale applied to q.k (READING: 1/sqrt(128))
 *   out     : [64][128]; head h belongs to group h/16 (READING: contiguous GQA groups).
 * A head with no valid key gets 0. */
void orc_sparse_attention_token(const uint16_t *q, const uint8_t *k_codes, const uint8_t *k_scales,
                                const uint8_t *v_codes, const uint8_t *v_scales, int32_t T,
                                const int32_t *ids, int32_t n_ids, int64_t p, double scale,
                                double *out) {
    int64_t cap = (int64_t)n_ids * 128;
    double *logit = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
    double kd[128], vd[128], qv[128];
    for (int h = 0; h < 64; h++) {
        int g = h / 16;
        for (int d = 0; d < 128; d++) qv[d] = orc_bf16_value(q[h * 128 + d]);
        int64_t n_keys = 0;
        for (int i = 0; i < n_ids; i++) {
            int32_t blk = ids[g * n_ids + i];
            if (blk < 0) continue;
            for (int64_t t = (int64_t)blk * 128; t < (int64_t)blk * 128 + 128; t++) {
                if (t > p || t >= T) break;
                orc_nvfp4_dequantize(k_codes + (t * 4 + g) * 64, k_scales + (t * 4 + g) * 8, 1, kd);
                double s = 0.0;
                for (int d = 0; d < 128; d++) s += qv[d] * kd[d];
                logit[n_keys] = s * scale;
                tok[n_keys] = t;
                n_keys++;
            }
        }
        for (int d = 0; d < 128; d++) out[h * 128 + d] = 0.0;
        if (n_keys == 0) continue;
        double mx = -INFINITY;
        for (int64_t i = 0; i < n_keys; i++)
            if (logit[i] > mx) mx = logit[i];
        double denom = 0.0;
        for (int64_t i = 0; i < n_keys; i++) {
            logit[i] = exp(logit[i] - mx);
            denom += logit[i];
        }
        for (int64_t i = 0; i < n_keys; i++) {
            int64_t t = tok[i];
            orc_nvfp4_dequantize(v_codes + (t * 4 + g) * 64, v_scales + (t * 4 + g) * 8, 1, vd);
            double w = logit[i] / denom;
            for (int d = 0; d < 128; d++) out[h * 128 + d] += w * vd[d];
        }
    }
    free(logit);
    free(tok);
}

/* Plain CPU oracle for the MSA decode path (test infrastructure only; see msa_oracle.c).
 * This header belongs to the oracle alone and is not shared with the HIP library. */
#ifndef MSA_ORACLE_H
#define MSA_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif
double orc_e4m3_value(uint8_t b);
double orc_e2m1_value(uint8_t nibble);
uint8_t orc_e4m3_encode(float x);
uint8_t orc_e2m1_encode_magnitude(float r);
void orc_nvfp4_quantize_group(const float *x, uint8_t *nibbles, uint8_t *scale_byte);
void orc_nvfp4_quantize(const float *x, int64_t n_vec, uint8_t *codes, uint8_t *scales);
void orc_nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t n_vec, double *out);
double orc_bf16_value(uint16_t bits);
void orc_index_scores(const uint16_t *q_idx, const uint8_t *ik_codes, const uint8_t *ik_scales,
                      int32_t T, int32_t q, int32_t nb_out, double *out);
void orc_index_scores_lse(const uint16_t *q_idx, const uint8_t *ik_codes, const uint8_t *ik_scales,
                          int32_t T, int32_t q, int32_t nb_out, double *out);
int orc_block_topk(const double *scores, int32_t n, int32_t topk, int32_t *ids_out, double *margin);
void orc_sparse_attention_token(const uint16_t *q, const uint8_t *k_codes, const uint8_t *k_scales,
                                const uint8_t *v_codes, const uint8_t *v_scales, int32_t T,
                                const int32_t *ids, int32_t n_ids, int64_t p, double scale,
                                double *out);
#ifdef __cplusplus
}
#endif
#endif

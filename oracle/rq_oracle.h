/*
 * CPU oracle for the ResidualQuant decode path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. The product library never links, includes or calls it, and
 * this oracle includes nothing from the product (no HIP header, no shared
 * source, no shared tables).
 *
 * Citations name the paper page "KV Cache Quantization for Looped Transformers
 * with 2-Bit Residuals" (ResidualQuant) by section, table or appendix.
 *
 * Everything is computed in IEEE binary64 with plain loops, in the order the
 * paper states the method. fp16/bf16 are decoded and encoded by hand-written
 * routines in this file.
 */
#ifndef RQ_ORACLE_H
#define RQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats ---------------------------------------------------- */
enum { RQO_RNE = 0, RQO_RD = 1, RQO_RU = 2 };   /* to nearest-even, toward -inf, toward +inf */

uint16_t rqo_f16_encode(double x, int mode);
double rqo_f16_decode(uint16_t h);
double rqo_bf16_decode(uint16_t h);
void rqo_f16_encode_array(const double* x, int64_t n, int mode, uint16_t* out);
void rqo_f16_decode_array(const uint16_t* h, int64_t n, double* out);
void rqo_bf16_decode_array(const uint16_t* h, int64_t n, double* out);

/* ---- rotation (§2.2, App. G.2): randomized Sylvester-Hadamard ------------ */
/* W[n][n] with W_1 = [1], W_2m = [[W_m, W_m], [W_m, -W_m]]; n a power of two. */
int rqo_sylvester(int n, double* W);
/* H[D][D] = block-diag over D/nb blocks of (W_nb / sqrt(nb)) * diag(sign[block]);
 * z = H x. Returns 0, or -1 if nb is not a power of two dividing D. */
int rqo_rotation(int D, int nb, const int8_t* sign, double* H);

/* ---- quantizer (§2.1) ---------------------------------------------------- */
/* One group of g values -> fp16 offset o, fp16 scale s, integer codes.
 *   o = fp16 round-toward--inf of min(v); s = fp16 round-toward-+inf of
 *   (max(v) - o) / (2^bits - 1); code_i = clamp(rne((v_i - o) / s), 0, 2^bits - 1);
 *   s == 0 (all values equal o) gives code 0 everywhere. An o or s whose fp16
 *   rounding overflows is held at +-65504 (the largest finite fp16 magnitude of
 *   its sign), so values outside [o, o + (2^bits - 1) s] clip to the end codes.
 * Optional outputs (may be NULL): delta[i] = distance, in code units, of
 * (v_i - o)/s from the nearest rounding boundary k + 1/2; pre_o = min(v);
 * pre_s = (max(v) - o)/(2^bits - 1) before fp16 rounding. */
void rqo_group_quant(const double* v, int g, int bits, uint16_t* o16, uint16_t* s16,
                     uint16_t* codes, double* delta, double* pre_o, double* pre_s);

/* ---- packed layout ------------------------------------------------------- */
/* A group of g codes of `bits` bits fills g*bits/8 bytes, as g*bits/32
 * little-endian 32-bit words. Element e lies in half h = e / (g/2) at index
 * k = e % (g/2); 16/bits consecutive k share one 16-bit half-word j =
 * k / (16/bits), at bit offset bits*(k % (16/bits)); word j holds half-word j of
 * half 0 in bits 0..15 and half-word j of half 1 in bits 16..31.
 * bits in {2, 4, 8, 16}; g a multiple of 32/bits*2. */
int rqo_pack_group(const uint16_t* codes, int g, int bits, uint8_t* out);
int rqo_unpack_group(const uint8_t* in, int g, int bits, uint16_t* codes);

/* ---- configuration of one cache series --------------------------------- */
/* Reference policies (§3.2), applied within each loop group (§5 "Models":
 * Huginn's 32 loops as eight independent groups of four, App. D):
 *   RQO_LAST_LOOP:  anchor = last loop of the group, R_r = its reconstruction;
 *   RQO_PREV_LOOP:  anchor = first loop of the group, R_r = reconstruction of
 *                   loop r-1 (a chain);
 *   RQO_FIRST_LOOP: anchor = first loop of the group, R_r = its reconstruction. */
enum { RQO_LAST_LOOP = 0, RQO_PREV_LOOP = 1, RQO_FIRST_LOOP = 2 };
#define RQO_MAX_LOOPS 32
typedef struct {
  int32_t D;          /* head dimension */
  int32_t L;          /* loops, 1 .. RQO_MAX_LOOPS */
  int32_t policy;     /* RQO_LAST_LOOP, RQO_PREV_LOOP or RQO_FIRST_LOOP */
  int32_t loop_group; /* loops per anchor group (divides L); 0 = one group of all L loops */
  int32_t bits[RQO_MAX_LOOPS];   /* bit width per loop (0-based loop index) */
  int32_t group[RQO_MAX_LOOPS];  /* quantization group size per loop (divides D) */
} rqo_cfg;

/* Bytes of one token's packed codes for loop r: D * bits[r] / 8. */
int rqo_row_bytes(const rqo_cfg* c, int r);

/* Quantize one (tensor, batch, head) series of T tokens.
 * X: bf16 [L][T][D] (original domain). H: fp32 [D][D], z = H x.
 * codes[r]: [T][row_bytes(r)]; meta[r]: fp16 [T][D/group[r]][2] as (o, s);
 * alpha[r]: fp16 [T] for every non-anchor loop (ignored for the anchor; may be NULL there);
 *   an LS coefficient whose fp16 rounding overflows is held at +-65504.
 * Diagnostics (each may be NULL): delta [L][T][D]; alpha_pre [L][T];
 * pre_o, pre_s [L][T][D], of which entry [r][t][j] for j < D/group[r] holds
 * group j's value before fp16 rounding.
 * Returns 0 or a negative error code. */
int rqo_quantize_series(const rqo_cfg* c, const uint16_t* X, int T, const float* H,
                        uint8_t* const* codes, uint16_t* const* meta, uint16_t* const* alpha,
                        double* delta, double* alpha_pre, double* pre_o, double* pre_s);

/* Rebuild the rotated-domain reconstruction zhat of loop r for tokens [0, T):
 * out [T][D]. With a the anchor of r's group: Last-loop and First-loop:
 * zhat_a = A, zhat_r = alpha_r * A + D(c_r); Previous-loop: zhat_a = A,
 * zhat_r = alpha_r * zhat_{r-1} + D(c_r) back to the group's first loop. */
int rqo_reconstruct(const rqo_cfg* c, int r, int T, const uint8_t* const* codes,
                    const uint16_t* const* meta, const uint16_t* const* alpha, double* out);

/* Decode attention of one query against T cached tokens of loop r plus the
 * current token kept in bf16 (§4.1, §4.2 Decode, App. G.2 Reconstruction):
 * q' = HK q; s_t = scale <q', zhatK_t>; s_cur = scale <q, kcur>;
 * p = softmax; out = (HV^T sum_t p_t zhatV_t + p_cur vcur) -- fp64 [D]. */
int rqo_attend(const rqo_cfg* c, int r, int T,
               const uint8_t* const* kcodes, const uint16_t* const* kmeta, const uint16_t* const* kalpha,
               const uint8_t* const* vcodes, const uint16_t* const* vmeta, const uint16_t* const* valpha,
               const float* HK, const float* HV, const uint16_t* q, const uint16_t* kcur,
               const uint16_t* vcur, double scale, double* out);

/* The same attention by brute force: materialize Khat_t = HK^T zhatK_t and
 * Vhat_t = HV^T zhatV_t, then textbook softmax(scale q Khat^T) Vhat. */
int rqo_attend_bruteforce(const rqo_cfg* c, int r, int T,
                          const uint8_t* const* kcodes, const uint16_t* const* kmeta, const uint16_t* const* kalpha,
                          const uint8_t* const* vcodes, const uint16_t* const* vmeta, const uint16_t* const* valpha,
                          const float* HK, const float* HV, const uint16_t* q, const uint16_t* kcur,
                          const uint16_t* vcur, double scale, double* out);

/* Textbook attention over an uncompressed bf16 cache K, V [T][D] plus the
 * current token (the BF16 decode baseline of §5.3). */
int rqo_attend_bf16(int D, int T, const uint16_t* K, const uint16_t* V, const uint16_t* q,
                    const uint16_t* kcur, const uint16_t* vcur, double scale, double* out);

/* Prefill attention of one loop (§4.2 "Prefill": every loop attends causally
 * over its own BF16 prompt K/V before the prompt is quantized). Q, K, V are
 * bf16 [T][D] of one (sequence, head); row i of out (fp64 [T][D]) is the
 * softmax(scale q_i . k_j) weighted sum of v_j over j <= i. */
int rqo_prefill_attend(int D, int T, const uint16_t* Q, const uint16_t* K, const uint16_t* V, double scale,
                       double* out);

#ifdef __cplusplus
}
#endif
#endif

/*
 * CPU oracle for the ResidualQuant decode path -- TEST INFRASTRUCTURE ONLY.
 * See rq_oracle.h for the contract of every entry point.
 *
 * Citations name the paper page "KV Cache Quantization for Looped Transformers
 * with 2-Bit Residuals" (ResidualQuant) by section, table or appendix.
 *
 * Style: plain binary64 loops in the order the paper states each step; no
 * blocking, no fusion, no reordering. Build with -ffp-contract=off so that
 * every written product and sum is its own rounding.
 */
#include "rq_oracle.h"

#include <cmath>
#include <cstring>
#include <vector>

namespace {

bool is_pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

/* Correctly rounded binary64 -> binary16 with a selectable direction.
 * The magnitude is scaled by the exact power of two that makes one unit the
 * spacing of binary16 numbers in its binade; the integer part and the
 * remainder then decide the rounding. */
uint16_t f16_encode(double x, int mode) {
  if (std::isnan(x)) return 0x7e00;
  const bool neg = std::signbit(x);
  const uint16_t sign = neg ? 0x8000 : 0;
  const double a = std::fabs(x);
  if (std::isinf(a)) return sign | 0x7c00;
  if (a == 0.0) return sign;
  int e = 0;
  std::frexp(a, &e);                            /* a = f * 2^e with f in [0.5, 1) */
  const int lead = e - 1;                       /* exponent of the leading bit */
  const int qexp = (lead < -14) ? -24 : lead - 10;  /* spacing 2^qexp in this binade */
  const double n = std::ldexp(a, -qexp);        /* exact */
  const double fl = std::floor(n);
  const double frac = n - fl;                   /* exact */
  bool up = false;                              /* round the magnitude up? */
  if (mode == RQO_RNE) {
    up = frac > 0.5 || (frac == 0.5 && std::fmod(fl, 2.0) == 1.0);
  } else if (mode == RQO_RD) {                  /* toward -inf: negative magnitudes grow */
    up = neg && frac > 0.0;
  } else {                                      /* toward +inf: positive magnitudes grow */
    up = !neg && frac > 0.0;
  }
  const double v = std::ldexp(fl + (up ? 1.0 : 0.0), qexp);
  if (v > 65504.0) {
    const bool toward_zero = (mode == RQO_RD && !neg) || (mode == RQO_RU && neg);
    return toward_zero ? (uint16_t)(sign | 0x7bff) : (uint16_t)(sign | 0x7c00);
  }
  if (v == 0.0) return sign;
  int e2 = 0;
  std::frexp(v, &e2);
  const int lead2 = e2 - 1;
  if (lead2 < -14) return (uint16_t)(sign | (uint16_t)std::ldexp(v, 24));  /* subnormal */
  const uint16_t mant = (uint16_t)(std::ldexp(v, -(lead2 - 10)) - 1024.0);
  return (uint16_t)(sign | (uint16_t)((lead2 + 15) << 10) | mant);
}

/* The cache holds o, s and alpha as finite fp16 numbers. A value whose rounding
 * leaves the fp16 range (rotated inputs or residuals beyond +-65504, or an LS
 * coefficient of that size) is held at the largest finite magnitude of its
 * sign; the pages do not discuss overflow. */
uint16_t f16_saturate(uint16_t h) {
  return (h & 0x7fff) == 0x7c00 ? (uint16_t)((h & 0x8000) | 0x7bff) : h;
}

double f16_decode(uint16_t h) {
  const int e = (h >> 10) & 31;
  const int m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(1024.0 + m, e - 25);
  return (h & 0x8000) ? -v : v;
}

double bf16_decode(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

/* z = H x with H fp32 [D][D] and x already decoded. */
void rotate(int D, const float* H, const double* x, double* z) {
  for (int i = 0; i < D; ++i) {
    double acc = 0.0;
    for (int j = 0; j < D; ++j) acc += (double)H[(size_t)i * D + j] * x[j];
    z[i] = acc;
  }
}

double dot(int n, const double* a, const double* b) {
  double acc = 0.0;
  for (int i = 0; i < n; ++i) acc += a[i] * b[i];
  return acc;
}

bool bits_ok(int b) { return b == 2 || b == 4 || b == 8 || b == 16; }

int check_cfg(const rqo_cfg* c) {
  if (!c || c->D <= 0 || c->L < 1 || c->L > RQO_MAX_LOOPS) return -1;
  if (c->policy != RQO_LAST_LOOP && c->policy != RQO_PREV_LOOP && c->policy != RQO_FIRST_LOOP) return -1;
  if (c->loop_group < 0 || (c->loop_group > 0 && c->L % c->loop_group != 0)) return -1;
  for (int r = 0; r < c->L; ++r) {
    if (!bits_ok(c->bits[r])) return -2;
    const int g = c->group[r];
    if (g <= 0 || c->D % g != 0 || g % (2 * (16 / c->bits[r])) != 0) return -3;
  }
  return 0;
}

/* Loops per anchor group, the first loop of r's group and its anchor (§3.2, §5 "Models"). */
int group_len(const rqo_cfg* c) { return c->loop_group > 0 ? c->loop_group : c->L; }
int group_first(const rqo_cfg* c, int r) { return r / group_len(c) * group_len(c); }
int anchor_of(const rqo_cfg* c, int r) {
  return c->policy == RQO_LAST_LOOP ? group_first(c, r) + group_len(c) - 1 : group_first(c, r);
}

/* Quantize a whole D-vector group by group at loop r; returns the
 * dequantized vector D(c) in deq (§2.1). */
void quantize_vector(const rqo_cfg* c, int r, const double* v, uint8_t* code_row, uint16_t* meta_row,
                     double* delta_row, double* pre_o_row, double* pre_s_row, double* deq) {
  const int g = c->group[r];
  const int b = c->bits[r];
  std::vector<uint16_t> codes(g);
  const int group_bytes = g * b / 8;
  for (int j = 0; j < c->D / g; ++j) {
    uint16_t o16 = 0, s16 = 0;
    double po = 0.0, ps = 0.0;
    rqo_group_quant(v + (size_t)j * g, g, b, &o16, &s16, codes.data(),
                    delta_row ? delta_row + (size_t)j * g : nullptr, &po, &ps);
    meta_row[2 * j] = o16;
    meta_row[2 * j + 1] = s16;
    if (pre_o_row) pre_o_row[j] = po;
    if (pre_s_row) pre_s_row[j] = ps;
    rqo_pack_group(codes.data(), g, b, code_row + (size_t)j * group_bytes);
    const double o = f16_decode(o16), s = f16_decode(s16);
    for (int i = 0; i < g; ++i) deq[(size_t)j * g + i] = o + s * (double)codes[i];
  }
}

/* D(c) of loop r for one token, from the packed row and its metadata. */
void dequant_row(const rqo_cfg* c, int r, const uint8_t* code_row, const uint16_t* meta_row, double* out) {
  const int g = c->group[r];
  const int b = c->bits[r];
  std::vector<uint16_t> codes(g);
  const int group_bytes = g * b / 8;
  for (int j = 0; j < c->D / g; ++j) {
    rqo_unpack_group(code_row + (size_t)j * group_bytes, g, b, codes.data());
    const double o = f16_decode(meta_row[2 * j]), s = f16_decode(meta_row[2 * j + 1]);
    for (int i = 0; i < g; ++i) out[(size_t)j * g + i] = o + s * (double)codes[i];
  }
}

/* zhat of loop r, token t, rotated domain (§3.2, App. D, App. G.2 Reconstruction). */
void reconstruct_token(const rqo_cfg* c, int r, int t, const uint8_t* const* codes,
                       const uint16_t* const* meta, const uint16_t* const* alpha, double* z) {
  const int D = c->D;
  const int a = anchor_of(c, r);
  std::vector<double> res(D);
  auto row = [&](int loop, double* out) {
    dequant_row(c, loop, codes[loop] + (size_t)t * rqo_row_bytes(c, loop),
                meta[loop] + (size_t)t * (D / c->group[loop]) * 2, out);
  };
  row(a, z);                                           /* anchor A */
  if (r == a) return;
  if (c->policy != RQO_PREV_LOOP) {                    /* shared anchor */
    const double al = f16_decode(alpha[r][t]);
    row(r, res.data());
    for (int i = 0; i < D; ++i) z[i] = al * z[i] + res[i];   /* alpha_r A + D(c_r) */
  } else {
    for (int j = a + 1; j <= r; ++j) {                 /* zhat_j = alpha_j zhat_{j-1} + D(c_j) */
      const double al = f16_decode(alpha[j][t]);
      row(j, res.data());
      for (int i = 0; i < D; ++i) z[i] = al * z[i] + res[i];
    }
  }
}

void decode_bf16_vec(int D, const uint16_t* h, double* out) {
  for (int i = 0; i < D; ++i) out[i] = bf16_decode(h[i]);
}

}  // namespace

extern "C" {

uint16_t rqo_f16_encode(double x, int mode) { return f16_encode(x, mode); }
double rqo_f16_decode(uint16_t h) { return f16_decode(h); }
double rqo_bf16_decode(uint16_t h) { return bf16_decode(h); }

void rqo_f16_encode_array(const double* x, int64_t n, int mode, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_encode(x[i], mode);
}
void rqo_f16_decode_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_decode(h[i]);
}
void rqo_bf16_decode_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_decode(h[i]);
}

int rqo_sylvester(int n, double* W) {
  if (!is_pow2(n)) return -1;
  W[0] = 1.0;
  for (int m = 1; m < n; m *= 2) {
    for (int i = 0; i < m; ++i) {
      for (int j = 0; j < m; ++j) {
        const double w = W[(size_t)i * n + j];
        W[(size_t)i * n + j + m] = w;
        W[(size_t)(i + m) * n + j] = w;
        W[(size_t)(i + m) * n + j + m] = -w;
      }
    }
  }
  return 0;
}

int rqo_rotation(int D, int nb, const int8_t* sign, double* H) {
  if (!is_pow2(nb) || D % nb != 0) return -1;
  std::vector<double> W((size_t)nb * nb);
  rqo_sylvester(nb, W.data());
  const double inv = 1.0 / std::sqrt((double)nb);
  for (size_t i = 0; i < (size_t)D * D; ++i) H[i] = 0.0;
  for (int blk = 0; blk < D / nb; ++blk) {
    for (int i = 0; i < nb; ++i) {
      for (int j = 0; j < nb; ++j) {
        const int gi = blk * nb + i, gj = blk * nb + j;
        H[(size_t)gi * D + gj] = W[(size_t)i * nb + j] * inv * (double)sign[gj];
      }
    }
  }
  return 0;
}

void rqo_group_quant(const double* v, int g, int bits, uint16_t* o16, uint16_t* s16,
                     uint16_t* codes, double* delta, double* pre_o, double* pre_s) {
  double mn = v[0], mx = v[0];
  for (int i = 1; i < g; ++i) {
    if (v[i] < mn) mn = v[i];
    if (v[i] > mx) mx = v[i];
  }
  const double qmax = (double)((1 << bits) - 1);
  const uint16_t o = f16_saturate(f16_encode(mn, RQO_RD));
  const double od = f16_decode(o);
  const double sp = (mx - od) / qmax;
  const uint16_t s = f16_saturate(f16_encode(sp, RQO_RU));
  const double sd = f16_decode(s);
  *o16 = o;
  *s16 = s;
  if (pre_o) *pre_o = mn;
  if (pre_s) *pre_s = sp;
  for (int i = 0; i < g; ++i) {
    if (sd == 0.0) {
      codes[i] = 0;
      if (delta) delta[i] = INFINITY;
      continue;
    }
    const double t = (v[i] - od) / sd;
    double k = std::nearbyint(t);                      /* ties to even (default rounding mode) */
    if (k < 0.0) k = 0.0;
    if (k > qmax) k = qmax;
    codes[i] = (uint16_t)k;
    if (delta) delta[i] = std::fabs(t - std::floor(t) - 0.5);
  }
}

int rqo_pack_group(const uint16_t* codes, int g, int bits, uint8_t* out) {
  if (!bits_ok(bits) || g % (2 * (16 / bits)) != 0) return -1;
  const int half = g / 2;
  const int per_hw = 16 / bits;                        /* codes per 16-bit half-word */
  const int words = g * bits / 32;
  for (int w = 0; w < words; ++w) {
    uint32_t word = 0;
    for (int h = 0; h < 2; ++h) {
      for (int p = 0; p < per_hw; ++p) {
        const int k = w * per_hw + p;
        const uint32_t code = codes[h * half + k] & ((1u << bits) - 1u);
        word |= code << (16 * h + bits * p);
      }
    }
    for (int byte = 0; byte < 4; ++byte) out[4 * w + byte] = (uint8_t)(word >> (8 * byte));
  }
  return 0;
}

int rqo_unpack_group(const uint8_t* in, int g, int bits, uint16_t* codes) {
  if (!bits_ok(bits) || g % (2 * (16 / bits)) != 0) return -1;
  const int half = g / 2;
  const int per_hw = 16 / bits;
  const int words = g * bits / 32;
  for (int w = 0; w < words; ++w) {
    uint32_t word = 0;
    for (int byte = 0; byte < 4; ++byte) word |= (uint32_t)in[4 * w + byte] << (8 * byte);
    for (int h = 0; h < 2; ++h) {
      for (int p = 0; p < per_hw; ++p) {
        const int k = w * per_hw + p;
        codes[h * half + k] = (uint16_t)((word >> (16 * h + bits * p)) & ((1u << bits) - 1u));
      }
    }
  }
  return 0;
}

int rqo_row_bytes(const rqo_cfg* c, int r) { return c->D * c->bits[r] / 8; }

int rqo_quantize_series(const rqo_cfg* c, const uint16_t* X, int T, const float* H,
                        uint8_t* const* codes, uint16_t* const* meta, uint16_t* const* alpha,
                        double* delta, double* alpha_pre, double* pre_o, double* pre_s) {
  const int err = check_cfg(c);
  if (err) return err;
  const int D = c->D, L = c->L, G = group_len(c);
  std::vector<double> x(D);
  std::vector<double> Z((size_t)L * D);                /* rotated loops of this token */
  std::vector<double> ref(D), E(D), deq(D);
  for (int t = 0; t < T; ++t) {
    for (int r = 0; r < L; ++r) {                      /* Z_r = H X_r (§3.3, App. G.1) */
      decode_bf16_vec(D, X + ((size_t)r * T + t) * D, x.data());
      rotate(D, H, x.data(), &Z[(size_t)r * D]);
    }
    auto out_ptrs = [&](int r, uint8_t** crow, uint16_t** mrow, double** drow, double** porow, double** psrow) {
      *crow = codes[r] + (size_t)t * rqo_row_bytes(c, r);
      *mrow = meta[r] + (size_t)t * (D / c->group[r]) * 2;
      *drow = delta ? delta + ((size_t)r * T + t) * D : nullptr;
      *porow = pre_o ? pre_o + ((size_t)r * T + t) * D : nullptr;
      *psrow = pre_s ? pre_s + ((size_t)r * T + t) * D : nullptr;
    };
    uint8_t* crow; uint16_t* mrow; double *drow, *porow, *psrow;
    for (int g0 = 0; g0 < L; g0 += G) {                /* each loop group independently (§5 "Models") */
      const int a = anchor_of(c, g0);
      /* anchor: quantized directly; its reconstruction is the reference (§3.2, App. G.1) */
      out_ptrs(a, &crow, &mrow, &drow, &porow, &psrow);
      quantize_vector(c, a, &Z[(size_t)a * D], crow, mrow, drow, porow, psrow, ref.data());
      if (alpha_pre) alpha_pre[(size_t)a * T + t] = 0.0;
      /* Last-loop / First-loop: every other loop of the group refers to the
       * anchor; Previous-loop: loop r refers to the reconstruction of loop r-1,
       * walking away from the group's first loop. */
      for (int r = g0; r < g0 + G; ++r) {
        if (r == a) continue;
        const double* Zr = &Z[(size_t)r * D];
        const double den = dot(D, ref.data(), ref.data());
        const double al = den > 0.0 ? dot(D, Zr, ref.data()) / den : 0.0;   /* LS alpha (§3.2) */
        const uint16_t al16 = f16_saturate(f16_encode(al, RQO_RNE));
        const double alt = f16_decode(al16);
        alpha[r][t] = al16;
        if (alpha_pre) alpha_pre[(size_t)r * T + t] = al;
        for (int i = 0; i < D; ++i) E[i] = Zr[i] - alt * ref[i];           /* residual */
        out_ptrs(r, &crow, &mrow, &drow, &porow, &psrow);
        quantize_vector(c, r, E.data(), crow, mrow, drow, porow, psrow, deq.data());
        if (c->policy == RQO_PREV_LOOP) {
          for (int i = 0; i < D; ++i) ref[i] = alt * ref[i] + deq[i];    /* zhat_r, next reference */
        }
      }
    }
  }
  return 0;
}

int rqo_reconstruct(const rqo_cfg* c, int r, int T, const uint8_t* const* codes,
                    const uint16_t* const* meta, const uint16_t* const* alpha, double* out) {
  const int err = check_cfg(c);
  if (err) return err;
  if (r < 0 || r >= c->L) return -4;
  for (int t = 0; t < T; ++t) reconstruct_token(c, r, t, codes, meta, alpha, out + (size_t)t * c->D);
  return 0;
}

int rqo_attend(const rqo_cfg* c, int r, int T,
               const uint8_t* const* kcodes, const uint16_t* const* kmeta, const uint16_t* const* kalpha,
               const uint8_t* const* vcodes, const uint16_t* const* vmeta, const uint16_t* const* valpha,
               const float* HK, const float* HV, const uint16_t* q, const uint16_t* kcur,
               const uint16_t* vcur, double scale, double* out) {
  const int err = check_cfg(c);
  if (err) return err;
  if (r < 0 || r >= c->L || T < 0) return -4;
  const int D = c->D;
  std::vector<double> qd(D), qr(D), kc(D), vc(D), z(D), acc(D, 0.0), s(T > 0 ? T : 1);
  decode_bf16_vec(D, q, qd.data());
  decode_bf16_vec(D, kcur, kc.data());
  decode_bf16_vec(D, vcur, vc.data());
  rotate(D, HK, qd.data(), qr.data());                 /* q' = HK q (App. G.2) */
  double m = scale * dot(D, qd.data(), kc.data());    /* current token, original domain (§4.2) */
  const double s_cur = m;
  for (int t = 0; t < T; ++t) {
    reconstruct_token(c, r, t, kcodes, kmeta, kalpha, z.data());
    s[t] = scale * dot(D, qr.data(), z.data());
    if (s[t] > m) m = s[t];
  }
  double l = 0.0;
  for (int t = 0; t < T; ++t) {
    const double p = std::exp(s[t] - m);
    l += p;
    reconstruct_token(c, r, t, vcodes, vmeta, valpha, z.data());
    for (int i = 0; i < D; ++i) acc[i] += p * z[i];    /* rotated-domain value sum */
  }
  const double p_cur = std::exp(s_cur - m);
  l += p_cur;
  for (int j = 0; j < D; ++j) {                        /* one inverse rotation: HV^T acc */
    double o = 0.0;
    for (int i = 0; i < D; ++i) o += (double)HV[(size_t)i * D + j] * acc[i];
    out[j] = (o + p_cur * vc[j]) / l;
  }
  return 0;
}

int rqo_attend_bruteforce(const rqo_cfg* c, int r, int T,
                          const uint8_t* const* kcodes, const uint16_t* const* kmeta, const uint16_t* const* kalpha,
                          const uint8_t* const* vcodes, const uint16_t* const* vmeta, const uint16_t* const* valpha,
                          const float* HK, const float* HV, const uint16_t* q, const uint16_t* kcur,
                          const uint16_t* vcur, double scale, double* out) {
  const int err = check_cfg(c);
  if (err) return err;
  if (r < 0 || r >= c->L || T < 0) return -4;
  const int D = c->D;
  std::vector<double> qd(D), z(D);
  std::vector<double> K((size_t)(T + 1) * D), V((size_t)(T + 1) * D), s(T + 1);
  decode_bf16_vec(D, q, qd.data());
  for (int t = 0; t < T; ++t) {                        /* Khat = HK^T zhat, Vhat = HV^T zhat */
    reconstruct_token(c, r, t, kcodes, kmeta, kalpha, z.data());
    for (int j = 0; j < D; ++j) {
      double v = 0.0;
      for (int i = 0; i < D; ++i) v += (double)HK[(size_t)i * D + j] * z[i];
      K[(size_t)t * D + j] = v;
    }
    reconstruct_token(c, r, t, vcodes, vmeta, valpha, z.data());
    for (int j = 0; j < D; ++j) {
      double v = 0.0;
      for (int i = 0; i < D; ++i) v += (double)HV[(size_t)i * D + j] * z[i];
      V[(size_t)t * D + j] = v;
    }
  }
  decode_bf16_vec(D, kcur, &K[(size_t)T * D]);
  decode_bf16_vec(D, vcur, &V[(size_t)T * D]);
  double m = -INFINITY;
  for (int t = 0; t <= T; ++t) {
    s[t] = scale * dot(D, qd.data(), &K[(size_t)t * D]);
    if (s[t] > m) m = s[t];
  }
  double l = 0.0;
  for (int t = 0; t <= T; ++t) l += std::exp(s[t] - m);
  for (int j = 0; j < D; ++j) {
    double o = 0.0;
    for (int t = 0; t <= T; ++t) o += std::exp(s[t] - m) / l * V[(size_t)t * D + j];
    out[j] = o;
  }
  return 0;
}

int rqo_attend_bf16(int D, int T, const uint16_t* K, const uint16_t* V, const uint16_t* q,
                    const uint16_t* kcur, const uint16_t* vcur, double scale, double* out) {
  if (D <= 0 || T < 0) return -1;
  std::vector<double> qd(D), k(D), v(D), s(T + 1), acc(D, 0.0);
  decode_bf16_vec(D, q, qd.data());
  double m = -INFINITY;
  for (int t = 0; t <= T; ++t) {
    decode_bf16_vec(D, t < T ? K + (size_t)t * D : kcur, k.data());
    s[t] = scale * dot(D, qd.data(), k.data());
    if (s[t] > m) m = s[t];
  }
  double l = 0.0;
  for (int t = 0; t <= T; ++t) {
    const double p = std::exp(s[t] - m);
    l += p;
    decode_bf16_vec(D, t < T ? V + (size_t)t * D : vcur, v.data());
    for (int i = 0; i < D; ++i) acc[i] += p * v[i];
  }
  for (int i = 0; i < D; ++i) out[i] = acc[i] / l;
  return 0;
}

int rqo_prefill_attend(int D, int T, const uint16_t* Q, const uint16_t* K, const uint16_t* V, double scale,
                       double* out) {
  if (D <= 0 || T < 0) return -1;
  std::vector<double> q(D), k(D), v(D), s(T);
  for (int i = 0; i < T; ++i) {                 /* query i sees keys 0..i (causal) */
    decode_bf16_vec(D, Q + (size_t)i * D, q.data());
    double m = -INFINITY;
    for (int j = 0; j <= i; ++j) {
      decode_bf16_vec(D, K + (size_t)j * D, k.data());
      s[j] = scale * dot(D, q.data(), k.data());
      if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    double* o = out + (size_t)i * D;
    for (int c = 0; c < D; ++c) o[c] = 0.0;
    for (int j = 0; j <= i; ++j) {
      const double p = std::exp(s[j] - m);
      l += p;
      decode_bf16_vec(D, V + (size_t)j * D, v.data());
      for (int c = 0; c < D; ++c) o[c] += p * v[c];
    }
    for (int c = 0; c < D; ++c) o[c] /= l;
  }
  return 0;
}

}  // extern "C"

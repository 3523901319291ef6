/*
 * oracle.c -- plain, slow CPU oracle for one gated-attention decode / verify
 * step (one decoder layer, one GPU's head share).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library; the two are written independently from the
 * same definition.
 *
 * Source of the definition: the page "012-attention-local-splits.py"
 * (bishal.us open-kernel-challenge experiment, SGLang's Muse Spark Open
 * gated attention on H200): its module docstring (the ordered list of steps),
 * the `_prepare_qkv` Triton kernel (norm, RoPE, q cast, K/V store), the
 * `_cos_sin` table recipe, and `kernel_fn` (attention call and the
 * `rms_norm_gate` epilogue).  Readings of points the page leaves open are
 * marked READING in the comments below.
 *
 * Precision: the prologue follows the page's fp32 steps with every
 * intermediate bf16 rounding the page writes; attention and the epilogue are
 * evaluated in double (the page fixes no precision there beyond bf16 output).
 *
 * Build: gcc -O2 -fPIC -shared -fopenmp -ffp-contract=off -fno-fast-math oracle.c -lm
 * (contraction must stay off so every fp32 step rounds exactly once).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD_ARG (-1)
#define ORC_BAD_ROW (-2)

/* ------------------------------------------------------------------------ */
/* Configuration (mirrors the page's Config dict; its own struct).           */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t batch;        /* B                                                   */
  int32_t q_len;        /* L: 1 decode, 8 speculative verify                  */
  int32_t num_q_heads;  /* Hq                                                  */
  int32_t num_kv_heads; /* Hkv                                                 */
  int32_t head_dim;     /* D (64)                                              */
  int32_t page_size;    /* P                                                   */
  int32_t window;       /* W: key j visible to a query at p iff p-W < j <= p;  */
                        /*    0 = unbounded                                    */
  int32_t max_pages;    /* page_table row stride                               */
  int64_t num_pages;    /* pages in the cache pool                             */
  float rope_theta;     /* 0 = no RoPE                                         */
  float sm_scale;       /* applied softmax scale                               */
  float kv_scale;       /* != 1 selects the divided store / descaled read     */
  float q_scale;        /* q's norm output scale before its one bf16 rounding */
                        /*    (page "qk_norm"); 1 = page 1's prologue         */
} orc_config;

/* ------------------------------------------------------------------------ */
/* Number formats.                                                           */
/* ------------------------------------------------------------------------ */

/* bfloat16 bit pattern -> value (exact). */
float orc_bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint16_t float_bits_hi(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* Round a real number to bfloat16, to nearest with ties to even (the
 * rounding of torch's `.to(torch.bfloat16)` and of Triton's `.to(tl.bfloat16)`).
 * Written from the format: 8 significant bits, normal exponents down to
 * 2^-126, subnormal quantum 2^-133, overflow to infinity. */
uint16_t orc_bf16_round(double x) {
  if (isnan(x)) return 0x7FC0;
  if (isinf(x)) return x > 0 ? 0x7F80 : 0xFF80;
  double ax = fabs(x);
  /* largest finite bf16 is (2 - 2^-7) * 2^127; the halfway point to 2^128
   * rounds (ties-to-even, odd last bit) up to infinity. */
  const double max_finite = (2.0 - ldexp(1.0, -7)) * ldexp(1.0, 127);
  const double overflow_mid = (2.0 - ldexp(1.0, -8)) * ldexp(1.0, 127);
  if (ax >= overflow_mid) return signbit(x) ? 0xFF80 : 0x7F80;
  double r;
  if (ax == 0.0) {
    r = 0.0;
  } else {
    int e;
    frexp(ax, &e); /* ax = f * 2^e, f in [0.5, 1) -> leading bit 2^(e-1) */
    int lead = e - 1;
    if (lead < -126) lead = -126; /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, lead - 7);
    r = nearbyint(ax / quantum) * quantum; /* default mode: ties to even */
    if (r > max_finite) r = max_finite;    /* cannot happen below overflow_mid */
  }
  float f = (float)r; /* exact: r has <= 8 significant bits */
  if (signbit(x)) f = -f;
  return float_bits_hi(f);
}

/* Round-trip helper: value of bf16_round(x). */
static float bf16r(double x) { return orc_bf16_to_float(orc_bf16_round(x)); }

/* OCP float8 e4m3 ("fn") code -> value: sign, 4 exponent bits (bias 7),
 * 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); 0x7F and 0xFF
 * are NaN; there are no infinities. */
double orc_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Real number -> OCP e4m3 code, round to nearest, ties to even code, keeping
 * the sign of zero.
 * READING: magnitudes above the largest finite value (448) saturate to +-448
 * (the page stores through Triton's fp32->e4m3 conversion, which saturates to
 * the finite range); NaN maps to the NaN code with the input's sign. */
uint8_t orc_e4m3_encode(double x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return sign | 0x7F;
  double ax = fabs(x);
  if (ax >= 448.0) return sign | 0x7E; /* saturate (also +-inf) */
  if (ax < ldexp(1.0, -6)) {
    /* subnormal band: quantum 2^-9, codes 0..8 (8 is the smallest normal) */
    double q = nearbyint(ax / ldexp(1.0, -9));
    return sign | (uint8_t)q;
  }
  int e;
  frexp(ax, &e);
  int lead = e - 1; /* 2^lead <= ax < 2^(lead+1), lead in [-6, 8] */
  double q = nearbyint(ax / ldexp(1.0, lead - 3)); /* 8..16 */
  if (q == 16.0) {
    q = 8.0;
    lead += 1;
  }
  /* lead <= 8 here; at lead 8, q <= 14 because ax < 448 rounds to <= 448 */
  return sign | (uint8_t)(((lead + 7) << 3) | ((int)q - 8));
}

/* fp32 1/sqrt(a), correctly rounded (READING: the page calls tl.rsqrt whose
 * accuracy it does not state; the oracle takes the exact value rounded once).
 * The double estimate is within one float ulp; each candidate midpoint m
 * (25 significant bits, so m*m is exact in double) is tested exactly by the
 * sign of fma(m*m, a, -1). */
float orc_rsqrt_cr(float a) {
  if (!(a > 0.0f)) return a == 0.0f ? INFINITY : NAN;
  if (isinf(a)) return 0.0f;
  float y = (float)(1.0 / sqrt((double)a));
  for (int it = 0; it < 2; ++it) {
    float up = nextafterf(y, INFINITY);
    double mid_up = ((double)y + (double)up) * 0.5;
    if (fma(mid_up * mid_up, (double)a, -1.0) < 0.0) { /* true value above mid_up */
      y = up;
      continue;
    }
    float dn = nextafterf(y, 0.0f);
    double mid_dn = ((double)y + (double)dn) * 0.5;
    if (fma(mid_dn * mid_dn, (double)a, -1.0) > 0.0) { /* true value below mid_dn */
      y = dn;
      continue;
    }
    break;
  }
  return y;
}

/* RoPE inverse frequencies, as the page's `_cos_sin` builds them in fp32:
 * exponent 2i/D (exact in fp32), theta**exponent rounded to fp32, then the
 * fp32 reciprocal.  READING: the fp32 power is the exactly rounded value. */
void orc_inv_freq(float theta, int head_dim, float* out) {
  for (int i = 0; i < head_dim / 2; ++i) {
    float ex = (float)(2 * i) / (float)head_dim;
    float pw = (float)pow((double)theta, (double)ex);
    out[i] = 1.0f / pw;
  }
}

/* cos and sin of an fp32 angle, each rounded once to fp32 (READING: the page
 * evaluates torch's fp32 cos/sin; the oracle takes the exactly rounded value). */
static void cos_sin_f32(float ang, float* c, float* s) {
  *c = (float)cos((double)ang);
  *s = (float)sin((double)ang);
}

/* ------------------------------------------------------------------------ */
/* Step 1-4: the prologue (page: `_prepare_qkv`).                            */
/* ------------------------------------------------------------------------ */

static int cfg_ok(const orc_config* c) {
  if (!c) return 0;
  if (c->batch < 0 || c->q_len < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1) return 0;
  if (c->head_dim != 64) return 0;
  if (c->num_q_heads % c->num_kv_heads) return 0;
  if (c->page_size < 1 || c->window < 0 || c->max_pages < 0 || c->num_pages < 0) return 0;
  if (!(c->q_scale > 0.0f) || isinf(c->q_scale)) return 0;
  return 1;
}

/* Per-head unweighted RMSNorm of one 64-wide bf16 row, page order:
 * fp32 sum of squares (each square is exact in fp32; the sum is formed exactly
 * in double and rounded once), /D, + 1e-5 in fp32, rsqrt, fp32 product,
 * bf16 rounding.  With scale != 1 the fp32 product is multiplied by it before
 * that one rounding (page "qk_norm": QKNormDirectKernel's output scale). */
static void norm_row(const uint16_t* xin, int d, float scale, float* y_out, float* inv_out) {
  double ss = 0.0;
  for (int c = 0; c < d; ++c) {
    float x = orc_bf16_to_float(xin[c]);
    ss += (double)(x * x);
  }
  float ms = (float)ss / (float)d;
  float a = ms + 1.0e-5f;
  float inv = orc_rsqrt_cr(a);
  for (int c = 0; c < d; ++c) {
    float x = orc_bf16_to_float(xin[c]);
    float prod = x * inv;
    if (scale != 1.0f) prod = prod * scale;
    y_out[c] = bf16r(prod);
  }
  if (inv_out) *inv_out = inv;
}

/* Interleaved RoPE of a normed row at position pos: pairs (2i, 2i+1) share
 * frequency i; even column e*c - o*s, odd column o*c + e*s, each product and
 * the sum rounded in fp32, then bf16. */
static void rope_row(float* y, int d, int64_t pos, const float* inv_freq) {
  float out[256];
  for (int i = 0; i < d / 2; ++i) {
    float ang = (float)pos * inv_freq[i];
    float c, s;
    cos_sin_f32(ang, &c, &s);
    float e = y[2 * i], o = y[2 * i + 1];
    float ec = e * c, os = o * s, oc = o * c, es = e * s;
    float re = ec - os;
    float ro = oc + es;
    out[2 * i] = bf16r(re);
    out[2 * i + 1] = bf16r(ro);
  }
  memcpy(y, out, sizeof(float) * (size_t)d);
}

/* One q or k head row through the norm and, when theta != 0, RoPE at pos;
 * y receives the bf16-valued results (exposed for the tests' pins). */
void orc_norm_rope_row(const uint16_t* x, int d, int64_t pos, float theta, float* y) {
  float inv_freq[128];
  norm_row(x, d, 1.0f, y, NULL);
  if (theta != 0.0f) {
    orc_inv_freq(theta, d, inv_freq);
    rope_row(y, d, pos, inv_freq);
  }
}

/*
 * Prologue for all T = B*L new tokens.
 *   qkv       bf16 [T, (2Hq + 2Hkv) * D]: q heads | k heads | v heads | gate
 *   positions int64 [T]       RoPE position of each token
 *   cache_loc int64 [T]       flat cache row of each token
 *   k_cache, v_cache  e4m3 [num_pages * P, Hkv, D], updated in place
 *   k_scale, v_scale  divisors used when cfg->kv_scale != 1
 *   q_out     e4m3 [T, Hq, D]
 */
int orc_prologue(const orc_config* cfg, const uint16_t* qkv, const int64_t* positions,
                 const int64_t* cache_loc, uint8_t* k_cache, uint8_t* v_cache, float k_scale,
                 float v_scale, uint8_t* q_out) {
  if (!cfg_ok(cfg)) return ORC_BAD_ARG;
  const int hq = cfg->num_q_heads, hkv = cfg->num_kv_heads, d = cfg->head_dim;
  const int64_t T = (int64_t)cfg->batch * cfg->q_len;
  const int64_t width = (int64_t)(2 * hq + 2 * hkv) * d;
  const int64_t rows = cfg->num_pages * cfg->page_size;
  const int scaled = cfg->kv_scale != 1.0f;
  float inv_freq[128];
  if (cfg->rope_theta != 0.0f) orc_inv_freq(cfg->rope_theta, d, inv_freq);
  float y[256];
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* row = qkv + t * width;
    int64_t slot = cache_loc[t];
    /* READING: a token whose cache row lies outside the pool (e.g. a padded
     * request slot) stores nothing; its q is still produced. */
    const int store = slot >= 0 && slot < rows;
    for (int h = 0; h < hq + hkv; ++h) { /* q heads then k heads */
      /* READING: the q scale (page "qk_norm", folding the query factor into q
       * before its e4m3 cast) applies to the q heads' norm only; RoPE follows
       * on the scaled, rounded values as on page 1. */
      norm_row(row + (int64_t)h * d, d, h < hq ? cfg->q_scale : 1.0f, y, NULL);
      if (cfg->rope_theta != 0.0f) rope_row(y, d, positions[t], inv_freq);
      if (h < hq) {
        for (int c = 0; c < d; ++c) q_out[(t * hq + h) * d + c] = orc_e4m3_encode(y[c]);
      } else {
        int g = h - hq;
        for (int c = 0; c < d; ++c) {
          float key = y[c];
          if (scaled) key = bf16r(key / k_scale); /* fp32 quotient, then bf16 */
          if (store) k_cache[(slot * hkv + g) * d + c] = orc_e4m3_encode(key);
        }
      }
    }
    for (int g = 0; g < hkv; ++g) { /* value heads: the raw projection, not normed */
      const uint16_t* vin = row + (int64_t)(hq + hkv + g) * d;
      for (int c = 0; c < d; ++c) {
        float val = orc_bf16_to_float(vin[c]);
        if (scaled) val = bf16r(val / v_scale);
        if (store) v_cache[(slot * hkv + g) * d + c] = orc_e4m3_encode(val);
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 5: paged causal sliding-window GQA attention (page: the FA3 call).   */
/* ------------------------------------------------------------------------ */

/* Key range of query i of request b: its position is p = cache_seqlens[b] - L + i
 * (causal, bottom-right aligned: the block's last query sees the last key);
 * with a window W > 0 it sees keys p-W+1 .. p (the token and the W-1 before
 * it), clamped at 0.  Returns the count; *lo gets the first key. */
static int64_t key_range(const orc_config* cfg, const int32_t* cache_seqlens, int64_t t,
                         int64_t* lo) {
  int64_t b = t / cfg->q_len, i = t % cfg->q_len;
  int64_t p = (int64_t)cache_seqlens[b] - cfg->q_len + i;
  int64_t first = 0;
  if (cfg->window > 0) first = p - cfg->window + 1;
  if (first < 0) first = 0;
  *lo = first;
  return p >= first ? p - first + 1 : 0;
}

/* Flat cache row holding logical key j of request b. */
static int64_t key_row(const orc_config* cfg, const int32_t* page_table, int64_t b, int64_t j) {
  int64_t pg = j / cfg->page_size;
  if (pg >= cfg->max_pages) return -1;
  int64_t phys = page_table[b * cfg->max_pages + pg];
  if (phys < 0 || phys >= cfg->num_pages) return -1;
  return phys * cfg->page_size + j % cfg->page_size;
}

/* One (token t, q head h) pair of orc_attention; sc: scratch of at least
 * the pair's key count. */
static int attend_pair(const orc_config* cfg, const uint8_t* q, const uint8_t* k_cache,
                       const uint8_t* v_cache, const int32_t* page_table,
                       const int32_t* cache_seqlens, double kd, double vd, int64_t t, int h,
                       double* sc, double* o) {
  const int hq = cfg->num_q_heads, hkv = cfg->num_kv_heads, d = cfg->head_dim;
  const int64_t b = t / cfg->q_len;
  const int g = h / (hq / hkv);
  double qv[256];
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  int64_t lo;
  const int64_t cnt = key_range(cfg, cache_seqlens, t, &lo);
  if (cnt == 0) return ORC_OK;
  for (int c = 0; c < d; ++c) qv[c] = orc_e4m3_decode(q[(t * hq + h) * d + c]);
  double mx = -INFINITY;
  for (int64_t k = 0; k < cnt; ++k) {
    const int64_t r = key_row(cfg, page_table, b, lo + k);
    if (r < 0) return ORC_BAD_ROW;
    const uint8_t* kr = k_cache + (r * hkv + g) * d;
    double dot = 0.0;
    for (int c = 0; c < d; ++c) dot += qv[c] * orc_e4m3_decode(kr[c]);
    sc[k] = dot * kd * (double)cfg->sm_scale;
    if (sc[k] > mx) mx = sc[k];
  }
  double wsum = 0.0;
  for (int64_t k = 0; k < cnt; ++k) {
    const double w = exp(sc[k] - mx);
    wsum += w;
    const int64_t r = key_row(cfg, page_table, b, lo + k);
    const uint8_t* vr = v_cache + (r * hkv + g) * d;
    for (int c = 0; c < d; ++c) o[c] += w * orc_e4m3_decode(vr[c]);
  }
  for (int c = 0; c < d; ++c) o[c] = vd * o[c] / wsum;
  return ORC_OK;
}

/*
 * Attention output before any rounding, for selected (token, q head) pairs.
 *   q          e4m3 [T, Hq, D]
 *   sel_t/h    n_sel pairs; NULL for all T*Hq pairs in (t, h) order
 *   o_out      double [n_sel, D]
 * Scores s_j = (q . k_j) * k_descale * sm_scale over the visible keys, weights
 * exp(s_j - max s), o = v_descale * sum w_j v_j / sum w_j.  Query head h reads
 * KV head h / (Hq/Hkv) (READING: the usual grouped-query map).  The descales
 * are the cache scales on the scaled path and 1 otherwise (the page passes
 * k_descale / v_descale only when the scales are set).  A query with no
 * visible key gets o = 0 (READING).
 * The pairs are independent, so they are spread over OpenMP threads (when
 * the library is built with OpenMP); each pair's arithmetic and its order
 * are the same whatever the thread count.
 */
int orc_attention(const orc_config* cfg, const uint8_t* q, const uint8_t* k_cache,
                  const uint8_t* v_cache, const int32_t* page_table, const int32_t* cache_seqlens,
                  float k_scale, float v_scale, int64_t n_sel, const int64_t* sel_t,
                  const int32_t* sel_h, double* o_out) {
  if (!cfg_ok(cfg)) return ORC_BAD_ARG;
  const int hq = cfg->num_q_heads, d = cfg->head_dim;
  const int64_t T = (int64_t)cfg->batch * cfg->q_len;
  const int scaled = cfg->kv_scale != 1.0f;
  const double kd = scaled ? (double)k_scale : 1.0, vd = scaled ? (double)v_scale : 1.0;
  if (!sel_t) n_sel = T * hq;
  for (int64_t n = 0; n < n_sel; ++n) {
    const int64_t t = sel_t ? sel_t[n] : n / hq;
    const int h = sel_h ? sel_h[n] : (int)(n % hq);
    if (t < 0 || t >= T || h < 0 || h >= hq) return ORC_BAD_ARG;
  }
  int rc = ORC_OK;
#pragma omp parallel
  {
    double* sc = NULL;
    int64_t sc_cap = 0;
#pragma omp for schedule(dynamic, 4)
    for (int64_t n = 0; n < n_sel; ++n) {
      const int64_t t = sel_t ? sel_t[n] : n / hq;
      const int h = sel_h ? sel_h[n] : (int)(n % hq);
      int64_t lo;
      const int64_t cnt = key_range(cfg, cache_seqlens, t, &lo);
      if (cnt > sc_cap) {
        free(sc);
        sc_cap = cnt;
        sc = (double*)malloc(sizeof(double) * (size_t)cnt);
      }
      int r = (cnt > 0 && !sc) ? ORC_BAD_ARG
                               : attend_pair(cfg, q, k_cache, v_cache, page_table, cache_seqlens,
                                             kd, vd, t, h, sc, o_out + n * d);
      if (r != ORC_OK) {
#pragma omp critical
        rc = r;
      }
    }
    free(sc);
  }
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Page-list-driven (top-k block-sparse) decode (page "msa.py":              */
/* msa_sparse_decode_main and build_msa_decode_meta): each request is one    */
/* decode query at position cache_seqlens[b] - 1 attending to its cached     */
/* keys through the blocks a per-KV-head top-k list selects.                 */
/* block_idx int32 [Hkv, B, topk]: logical block indices, -1 padding; block  */
/* j holds keys j*BS .. (j+1)*BS - 1 of the request, those below             */
/* cache_seqlens[b] being visible (READING: the plan's qo_offset places the  */
/* query at the last cached position, and non-causal decode sees every      */
/* cached key of a selected block).  Query head h reads the list of KV head  */
/* h / (Hq/Hkv).  The key set is the union of the selected blocks (a         */
/* repeated index adds nothing); no window applies.  Scores, weights,        */
/* descales and the empty-set output 0 are as in orc_attention.              */
/* ------------------------------------------------------------------------ */
/* One (request b, KV head g) of orc_sparse_attention: its visible-key set and
 * its grp query heads; vis and sc hold at least max(cs, 1) entries. */
static int sparse_head(const orc_config* cfg, const uint8_t* q, const uint8_t* k_cache,
                       const uint8_t* v_cache, const int32_t* page_table, int64_t cs,
                       const int32_t* block_idx, int32_t block_size, int32_t topk, double kd,
                       double vd, int64_t b, int g, unsigned char* vis, double* sc,
                       double* o_out) {
  const int hq = cfg->num_q_heads, hkv = cfg->num_kv_heads, d = cfg->head_dim;
  const int grp = hq / hkv;
  const int64_t B = cfg->batch;
  double qv[256];
  /* visible keys of this KV head: the union of its selected blocks, below cs */
  memset(vis, 0, (size_t)(cs > 0 ? cs : 1));
  for (int i = 0; i < topk; ++i) {
    const int64_t j = block_idx[((int64_t)g * B + b) * topk + i];
    if (j < 0) continue;
    for (int64_t key = j * block_size; key < (j + 1) * block_size && key < cs; ++key) vis[key] = 1;
  }
  for (int hh = 0; hh < grp; ++hh) {
    const int h = g * grp + hh;
    double* o = o_out + (b * hq + h) * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int c = 0; c < d; ++c) qv[c] = orc_e4m3_decode(q[(b * hq + h) * d + c]);
    double mx = -INFINITY;
    int64_t cnt = 0;
    for (int64_t key = 0; key < cs; ++key) {
      if (!vis[key]) continue;
      const int64_t r = key_row(cfg, page_table, b, key);
      if (r < 0) return ORC_BAD_ROW;
      const uint8_t* kr = k_cache + (r * hkv + g) * d;
      double dot = 0.0;
      for (int c = 0; c < d; ++c) dot += qv[c] * orc_e4m3_decode(kr[c]);
      sc[key] = dot * kd * (double)cfg->sm_scale;
      if (sc[key] > mx) mx = sc[key];
      ++cnt;
    }
    if (cnt == 0) continue;
    double wsum = 0.0;
    for (int64_t key = 0; key < cs; ++key) {
      if (!vis[key]) continue;
      const double w = exp(sc[key] - mx);
      wsum += w;
      const int64_t r = key_row(cfg, page_table, b, key);
      const uint8_t* vr = v_cache + (r * hkv + g) * d;
      for (int c = 0; c < d; ++c) o[c] += w * orc_e4m3_decode(vr[c]);
    }
    for (int c = 0; c < d; ++c) o[c] = vd * o[c] / wsum;
  }
  return ORC_OK;
}

/* The (request, KV head) pairs are independent and spread over OpenMP
 * threads; each pair's arithmetic is the same whatever the thread count. */
int orc_sparse_attention(const orc_config* cfg, const uint8_t* q, const uint8_t* k_cache,
                         const uint8_t* v_cache, const int32_t* page_table,
                         const int32_t* cache_seqlens, const int32_t* block_idx,
                         int32_t block_size, int32_t topk, float k_scale, float v_scale,
                         double* o_out) {
  if (!cfg_ok(cfg) || cfg->q_len != 1 || block_size < 1 || topk < 1) return ORC_BAD_ARG;
  const int hkv = cfg->num_kv_heads;
  const int64_t B = cfg->batch;
  const int scaled = cfg->kv_scale != 1.0f;
  const double kd = scaled ? (double)k_scale : 1.0, vd = scaled ? (double)v_scale : 1.0;
  int rc = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bg = 0; bg < B * hkv; ++bg) {
    const int64_t b = bg / hkv;
    const int g = (int)(bg % hkv);
    const int64_t cs = cache_seqlens[b];
    unsigned char* vis = (unsigned char*)calloc((size_t)(cs > 0 ? cs : 1), 1);
    double* sc = (double*)malloc(sizeof(double) * (size_t)(cs > 0 ? cs : 1));
    int r = (!vis || !sc) ? ORC_BAD_ARG
                          : sparse_head(cfg, q, k_cache, v_cache, page_table, cs, block_idx,
                                        block_size, topk, kd, vd, b, g, vis, sc, o_out);
    free(vis);
    free(sc);
    if (r != ORC_OK) {
#pragma omp critical
      rc = r;
    }
  }
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Step 6: the gated epilogue (page: rms_norm_gate on the bf16 attention     */
/* output, weight None, eps 1e-5).                                          */
/* ------------------------------------------------------------------------ */

/*
 * For each selected pair: ob = bf16(o) (the attention result is bf16 on the
 * page), r = 1/sqrt(mean(ob^2) + 1e-5), out = bf16(ob * r * sigmoid(gate)),
 * with gate = qkv[t, (Hq + 2Hkv)*D + h*D + c].  One rounding at the end
 * (READING: the epilogue's internal precision is not shown on the page).
 *   o_in   double [n_sel, D];  out  bf16 bits [n_sel, D]
 */
int orc_epilogue(const orc_config* cfg, const double* o_in, const uint16_t* qkv, int64_t n_sel,
                 const int64_t* sel_t, const int32_t* sel_h, uint16_t* out) {
  if (!cfg_ok(cfg)) return ORC_BAD_ARG;
  const int hq = cfg->num_q_heads, hkv = cfg->num_kv_heads, d = cfg->head_dim;
  const int64_t T = (int64_t)cfg->batch * cfg->q_len;
  const int64_t width = (int64_t)(2 * hq + 2 * hkv) * d;
  const int64_t gate_off = (int64_t)(hq + 2 * hkv) * d;
  if (!sel_t) n_sel = T * hq;
  double ob[256];
  for (int64_t n = 0; n < n_sel; ++n) {
    int64_t t = sel_t ? sel_t[n] : n / hq;
    int h = sel_h ? sel_h[n] : (int)(n % hq);
    if (t < 0 || t >= T || h < 0 || h >= hq) return ORC_BAD_ARG;
    double ss = 0.0;
    for (int c = 0; c < d; ++c) {
      ob[c] = (double)bf16r(o_in[n * d + c]);
      ss += ob[c] * ob[c];
    }
    double r = 1.0 / sqrt(ss / d + 1.0e-5);
    for (int c = 0; c < d; ++c) {
      double gt = (double)orc_bf16_to_float(qkv[t * width + gate_off + (int64_t)h * d + c]);
      double sig = 1.0 / (1.0 + exp(-gt));
      out[n * d + c] = orc_bf16_round(ob[c] * r * sig);
    }
  }
  return ORC_OK;
}

/* The sparse decode step: the same prologue and epilogue around the         */
/* block-sparse attention (every cache store before any attention read).     */
int orc_sparse_step(const orc_config* cfg, const uint16_t* qkv, const int64_t* positions,
                    const int64_t* cache_loc, const int32_t* cache_seqlens,
                    const int32_t* page_table, const int32_t* block_idx, int32_t block_size,
                    int32_t topk, uint8_t* k_cache, uint8_t* v_cache, float k_scale,
                    float v_scale, uint8_t* q_out, double* o_scratch, uint16_t* out) {
  int rc = orc_prologue(cfg, qkv, positions, cache_loc, k_cache, v_cache, k_scale, v_scale, q_out);
  if (rc) return rc;
  rc = orc_sparse_attention(cfg, q_out, k_cache, v_cache, page_table, cache_seqlens, block_idx,
                            block_size, topk, k_scale, v_scale, o_scratch);
  if (rc) return rc;
  return orc_epilogue(cfg, o_scratch, qkv, 0, NULL, NULL, out);
}

/* ------------------------------------------------------------------------ */
/* The whole step, in the page's order: every cache store happens before any */
/* attention read.  o_scratch: double [T*Hq*D] caller-provided.              */
/* ------------------------------------------------------------------------ */
int orc_step(const orc_config* cfg, const uint16_t* qkv, const int64_t* positions,
             const int64_t* cache_loc, const int32_t* cache_seqlens, const int32_t* page_table,
             uint8_t* k_cache, uint8_t* v_cache, float k_scale, float v_scale, uint8_t* q_out,
             double* o_scratch, uint16_t* out) {
  int rc = orc_prologue(cfg, qkv, positions, cache_loc, k_cache, v_cache, k_scale, v_scale, q_out);
  if (rc) return rc;
  rc = orc_attention(cfg, q_out, k_cache, v_cache, page_table, cache_seqlens, k_scale, v_scale, 0,
                     NULL, NULL, o_scratch);
  if (rc) return rc;
  return orc_epilogue(cfg, o_scratch, qkv, 0, NULL, NULL, out);
}

/* ------------------------------------------------------------------------ */
/* Step metadata: the per-token positions and cache rows and the per-request */
/* key counts that every layer of a step shares, from the cached lengths and */
/* the page table.                                                           */
/*                                                                          */
/* Page "012-attention-local-splits.py", `Inputs`: token t = b*L + i sits at */
/* position seq_lens[b] + i; cache_loc[t] is the flat cache row the page     */
/* table gives that position (physical page * page_size + offset in page);   */
/* cache_seqlens = seq_lens + L.  Page "msa.py" (update_msa_decode_cg_meta): */
/* graph replay pads the batch with seq_len == 0 slots, masked by a zero key */
/* count.                                                                    */
/* READING: in a decode or verify step (q_len <= 8) a slot with seq_lens[b]  */
/* <= 0 is padding (a decode request always has cached tokens); in an extend */
/* step (q_len > 8) seq_lens[b] == 0 is a new request with an empty prefix   */
/* and only seq_lens[b] < 0 is padding.  A padded slot's tokens get position */
/* 0 and cache row -1 (nothing is stored) and the slot key count 0 (no key,  */
/* output 0).  A position whose page-table entry lies beyond max_pages or is */
/* negative also gets cache row -1.                                          */
/* ------------------------------------------------------------------------ */
int orc_step_meta(const orc_config* cfg, const int32_t* seq_lens, const int32_t* page_table,
                  int64_t* positions, int64_t* cache_loc, int32_t* cache_seqlens) {
  if (!cfg_ok(cfg)) return ORC_BAD_ARG;
  const int64_t P = cfg->page_size;
  for (int64_t b = 0; b < cfg->batch; ++b) {
    const int64_t len = seq_lens[b];
    const int pad = cfg->q_len <= 8 ? len <= 0 : len < 0;
    cache_seqlens[b] = pad ? 0 : (int32_t)(len + cfg->q_len);
    for (int64_t i = 0; i < cfg->q_len; ++i) {
      const int64_t t = b * cfg->q_len + i;
      if (pad) {
        positions[t] = 0;
        cache_loc[t] = -1;
        continue;
      }
      const int64_t p = len + i;
      positions[t] = p;
      const int64_t page = p / P;
      int64_t entry = -1;
      if (page < cfg->max_pages) entry = page_table[b * cfg->max_pages + page];
      cache_loc[t] = entry < 0 ? -1 : entry * P + p % P;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* The physical page table of a step from the allocator's map (page          */
/* "msa.py", _build_page_table): req_to_token[r, p] is the physical slot of  */
/* logical position p of request row r; pages hold page_size contiguous      */
/* slots, so the physical page of logical page i of request b is             */
/* req_to_token[slot_ids[b], i * P] / P, for i < ceil(kv_lens[b] / P).       */
/*   page_table  int32 [B, max_pages] (NULL: not built): those pages, then   */
/*               -1 to the end of the row (page 1's layout)                  */
/*   kv_indices  int32 [sum of page counts] (NULL: not built): the same      */
/*               pages packed request after request (page 2's kv_indices),   */
/*               request b's from kv_indptr[b]                               */
/*   kv_indptr   int32 [B + 1] (needed with kv_indices): exclusive prefix    */
/*               sums of the page counts                                     */
/* READING: kv_lens[b] <= 0 gives no page (a padded slot); a negative map    */
/* entry is no slot and gives -1.  A slot id outside 0..max_reqs-1, a page   */
/* whose first position lies past the map's row, or more pages than          */
/* max_pages for the padded table is a caller error (ORC_BAD_ARG).           */
/* ------------------------------------------------------------------------ */
int orc_page_table(const int32_t* req_to_token, int64_t req_stride, int64_t max_reqs,
                   const int32_t* slot_ids, const int32_t* kv_lens, int32_t batch,
                   int32_t page_size, int32_t max_pages, int32_t* page_table,
                   int32_t* kv_indices, int32_t* kv_indptr) {
  if (batch < 0 || page_size < 1 || req_stride < 1 || max_reqs < 1) return ORC_BAD_ARG;
  if (page_table && max_pages < 1) return ORC_BAD_ARG;
  if (kv_indices && !kv_indptr) return ORC_BAD_ARG;
  int64_t packed = 0;
  if (kv_indptr) kv_indptr[0] = 0;
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t r = slot_ids[b];
    if (r < 0 || r >= max_reqs) return ORC_BAD_ARG;
    const int64_t len = kv_lens[b];
    const int64_t n = len > 0 ? (len + page_size - 1) / page_size : 0;
    if (n > 0 && (n - 1) * page_size >= req_stride) return ORC_BAD_ARG;
    if (page_table && n > max_pages) return ORC_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t slot = req_to_token[r * req_stride + i * page_size];
      const int32_t page = slot < 0 ? -1 : (int32_t)(slot / page_size);
      if (page_table) page_table[b * max_pages + i] = page;
      if (kv_indices) kv_indices[packed + i] = page;
    }
    if (page_table)
      for (int64_t i = n; i < max_pages; ++i) page_table[b * max_pages + i] = -1;
    packed += n;
    if (kv_indptr) kv_indptr[b + 1] = (int32_t)packed;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Page "qk_norm" (vLLM's CuTeDSL fused QK-norm for MuseSpark1x attention):  */
/* the `qk_norm` function and the kernel of its `QKNormDirectKernel` class.  */
/* Each head_dim-wide group of a row of x [M, heads * head_dim] (rows        */
/* `row_stride` elements apart, the last dimension contiguous) is normed     */
/* without a weight: rstd = rsqrt(sum of squares / head_dim + eps); the      */
/* kernel keeps x * rstd in fp32, multiplies by the output scale when one is */
/* given, and rounds once, on the store, to the input's 16-bit type.         */
/* READING: the page's fp32 sum and fastmath rsqrt are taken exactly: the    */
/* sum of squares (each square exact in fp32) is formed in double and        */
/* rounded once to fp32, and rsqrt is correctly rounded; the divide by       */
/* head_dim and the + eps are fp32 operations.  The scale multiplies only    */
/* when it is not 1 (the page compiles the product out otherwise; a product  */
/* by 1 changes nothing either way).                                         */
/* ------------------------------------------------------------------------ */

/* IEEE binary16 bit pattern -> value (exact). */
double orc_fp16_to_double(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0x1F) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -24); /* subnormal: quantum 2^-24 */
  else v = ldexp(1024.0 + (double)m, e - 25);
  return s ? -v : v;
}

/* Round a real number to binary16, to nearest with ties to even.  Written
 * from the format: 11 significant bits, normal exponents down to 2^-14,
 * subnormal quantum 2^-24, largest finite 65504; from the halfway point
 * 65520 up the result is infinity. */
uint16_t orc_fp16_round(double x) {
  if (isnan(x)) return 0x7E00;
  const uint16_t sign = signbit(x) ? 0x8000 : 0;
  const double ax = fabs(x);
  if (ax >= 65520.0) return sign | 0x7C00;
  if (ax == 0.0) return sign;
  int e;
  frexp(ax, &e); /* leading bit 2^(e-1) */
  int lead = e - 1;
  if (lead < -14) lead = -14;
  const double quantum = ldexp(1.0, lead - 10);
  const double q = nearbyint(ax / quantum); /* ties to even */
  const double r = q * quantum;
  if (r < ldexp(1.0, -14)) return sign | (uint16_t)q; /* subnormal (q < 1024) */
  int re;
  frexp(r, &re);
  const int rl = re - 1; /* rounding may carry into the next binade */
  const double mant = r / ldexp(1.0, rl) - 1.0;
  return sign | (uint16_t)(((rl + 15) << 10) | (int)nearbyint(mant * 1024.0));
}

/* dtype 0: bfloat16, 1: binary16. */
int orc_qk_norm(const uint16_t* x, int64_t M, int32_t num_heads, int32_t head_dim,
                int64_t row_stride, int32_t dtype, float eps, float scale, uint16_t* out) {
  if (M < 0 || num_heads < 1 || head_dim < 1 || (dtype != 0 && dtype != 1) ||
      row_stride < (int64_t)num_heads * head_dim)
    return ORC_BAD_ARG;
  const int64_t n = (int64_t)num_heads * head_dim;
  for (int64_t r = 0; r < M; ++r) {
    for (int32_t h = 0; h < num_heads; ++h) {
      const uint16_t* xs = x + r * row_stride + (int64_t)h * head_dim;
      uint16_t* os = out + r * n + (int64_t)h * head_dim;
      double ss = 0.0;
      for (int32_t c = 0; c < head_dim; ++c) {
        const float v = dtype ? (float)orc_fp16_to_double(xs[c]) : orc_bf16_to_float(xs[c]);
        ss += (double)(v * v);
      }
      const float ms = (float)ss / (float)head_dim;
      const float rstd = orc_rsqrt_cr(ms + eps);
      for (int32_t c = 0; c < head_dim; ++c) {
        const float v = dtype ? (float)orc_fp16_to_double(xs[c]) : orc_bf16_to_float(xs[c]);
        float y = v * rstd;
        if (scale != 1.0f) y = y * scale;
        os[c] = dtype ? orc_fp16_round((double)y) : orc_bf16_round((double)y);
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Thread control of the OpenMP loops above (test and benchmark use only):   */
/* n > 0 sets the thread count; returns the count the next loop will use (1  */
/* when the library was built without OpenMP).                               */
/* ------------------------------------------------------------------------ */
#ifdef _OPENMP
#include <omp.h>
#endif
int orc_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

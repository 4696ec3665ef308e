/*
 * oracle.c -- plain fp64 CPU oracle for Flint's decode-attention hot path.
 *
 * TEST INFRASTRUCTURE: loaded only by the tests, the smoke check and the
 * bench's cpu_baseline leg.  It shares no code with the HIP library.  Every
 * function is the plain definition written out in double precision; there is
 * no tiling, fusion or reordering of the arithmetic beyond what the
 * definition states.  See oracle.h for the sources and the cache layout.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* O1: bf16 from its definition.  A bf16 number is sign, 8 exponent bits and
 * 7 fraction bits with IEEE-754 binary semantics (bias 127).               */

/* value of a 15-bit magnitude field, treating exponent 255 as an ordinary
 * exponent (so the field after the largest finite value reads as 2^128). */
static double mag_value(uint32_t m) {
  uint32_t e = m >> 7, f = m & 0x7Fu;
  if (e == 0) return ldexp((double)f, -133); /* subnormal: f/128 * 2^-126 */
  return ldexp(1.0 + (double)f / 128.0, (int)e - 127);
}

double orc_bf16_value(uint16_t b) {
  double sgn = (b & 0x8000u) ? -1.0 : 1.0;
  uint32_t m = b & 0x7FFFu;
  if ((m >> 7) == 0xFFu) return (m & 0x7Fu) ? NAN : sgn * INFINITY;
  return sgn * mag_value(m);
}

/* Round a real value to the nearest bf16; ties go to the even fraction. */
static uint16_t bf16_rne_double(double x) {
  if (isnan(x)) return 0x7FC0u;
  uint16_t sign = signbit(x) ? 0x8000u : 0;
  double a = fabs(x);
  if (a >= ldexp(1.0, 128)) return sign | 0x7F80u;
  /* largest magnitude field lo with value(lo) <= a; value(0x7F80) = 2^128 > a */
  uint32_t lo = 0, hi = 0x7F80u;
  while (hi - lo > 1) {
    uint32_t mid = (lo + hi) / 2;
    if (mag_value(mid) <= a) lo = mid; else hi = mid;
  }
  double dlo = a - mag_value(lo), dhi = mag_value(lo + 1) - a; /* both exact */
  uint32_t m;
  if (dlo < dhi) m = lo;
  else if (dhi < dlo) m = lo + 1;
  else m = (lo & 1u) ? lo + 1 : lo;
  return sign | (uint16_t)m; /* m == 0x7F80 is infinity */
}

uint16_t orc_bf16_rne(float x) {
  if (isnan(x)) { /* keep the payload, set the quiet bit */
    uint32_t u; memcpy(&u, &x, 4);
    return (uint16_t)((u >> 16) | 0x0040u);
  }
  return bf16_rne_double((double)x);
}

void orc_bf16_rne_array(const double* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = bf16_rne_double(x[i]);
}

static double g_bf16[65536];
__attribute__((constructor)) static void init_table(void) {
  for (uint32_t b = 0; b < 65536u; ++b) g_bf16[b] = orc_bf16_value((uint16_t)b);
}
static inline double bf(uint16_t b) { return g_bf16[b]; }

/* ------------------------------------------------------------------------ */
/* fp8 E4M3 by its definition: code c (0..126 for the finite magnitudes) is
 * m/8 * 2^-6 for exponent field 0 and (1 + m/8) * 2^(e-7) otherwise. */
static double fp8_mag(int c) {
  const int e = c >> 3, m = c & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

double orc_fp8_value(uint8_t c) {
  if ((c & 0x7F) == 0x7F) return NAN;
  const double v = fp8_mag(c & 0x7F);
  return (c & 0x80) ? -v : v;
}

uint8_t orc_fp8_rne(double x) {
  const uint8_t s = signbit(x) ? 0x80 : 0;
  if (isnan(x)) return s | 0x7F;
  const double a = fabs(x);
  if (a >= 448.0) return s | 0x7E; /* saturate to the largest finite value */
  /* codes 0..0x7E grow with their value: bracket a as mag(lo) <= a < mag(hi) */
  int lo = 0, hi = 0x7E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (fp8_mag(mid) <= a) lo = mid; else hi = mid;
  }
  const double dl = a - fp8_mag(lo), dh = fp8_mag(hi) - a;
  const int c = dl < dh ? lo : (dh < dl ? hi : ((lo & 1) ? hi : lo));
  return (uint8_t)(s | c);
}

static double g_fp8[256];
__attribute__((constructor)) static void init_fp8_table(void) {
  for (int c = 0; c < 256; ++c) g_fp8[c] = orc_fp8_value((uint8_t)c);
}

/* element i of the K (resp. V) cache as a real number */
static inline double k_at(const orc_layer* L, const void* kc, int64_t i) {
  return L->kv_fp8 ? g_fp8[((const uint8_t*)kc)[i]] * L->k_scale : bf(((const uint16_t*)kc)[i]);
}
static inline double v_at(const orc_layer* L, const void* vc, int64_t i) {
  return L->kv_fp8 ? g_fp8[((const uint8_t*)vc)[i]] * L->v_scale : bf(((const uint16_t*)vc)[i]);
}

/* ------------------------------------------------------------------------ */
/* O2: per-head RMSNorm (hnkhoi "Model architecture": per-head Q/K RMSNorm). */
void orc_rmsnorm(const float* x, const float* w, int n, double eps, double* y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
  double r = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) y[i] = (double)x[i] * r * (double)w[i];
}

/* O3: rotate-half RoPE on the sliding layers (hnkhoi "Model architecture").
 * Reading: base theta, all d dims rotate, pairs (i, i+d/2), absolute
 * 0-based positions. */
void orc_rope(double* x, int d, double pos, double theta) {
  int half = d / 2;
  for (int i = 0; i < half; ++i) {
    double a = pos * pow(theta, -2.0 * i / d);
    double c = cos(a), s = sin(a);
    double x0 = x[i], x1 = x[i + half];
    x[i] = x0 * c - x1 * s;
    x[i + half] = x1 * c + x0 * s;
  }
}

/* ------------------------------------------------------------------------ */
/* O8: page walk. */
int64_t orc_slot(const int32_t* bt, int bt_stride, int bs, int b, int pos) {
  int32_t page = bt[(int64_t)b * bt_stride + pos / bs];
  return (int64_t)page * bs + pos % bs;
}

/* Cache layout (the library's own convention; the pages fix none).  Each
 * (page, KV head g) owns one contiguous tile of bs * d elements.
 * bf16 (d a multiple of 8): K in blocks of 32 dims, each in groups of 8 dims,
 * each group holding the 8 dims of every row in turn:
 *   (dim >> 5) * bs * 32 + ((dim >> 3) & 3) * bs * 8 + row * 8 + (dim & 7);
 * V dim-major: dim * bs + row.
 * fp8 (d = 128, bs = 16 only), within the 2048-byte tile:
 *   K: ((dim >> 4) & 1) * 1024 + (dim >> 5) * 256 + row * 16 + (dim & 15)
 *   V: (dim >> 6) * 1024 + ((row >> 2) * 16 + (dim & 15)) * 16
 *      + ((dim >> 4) & 3) * 4 + (row & 3) */
int64_t orc_k_offset(const orc_layer* L, int64_t page, int g, int row, int dim) {
  const int64_t tile = (page * L->hkv + g) * (int64_t)L->bs * L->d;
  if (L->kv_fp8) return tile + ((dim >> 4) & 1) * 1024 + (dim >> 5) * 256 + row * 16 + (dim & 15);
  return tile + (int64_t)(dim >> 5) * L->bs * 32 + ((dim >> 3) & 3) * L->bs * 8 + row * 8 + (dim & 7);
}
int64_t orc_v_offset(const orc_layer* L, int64_t page, int g, int row, int dim) {
  const int64_t tile = (page * L->hkv + g) * (int64_t)L->bs * L->d;
  if (L->kv_fp8)
    return tile + (dim >> 6) * 1024 + ((row >> 2) * 16 + (dim & 15)) * 16 + ((dim >> 4) & 3) * 4 +
           (row & 3);
  return tile + (int64_t)dim * L->bs + row;
}

/* the fp8 tile order above is defined for d = 128 and bs = 16 only */
static int bad_shape(const orc_layer* L) { return L->kv_fp8 && (L->d != 128 || L->bs != 16); }

/* O4: norm -> rope -> cache write, in that order (reading of the vLLM day-0
 * post, "What happened": fused normalisation, rotary and cache operations). */
int orc_append(const orc_layer* L, int T, const float* q_in, const float* k_in,
               const float* v_in, const float* qw, const float* kw,
               const int32_t* positions, const int32_t* slots,
               double* q_out, void* kc, void* vc, int num_blocks) {
  const int d = L->d;
  if (bad_shape(L)) return -2;
  double* tmp = (double*)malloc(sizeof(double) * d);
  int rc = 0;
  for (int t = 0; t < T; ++t) {
    double pos = positions[t];
    if (q_out) {
      for (int h = 0; h < L->hq; ++h) {
        double* y = q_out + ((int64_t)t * L->hq + h) * d;
        orc_rmsnorm(q_in + ((int64_t)t * L->hq + h) * d, qw, d, L->eps, y);
        if (L->use_rope) orc_rope(y, d, pos, L->theta);
      }
    }
    int32_t slot = slots[t];
    if (slot < 0) continue;
    if ((int64_t)slot >= (int64_t)num_blocks * L->bs) { rc = -1; continue; }
    int64_t page = slot / L->bs;
    int row = slot % L->bs;
    for (int g = 0; g < L->hkv; ++g) {
      orc_rmsnorm(k_in + ((int64_t)t * L->hkv + g) * d, kw, d, L->eps, tmp);
      if (L->use_rope) orc_rope(tmp, d, pos, L->theta);
      const float* v = v_in + ((int64_t)t * L->hkv + g) * d;
      for (int i = 0; i < d; ++i) {
        const int64_t ko = orc_k_offset(L, page, g, row, i), vo = orc_v_offset(L, page, g, row, i);
        if (L->kv_fp8) {
          ((uint8_t*)kc)[ko] = orc_fp8_rne(tmp[i] / L->k_scale);
          ((uint8_t*)vc)[vo] = orc_fp8_rne((double)v[i] / L->v_scale);
        } else {
          ((uint16_t*)kc)[ko] = bf16_rne_double(tmp[i]);
          ((uint16_t*)vc)[vo] = orc_bf16_rne(v[i]);
        }
      }
    }
  }
  free(tmp);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* O5: attention of one query row, one head, with the sink.
 * Reading (the pages only say "learned attention sinks"): the sink is one
 * scalar logit per query head that joins the softmax denominator, is not
 * multiplied by the softmax scale and carries no value.
 * Keys: lo..t with lo = 0 (full layers) or max(0, t-window+1) (sliding). */
static int attend_row(const orc_layer* L, const double* qh, int h, const void* kc,
                      const void* vc, int num_blocks, const int32_t* bt, int bt_stride,
                      int b, int t, double sink, double* out) {
  const int d = L->d, g = h / (L->hq / L->hkv);
  int lo = (L->window > 0) ? t - L->window + 1 : 0;
  if (lo < 0) lo = 0;
  int n = t - lo + 1;
  double* s = (double*)malloc(sizeof(double) * (size_t)n);
  int32_t* pages = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  double m = sink;
  for (int j = lo; j <= t; ++j) {
    int32_t page = bt[(int64_t)b * bt_stride + j / L->bs];
    if (page < 0 || page >= num_blocks) { free(s); free(pages); return -1; }
    pages[j - lo] = page;
    double dot = 0.0;
    for (int i = 0; i < d; ++i) dot += qh[i] * k_at(L, kc, orc_k_offset(L, page, g, j % L->bs, i));
    s[j - lo] = L->scale * dot;
    if (s[j - lo] > m) m = s[j - lo];
  }
  double z = exp(sink - m);
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  for (int j = 0; j < n; ++j) {
    double e = exp(s[j] - m);
    z += e;
    const int row = (lo + j) % L->bs;
    for (int i = 0; i < d; ++i) out[i] += e * v_at(L, vc, orc_v_offset(L, pages[j], g, row, i));
  }
  for (int i = 0; i < d; ++i) out[i] /= z;
  free(s);
  free(pages);
  return 0;
}

int orc_default_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int orc_attn_decode(const orc_layer* L, int B, const double* q, const void* kc,
                    const void* vc, int num_blocks, const int32_t* bt, int bt_stride,
                    const int32_t* seq_lens, const float* sinks, double* out, int nthreads) {
  if (bad_shape(L)) return -2;
  if (nthreads <= 0) nthreads = orc_default_threads();
  int bad = 0;
  const int64_t items = (int64_t)B * L->hq;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
  for (int64_t it = 0; it < items; ++it) {
    int b = (int)(it / L->hq), h = (int)(it % L->hq);
    int t = seq_lens[b] - 1;
    if (t < 0) { bad |= 1; continue; }
    const double* qh = q + ((int64_t)b * L->hq + h) * L->d;
    double* o = out + ((int64_t)b * L->hq + h) * L->d;
    if (attend_row(L, qh, h, kc, vc, num_blocks, bt, bt_stride, b, t, (double)sinks[h], o))
      bad |= 1;
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* O6: partial softmax over a key range and the log-sum-exp merge. */
void orc_attn_partial(const orc_layer* L, const double* qh, int h, const void* kc,
                      const void* vc, const int32_t* bt, int bt_stride, int b,
                      int j0, int j1, double* ot, double* lse) {
  const int d = L->d, g = h / (L->hq / L->hkv);
  for (int i = 0; i < d; ++i) ot[i] = 0.0;
  if (bad_shape(L)) { *lse = NAN; return; }
  if (j1 <= j0) { *lse = -INFINITY; return; }
  int n = j1 - j0;
  double* s = (double*)malloc(sizeof(double) * (size_t)n);
  double m = -INFINITY;
  for (int j = j0; j < j1; ++j) {
    const int32_t page = bt[(int64_t)b * bt_stride + j / L->bs];
    double dot = 0.0;
    for (int i = 0; i < d; ++i) dot += qh[i] * k_at(L, kc, orc_k_offset(L, page, g, j % L->bs, i));
    s[j - j0] = L->scale * dot;
    if (s[j - j0] > m) m = s[j - j0];
  }
  double l = 0.0;
  for (int j = j0; j < j1; ++j) {
    const int32_t page = bt[(int64_t)b * bt_stride + j / L->bs];
    double e = exp(s[j - j0] - m);
    l += e;
    for (int i = 0; i < d; ++i)
      ot[i] += e * v_at(L, vc, orc_v_offset(L, page, g, j % L->bs, i));
  }
  for (int i = 0; i < d; ++i) ot[i] /= l;
  *lse = m + log(l);
  free(s);
}

void orc_merge(int S, int d, const double* ot, const double* lse, double sink, double* out) {
  double M = sink;
  for (int s = 0; s < S; ++s) if (lse[s] > M) M = lse[s];
  double den = exp(sink - M);
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  for (int s = 0; s < S; ++s) {
    if (isinf(lse[s]) && lse[s] < 0) continue; /* empty range contributes 0 */
    double w = exp(lse[s] - M);
    den += w;
    for (int i = 0; i < d; ++i) out[i] += w * ot[(int64_t)s * d + i];
  }
  for (int i = 0; i < d; ++i) out[i] /= den;
}

/* ------------------------------------------------------------------------ */
/* O7: prefill = O5 for every query row at its own position. */
int orc_attn_prefill(const orc_layer* L, int B, const double* q, const int32_t* cu,
                     const void* kc, const void* vc, int num_blocks,
                     const int32_t* bt, int bt_stride, const int32_t* seq_lens,
                     const float* sinks, double* out, const int32_t* rows, int nrows,
                     int nthreads) {
  if (bad_shape(L)) return -2;
  if (nthreads <= 0) nthreads = orc_default_threads();
  const int64_t total_q = cu[B];
  const int64_t nr = rows ? nrows : total_q;
  const int64_t items = nr * L->hq;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
  for (int64_t it = 0; it < items; ++it) {
    int64_t ri = it / L->hq;
    int h = (int)(it % L->hq);
    int64_t row = rows ? rows[ri] : ri;
    if (row < 0 || row >= total_q) { bad |= 1; continue; }
    int b = 0;
    while (cu[b + 1] <= row) ++b; /* request owning this row */
    int q_len = cu[b + 1] - cu[b];
    int t = seq_lens[b] - q_len + (int)(row - cu[b]);
    if (t < 0) { bad |= 1; continue; }
    const double* qh = q + (row * L->hq + h) * L->d;
    double* o = out + (row * L->hq + h) * L->d;
    if (attend_row(L, qh, h, kc, vc, num_blocks, bt, bt_stride, b, t, (double)sinks[h], o))
      bad |= 1;
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Footprint ("What happened": 28 KiB per token over the full layers;
 * models JSON "kvCacheGiBPerRequest"). */
int64_t orc_full_kv_bytes_per_token(int full_layers, int hkv, int d, int elem_bytes) {
  return (int64_t)full_layers * 2 /* K and V */ * hkv * d * elem_bytes;
}

int64_t orc_kv_bytes_per_request(int64_t ctx, int full_layers, int sliding_layers,
                                 int window, int hkv, int d, int elem_bytes) {
  int64_t kept = ctx < window ? ctx : window;
  int64_t per_tok_layer = 2 * (int64_t)hkv * d * elem_bytes;
  return ctx * full_layers * per_tok_layer + kept * sliding_layers * per_tok_layer;
}

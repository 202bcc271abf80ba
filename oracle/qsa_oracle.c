/*
 * qsa_oracle.c -- plain, slow, fp64 CPU oracle for the QSA prompt-attention
 * path.  TEST INFRASTRUCTURE ONLY: nothing in the product path may call it.
 * It shares no code, header or constant with the HIP library.
 *
 * What the path computes, per prompt token t and KV group g (pages
 * "round 6 track b - qsa flash" and "opus_r9_qsa"):
 *   1. the token sees n = pos0 + t + 1 KV cells (itself included);
 *   2. selection: every cell when n <= budget ("identity ids"), otherwise the
 *      `budget` cells with the largest selection score, ties to the lower
 *      index, listed in ascending order ("round 6 track b - qsa flash",
 *      delivered change; experiment contract: selected-index semantics
 *      above budget);
 *   3. for each of the group's query heads h: s_c = 0.0625 * q_h . k_c with
 *      k_c[d] = kq[c][d] * ksc[c][d/64] ("opus_r9_qsa", what changed: the
 *      0.0625 combine; "round 6 track b - qsa flash", delivered change: four
 *      scales per cell);
 *   4. softmax over the selected cells and o = sum_c w_c v_c with
 *      v_c[d] = vq[c][d] * vsc[c][d/64].
 * The chunked online softmax and the (m, l) log-sum-exp merge of the pages
 * ("round 27 track b - qsa prep and merge", decision and correctness) are a
 * faster route to the same number; the oracle states the plain definition
 * and, separately, the chunk-partial and merge steps so that their
 * invariants can be checked.
 *
 * Everything is fp64.  fp16 inputs are widened by the caller (exact).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD -1

typedef struct {
  float s;
  int32_t c;
} scored_cell;

/* Order for selection: larger score first; equal scores, lower index
 * first.  IEEE comparison makes -0.0 equal to +0.0. */
static int by_score_desc_index_asc(const void *pa, const void *pb) {
  const scored_cell *a = (const scored_cell *)pa, *b = (const scored_cell *)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->c < b->c) ? -1 : (a->c > b->c);
}

static int by_int_asc(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

/* Selection scores.  The pages name the score kernel and its buffers
 * ("round 27 track b - qsa prep and merge", decision: four-value dot
 * products; correctness: qidx, pooled, scores) but not their content; the
 * reading taken: the score of cell c for token t in group g is the dot
 * product of the token's index query with the cell's pooled key,
 *   scores[t][g][c] = sum_d qidx[t][g][d] * pooled[g][c][d],
 * written for the rows above budget (n > budget, the rows whose selection
 * reads scores) at cells c < n; every other element is left as it was.
 * fp64 throughout (fp32 inputs widen exactly, and their products are exact
 * in fp64). */
int qsa_oracle_score(int T, int pos0, int G, int D, int budget, int64_t n_cells,
                     const double *qidx, const double *pooled, double *scores) {
  if (T < 0 || pos0 < 0 || G <= 0 || D <= 0 || budget <= 0 || n_cells < (int64_t)pos0 + T)
    return ORACLE_BAD;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < T * G; ++r) {
    int t = r / G, g = r % G;
    int64_t n = (int64_t)pos0 + t + 1;
    if (n <= budget) continue;
    const double *q = qidx + (int64_t)r * D;
    for (int64_t c = 0; c < n; ++c) {
      const double *p = pooled + ((int64_t)g * n_cells + c) * D;
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += q[d] * p[d];
      scores[(int64_t)r * n_cells + c] = acc;
    }
  }
  return ORACLE_OK;
}

/* Selected ids of every (t, g) row: ids[t][g][0..budget), identity rows
 * 0..n-1 then -1, above-budget rows exactly `budget` ascending ids.
 * scores is [T][G][n_cells] and is read only for rows with n > budget
 * (it may be NULL when no row is above budget). */
int qsa_oracle_select(int T, int pos0, int G, int budget, int64_t n_cells,
                      const float *scores, int32_t *ids) {
  if (T < 0 || pos0 < 0 || G <= 0 || budget <= 0 || n_cells < (int64_t)pos0 + T)
    return ORACLE_BAD;
  if (!scores && (int64_t)pos0 + T > budget) return ORACLE_BAD;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < T * G; ++r) {
    int t = r / G, g = r % G;
    int64_t n = (int64_t)pos0 + t + 1;
    int32_t *row = ids + (int64_t)r * budget;
    if (n <= budget) {
      for (int64_t i = 0; i < budget; ++i) row[i] = (i < n) ? (int32_t)i : -1;
      continue;
    }
    scored_cell *cells = (scored_cell *)malloc(sizeof(scored_cell) * (size_t)n);
    if (!cells) {
      bad = 1;
      continue;
    }
    const float *srow = scores + ((int64_t)t * G + g) * n_cells;
    for (int64_t c = 0; c < n; ++c) {
      cells[c].s = srow[c];
      cells[c].c = (int32_t)c;
    }
    qsort(cells, (size_t)n, sizeof(scored_cell), by_score_desc_index_asc);
    for (int i = 0; i < budget; ++i) row[i] = cells[i].c;
    qsort(row, (size_t)budget, sizeof(int32_t), by_int_asc);
    free(cells);
  }
  return bad ? ORACLE_BAD : ORACLE_OK;
}

/* Number of selected cells of token t. */
static int64_t n_selected(int pos0, int t, int budget) {
  int64_t n = (int64_t)pos0 + t + 1;
  return n <= budget ? n : budget;
}

/* The selected cell list of row (t, g): identity when under budget (ids may
 * then be NULL or poisoned and are not read), the ids row otherwise. */
static int64_t cell_at(const int32_t *ids, int pos0, int t, int g, int G, int budget, int64_t i) {
  int64_t n = (int64_t)pos0 + t + 1;
  if (n <= budget) return i;
  return ids[((int64_t)t * G + g) * budget + i];
}

/* s_c for one head over the row's selected cells, written to s[0..nsel). */
static void head_scores(const double *qh, const int8_t *kq_g, const double *ksc_g, int D,
                        int nblk, const int32_t *ids, int pos0, int t, int g, int G,
                        int budget, int64_t nsel, double scale, double *s) {
  int blk = D / nblk;
  for (int64_t i = 0; i < nsel; ++i) {
    int64_t c = cell_at(ids, pos0, t, g, G, budget, i);
    const int8_t *kc = kq_g + c * D;
    const double *sc = ksc_g + c * nblk;
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += qh[d] * ((double)kc[d] * sc[d / blk]);
    s[i] = scale * acc;
  }
}

/* Full attention output out[t][h][d] (fp64) given the selected ids.
 * q: [T][G*HPG][D]; kq, vq: [G][n_cells][D]; ksc, vsc: [G][n_cells][D/64]. */
int qsa_oracle_attend(int T, int pos0, int G, int HPG, int D, int budget, int64_t n_cells,
                      const double *q, const int8_t *kq, const double *ksc, const int8_t *vq,
                      const double *vsc, const int32_t *ids, double *out) {
  if (T < 0 || pos0 < 0 || G <= 0 || HPG <= 0 || D <= 0 || D % 64 || budget <= 0 ||
      n_cells < (int64_t)pos0 + T)
    return ORACLE_BAD;
  if (!ids && (int64_t)pos0 + T > budget) return ORACLE_BAD;
  const int nblk = D / 64;
  const double scale = 1.0 / sqrt((double)D); /* 0.0625 at D = 256 */
  const int H = G * HPG;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < T * G; ++r) {
    int t = r / G, g = r % G;
    int64_t nsel = n_selected(pos0, t, budget);
    double *s = (double *)malloc(sizeof(double) * (size_t)nsel);
    if (!s) {
      bad = 1;
      continue;
    }
    const int8_t *kq_g = kq + (int64_t)g * n_cells * D;
    const int8_t *vq_g = vq + (int64_t)g * n_cells * D;
    const double *ksc_g = ksc + (int64_t)g * n_cells * nblk;
    const double *vsc_g = vsc + (int64_t)g * n_cells * nblk;
    for (int j = 0; j < HPG; ++j) {
      int h = g * HPG + j;
      const double *qh = q + ((int64_t)t * H + h) * D;
      head_scores(qh, kq_g, ksc_g, D, nblk, ids, pos0, t, g, G, budget, nsel, scale, s);
      double m = -INFINITY;
      for (int64_t i = 0; i < nsel; ++i)
        if (s[i] > m) m = s[i];
      double l = 0.0;
      for (int64_t i = 0; i < nsel; ++i) {
        s[i] = exp(s[i] - m);
        l += s[i];
      }
      double *oh = out + ((int64_t)t * H + h) * D;
      for (int d = 0; d < D; ++d) oh[d] = 0.0;
      for (int64_t i = 0; i < nsel; ++i) {
        int64_t c = cell_at(ids, pos0, t, g, G, budget, i);
        const int8_t *vc = vq_g + c * D;
        const double *sc = vsc_g + c * nblk;
        for (int d = 0; d < D; ++d) oh[d] += s[i] * ((double)vc[d] * sc[d / 64]);
      }
      for (int d = 0; d < D; ++d) oh[d] /= l;
    }
    free(s);
  }
  return bad ? ORACLE_BAD : ORACLE_OK;
}

/* Chunk partials of the split form: the row's selected list is cut into
 * consecutive chunks of `chunk` cells; for chunk k and head h:
 *   m_k = max s_c,  l_k = sum exp(s_c - m_k),  o_k = sum exp(s_c - m_k) v_c
 * (o_k unnormalised).  m, l: [T][KC][H]; o: [T][KC][H][D], KC = ceil(budget /
 * chunk); entries of chunks a token does not have are left untouched. */
int qsa_oracle_partials(int T, int pos0, int G, int HPG, int D, int budget, int64_t n_cells,
                        int chunk, const double *q, const int8_t *kq, const double *ksc,
                        const int8_t *vq, const double *vsc, const int32_t *ids, double *m,
                        double *l, double *o) {
  if (T < 0 || pos0 < 0 || G <= 0 || HPG <= 0 || D <= 0 || D % 64 || budget <= 0 ||
      chunk <= 0 || n_cells < (int64_t)pos0 + T)
    return ORACLE_BAD;
  if (!ids && (int64_t)pos0 + T > budget) return ORACLE_BAD;
  const int nblk = D / 64;
  const double scale = 1.0 / sqrt((double)D);
  const int H = G * HPG;
  const int KC = (budget + chunk - 1) / chunk;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < T * G; ++r) {
    int t = r / G, g = r % G;
    int64_t nsel = n_selected(pos0, t, budget);
    double *s = (double *)malloc(sizeof(double) * (size_t)nsel);
    if (!s) {
      bad = 1;
      continue;
    }
    const int8_t *kq_g = kq + (int64_t)g * n_cells * D;
    const int8_t *vq_g = vq + (int64_t)g * n_cells * D;
    const double *ksc_g = ksc + (int64_t)g * n_cells * nblk;
    const double *vsc_g = vsc + (int64_t)g * n_cells * nblk;
    for (int j = 0; j < HPG; ++j) {
      int h = g * HPG + j;
      const double *qh = q + ((int64_t)t * H + h) * D;
      head_scores(qh, kq_g, ksc_g, D, nblk, ids, pos0, t, g, G, budget, nsel, scale, s);
      for (int64_t k0 = 0, k = 0; k0 < nsel; k0 += chunk, ++k) {
        int64_t k1 = k0 + chunk < nsel ? k0 + chunk : nsel;
        double mk = -INFINITY;
        for (int64_t i = k0; i < k1; ++i)
          if (s[i] > mk) mk = s[i];
        int64_t rec = ((int64_t)t * KC + k) * H + h;
        double lk = 0.0;
        double *ok = o + rec * D;
        for (int d = 0; d < D; ++d) ok[d] = 0.0;
        for (int64_t i = k0; i < k1; ++i) {
          double w = exp(s[i] - mk);
          lk += w;
          int64_t c = cell_at(ids, pos0, t, g, G, budget, i);
          const int8_t *vc = vq_g + c * D;
          const double *sc = vsc_g + c * nblk;
          for (int d = 0; d < D; ++d) ok[d] += w * ((double)vc[d] * sc[d / 64]);
        }
        m[rec] = mk;
        l[rec] = lk;
      }
    }
    free(s);
  }
  return bad ? ORACLE_BAD : ORACLE_OK;
}

/* Log-sum-exp merge of chunk partials ("round 27 track b - qsa prep and
 * merge", decision: the (m, l) merge of chunk partials).  part is the fp32 record layout of the split
 * form: part[((t*KC + k)*H + h)*(D+2) + 0..D-1] = o_k (unnormalised),
 * [+D] = m_k, [+D+1] = l_k.  nchunks[t] chunks are merged for token t:
 *   M = max_k m_k,  L = sum_k l_k e^{m_k - M},  out = sum_k e^{m_k - M} o_k / L.
 */
int qsa_oracle_merge(int T, int H, int D, int KC, const int32_t *nchunks, const float *part,
                     double *out) {
  if (T < 0 || H <= 0 || D <= 0 || KC <= 0 || !nchunks || !part || !out) return ORACLE_BAD;
  const int64_t rs = D + 2;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < T * H; ++r) {
    int t = r / H, h = r % H;
    int nk = nchunks[t];
    double *oh = out + (int64_t)r * D;
    for (int d = 0; d < D; ++d) oh[d] = 0.0;
    if (nk <= 0) continue;
    double M = -INFINITY;
    for (int k = 0; k < nk; ++k) {
      double mk = part[(((int64_t)t * KC + k) * H + h) * rs + D];
      if (mk > M) M = mk;
    }
    double L = 0.0;
    for (int k = 0; k < nk; ++k) {
      const float *rec = part + (((int64_t)t * KC + k) * H + h) * rs;
      double e = exp((double)rec[D] - M);
      L += (double)rec[D + 1] * e;
      for (int d = 0; d < D; ++d) oh[d] += e * (double)rec[d];
    }
    for (int d = 0; d < D; ++d) oh[d] /= L;
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * K/V quantiser: the step that fills the int8 cache the path reads (the
 * quantiser part of the pages' prep step; "round 6 track b - qsa flash",
 * delivered change: int8 codes with one fp16 scale per 64 dims).  The pages do not state the
 * rounding rule; the reading taken is the plain absmax one, per row and
 * 64-dim block b:
 *   amax  = max_d |x[d]|                        (exact)
 *   scale = fp16_rne(amax / 127)                (fp32 division, correctly rounded)
 *   code  = clamp(rint(x[d] / scale), -127, 127)  (fp32 division, ties to even)
 * and code = 0 for every d of a block whose scale is 0.  The decisions are
 * taken in IEEE fp32 (the precision the GPU kernel uses), so codes and scales
 * must match bit for bit.  Inputs are fp16 bit patterns and must be finite.
 */

/* fp16 bits -> float (exact). */
static float f16_bits_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31;
  const int exp = (h >> 10) & 31;
  const uint32_t man = h & 1023u;
  float v;
  if (exp == 0) {
    v = ldexpf((float)man, -24);                 /* zero or subnormal */
  } else if (exp == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexpf((float)(man | 1024u), exp - 25);  /* 1.man * 2^(exp-15) */
  }
  uint32_t bits;
  memcpy(&bits, &v, 4);
  bits |= sign;
  memcpy(&v, &bits, 4);
  return v;
}

/* float -> fp16 bits, round to nearest, ties to even (IEEE 754 binary16). */
static uint16_t f32_to_f16_bits_rne(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  const float a = fabsf(f);
  if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
  if (a >= 65520.0f) return (uint16_t)(sign | 0x7c00u);   /* rounds past the largest finite */
  if (a < ldexpf(1.0f, -14)) {
    /* subnormal range: value = m * 2^-24, m = rint(a * 2^24) (exact scaling) */
    const float m = rintf(ldexpf(a, 24));
    return (uint16_t)(sign | (uint16_t)m);             /* m == 1024 gives the smallest normal */
  }
  int e;
  const float fr = frexpf(a, &e);                      /* a = fr * 2^e, fr in [0.5, 1) */
  const float m = rintf(ldexpf(fr, 11));               /* 11 significant bits, in [1024, 2048] */
  uint32_t man = (uint32_t)m;
  int exp = e - 1 + 15;                                /* biased exponent of 1.xxx * 2^(e-1) */
  if (man == 2048u) {                                  /* rounded up to the next binade */
    man = 1024u;
    exp += 1;
  }
  if (exp >= 31) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)(exp << 10) | (uint16_t)(man & 1023u));
}

int qsa_oracle_f32_to_f16(int64_t n, const float *in, uint16_t *out) {
  if (n < 0 || (n && (!in || !out))) return ORACLE_BAD;
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16_bits_rne(in[i]);
  return ORACLE_OK;
}

int qsa_oracle_quantize(int64_t rows, int D, int block, const uint16_t *x, int8_t *codes,
                        uint16_t *scales) {
  if (rows < 0 || D <= 0 || block <= 0 || D % block != 0) return ORACLE_BAD;
  if (rows && (!x || !codes || !scales)) return ORACLE_BAD;
  const int nb = D / block;
  for (int64_t r = 0; r < rows; ++r) {
    for (int b = 0; b < nb; ++b) {
      const uint16_t *xb = x + r * D + (int64_t)b * block;
      int8_t *cb = codes + r * D + (int64_t)b * block;
      float amax = 0.0f;
      for (int d = 0; d < block; ++d) {
        const float v = fabsf(f16_bits_to_f32(xb[d]));
        if (v > amax) amax = v;
      }
      const uint16_t sbits = f32_to_f16_bits_rne(amax / 127.0f);
      scales[r * nb + b] = sbits;
      const float s = f16_bits_to_f32(sbits);
      for (int d = 0; d < block; ++d) {
        float c = 0.0f;
        if (s > 0.0f) {
          c = rintf(f16_bits_to_f32(xb[d]) / s);
          if (c > 127.0f) c = 127.0f;
          if (c < -127.0f) c = -127.0f;
        }
        cb[d] = (int8_t)c;
      }
    }
  }
  return ORACLE_OK;
}

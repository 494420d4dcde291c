/*
 * Plain CPU oracle for selected-KV paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is compiled into liboracle.so, which is
 * loaded by tests/, by __graft_entry__.smoke() and by the cpu_baseline leg of
 * bench.py -- never by the product library.  It shares no source, header or
 * constant with the HIP path.
 *
 * Every result is the plain definition written out: nested loops, inputs widened
 * exactly to double, fp64 accumulation, no blocking, no fusion, no reordering.
 * OpenMP only splits independent output rows across threads; each output value
 * is computed by one thread in a fixed order.
 *
 * Sources (titles of the pages the method is described on):
 *   [KAP]   "KAP: Bridging the Knowledge Selection-Runtime Consumption Gap in LLM
 *            Systems" (arXiv 2607.24260): selected-KV view, executor, verifier.
 *   [KRI]   knlp.io "KRI" page: KRI-Q variant (Q.K against block-mean K), the
 *            A<a>R<r>K<k> split tag, and the connector that mean-pools over heads
 *            before the per-request top-K.
 *   [ESKV]  EarlySelectKV news item, Interpretation: selector scores and top-k
 *            over a K-summary cache.
 *
 * Layouts (element offsets, dense):
 *   K pool   [num_pages][Hkv][page_size][D]      (token-major inside a page)
 *   V pool   [num_pages][Hkv][D][page_size]      (dim-major inside a page)
 *   summary  [num_pages][Hkv][D]
 *   q        [B][q_len][Hq][D]
 *   block table [B][max_pages], compact tables [B][G][cap]
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { KOR_F32 = 0, KOR_BF16 = 1 };

/* Threads the OpenMP loops below use. */
int kor_num_threads(void) { return omp_get_max_threads(); }

/* Sets that thread count (for timing the oracle on one core). */
void kor_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* Exact widening of one stored element to double. */
static double widen(const void* base, int dtype, int64_t i) {
  if (dtype == KOR_F32) return (double)((const float*)base)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/*
 * O1. Rotary position embedding of one vector at a logical position.
 * [KAP] executor: the proposal token is fed at its full-sequence logical
 * position, so its query is rotated there.  Pairing is rotate-half: element i
 * pairs with element i + D/2, frequency theta^(-2i/D); all in fp64.
 */
void kor_rope(const double* x, int D, double pos, double theta, double* out) {
  int half = D / 2;
  for (int i = 0; i < half; i++) {
    double inv_freq = pow(theta, -2.0 * (double)i / (double)D);
    double angle = pos * inv_freq;
    double c = cos(angle), s = sin(angle);
    double a = x[i], b = x[i + half];
    out[i] = a * c - b * s;
    out[i + half] = b * c + a * s;
  }
}

/* Load query row (b, i, h) widened and rotated at position pos. */
static void load_rotated_q(const void* q, int q_dt, int64_t row_off, int D, double pos,
                           double theta, double* tmp, double* out) {
  for (int d = 0; d < D; d++) tmp[d] = widen(q, q_dt, row_off + d);
  kor_rope(tmp, D, pos, theta, out);
}

/*
 * O2. Block-mean K summary: for every page listed in a request's block table,
 * the mean over that page's valid tokens of its cached keys, per KV head.
 * [KRI] KRI-Q scores against block-mean K; [ESKV] keeps it as the K-summary
 * cache.  Valid tokens of logical page p: min(page_size, L - p*page_size).
 * Output is fp64 [num_pages][Hkv][D]; pages not referenced are left untouched.
 */
void kor_summary(const void* K, int kv_dt, int num_pages, const int32_t* bt, int max_pages,
                 const int32_t* seq_lens, int B, int Hkv, int D, int page_size, double* out) {
  (void)num_pages;
  for (int b = 0; b < B; b++) {
    int L = seq_lens[b];
    int N = (L + page_size - 1) / page_size;
    for (int p = 0; p < N; p++) {
      int phys = bt[(int64_t)b * max_pages + p];
      int nvalid = L - p * page_size;
      if (nvalid > page_size) nvalid = page_size;
      for (int g = 0; g < Hkv; g++) {
        for (int d = 0; d < D; d++) {
          double acc = 0.0;
          for (int t = 0; t < nvalid; t++) {
            int64_t off = (((int64_t)phys * Hkv + g) * page_size + t) * D + d;
            acc += widen(K, kv_dt, off);
          }
          out[((int64_t)phys * Hkv + g) * D + d] = acc / (double)nvalid;
        }
      }
    }
  }
}

/*
 * O3. Page scores.  u_g = sum over the query heads of KV group g of the rotated
 * query; S[b][g][p] = u_g . summary[bt[b][p]][g] for p < N_b, -inf otherwise.
 * A raw dot product: no 1/sqrt(D), no softmax ([KRI] KRI-Q: Q.K agreement
 * against block-mean K; per KV head, summed over the query group).
 * Query heads map to KV heads in contiguous groups: g(h) = h / (Hq/Hkv).
 * q is [B][Hq][D] (one query per request); output fp64 [B][Hkv][max_pages].
 */
void kor_score(const void* q, int q_dt, const int32_t* pos, double theta, const void* summ,
               int s_dt, const int32_t* bt, int max_pages, const int32_t* seq_lens, int B,
               int Hq, int Hkv, int D, int page_size, double* scores) {
  int grp = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; b++) {
    for (int g = 0; g < Hkv; g++) {
      double* tmp = (double*)malloc(sizeof(double) * D);
      double* rot = (double*)malloc(sizeof(double) * D);
      double* u = (double*)calloc((size_t)D, sizeof(double));
      for (int hh = 0; hh < grp; hh++) {
        int h = g * grp + hh;
        load_rotated_q(q, q_dt, ((int64_t)b * Hq + h) * D, D, (double)pos[b], theta, tmp, rot);
        for (int d = 0; d < D; d++) u[d] += rot[d];
      }
      int N = (seq_lens[b] + page_size - 1) / page_size;
      for (int p = 0; p < max_pages; p++) {
        double s = -INFINITY;
        if (p < N) {
          int phys = bt[(int64_t)b * max_pages + p];
          s = 0.0;
          for (int d = 0; d < D; d++)
            s += u[d] * widen(summ, s_dt, ((int64_t)phys * Hkv + g) * D + d);
        }
        scores[((int64_t)b * Hkv + g) * max_pages + p] = s;
      }
      free(tmp);
      free(rot);
      free(u);
    }
  }
}

/*
 * O3'. Proxy query for early routing ([ESKV] Interpretation: the side flow
 * builds a proxy query from a preceding hidden state through the query
 * projection).  q[b][n] = sum_c hidden[b][c] * Wq[c][n], exact bf16 products
 * summed in fp64.  hidden [B][dm], Wq [dm][n_out]; output fp64 [B][n_out].
 */
void kor_proxy_query(const void* hidden, int h_dt, const void* wq, int w_dt, int B, int dm,
                     int n_out, double* out) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; b++) {
    for (int n = 0; n < n_out; n++) {
      double acc = 0.0;
      for (int c = 0; c < dm; c++)
        acc += widen(hidden, h_dt, (int64_t)b * dm + c) * widen(wq, w_dt, (int64_t)c * n_out + n);
      out[(int64_t)b * n_out + n] = acc;
    }
  }
}

/* ---------------------------------------------------------------------------
 * O4. Top-K under the A<a>R<r>K<k> split ([KRI] A<a>R<r>K<k> tag): anchors are
 * the first a pages, recents the last r pages, and the best k pages of the
 * middle [a, N-r) by score.  Ranking key: descending score, ties to the lowest
 * page index.  -0.0 equals +0.0; NaN ranks below -inf and NaNs tie.  The
 * result is the ascending list of chosen logical pages ([KAP] selected pages
 * are compacted in access order).
 *
 * Pooled mode ([KRI] the connector mean-pools across heads, then takes top-K
 * per request): key = (((S0 + S1) + S2) + ... + S_{H-1}) / H, every operation a
 * single fp32 round-to-nearest-even (this file is compiled without FMA
 * contraction).  Per-head mode: key = S[g][p].
 * Selection is defined on fp32 scores: the decision is taken in the kernel's
 * precision.
 * ------------------------------------------------------------------------- */
typedef struct {
  float key;
  int idx;
} kor_cand;

/* returns <0 when x ranks before y */
static int rank_cmp(const void* px, const void* py) {
  const kor_cand* x = (const kor_cand*)px;
  const kor_cand* y = (const kor_cand*)py;
  int xn = isnan(x->key), yn = isnan(y->key);
  if (xn != yn) return xn ? 1 : -1;      /* NaN ranks last */
  if (!xn && x->key != y->key) return (x->key > y->key) ? -1 : 1;
  return (x->idx < y->idx) ? -1 : (x->idx > y->idx ? 1 : 0);
}

void kor_select(const float* scores, int B, int Hkv, int max_pages, const int32_t* seq_lens,
                int page_size, int per_head, const int32_t* anchor, const int32_t* recent,
                const int32_t* k_mid, int cap, int32_t* sel, int32_t* cnt) {
  int G = per_head ? Hkv : 1;
  kor_cand* cand = (kor_cand*)malloc(sizeof(kor_cand) * (size_t)(max_pages > 0 ? max_pages : 1));
  char* chosen = (char*)malloc((size_t)(max_pages > 0 ? max_pages : 1));
  for (int b = 0; b < B; b++) {
    int N = (seq_lens[b] + page_size - 1) / page_size;
    int a = anchor[b], r = recent[b], k = k_mid[b];
    for (int gr = 0; gr < G; gr++) {
      memset(chosen, 0, (size_t)(max_pages > 0 ? max_pages : 1));
      if (a + r >= N) {
        for (int p = 0; p < N; p++) chosen[p] = 1;
      } else {
        for (int p = 0; p < a; p++) chosen[p] = 1;
        for (int p = N - r; p < N; p++) chosen[p] = 1;
        int nm = 0;
        for (int p = a; p < N - r; p++) {
          float key;
          if (per_head) {
            key = scores[((int64_t)b * Hkv + gr) * max_pages + p];
          } else {
            volatile float acc = scores[((int64_t)b * Hkv + 0) * max_pages + p];
            for (int g = 1; g < Hkv; g++) acc = acc + scores[((int64_t)b * Hkv + g) * max_pages + p];
            volatile float mean = acc / (float)Hkv;
            key = mean;
          }
          cand[nm].key = key;
          cand[nm].idx = p;
          nm++;
        }
        qsort(cand, (size_t)nm, sizeof(kor_cand), rank_cmp);
        int take = k < nm ? k : nm;
        for (int j = 0; j < take; j++) chosen[cand[j].idx] = 1;
      }
      int c = 0;
      int32_t* row = sel + ((int64_t)b * G + gr) * cap;
      for (int p = 0; p < N; p++)
        if (chosen[p] && c < cap) row[c++] = p;
      for (int j = c; j < cap; j++) row[j] = -1;
      cnt[(int64_t)b * G + gr] = c;
    }
  }
  free(cand);
  free(chosen);
}

/*
 * Budget from a retention ratio s = s_num/s_den for N pages: ceil(N*s) in
 * integer arithmetic, raised to at least a+r and capped at N; the middle count
 * is what remains after anchors and recents.
 */
int kor_budget_from_ratio(int N, int64_t s_num, int64_t s_den, int a, int r) {
  int64_t budget = ((int64_t)N * s_num + s_den - 1) / s_den;
  if (budget < a + r) budget = a + r;
  if (budget > N) budget = N;
  return (int)budget;
}

/*
 * O5. Compact view ([KAP] selected-KV view: the chosen logical pages, in
 * ascending order, with their physical pages; the slot mapping gives each new
 * token its physical page and offset).
 *   cbt[j]  = bt[sel[j]]           clog[j] = sel[j]        (j < cnt; -1 after)
 *   clen    = sum over j of the valid tokens of logical page sel[j]
 *   slot[i] = bt[(P+i)/ps]*ps + (P+i)%ps for the new token at P+i, or -1 when
 *             that logical page lies beyond the table or is unallocated (-1).
 */
void kor_compact(const int32_t* sel, const int32_t* cnt, int B, int G, int cap, const int32_t* bt,
                 int max_pages, const int32_t* seq_lens, int page_size, const int32_t* pos,
                 int q_new, int32_t* cbt, int32_t* clog, int32_t* clen, int64_t* slot) {
  for (int b = 0; b < B; b++) {
    int L = seq_lens[b];
    for (int gr = 0; gr < G; gr++) {
      int64_t base = ((int64_t)b * G + gr) * cap;
      int c = cnt[(int64_t)b * G + gr];
      int64_t tokens = 0;
      for (int j = 0; j < cap; j++) {
        if (j < c) {
          int p = sel[base + j];
          cbt[base + j] = bt[(int64_t)b * max_pages + p];
          clog[base + j] = p;
          int nvalid = L - p * page_size;
          if (nvalid > page_size) nvalid = page_size;
          tokens += nvalid;
        } else {
          cbt[base + j] = -1;
          clog[base + j] = -1;
        }
      }
      clen[(int64_t)b * G + gr] = (int32_t)tokens;
    }
    for (int i = 0; i < q_new; i++) {
      int64_t t = (int64_t)pos[b] + i;
      int64_t p = t / page_size;
      int64_t s = -1;
      if (p < max_pages) {
        int phys = bt[(int64_t)b * max_pages + p];
        if (phys >= 0) s = (int64_t)phys * page_size + t % page_size;
      }
      slot[(int64_t)b * q_new + i] = s;
    }
  }
}

/*
 * O6/O7. Softmax attention of rotated queries over an explicit set of logical
 * token positions, read through the full block table.
 *
 * [KAP] executor: a proposal step is a q=1 decode over the selected pages with
 * the token at its full-sequence logical position; verifier: a short query
 * window over the full KV with the original logical positions.  Both are plain
 * softmax attention over the keys the view exposes, so this one definition
 * serves both: keys for (b, G-row) are the positions keys[key_off[row] ..
 * key_off[row+1]); query i of request b sits at pos0[b] + i and sees key t iff
 * t <= pos0[b] + i.
 *   z_t = scale * RoPE(q, pos0+i) . K(t)
 *   out = sum_t exp(z_t - m) V(t) / sum_t exp(z_t - m),  lse = m + log sum_t exp(z_t - m)
 * K(t) = K[bt[b][t/ps]][g][t%ps][:], V(t) = V[bt[b][t/ps]][g][:][t%ps].
 * Rows with no visible key get out = 0 and lse = -inf.
 * G = 1 shares one key set for all heads; G = Hkv gives each KV head its own.
 * out fp64 [B][q_len][Hq][D], lse fp64 [B][q_len][Hq].
 */
void kor_attend(const void* q, int q_dt, int q_len, const int32_t* pos0, double theta,
                double scale, const void* K, const void* V, int kv_dt, int Hkv, int D,
                int page_size, const int32_t* bt, int max_pages, const int32_t* keys,
                const int64_t* key_off, int G, int B, int Hq, double* out, double* lse) {
  int grp = Hq / Hkv;
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int b = 0; b < B; b++) {
    for (int i = 0; i < q_len; i++) {
      for (int h = 0; h < Hq; h++) {
        int g = h / grp;
        int row = (G == 1) ? 0 : g;
        int64_t k0 = key_off[(int64_t)b * G + row], k1 = key_off[(int64_t)b * G + row + 1];
        double qpos = (double)pos0[b] + (double)i;
        double* tmp = (double*)malloc(sizeof(double) * D);
        double* qr = (double*)malloc(sizeof(double) * D);
        double* z = (double*)malloc(sizeof(double) * (size_t)((k1 - k0) > 0 ? (k1 - k0) : 1));
        double* acc = (double*)calloc((size_t)D, sizeof(double));
        load_rotated_q(q, q_dt, (((int64_t)b * q_len + i) * Hq + h) * D, D, qpos, theta, tmp, qr);
        double m = -INFINITY;
        for (int64_t j = k0; j < k1; j++) {
          int t = keys[j];
          if ((double)t > qpos) { z[j - k0] = -INFINITY; continue; }
          int phys = bt[(int64_t)b * max_pages + t / page_size];
          int slot = t % page_size;
          double dot = 0.0;
          for (int d = 0; d < D; d++)
            dot += qr[d] * widen(K, kv_dt, (((int64_t)phys * Hkv + g) * page_size + slot) * D + d);
          z[j - k0] = scale * dot;
          if (z[j - k0] > m) m = z[j - k0];
        }
        double denom = 0.0;
        if (m != -INFINITY) {
          for (int64_t j = k0; j < k1; j++) {
            if (z[j - k0] == -INFINITY) continue;
            int t = keys[j];
            int phys = bt[(int64_t)b * max_pages + t / page_size];
            int slot = t % page_size;
            double w = exp(z[j - k0] - m);
            denom += w;
            for (int d = 0; d < D; d++)
              acc[d] += w * widen(V, kv_dt, (((int64_t)phys * Hkv + g) * D + d) * page_size + slot);
          }
        }
        int64_t orow = ((int64_t)b * q_len + i) * Hq + h;
        for (int d = 0; d < D; d++) out[orow * D + d] = denom > 0.0 ? acc[d] / denom : 0.0;
        lse[orow] = denom > 0.0 ? m + log(denom) : -INFINITY;
        free(tmp);
        free(qr);
        free(z);
        free(acc);
      }
    }
  }
}

/*
 * O2'. KV append through a slot mapping: write one token's K row and V column
 * per KV head into the slot slot[b][i] (skipped when -1).  [KAP] verifier: a
 * verify pass moves the committed full-context KV forward; [KAP] selected-KV
 * view: the slot mapping gives each new token its physical page and offset.
 * k_new/v_new are [B][q_new][Hkv][D]; K and V are updated in place (same dtype).
 */
void kor_append_kv(const void* k_new, const void* v_new, int kv_dt, const int64_t* slot, int B,
                   int q_new, int Hkv, int D, int page_size, void* K, void* V) {
  size_t eb = kv_dt == KOR_F32 ? 4 : 2;
  for (int b = 0; b < B; b++)
    for (int i = 0; i < q_new; i++) {
      int64_t s = slot[(int64_t)b * q_new + i];
      if (s < 0) continue;
      int64_t page = s / page_size, t = s % page_size;
      for (int g = 0; g < Hkv; g++)
        for (int d = 0; d < D; d++) {
          int64_t src = (((int64_t)b * q_new + i) * Hkv + g) * D + d;
          int64_t kd = ((page * Hkv + g) * page_size + t) * D + d;
          int64_t vd = ((page * Hkv + g) * D + d) * page_size + t;
          memcpy((char*)K + kd * eb, (const char*)k_new + src * eb, eb);
          memcpy((char*)V + vd * eb, (const char*)v_new + src * eb, eb);
        }
    }
}

/*
 * O5'. Compact KV workspace ([KAP] selected-KV view: the executor materializes
 * a compact physical view of the selected pages; shape stabilization: a
 * reusable compact KV workspace).  Workspace page b*cap + j holds, in head slot
 * g, head g of compact page j of selection row (b, G == 1 ? 0 : g): K and V
 * tiles are copied bit for bit.  ws_table[b][gr][j] = b*cap + j where
 * cbt[b][gr][j] >= 0, else -1.  Workspace slots with no source stay untouched.
 */
void kor_materialize(const void* K, const void* V, int kv_dt, int Hkv, int D, int page_size,
                     const int32_t* cbt, int B, int G, int cap, void* Kws, void* Vws,
                     int32_t* ws_table) {
  size_t eb = kv_dt == KOR_F32 ? 4 : 2;
  size_t tile = (size_t)page_size * D * eb;   /* one (page, head) K or V tile */
  for (int b = 0; b < B; b++)
    for (int j = 0; j < cap; j++) {
      int64_t dst = (int64_t)b * cap + j;
      for (int g = 0; g < Hkv; g++) {
        int gr = G == 1 ? 0 : g;
        int32_t src = cbt[((int64_t)b * G + gr) * cap + j];
        if (src < 0) continue;
        memcpy((char*)Kws + (dst * Hkv + g) * tile, (const char*)K + ((int64_t)src * Hkv + g) * tile, tile);
        memcpy((char*)Vws + (dst * Hkv + g) * tile, (const char*)V + ((int64_t)src * Hkv + g) * tile, tile);
      }
      for (int gr = 0; gr < G; gr++) {
        int64_t t = ((int64_t)b * G + gr) * cap + j;
        ws_table[t] = cbt[t] >= 0 ? (int32_t)dst : -1;
      }
    }
}

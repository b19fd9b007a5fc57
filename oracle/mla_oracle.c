/*
 * mla_oracle.c — plain, slow fp64 CPU reference for multi-head latent
 * attention (MLA). TEST INFRASTRUCTURE ONLY: it exists to check the GPU
 * library, it is never part of the product path, and it shares no code,
 * header, table or helper with the HIP sources.
 *
 * Every function reads the stored element type (f32, bf16 bits, f64, or
 * e4m3 bytes) and widens it exactly to double; all arithmetic is in double,
 * in the order the defining formula states, with plain loops. OpenMP only
 * spreads independent (sequence, head) pairs or rows across threads; it does
 * not change any summation order. Dimensions are arguments, so tiny cases
 * can be checked by hand.
 *
 * Sources (web pages, by title and section):
 *   "KV Reconstruction" (DeepSeek-V3 note), "How it works": k^C = W^UK c,
 *       v^C = W^UV c, key = [k^C ; k^R]; the two absorb identities; the
 *       naive and absorbed paths agree under scale 1/sqrt(d_h + d_h^R).
 *   "DeepSeek-V3.2-Exp · Absorb key weights", MQA-decode code excerpt:
 *       absorb, latent + rotary scores times the scale, -inf index mask
 *       shared by all heads, softmax over positions, latent mix, W^UV.
 *   "Value up-projection", prefill code excerpt: wkv_b applied to the
 *       latent, viewed per head, split into k_nope and v, k^R broadcast
 *       and concatenated; ordinary attention over the result.
 *   "DeepSeek-V3.2-Exp · Key–value latent", linear excerpt: one fp32 scale
 *       per 128x128 block of a 1-byte weight, grid of ceil(out/128) by
 *       ceil(in/128).
 * Parity status of each function is listed next to it; all are pinned by
 * the CPU test suite (closed forms, naive/absorbed agreement, library
 * routines, brute force on tiny inputs).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

/* ---- element access ---------------------------------------------------- */

/* bfloat16 is the upper half of an IEEE binary32: widening is exact. */
double orc_bf16_to_f64(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load(const void* p, int64_t i, int dt) {
  switch (dt) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t*)p)[i]);
    default: return ((const double*)p)[i];
  }
}

/* ---- rounding ------------------------------------------------------------ */

/* Round a double to the nearest bfloat16 (ties to even), returning its bits.
 * bfloat16 keeps 8 significant bits and the binary32 exponent range; the
 * double is first examined exactly, so there is a single rounding. */
uint16_t orc_f64_to_bf16(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
  uint16_t sign = signbit(x) ? 0x8000u : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  /* quantum of the bf16 binade that holds a: 2^(e-7) for normals
   * (a in [2^e, 2^(e+1))), 2^-133 for subnormals (e < -126). */
  int e;
  frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  e -= 1;       /* now a in [2^e, 2^(e+1)) */
  int qexp = (e < -126 ? -126 : e) - 7;
  double q = ldexp(1.0, qexp);
  double n = a / q; /* exact: scaling by a power of two */
  double r = floor(n);
  double frac = n - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  double v = r * q; /* the rounded magnitude */
  if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u); /* overflow */
  float f = (float)v; /* exact: v has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

/* ---- FP8 ----------------------------------------------------------------- */

/* OCP 8-bit floating point, E4M3 variant ("e4m3fn"): 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
 * m * 2^-9; S.1111.111 is NaN; there are no infinities. */
double orc_e4m3_to_f64(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
  double v;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Block dequantisation: out = bf16( f32( decode(w) * scale[i/128][j/128] ) ).
 * The product of a 4-bit and a 24-bit significand is exact in double; it is
 * then rounded to binary32 (the precision of the scale) and to bfloat16,
 * each to nearest-even. Parity: pinned (torch e4m3fn decode and torch CPU
 * float32 multiply + bfloat16 cast). */
int orc_dequant_fp8_block(const uint8_t* w, const float* scale, int64_t rows,
                          int64_t cols, uint16_t* out) {
  if (rows < 0 || cols < 0) return -1;
  int64_t scols = (cols + 127) / 128;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < rows; i++) {
    for (int64_t j = 0; j < cols; j++) {
      double d = orc_e4m3_to_f64(w[i * cols + j]);
      double s = (double)scale[(i / 128) * scols + j / 128];
      float p = (float)(d * s); /* C conversion: round to nearest-even */
      out[i * cols + j] = orc_f64_to_bf16((double)p);
    }
  }
  return 0;
}

/* ---- absorb W^UK into the query ------------------------------------------ */

/* q_lat[b,h,c] = sum_{d<d_n} q_nope[b,h,d] * W[h*(d_n+d_v) + d, c]
 * ("Absorb key weights" equation and excerpt). Parity: pinned via the
 * naive/absorbed identity and closed forms. */
int orc_absorb_q(const void* q_nope, int dt_q, const void* w, int dt_w, int B,
                 int n_h, int d_n, int d_v, int d_c, double* q_lat) {
  if (B < 0 || n_h < 1 || d_n < 1 || d_v < 1 || d_c < 1) return -1;
  int64_t rows_per_head = (int64_t)d_n + d_v;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; b++)
    for (int h = 0; h < n_h; h++)
      for (int c = 0; c < d_c; c++) {
        double acc = 0.0;
        for (int d = 0; d < d_n; d++)
          acc += load(q_nope, ((int64_t)b * n_h + h) * d_n + d, dt_q) *
                 load(w, ((int64_t)h * rows_per_head + d) * d_c + c, dt_w);
        q_lat[((int64_t)b * n_h + h) * d_c + c] = acc;
      }
  return 0;
}

/* ---- index mask ------------------------------------------------------------ */

/* Fills allowed[0..T) for one sequence and returns how many positions are
 * allowed: every position when idx is NULL, otherwise the set the index
 * mask of the excerpts marks. Both excerpts build that mask by scattering 0
 * into a row of -inf at the listed positions, so the listed entries form a
 * set: a repeated entry marks its position once, and an entry outside
 * [0, T) addresses no position and marks nothing. */
static int build_allowed(const int32_t* idx, int K, int T, unsigned char* allowed) {
  if (!idx) {
    memset(allowed, 1, (size_t)T);
    return T;
  }
  memset(allowed, 0, (size_t)T);
  int n = 0;
  for (int k = 0; k < K; k++) {
    int32_t t = idx[k];
    if (t < 0 || t >= T || allowed[t]) continue;
    allowed[t] = 1;
    n++;
  }
  return n;
}

/* softmax over the allowed positions of z[0..T) (disallowed entries are -inf
 * and get probability exactly 0). Returns log-sum-exp. */
static double softmax_inplace(double* z, const unsigned char* allowed, int T) {
  double m = -INFINITY;
  for (int t = 0; t < T; t++)
    if (allowed[t] && z[t] > m) m = z[t];
  double sum = 0.0;
  for (int t = 0; t < T; t++) {
    z[t] = allowed[t] ? exp(z[t] - m) : 0.0;
    sum += z[t];
  }
  for (int t = 0; t < T; t++) z[t] /= sum;
  return m + log(sum);
}

/* ---- latent attention (absorbed decode core) ------------------------------ */

/* For each sequence b and head h, with one query token:
 *   z[t] = scale * ( sum_c q_lat[b,h,c] latent[b,t,c] + sum_r q_pe[b,h,r] rope[b,t,r] )
 *   z[t] = -inf for t outside the index set (shared by all heads)
 *   p = softmax(z);  out_lat[b,h,c] = sum_t p[t] latent[b,t,c]
 * ("Absorb key weights" excerpt; "KV Reconstruction", "How it works").
 * Latent element (b,t,c) is at latent[b*lat_bs + t*lat_rs + c], rotary
 * element (b,t,r) at rope[b*rope_bs + t*rope_rs + r].
 * Optional outputs: lse[b,h] = log sum_t exp z[t]; probs[b,h,t] = p[t].
 * A sequence whose index set marks no position gets the empty sum: zero
 * output, lse = -inf, zero probabilities.
 * Parity: pinned (naive-path identity, closed forms, permutation, torch
 * SDPA with the set's boolean mask). */
int orc_latent_attention(const void* q_lat, int dt_ql, const void* q_pe, int dt_qp,
                         const void* latent, const void* rope, int dt_cache,
                         int64_t lat_bs, int64_t lat_rs, int64_t rope_bs,
                         int64_t rope_rs, int B, int n_h,
                         int T, int d_c, int d_r, const int32_t* idx, int K,
                         double scale, double* out_lat, double* lse, double* probs) {
  if (B < 0 || n_h < 1 || T < 1 || d_c < 1 || d_r < 0) return -1;
  if (idx && (K < 1 || K > T)) return -1;
  unsigned char* allowed = (unsigned char*)malloc((size_t)B * T);
  int* nallowed = (int*)malloc(sizeof(int) * (size_t)(B ? B : 1));
  if (!allowed || !nallowed) {
    free(allowed);
    free(nallowed);
    return -2;
  }
  for (int b = 0; b < B; b++)
    nallowed[b] = build_allowed(idx ? idx + (int64_t)b * K : NULL, K, T, allowed + (int64_t)b * T);
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; b++)
    for (int h = 0; h < n_h; h++) {
      const unsigned char* al = allowed + (int64_t)b * T;
      int64_t qrow = (int64_t)b * n_h + h;
      if (nallowed[b] == 0) { /* no position in the set: empty sum, zero output */
        for (int c = 0; c < d_c; c++) out_lat[qrow * d_c + c] = 0.0;
        if (lse) lse[qrow] = -INFINITY;
        if (probs)
          for (int t = 0; t < T; t++) probs[qrow * T + t] = 0.0;
        continue;
      }
      double* z = (double*)malloc(sizeof(double) * (size_t)T);
      if (!z) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      for (int t = 0; t < T; t++) {
        if (!al[t]) {
          z[t] = -INFINITY;
          continue;
        }
        int64_t lbase = (int64_t)b * lat_bs + (int64_t)t * lat_rs;
        int64_t rbase = (int64_t)b * rope_bs + (int64_t)t * rope_rs;
        double content = 0.0, rotary = 0.0;
        for (int c = 0; c < d_c; c++)
          content += load(q_lat, qrow * d_c + c, dt_ql) * load(latent, lbase + c, dt_cache);
        for (int r = 0; r < d_r; r++)
          rotary += load(q_pe, qrow * d_r + r, dt_qp) * load(rope, rbase + r, dt_cache);
        z[t] = scale * (content + rotary);
      }
      double l = softmax_inplace(z, al, T);
      if (lse) lse[qrow] = l;
      for (int c = 0; c < d_c; c++) {
        double acc = 0.0;
        for (int t = 0; t < T; t++)
          if (al[t])
            acc += z[t] * load(latent, (int64_t)b * lat_bs + (int64_t)t * lat_rs + c, dt_cache);
        out_lat[qrow * d_c + c] = acc;
      }
      if (probs)
        for (int t = 0; t < T; t++) probs[qrow * T + t] = z[t];
      free(z);
    }
  free(allowed);
  free(nallowed);
  return bad ? -2 : 0;
}

/* ---- latent attention with several query tokens per sequence ---------------
 * The same equation with the query-token axis s that the "Absorb key weights"
 * decode excerpt carries in its einsums (q [b,s,h,c] against the cache
 * [b,t,c], scores [b,s,h,t]): for sequence b, token j < s_q and head h,
 *   z[t] = scale * ( q_lat[b,j,h,:] . latent[b,t,:] + q_pe[b,j,h,:] . rope[b,t,:] )
 * over t < T, where T counts the cached positions including the s_q new
 * tokens (they occupy positions T - s_q .. T - 1). The index set, when
 * given, is one per sequence, shared by every token and head (the excerpt's
 * mask has a singleton token axis). With causal != 0, token j also may not
 * see positions after its own: t <= T - s_q + j (the reading of the causal
 * mask of the prefill excerpt, "Value up-projection", for queries that sit
 * at the end of the cache). p = softmax(z); out_lat[b,j,h,:] = sum_t p[t]
 * latent[b,t,:]; lse[b,j,h] = log sum_t exp z[t]. Layouts [B, s_q, n_h, .].
 * Parity: pinned (s_q = 1 is the single-token function; token j equals the
 * single-token function over the first T - s_q + j + 1 positions when causal,
 * over all T otherwise; hand-checked causal corner). */
int orc_latent_attention_multi(const void* q_lat, int dt_ql, const void* q_pe, int dt_qp,
                               const void* latent, const void* rope, int dt_cache,
                               int64_t lat_bs, int64_t lat_rs, int64_t rope_bs,
                               int64_t rope_rs, int B, int s_q, int n_h, int T, int d_c,
                               int d_r, const int32_t* idx, int K, int causal, double scale,
                               double* out_lat, double* lse) {
  if (B < 0 || s_q < 1 || n_h < 1 || T < 1 || d_c < 1 || d_r < 0) return -1;
  if (idx && (K < 1 || K > T)) return -1;
  if (causal && T < s_q) return -1;
  unsigned char* allowed = (unsigned char*)malloc((size_t)B * T);
  if (!allowed) return -2;
  for (int b = 0; b < B; b++)
    build_allowed(idx ? idx + (int64_t)b * K : NULL, K, T, allowed + (int64_t)b * T);
  int bad = 0;
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int b = 0; b < B; b++)
    for (int j = 0; j < s_q; j++)
      for (int h = 0; h < n_h; h++) {
        unsigned char* al = (unsigned char*)malloc((size_t)T);
        double* z = (double*)malloc(sizeof(double) * (size_t)T);
        if (!al || !z) {
#pragma omp atomic write
          bad = 1;
          free(al);
          free(z);
          continue;
        }
        for (int t = 0; t < T; t++)
          al[t] = allowed[(int64_t)b * T + t] && !(causal && t > T - s_q + j);
        int any = 0;
        for (int t = 0; t < T; t++) any |= al[t];
        int64_t qrow = ((int64_t)b * s_q + j) * n_h + h;
        if (!any) { /* nothing visible: empty sum, zero output, lse = -inf */
          for (int c = 0; c < d_c; c++) out_lat[qrow * d_c + c] = 0.0;
          if (lse) lse[qrow] = -INFINITY;
          free(al);
          free(z);
          continue;
        }
        for (int t = 0; t < T; t++) {
          if (!al[t]) {
            z[t] = -INFINITY;
            continue;
          }
          int64_t lbase = (int64_t)b * lat_bs + (int64_t)t * lat_rs;
          int64_t rbase = (int64_t)b * rope_bs + (int64_t)t * rope_rs;
          double content = 0.0, rotary = 0.0;
          for (int c = 0; c < d_c; c++)
            content += load(q_lat, qrow * d_c + c, dt_ql) * load(latent, lbase + c, dt_cache);
          for (int r = 0; r < d_r; r++)
            rotary += load(q_pe, qrow * d_r + r, dt_qp) * load(rope, rbase + r, dt_cache);
          z[t] = scale * (content + rotary);
        }
        double l = softmax_inplace(z, al, T);
        if (lse) lse[qrow] = l;
        for (int c = 0; c < d_c; c++) {
          double acc = 0.0;
          for (int t = 0; t < T; t++)
            if (al[t])
              acc += z[t] * load(latent, (int64_t)b * lat_bs + (int64_t)t * lat_rs + c, dt_cache);
          out_lat[qrow * d_c + c] = acc;
        }
        free(al);
        free(z);
      }
  free(allowed);
  return bad ? -2 : 0;
}

/* ---- W^UV after the sum ----------------------------------------------------- */

/* out[b,h,d] = sum_c o_lat[b,h,c] * W[h*(d_n+d_v) + d_n + d, c]
 * ("Absorb key weights" excerpt, last einsum; "Value up-projection",
 * "Explanation": value rows are the last d_v of each head).
 * Parity: pinned via the naive/absorbed identity and closed forms. */
int orc_out_up(const void* o_lat, int dt_o, const void* w, int dt_w, int B,
               int n_h, int d_n, int d_v, int d_c, double* out) {
  if (B < 0 || n_h < 1 || d_n < 1 || d_v < 1 || d_c < 1) return -1;
  int64_t rows_per_head = (int64_t)d_n + d_v;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; b++)
    for (int h = 0; h < n_h; h++)
      for (int d = 0; d < d_v; d++) {
        double acc = 0.0;
        for (int c = 0; c < d_c; c++)
          acc += load(o_lat, ((int64_t)b * n_h + h) * d_c + c, dt_o) *
                 load(w, ((int64_t)h * rows_per_head + d_n + d) * d_c + c, dt_w);
        out[((int64_t)b * n_h + h) * d_v + d] = acc;
      }
  return 0;
}

/* ---- full absorbed decode ------------------------------------------------- */

/* The whole absorbed path in double: absorb, latent attention, W^UV, with no
 * intermediate rounding. out [B,n_h,d_v]; optional o_lat [B,n_h,d_c],
 * lse [B,n_h], probs [B,n_h,T]. Parity: pinned (equals the naive path). */
int orc_decode_absorbed(const void* q_nope, const void* q_pe, int dt_q,
                        const void* latent, const void* rope, int dt_cache,
                        int64_t lat_bs, int64_t lat_rs, int64_t rope_bs,
                        int64_t rope_rs, const void* w,
                        int dt_w, int B, int n_h, int T, int d_c, int d_r, int d_n,
                        int d_v, const int32_t* idx, int K, double scale, double* out,
                        double* o_lat_out, double* lse, double* probs) {
  if (B < 0 || n_h < 1) return -1;
  size_t nq = (size_t)B * n_h * d_c;
  double* q_lat = (double*)malloc(sizeof(double) * (nq ? nq : 1));
  double* o_lat = o_lat_out ? o_lat_out : (double*)malloc(sizeof(double) * (nq ? nq : 1));
  int rc = (q_lat && o_lat) ? 0 : -2;
  if (!rc) rc = orc_absorb_q(q_nope, dt_q, w, dt_w, B, n_h, d_n, d_v, d_c, q_lat);
  if (!rc)
    rc = orc_latent_attention(q_lat, ORC_F64, q_pe, dt_q, latent, rope, dt_cache,
                              lat_bs, lat_rs, rope_bs, rope_rs, B, n_h, T, d_c, d_r, idx, K,
                              scale, o_lat, lse, probs);
  if (!rc) rc = orc_out_up(o_lat, ORC_F64, w, dt_w, B, n_h, d_n, d_v, d_c, out);
  free(q_lat);
  if (!o_lat_out) free(o_lat);
  return rc;
}

/* ---- naive path: reconstruct, then ordinary attention --------------------- */

/* Reconstruct one token's per-head key and value from its latent row:
 *   kv[h,e] = sum_c W[h*(d_n+d_v) + e, c] * c_row[c]
 *   K[h] = [kv[h,0:d_n] ; k_rope],  V[h] = kv[h, d_n:d_n+d_v]
 * ("KV Reconstruction", "How it works"; "Value up-projection" prefill
 * excerpt). The rotary part is copied, never re-rotated ("Watch-outs"). */
static void reconstruct_row(const void* c_row, const void* kr_row, int dt_in,
                            const void* w, int dt_w, int n_h, int d_c, int d_r,
                            int d_n, int d_v, double* K_row, double* V_row) {
  int64_t rows_per_head = (int64_t)d_n + d_v;
  for (int h = 0; h < n_h; h++) {
    for (int e = 0; e < d_n + d_v; e++) {
      double acc = 0.0;
      for (int c = 0; c < d_c; c++)
        acc += load(w, ((int64_t)h * rows_per_head + e) * d_c + c, dt_w) * load(c_row, c, dt_in);
      if (e < d_n)
        K_row[(int64_t)h * (d_n + d_r) + e] = acc;
      else
        V_row[(int64_t)h * d_v + (e - d_n)] = acc;
    }
    for (int r = 0; r < d_r; r++) K_row[(int64_t)h * (d_n + d_r) + d_n + r] = load(kr_row, r, dt_in);
  }
}

/* K [N, n_h, d_n+d_r], V [N, n_h, d_v] from c [N, d_c], k_rope [N, d_r].
 * Parity: pinned (structured weights with a closed form; the naive path
 * built on it agrees with torch attention and with the absorbed path). */
int orc_kv_reconstruct(const void* c, const void* k_rope, int dt_in, const void* w,
                       int dt_w, int64_t N, int n_h, int d_c, int d_r, int d_n, int d_v,
                       double* K, double* V) {
  if (N < 0 || n_h < 1 || d_c < 1 || d_r < 0 || d_n < 1 || d_v < 1) return -1;
  const size_t esz = dt_in == ORC_F32 ? 4 : dt_in == ORC_BF16 ? 2 : 8;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++)
    reconstruct_row((const char*)c + (size_t)n * d_c * esz,
                    (const char*)k_rope + (size_t)n * d_r * esz, dt_in, w, dt_w, n_h,
                    d_c, d_r, d_n, d_v, K + n * n_h * (d_n + d_r), V + n * n_h * d_v);
  return 0;
}

/* Naive decode with one query token per sequence: reconstruct K, V for the T
 * cached positions of each sequence, then
 *   z[t] = scale * <[q_nope ; q_pe], K[t,h]>,  -inf outside the index set,
 *   p = softmax(z),  out[b,h] = sum_t p[t] V[t,h]
 * ("Value up-projection" prefill excerpt, restricted to the last query row,
 * which sees every cached position). out [B,n_h,d_v], probs optional; a
 * sequence whose index set marks no position gets a zero output.
 * Parity: pinned (torch scaled_dot_product_attention in double, incl. index
 * sets with repeats and out-of-range entries). */
int orc_decode_naive(const void* q_nope, const void* q_pe, int dt_q, const void* latent,
                     const void* rope, int dt_cache, int64_t lat_bs, int64_t lat_rs,
                     int64_t rope_bs, int64_t rope_rs, const void* w, int dt_w, int B,
                     int n_h, int T,
                     int d_c, int d_r, int d_n, int d_v, const int32_t* idx, int K,
                     double scale, double* out, double* probs) {
  if (B < 0 || n_h < 1 || T < 1) return -1;
  if (idx && (K < 1 || K > T)) return -1;
  const size_t esz = dt_cache == ORC_F32 ? 4 : dt_cache == ORC_BF16 ? 2 : 8;
  int dk = d_n + d_r;
  double* Kb = (double*)malloc(sizeof(double) * (size_t)T * n_h * dk);
  double* Vb = (double*)malloc(sizeof(double) * (size_t)T * n_h * d_v);
  double* z = (double*)malloc(sizeof(double) * (size_t)T * n_h);
  unsigned char* al = (unsigned char*)malloc((size_t)T);
  int rc = (Kb && Vb && z && al) ? 0 : -2;
  for (int b = 0; b < B && !rc; b++) {
    if (build_allowed(idx ? idx + (int64_t)b * K : NULL, K, T, al) == 0) {
      /* no position in the set: empty sum, zero output */
      for (int h = 0; h < n_h; h++) {
        int64_t qrow = (int64_t)b * n_h + h;
        for (int d = 0; d < d_v; d++) out[qrow * d_v + d] = 0.0;
        if (probs)
          for (int t = 0; t < T; t++) probs[qrow * T + t] = 0.0;
      }
      continue;
    }
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
      int64_t lbase = (int64_t)b * lat_bs + (int64_t)t * lat_rs;
      int64_t rbase = (int64_t)b * rope_bs + (int64_t)t * rope_rs;
      reconstruct_row((const char*)latent + (size_t)lbase * esz,
                      (const char*)rope + (size_t)rbase * esz, dt_cache, w, dt_w, n_h, d_c,
                      d_r, d_n, d_v, Kb + (int64_t)t * n_h * dk, Vb + (int64_t)t * n_h * d_v);
    }
#pragma omp parallel for schedule(static)
    for (int h = 0; h < n_h; h++) {
      int64_t qrow = (int64_t)b * n_h + h;
      double* zh = z + (int64_t)h * T;
      for (int t = 0; t < T; t++) {
        if (!al[t]) {
          zh[t] = -INFINITY;
          continue;
        }
        const double* k = Kb + ((int64_t)t * n_h + h) * dk;
        double acc = 0.0;
        for (int d = 0; d < d_n; d++) acc += load(q_nope, qrow * d_n + d, dt_q) * k[d];
        for (int r = 0; r < d_r; r++) acc += load(q_pe, qrow * d_r + r, dt_q) * k[d_n + r];
        zh[t] = scale * acc;
      }
      softmax_inplace(zh, al, T);
      for (int d = 0; d < d_v; d++) {
        double acc = 0.0;
        for (int t = 0; t < T; t++)
          if (al[t]) acc += zh[t] * Vb[((int64_t)t * n_h + h) * d_v + d];
        out[qrow * d_v + d] = acc;
      }
      if (probs)
        for (int t = 0; t < T; t++) probs[qrow * T + t] = zh[t];
    }
  }
  free(Kb);
  free(Vb);
  free(z);
  free(al);
  return rc;
}

/* ---- softmax scale ----------------------------------------------------------
 * "DeepSeek-V3.2-Exp · Key–value latent", mla-init excerpt: the scale is
 * qk_head_dim^(-1/2); when the model runs past its original context length
 * it is multiplied by mscale^2 with mscale = 0.1 * m * ln(rope_factor) + 1.
 * Returns NaN for a non-positive head dimension, or a non-positive
 * rope_factor when the extension applies. */
double orc_softmax_scale(int qk_head_dim, int64_t max_seq_len, int64_t original_seq_len,
                         double m, double rope_factor) {
  if (qk_head_dim <= 0) return NAN;
  double scale = 1.0 / sqrt((double)qk_head_dim);
  if (max_seq_len > original_seq_len) {
    if (!(rope_factor > 0.0)) return NAN;
    const double ms = 0.1 * m * log(rope_factor) + 1.0;
    scale = scale * ms * ms;
  }
  return scale;
}

/* ---- cache append ----------------------------------------------------------
 * The new token's entries of the compressed cache. "DeepSeek-V3.2-Exp ·
 * Key–value latent", section "Key–value down-projection" (mla-kv excerpt):
 * the joint down-projection is split into the latent and the rotary key; the
 * latent is normalised and the key rotated. Section "Key–value latent
 * RMSNorm" (rmsnorm excerpt): in float32, var = mean of the squares over the
 * feature axis, x * rsqrt(var + eps), times a per-feature gain, then cast
 * back once. "DeepSeek V3" (inference notes), "Decoupled RoPE": the rotary
 * key is computed once per token, shared by all heads and cached.
 *
 * Rotation reading (the pages show neither the body of the rotary helper nor
 * its frequency table): features (2i, 2i+1) form a pair that is rotated by
 * the angle of entry i of the table row for the token's position, given as
 * (cos, sin) in freqs[pos][i][0..1]:
 *   y[2i]   = x[2i] cos - x[2i+1] sin
 *   y[2i+1] = x[2i] sin + x[2i+1] cos
 * i.e. (x[2i] + i x[2i+1]) times the unit complex number (cos + i sin).
 *
 * kv [N, d_c], k_pe [N, d_r] (dt_in), gamma [d_c] f32, freqs [P, d_r/2, 2]
 * f32, pos [N] int32 (each < P). Out: lat_out [N, d_c], rope_out [N, d_r]
 * doubles (unrounded). Parity: pinned (closed forms for constant and scaled
 * rows, unit RMS, quarter-turn and composed rotations, single-feature pairing).
 */
int orc_cache_append(const void* kv, const void* k_pe, int dt_in, const float* gamma,
                     const float* freqs, const int32_t* pos, int64_t N, int64_t P,
                     int d_c, int d_r, double eps, double* lat_out, double* rope_out) {
  if (N < 0 || P < 0 || d_c <= 0 || d_r <= 0 || (d_r & 1) || eps < 0) return -1;
  for (int64_t n = 0; n < N; n++)
    if (pos[n] < 0 || pos[n] >= P) return -1;
  for (int64_t n = 0; n < N; n++) {
    double ss = 0.0;
    for (int c = 0; c < d_c; c++) {
      const double x = load(kv, n * d_c + c, dt_in);
      ss += x * x;
    }
    const double var = ss / d_c;
    const double inv = 1.0 / sqrt(var + eps);
    for (int c = 0; c < d_c; c++)
      lat_out[n * d_c + c] = (double)gamma[c] * (load(kv, n * d_c + c, dt_in) * inv);
    const float* f = freqs + (int64_t)pos[n] * d_r;
    for (int i = 0; i < d_r / 2; i++) {
      const double x0 = load(k_pe, n * d_r + 2 * i, dt_in);
      const double x1 = load(k_pe, n * d_r + 2 * i + 1, dt_in);
      const double c = f[2 * i], s = f[2 * i + 1];
      rope_out[n * d_r + 2 * i] = x0 * c - x1 * s;
      rope_out[n * d_r + 2 * i + 1] = x0 * s + x1 * c;
    }
  }
  return 0;
}

/* ---- ordinary attention over reconstructed keys and values ---------------
 * "Value up-projection", prefill excerpt: q = [q_nope ; q_pe] per head,
 * scores = q . k for every (query s, key t) times the scale, plus the index
 * mask (per query token: -inf outside that token's index set, scattered from
 * its own row of indices) and the causal mask, softmax over t, then the
 * probability-weighted sum of the values. Queries sit at the end of the key
 * sequence: query s is position T - S + s (T == S in the excerpt, where the
 * causal mask lets s see t <= s).
 *   q   [B, S, n_h, d_qk],  k [B, T, n_h, d_qk],  v [B, T, n_h, d_v]
 *   idx int32 [B, S, K] or NULL;  causal: t <= T - S + s
 *   out [B, S, n_h, d_v] (double), lse [B, S, n_h] (optional)
 * A query with no visible key gets a zero output and lse = -inf.
 * Parity: pinned (torch scaled_dot_product_attention in double with the
 * same boolean mask; hand-checked first causal row; reduction of one query
 * to the naive decode path). */
int orc_attention_naive(const void* q, const void* k, const void* v, int dt, int B, int S,
                        int T, int n_h, int d_qk, int d_v, const int32_t* idx, int K,
                        int causal, double scale, double* out, double* lse) {
  if (B < 0 || S < 0 || T < 1 || n_h < 1 || d_qk < 1 || d_v < 1) return -1;
  if (idx && (K < 1 || K > T)) return -1;
  if (causal && T < S) return -1;
  int bad = 0;
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int b = 0; b < B; b++)
    for (int s = 0; s < S; s++)
      for (int h = 0; h < n_h; h++) {
        unsigned char* al = (unsigned char*)malloc((size_t)T);
        double* z = (double*)malloc(sizeof(double) * (size_t)T);
        if (!al || !z) {
#pragma omp atomic write
          bad = 1;
          free(al);
          free(z);
          continue;
        }
        build_allowed(idx ? idx + ((int64_t)b * S + s) * K : NULL, K, T, al);
        int any = 0;
        for (int t = 0; t < T; t++) {
          if (causal && t > T - S + s) al[t] = 0;
          any |= al[t];
        }
        const int64_t row = ((int64_t)b * S + s) * n_h + h;
        if (!any) {
          for (int d = 0; d < d_v; d++) out[row * d_v + d] = 0.0;
          if (lse) lse[row] = -INFINITY;
          free(al);
          free(z);
          continue;
        }
        for (int t = 0; t < T; t++) {
          if (!al[t]) {
            z[t] = -INFINITY;
            continue;
          }
          const int64_t krow = ((int64_t)b * T + t) * n_h + h;
          double acc = 0.0;
          for (int e = 0; e < d_qk; e++)
            acc += load(q, row * d_qk + e, dt) * load(k, krow * d_qk + e, dt);
          z[t] = scale * acc;
        }
        double l = softmax_inplace(z, al, T);
        if (lse) lse[row] = l;
        for (int d = 0; d < d_v; d++) {
          double acc = 0.0;
          for (int t = 0; t < T; t++)
            if (al[t]) acc += z[t] * load(v, (((int64_t)b * T + t) * n_h + h) * d_v + d, dt);
          out[row * d_v + d] = acc;
        }
        free(al);
        free(z);
      }
  return bad ? -1 : 0;
}

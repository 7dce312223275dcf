/*
 * vga_oracle.c -- plain fp64 CPU oracle for alternating attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code with the HIP library.
 *
 * Everything here is written to be read against the pages, not to be fast:
 * every attention output is computed from its definition with a max-shifted
 * softmax over an explicit list of columns, in double precision.
 *
 * Sources (web pages, cited by title and section):
 *  - "VGGT CVPR25 Best Paper" notes, section "Alternating-Attention":
 *    frame-wise self-attention inside each frame, then global self-attention
 *    over all N*L tokens of all frames; no cross-attention.
 *  - "AVGGT: Rethinking Global Attention for Accelerating VGGT", technical
 *    summary section 3 (Methodology): step one turns early global layers into
 *    frame attention; step two, Subsampled Global Attention (SGA), keeps every
 *    query, samples K/V on a strided patch grid, keeps each token's diagonal
 *    term, approximates every dropped K/V column by one global mean vector,
 *    and normalises the three parts under one shared softmax.
 *  - "VGGT-Omega" notes, section 2 (first architectural change, Register
 *    Attention) and architecture section 2.3: in some global layers the
 *    cross-frame exchange runs only among the per-frame register and camera
 *    tokens, while image tokens attend inside their own frame.
 *
 * Readings where the pages leave a step open (all documented in the design
 * notes, and each one a parameter or a single line below):
 *  - softmax scale: caller-supplied (textbook 1/sqrt(d) by default upstream);
 *  - grid sampling: patch (r, c) is kept iff r mod sh == oh and c mod sw == ow;
 *    a truncated window at the grid edge gets no extra sample;
 *  - special tokens (local index >= gh*gw) are never dropped;
 *  - the mean-fill column stands for |D| identical columns: its logit is
 *    scale*<q, kmean> + ln|D| and its value is vmean, where kmean/vmean are
 *    the means over ALL dropped tokens of all frames (one vector per head);
 *  - the diagonal column is added only when the query's own token was
 *    dropped, so no column is ever counted twice;
 *  - with |D| == 0 there is no mean column;
 *  - mean_fill == 2 is the unit-weight alternative: the same column with
 *    logit scale*<q, kmean> (it stands for one column, not |D|);
 *  - register attention: a special-token query (camera and registers are the
 *    special tokens) attends over the special tokens of all frames; a patch
 *    query attends over its own frame's tokens, as in frame attention.
 *
 * Layout: Q, K, V are [T, H, d] row-major with T = N*L, token t = f*L + u,
 * u < gh*gw a patch at (u / gw, u % gw) and u >= gh*gw a special token.
 * Element type: dtype 0 = IEEE fp32, dtype 1 = bf16 given as raw uint16 bits.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_MODE_FRAME = 0, ORC_MODE_GLOBAL = 1, ORC_MODE_SGA = 2,
       ORC_MODE_REGISTER = 3 };
enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* Read element idx of a fp32 or bf16 array exactly into a double. */
static double elem(const void* base, int dtype, int64_t idx) {
  if (dtype == ORC_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Is local token u of a frame kept as a K/V column by SGA grid sampling? */
static int sga_keeps(int32_t u, int32_t gh, int32_t gw, int32_t sh, int32_t sw,
                     int32_t oh, int32_t ow) {
  if (u >= gh * gw) return 1; /* special tokens are not grid points: kept */
  int32_t r = u / gw, c = u % gw;
  return (r % sh == oh) && (c % sw == ow);
}

/* SGA key selection.  Walks every token in ascending order and records the
 * kept ones.  keep_idx (length >= returned count) and keep_mask (length N*L)
 * may be NULL.  Returns the number of kept tokens over all frames. */
int64_t vgao_select(int32_t N, int32_t L, int32_t gh, int32_t gw, int32_t sh,
                    int32_t sw, int32_t oh, int32_t ow, int64_t* keep_idx,
                    uint8_t* keep_mask) {
  int64_t n = 0;
  for (int32_t f = 0; f < N; ++f) {
    for (int32_t u = 0; u < L; ++u) {
      int64_t t = (int64_t)f * L + u;
      int kept = sga_keeps(u, gh, gw, sh, sw, oh, ow);
      if (keep_mask) keep_mask[t] = (uint8_t)kept;
      if (kept) {
        if (keep_idx) keep_idx[n] = t;
        ++n;
      }
    }
  }
  return n;
}

/* Per-head means of K and V over the dropped tokens: out [H, d] each.
 * Returns |D|; with |D| == 0 the outputs are left at zero. */
int64_t vgao_dropped_mean(int32_t N, int32_t L, int32_t gh, int32_t gw,
                          int32_t H, int32_t d, int32_t dtype, const void* k,
                          const void* v, int32_t sh, int32_t sw, int32_t oh,
                          int32_t ow, double* kmean, double* vmean) {
  int64_t T = (int64_t)N * L, nd = 0;
  memset(kmean, 0, sizeof(double) * (size_t)H * d);
  memset(vmean, 0, sizeof(double) * (size_t)H * d);
  for (int64_t t = 0; t < T; ++t) {
    if (sga_keeps((int32_t)(t % L), gh, gw, sh, sw, oh, ow)) continue;
    ++nd;
    for (int32_t h = 0; h < H; ++h)
      for (int32_t e = 0; e < d; ++e) {
        int64_t idx = (t * H + h) * d + e;
        kmean[h * d + e] += elem(k, dtype, idx);
        vmean[h * d + e] += elem(v, dtype, idx);
      }
  }
  if (nd > 0)
    for (int64_t i = 0; i < (int64_t)H * d; ++i) {
      kmean[i] /= (double)nd;
      vmean[i] /= (double)nd;
    }
  return nd;
}

/* Attention for a list of query rows.
 *
 * mode FRAME : the columns of row i are the L tokens of i's own frame.
 * mode GLOBAL: the columns of row i are all T tokens.
 * mode SGA   : the columns are the kept tokens; plus row i's own token when
 *              `diagonal` is set and that token was dropped; plus, when
 *              `mean_fill` is set and |D| > 0, one column with key kmean,
 *              value vmean and logit scale*<q,kmean> + ln|D| (mean_fill 1,
 *              count-weighted) or scale*<q,kmean> (mean_fill 2, unit weight).
 * mode REGISTER: a special row's columns are the special tokens of every
 *              frame in ascending token order; a patch row's columns are the
 *              L tokens of its own frame.
 * For every column j: z_j = scale * <q_i, k_j> (+ ln|D| for the
 * count-weighted mean column); O_i = sum_j exp(z_j - max z) v_j /
 * sum_j exp(z_j - max z).
 *
 * rows: query tokens (NULL => all T rows in order); out: [nrows, H, d].
 * threads <= 0 uses the OpenMP default.  Returns 0, or -1 on bad arguments
 * or allocation failure. */
int vgao_attention(int32_t mode, int32_t N, int32_t L, int32_t gh, int32_t gw,
                   int32_t H, int32_t d, int32_t dtype, double scale,
                   const void* q, const void* k, const void* v, int32_t sh,
                   int32_t sw, int32_t oh, int32_t ow, int32_t diagonal,
                   int32_t mean_fill, const int64_t* rows, int64_t nrows,
                   double* out, int32_t threads) {
  if (N < 1 || L < 1 || H < 1 || d < 1 || gh < 0 || gw < 0 || gh * gw > L)
    return -1;
  if (mode != ORC_MODE_FRAME && mode != ORC_MODE_GLOBAL &&
      mode != ORC_MODE_SGA && mode != ORC_MODE_REGISTER)
    return -1;
  if (mean_fill < 0 || mean_fill > 2) return -1;
  int64_t T = (int64_t)N * L;
  if (rows == NULL) nrows = T;

  int64_t nkeep = 0, ndrop = 0;
  int64_t* keep_idx = NULL;
  uint8_t* keep_mask = NULL;
  double *kmean = NULL, *vmean = NULL;
  if (mode == ORC_MODE_SGA) {
    if (sh < 1 || sw < 1 || oh < 0 || ow < 0 || oh >= sh || ow >= sw) return -1;
    keep_idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)T);
    keep_mask = (uint8_t*)malloc((size_t)T);
    kmean = (double*)malloc(sizeof(double) * (size_t)H * d);
    vmean = (double*)malloc(sizeof(double) * (size_t)H * d);
    if (!keep_idx || !keep_mask || !kmean || !vmean) {
      free(keep_idx); free(keep_mask); free(kmean); free(vmean);
      return -1;
    }
    nkeep = vgao_select(N, L, gh, gw, sh, sw, oh, ow, keep_idx, keep_mask);
    ndrop = vgao_dropped_mean(N, L, gh, gw, H, d, dtype, k, v, sh, sw, oh, ow,
                              kmean, vmean);
  }
  int use_mean = (mode == ORC_MODE_SGA) && mean_fill && ndrop > 0;

#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
  int failed = 0;
#pragma omp parallel reduction(|| : failed)
  {
    /* per-thread scratch: logits and the column list of one row */
    double* z = (double*)malloc(sizeof(double) * (size_t)(T + 2));
    int64_t* col = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T + 2));
    double* qi = (double*)malloc(sizeof(double) * (size_t)d);
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    if (!z || !col || !qi || !acc) failed = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < nrows * H; ++task) {
      if (!z || !col || !qi || !acc) continue;
      int64_t r = task / H;
      int32_t h = (int32_t)(task % H);
      int64_t i = rows ? rows[r] : r;
      if (i < 0 || i >= T) { failed = 1; continue; }

      /* 1. the column list of row i (index -1 marks the mean column) */
      int64_t nc = 0;
      if (mode == ORC_MODE_GLOBAL) {
        for (int64_t j = 0; j < T; ++j) col[nc++] = j;
      } else if (mode == ORC_MODE_FRAME ||
                 (mode == ORC_MODE_REGISTER && i % L < gh * gw)) {
        int64_t f0 = (i / L) * L;
        for (int64_t j = f0; j < f0 + L; ++j) col[nc++] = j;
      } else if (mode == ORC_MODE_REGISTER) {
        /* a special query: every special token of every frame */
        for (int64_t j = 0; j < T; ++j)
          if (j % L >= gh * gw) col[nc++] = j;
      } else {
        for (int64_t n = 0; n < nkeep; ++n) col[nc++] = keep_idx[n];
        if (diagonal && !keep_mask[i]) col[nc++] = i;
        if (use_mean) col[nc++] = -1;
      }

      /* 2. logits */
      for (int32_t e = 0; e < d; ++e) qi[e] = elem(q, dtype, (i * H + h) * d + e);
      for (int64_t c = 0; c < nc; ++c) {
        double dot = 0.0;
        if (col[c] >= 0) {
          for (int32_t e = 0; e < d; ++e)
            dot += qi[e] * elem(k, dtype, (col[c] * H + h) * d + e);
          z[c] = scale * dot;
        } else {
          for (int32_t e = 0; e < d; ++e) dot += qi[e] * kmean[h * d + e];
          z[c] = scale * dot + (mean_fill == 1 ? log((double)ndrop) : 0.0);
        }
      }

      /* 3. max-shifted softmax and weighted sum of values */
      double zmax = -INFINITY;
      for (int64_t c = 0; c < nc; ++c)
        if (z[c] > zmax) zmax = z[c];
      double wsum = 0.0;
      for (int32_t e = 0; e < d; ++e) acc[e] = 0.0;
      for (int64_t c = 0; c < nc; ++c) {
        double w = exp(z[c] - zmax);
        wsum += w;
        if (col[c] >= 0) {
          for (int32_t e = 0; e < d; ++e)
            acc[e] += w * elem(v, dtype, (col[c] * H + h) * d + e);
        } else {
          for (int32_t e = 0; e < d; ++e) acc[e] += w * vmean[h * d + e];
        }
      }
      for (int32_t e = 0; e < d; ++e) out[(r * H + h) * d + e] = acc[e] / wsum;
    }
    free(z); free(col); free(qi); free(acc);
  }
  free(keep_idx); free(keep_mask); free(kmean); free(vmean);
  return failed ? -1 : 0;
}

/* Layer schedule of the training-free pipeline: of the num_global global
 * attention slots, the first num_early become frame attention; the rest run
 * SGA when use_sga is set, else stay exact global attention.
 * out[g] is ORC_MODE_FRAME, ORC_MODE_GLOBAL or ORC_MODE_SGA.
 * Returns 0, or -1 when num_early is outside [0, num_global]. */
int vgao_schedule(int32_t num_global, int32_t num_early, int32_t use_sga,
                  int32_t* out) {
  if (num_global < 0 || num_early < 0 || num_early > num_global) return -1;
  for (int32_t g = 0; g < num_global; ++g)
    out[g] = g < num_early ? ORC_MODE_FRAME
                           : (use_sga ? ORC_MODE_SGA : ORC_MODE_GLOBAL);
  return 0;
}

/* Schedule with register attention: as vgao_schedule, except that of the
 * slots not converted to frame attention, every register_every-th slot
 * counted from slot 0 (g mod register_every == register_every - 1) runs
 * register attention.  register_every == 0 gives vgao_schedule.
 * Returns 0, or -1 on bad arguments. */
int vgao_schedule_register(int32_t num_global, int32_t num_early,
                           int32_t register_every, int32_t use_sga,
                           int32_t* out) {
  if (register_every < 0) return -1;
  if (vgao_schedule(num_global, num_early, use_sga, out) != 0) return -1;
  for (int32_t g = num_early; g < num_global; ++g)
    if (register_every > 0 && g % register_every == register_every - 1)
      out[g] = ORC_MODE_REGISTER;
  return 0;
}

/* Number of threads the oracle runs with (for reporting). */
/* The linear projections around an attention layer (the QKV projection
 * before it and the output projection after it), read as the plain
 * nn.Linear-style layer the pages leave open: y = x W^T + b with
 *   x [M, K] (M tokens, K input features), w [N, K] row-major (row n holds
 *   the weights of output feature n), b [N] or NULL (no bias),
 * all of one dtype, and y [M, N] in fp64:
 *   y[m][n] = sum_k x[m][k] * w[n][k] + b[n].                               */
int vgao_linear(int64_t M, int32_t K, int32_t N, int32_t dtype, const void* x,
                const void* w, const void* b, double* y, int32_t threads) {
  if (M < 0 || K < 1 || N < 1 || !x || !w || !y) return -1;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int32_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int32_t k = 0; k < K; ++k)
        acc += elem(x, dtype, m * K + k) * elem(w, dtype, (int64_t)n * K + k);
      y[m * N + n] = acc + (b ? elem(b, dtype, n) : 0.0);
    }
  }
  return 0;
}

/* QKV projection of H heads of 64: the C = 64*H input features of each of
 * the M tokens map to 3C outputs, y = x W^T + b with w [3C, C]; output
 * features [0, C) are q, [C, 2C) are k and [2C, 3C) are v, each stored
 * [M, H, 64] (feature c = 64*h + e of head h, dim e).                       */
int vgao_qkv_proj(int64_t M, int32_t H, int32_t dtype, const void* x, const void* w,
                  const void* b, double* q, double* k, double* v, int32_t threads) {
  const int32_t C = 64 * H;
  if (H < 1 || !q || !k || !v) return -1;
  double* y = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1) * 3 * C);
  if (!y) return -1;
  int rc = vgao_linear(M, C, 3 * C, dtype, x, w, b, y, threads);
  for (int64_t m = 0; rc == 0 && m < M; ++m)
    for (int32_t c = 0; c < C; ++c) {
      q[m * C + c] = y[m * 3 * C + c];
      k[m * C + c] = y[m * 3 * C + C + c];
      v[m * C + c] = y[m * 3 * C + 2 * C + c];
    }
  free(y);
  return rc;
}

int32_t vgao_max_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * CPU oracle for the MoE expert-compute-plus-return path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this file; only the
 * tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no code with the
 * GPU library (no headers, helpers, tables or constants).
 *
 * Source: "Fine-grained Computation-Communication Overlap via Tile-level Signaling and Scheduling for
 * Mixture-of-Experts" (Cui, Wingkvist, Ericsson; arXiv 2607.19539), as summarised on its review page:
 * the pith section ("The pith"), "What carries the argument", the referee's first major comment on
 * section 4.5 / Algorithm 1, and the ledger's third axiom (section 3.2.3, combine plan).
 *
 * Every floating-point step accumulates in double.  In bf16 mode the FFN hidden activation h and the
 * FFN output y are each rounded once, directly from double, to bf16 with round-to-nearest-even, and
 * so is the combined output; in fp32 mode nothing is rounded.  Plain loops, no blocking or fusion.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------------ */
/* bf16 helpers (oracle-private)                                                                     */

static double orc_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Correctly rounded double -> bf16 value (returned as a double), ties to even.
 * bf16: 8 significant bits, fp32 exponent range, subnormal spacing 2^-133. */
double orc_round_bf16(double v) {
  if (v == 0.0 || isnan(v) || isinf(v)) return v;
  int ex;
  (void)frexp(fabs(v), &ex);      /* |v| = m * 2^ex with m in [0.5, 1) */
  int q = ex - 8;                 /* quantum exponent of a normal bf16 with this binade */
  if (q < -133) q = -133;         /* subnormal range */
  double r = nearbyint(ldexp(fabs(v), -q)); /* default rounding mode: nearest, ties to even */
  double out = ldexp(r, q);
  if (out > 3.3895313892515355e38) out = INFINITY; /* beyond the largest finite bf16 */
  return v < 0 ? -out : out;
}

uint16_t orc_bf16_bits(double v) {
  float f = (float)orc_round_bf16(v); /* exact: the value is representable in fp32 */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------------------------------ */
/* Routing: per token, experts sorted by logit descending (ties to the lower id), first k taken;      */
/* weight = softmax over all G logits at the chosen ids, no renormalisation over the k.                */

typedef struct {
  float v;
  int id;
} orc_kv;

static int orc_kv_cmp(const void* a, const void* b) {
  const orc_kv* x = (const orc_kv*)a;
  const orc_kv* y = (const orc_kv*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->id < y->id) ? -1 : (x->id > y->id);
}

int orc_route(int64_t T, int G, int k, const float* logits, int32_t* topk_idx, float* topk_w) {
  if (T < 0 || G <= 0 || k <= 0 || k > G) return -1;
  orc_kv* buf = (orc_kv*)malloc(sizeof(orc_kv) * (size_t)G);
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * G;
    for (int g = 0; g < G; ++g) {
      buf[g].v = l[g];
      buf[g].id = g;
    }
    qsort(buf, (size_t)G, sizeof(orc_kv), orc_kv_cmp);
    double mx = buf[0].v, den = 0.0;
    for (int g = 0; g < G; ++g) den += exp((double)l[g] - mx);
    for (int j = 0; j < k; ++j) {
      topk_idx[t * k + j] = buf[j].id;
      topk_w[t * k + j] = (float)(exp((double)buf[j].v - mx) / den);
    }
  }
  free(buf);
  return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Layout (Algorithm 1 as restated by the referee: rows of each local expert grouped by owner rank,   */
/* each (expert, owner) group padded to a multiple of the tile height M).                             */

/* segment descriptor fields */
enum { SEG_OWNER = 0, SEG_EXPERT, SEG_FIRST_BAND, SEG_NBANDS, SEG_SRC_ROW, SEG_DST_ROW, SEG_ROWS, SEG_GROUP,
       SEG_FIELDS };

typedef struct {
  /* inputs */
  const int32_t* topk_idx; /* [T*k] global expert ids */
  int32_t R, T_o, G, E_l, k, self_rank, M, mgb;
  int64_t cap_rows; /* capacity of row_src */
  int64_t cap_tiles; /* capacity of the band tables, tile_order and seg_desc */
  /* outputs (caller-allocated) */
  int32_t* counts;     /* [E_l*R]   n_{e,r}, index e*R+r */
  int32_t* padded_off; /* [E_l*R]   exclusive prefix of P in (e, r) order */
  int32_t* recv_off;   /* [E_l*R]   sum over e' < e of n_{e',r} */
  int32_t* tile_owner; /* [n_tiles] */
  int32_t* tile_expert;
  int32_t* tile_valid; /* real rows in the band */
  int32_t* tile_order; /* [n_tiles] bands in remote-first order */
  int32_t* seg_desc;   /* [n_segs * SEG_FIELDS] */
  int32_t* row_src;    /* [M_pad] token row or -1 */
  int32_t* combine_plan; /* [T*k] row in the owner's receive buffer or -1 */
  int32_t* scalars;      /* [3+R] M_pad, n_tiles, n_segs, N_r[R] */
} orc_layout_args;


/* sort key of a group for the remote-first order: (is_self, -P, e, r) ascending */
typedef struct {
  int is_self, negP, e, r;
} orc_gkey;

static int orc_gkey_cmp(const void* a, const void* b) {
  const orc_gkey* x = (const orc_gkey*)a;
  const orc_gkey* y = (const orc_gkey*)b;
  if (x->is_self != y->is_self) return x->is_self < y->is_self ? -1 : 1;
  if (x->negP != y->negP) return x->negP < y->negP ? -1 : 1;
  if (x->e != y->e) return x->e < y->e ? -1 : 1;
  return (x->r > y->r) - (x->r < y->r);
}

/* Returns 0, -1 for a bad shape, -2 if a capacity is exceeded. */
int orc_layout(orc_layout_args* a) {
  const int R = a->R, T_o = a->T_o, E = a->E_l, k = a->k, M = a->M;
  if (R <= 0 || T_o < 0 || E <= 0 || k <= 0 || M <= 0 || a->mgb <= 0 || a->G <= 0) return -1;
  const int NG = E * R;
  const int lo = a->self_rank * E; /* global id of local expert 0 */

  /* 3a: group sizes n_{e,r}; a token's slot j is local when its expert id falls in [lo, lo+E) */
  for (int g = 0; g < NG; ++g) a->counts[g] = 0;
  for (int r = 0; r < R; ++r)
    for (int t = 0; t < T_o; ++t)
      for (int j = 0; j < k; ++j) {
        int e = a->topk_idx[((int64_t)r * T_o + t) * k + j] - lo;
        if (e >= 0 && e < E) a->counts[e * R + r] += 1;
      }

  /* 3b, 3c: padding to a multiple of M ((-n) mod M extra rows), offsets in (e, r) order */
  int64_t pad_total = 0;
  for (int e = 0; e < E; ++e)
    for (int r = 0; r < R; ++r) {
      int n = a->counts[e * R + r];
      int P = ((n + M - 1) / M) * M;
      a->padded_off[e * R + r] = (int32_t)pad_total;
      pad_total += P;
    }
  for (int r = 0; r < R; ++r) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      a->recv_off[e * R + r] = run;
      run += a->counts[e * R + r];
    }
    a->scalars[3 + r] = run; /* N_r */
  }
  const int64_t M_pad = pad_total;
  const int64_t n_tiles = M_pad / M;
  if (M_pad > a->cap_rows || n_tiles > a->cap_tiles) return -2;

  /* 3d: band tables */
  for (int e = 0; e < E; ++e)
    for (int r = 0; r < R; ++r) {
      int n = a->counts[e * R + r];
      int64_t off = a->padded_off[e * R + r];
      for (int64_t row = 0; row < n; row += M) {
        int64_t b = (off + row) / M;
        a->tile_owner[b] = r;
        a->tile_expert[b] = e;
        a->tile_valid[b] = (int32_t)((n - row) < M ? (n - row) : M);
      }
    }

  /* 3e: row map and combine plan; rank i inside a group follows ascending token index */
  for (int64_t p = 0; p < M_pad; ++p) a->row_src[p] = -1;
  int32_t* fill = (int32_t*)calloc((size_t)NG, sizeof(int32_t));
  for (int r = 0; r < R; ++r)
    for (int t = 0; t < T_o; ++t)
      for (int j = 0; j < k; ++j) {
        int64_t tok = (int64_t)r * T_o + t;
        int e = a->topk_idx[tok * k + j] - lo;
        if (e >= 0 && e < E) {
          int g = e * R + r;
          int i = fill[g]++;
          a->row_src[a->padded_off[g] + i] = (int32_t)tok;
          a->combine_plan[tok * k + j] = a->recv_off[g] + i;
        } else {
          a->combine_plan[tok * k + j] = -1;
        }
      }
  free(fill);

  /* 3f: remote-first order of non-empty groups, bands ascending inside each group; segments of up to
   * mgb bands cut at the group's real rows */
  orc_gkey* keys = (orc_gkey*)malloc(sizeof(orc_gkey) * (size_t)NG);
  int ng = 0;
  for (int e = 0; e < E; ++e)
    for (int r = 0; r < R; ++r) {
      int n = a->counts[e * R + r];
      if (n == 0) continue;
      keys[ng].is_self = (r == a->self_rank);
      keys[ng].negP = -(((n + M - 1) / M) * M);
      keys[ng].e = e;
      keys[ng].r = r;
      ++ng;
    }
  qsort(keys, (size_t)ng, sizeof(orc_gkey), orc_gkey_cmp);
  int64_t pos = 0, ns = 0;
  for (int q = 0; q < ng; ++q) {
    int e = keys[q].e, r = keys[q].r, g = e * R + r;
    int n = a->counts[g];
    int nb = (n + M - 1) / M;
    int64_t b0 = a->padded_off[g] / M;
    for (int b = 0; b < nb; ++b) a->tile_order[pos++] = (int32_t)(b0 + b);
    for (int b = 0; b < nb; b += a->mgb) {
      int cnt = (nb - b) < a->mgb ? (nb - b) : a->mgb;
      int rows = n - b * M;
      if (rows > cnt * M) rows = cnt * M;
      int32_t* s = a->seg_desc + ns * SEG_FIELDS;
      s[SEG_OWNER] = r;
      s[SEG_EXPERT] = e;
      s[SEG_FIRST_BAND] = (int32_t)(b0 + b);
      s[SEG_NBANDS] = cnt;
      s[SEG_SRC_ROW] = a->padded_off[g] + b * M;
      s[SEG_DST_ROW] = a->recv_off[g] + b * M;
      s[SEG_ROWS] = rows;
      s[SEG_GROUP] = g;
      ++ns;
    }
  }
  free(keys);
  a->scalars[0] = (int32_t)M_pad;
  a->scalars[1] = (int32_t)n_tiles;
  a->scalars[2] = (int32_t)ns;
  return 0;
}

/* Padding rows of a layout, sum over groups of ((-n) mod M).  With count_self = 0 the self rank's
 * groups are left out, which is the quantity the referee bounds for section 4.5. */
int64_t orc_padding_rows(const int32_t* counts, int E, int R, int M, int self_rank, int count_self) {
  int64_t s = 0;
  for (int e = 0; e < E; ++e)
    for (int r = 0; r < R; ++r) {
      if (!count_self && r == self_rank) continue;
      int64_t n = counts[e * R + r];
      s += (M - n % M) % M;
    }
  return s;
}

/* ------------------------------------------------------------------------------------------------ */
/* Expert SwiGLU FFN for a list of rows.                                                              */
/*   g_n = sum_c x_c Wg[e][n][c],  u_n = sum_c x_c Wu[e][n][c],  h_n = silu(g_n) u_n,                  */
/*   silu(g) = g / (1 + exp(-g)),  y_m = sum_n h_n Wd[e][m][n].                                        */
/* Wg = rows [0, f) of w_gate_up[e], Wu = rows [f, 2f); weights in (out, in) row-major order.         */
/* is_bf16: x and weights are bf16 bit patterns, h and y are rounded to bf16; else fp32, no rounding. */

static inline double orc_ld(const void* p, int64_t i, int is_bf16) {
  return is_bf16 ? orc_bf16_to_double(((const uint16_t*)p)[i]) : (double)((const float*)p)[i];
}

/* The bf16 value next to bf16 value h, above (up = 1) or below (up = 0). */
static double orc_bf16_step(double h, int up) {
  uint16_t b = orc_bf16_bits(h);
  if (h == 0.0) b = up ? 0x0001 : 0x8001;
  else if ((h > 0.0) == (up != 0)) b = (uint16_t)(b + 1);
  else b = (uint16_t)(b - 1);
  return orc_bf16_to_double(b);
}

typedef struct {
  double ratio; /* sort key */
  int n;
  double dh;    /* other bf16 candidate minus the rounded h */
} orc_cand;

static int orc_cand_cmp(const void* a, const void* b) {
  double x = ((const orc_cand*)a)->ratio, y = ((const orc_cand*)b)->ratio;
  return (x > y) - (x < y);
}

/*
 * orc_ffn_rows_ex: as orc_ffn_rows, and in bf16 mode also reports where rounding h to bf16 is not decided
 * by the kernel's fp32 arithmetic.  An fp32 evaluation of h_n = silu(g_n) u_n differs from the exact value
 * by accumulated rounding; its bound here is
 *   delta_n = 2^-21 sqrt(d) (|silu'(g_n) u_n| Qg_n + |silu(g_n)| Qu_n) + 2^-20 |h_n|,
 * Qg_n = sqrt(sum_c (x_c Wg[n][c])^2) and likewise Qu_n.  The first term bounds the rounding error of a
 * d-term fp32 sum: each addition errs by at most 2^-24 of its partial sum, the errors add like a random
 * walk, so their sum has a standard deviation near 0.4 * 2^-24 sqrt(d) Q; the bound is some twenty
 * standard deviations.  The second term allows for the evaluation of silu and the product.
 * When the exact h_n is within delta_n of the midpoint between its bf16 rounding and the neighbouring bf16
 * value, either rounding is a correct result; the row then lists n, the step dh to the other candidate
 * and the resulting change of y, dh * Wd[e][:, n], exactly.  Up to max_cand candidates per row are kept,
 * largest |dh| first (cand_vec may be NULL: the list without the vectors).  y_unr receives y before its final
 * rounding; h_out (optional, [nrows][f]) the
 * rounded hidden row; y_delta (optional, [nrows][d]) the same kind of bound for the fp32 evaluation of y
 * itself, 2^-21 sqrt(f) Qy_m + 2^-22 |y_m| with Qy_m = sqrt(sum_n (h_n Wd[e][m][n])^2): where y_unr lies
 * within y_delta of a bf16 rounding midpoint, both neighbouring bf16 values are correct results for y.
 */
int orc_ffn_rows_ex(int64_t nrows, const int32_t* src_row, const int32_t* expert, int d, int f, int is_bf16,
                    const void* x, const void* w_gate_up, const void* w_down, double* y_out, double* y_unr,
                    int max_cand, int32_t* cand_count, int32_t* cand_n, double* cand_vec, double* h_out,
                    double* y_delta) {
  if (nrows < 0 || d <= 0 || f <= 0) return -1;
#pragma omp parallel
  {
    double* xr = (double*)malloc(sizeof(double) * (size_t)d);
    double* h = (double*)malloc(sizeof(double) * (size_t)f);
    orc_cand* cands = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)f);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
      const int64_t tok = src_row[i];
      const int64_t e = expert[i];
      int nc = 0;
      for (int c = 0; c < d; ++c) xr[c] = orc_ld(x, tok * d + c, is_bf16);
      const int64_t wg0 = e * 2 * (int64_t)f * d;          /* gate row 0 of expert e */
      const int64_t wu0 = wg0 + (int64_t)f * d;            /* up row 0 */
      for (int n = 0; n < f; ++n) {
        double g = 0.0, u = 0.0, qg = 0.0, qu = 0.0;
        for (int c = 0; c < d; ++c) {
          const double tg = xr[c] * orc_ld(w_gate_up, wg0 + (int64_t)n * d + c, is_bf16);
          const double tu = xr[c] * orc_ld(w_gate_up, wu0 + (int64_t)n * d + c, is_bf16);
          g += tg;
          u += tu;
          qg += tg * tg;
          qu += tu * tu;
        }
        const double hv = (g / (1.0 + exp(-g))) * u;         /* silu(g) u */
        if (!is_bf16) {
          h[n] = hv;
          continue;
        }
        h[n] = orc_round_bf16(hv);
        if (cand_count != NULL && hv != h[n]) {
          const double sg = 1.0 / (1.0 + exp(-g)); /* sigmoid; silu'(g) = sg (1 + g (1 - sg)) */
          const double dsilu = sg * (1.0 + g * (1.0 - sg));
          const double delta = ldexp(sqrt((double)d) * (fabs(dsilu * u) * sqrt(qg) + fabs(g * sg) * sqrt(qu)), -21) +
                               ldexp(fabs(hv), -20);
          const double other = orc_bf16_step(h[n], hv > h[n]);
          const double margin = fabs(hv - 0.5 * (h[n] + other));
          if (margin <= delta) {
            cands[nc].ratio = -fabs(other - h[n]); /* sort key: largest step first */
            cands[nc].n = n;
            cands[nc].dh = other - h[n];
            ++nc;
          }
        }
      }
      if (h_out != NULL) memcpy(h_out + i * (int64_t)f, h, sizeof(double) * (size_t)f);
      const int64_t wd0 = e * (int64_t)d * f;
      for (int m = 0; m < d; ++m) {
        double acc = 0.0, qy = 0.0;
        for (int n = 0; n < f; ++n) {
          const double t = h[n] * orc_ld(w_down, wd0 + (int64_t)m * f + n, is_bf16);
          acc += t;
          qy += t * t;
        }
        if (y_unr != NULL) y_unr[i * d + m] = acc;
        if (y_delta != NULL) y_delta[i * d + m] = ldexp(sqrt((double)f) * sqrt(qy), -21) + ldexp(fabs(acc), -22);
        y_out[i * d + m] = is_bf16 ? orc_round_bf16(acc) : acc;
      }
      if (cand_count != NULL) {
        if (nc > max_cand) qsort(cands, (size_t)nc, sizeof(orc_cand), orc_cand_cmp);
        if (nc > max_cand) nc = max_cand;
        cand_count[i] = nc;
        for (int q = 0; q < nc; ++q) {
          cand_n[i * max_cand + q] = cands[q].n;
          if (cand_vec == NULL) continue; /* the list only */
          double* v = cand_vec + ((int64_t)i * max_cand + q) * d;
          for (int m = 0; m < d; ++m) v[m] = cands[q].dh * orc_ld(w_down, wd0 + (int64_t)m * f + cands[q].n, is_bf16);
        }
      }
    }
    free(xr);
    free(h);
    free(cands);
  }
  return 0;
}

int orc_ffn_rows(int64_t nrows, const int32_t* src_row, const int32_t* expert, int d, int f, int is_bf16,
                 const void* x, const void* w_gate_up, const void* w_down, double* y_out) {
  return orc_ffn_rows_ex(nrows, src_row, expert, d, f, is_bf16, x, w_gate_up, w_down, y_out, NULL, 0, NULL, NULL,
                         NULL, NULL, NULL);
}

/* ------------------------------------------------------------------------------------------------ */
/* Backward of the expert FFN for a list of rows (the review page, "Where Pith is reading between the lines": the same */
/* signalling applied to MoE training's backward pass).  Row i is token tok[i] routed to local expert expert[i]      */
/* with weight w[i]; d_out is the gradient of the combined output.  The combine made out = sum_j w_j y_j, so the     */
/* row's output gradient is dY = w dOut[tok], and through y = h Wd^T, h = silu(g) u, g = x Wg^T, u = x Wu^T:        */
/*   dH_n = sum_m dY_m Wd[m][n],  dU_n = dH_n silu(g_n),  dG_n = dH_n u_n silu'(g_n),                              */
/*   silu'(g) = s (1 + g (1 - s)) with s = 1 / (1 + exp(-g)),                                                       */
/*   dX_c = sum_n dG_n Wg[n][c] + dU_n Wu[n][c],                                                                    */
/* and the routing weight's gradient is <dOut[tok], y>.  The weight gradients are sums over an expert's rows of     */
/* dY h^T (Wd), dG x^T (Wg) and dU x^T (Wu); the caller forms them from the rows' dY, h and dG | dU.                */
/* is_bf16: the GPU feeds its GEMMs bf16 operands, so the values it rounds are rounded here at the same points:    */
/* dY = bf16(fp32(w * dOut)) (an fp32 product, then bf16), h = bf16(silu(g) u) as in the forward, dG and dU to      */
/* bf16, and the row dX to bf16 (the rows the return delivers); y = bf16(...) as delivered.  fp32: no rounding.    */
/* Every sum in double.                                                                                             */
/* adm_out (optional, bf16 mode, [nrows][3][2][f]): for h, dG and dU (in that order), the least and the greatest    */
/* bf16 values that an fp32 evaluation within its error bound can round to: the bf16 roundings of the exact value   */
/* minus and plus the bound (rounding is monotone, so every bf16 value between them is one such rounding).  The      */
/* bound adds, for each fp32 input of the value, the error of a d-term fp32 sum (2^-21 sqrt(d) times the root sum of */
/* squares of its terms, as in orc_ffn_rows_ex) times the value's derivative in that input, plus 2^-20 of the value  */
/* for its own evaluation: g, u and dH feed h = silu(g) u, dU = dH silu(g) and dG = dH u silu'(g).  dH's bound also */
/* holds sum_m |Wd[m][n]| times the widest step of dY[m] within its own admitted interval (below).                  */
/* dy_adm_out (optional, bf16 mode, [nrows][2][d]): dY's least and greatest admitted values, the bf16 roundings of  */
/* w dOut (1 -+ (w_rel + 2^-24)): a routing weight within relative w_rel of w (an fp32 softmax's weights are correct */
/* to that bound), times dOut, rounded to fp32.                                                                     */
int orc_bwd_rows(int64_t nrows, const int32_t* tok, const int32_t* expert, const float* w, int d, int f, int is_bf16,
                 const void* x, const void* w_gate_up, const void* w_down, const void* d_out, double* dx_row,
                 double* dy_out, double* h_out, double* dgu_out, double* y_out, double* adm_out, double w_rel,
                 double* dy_adm_out) {
  if (nrows < 0 || d <= 0 || f <= 0 || !(w_rel >= 0.0)) return -1;
#pragma omp parallel
  {
    double* xr = (double*)malloc(sizeof(double) * (size_t)d);
    double* dy = (double*)malloc(sizeof(double) * (size_t)d);
    double* wdy = (double*)malloc(sizeof(double) * (size_t)d); /* widest step of dY within its admitted interval */
    double* h = (double*)malloc(sizeof(double) * (size_t)f);
    double* dg = (double*)malloc(sizeof(double) * (size_t)f);
    double* du = (double*)malloc(sizeof(double) * (size_t)f);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
      const int64_t t = tok[i], e = expert[i];
      for (int c = 0; c < d; ++c) {
        xr[c] = orc_ld(x, t * d + c, is_bf16);
        const double o = orc_ld(d_out, t * d + c, is_bf16);
        dy[c] = is_bf16 ? orc_round_bf16((double)(float)(w[i] * (float)o)) : (double)w[i] * o;
        wdy[c] = 0.0;
        if (is_bf16 && (adm_out != NULL || dy_adm_out != NULL)) {
          const double v = (double)w[i] * o, b = fabs(v) * (w_rel + ldexp(1.0, -24));
          const double lo = orc_round_bf16(v - b), hi = orc_round_bf16(v + b);
          wdy[c] = fmax(hi - dy[c], dy[c] - lo);
          if (dy_adm_out != NULL) {
            dy_adm_out[(i * 2 + 0) * (int64_t)d + c] = lo;
            dy_adm_out[(i * 2 + 1) * (int64_t)d + c] = hi;
          }
        }
      }
      const int64_t wg0 = e * 2 * (int64_t)f * d, wu0 = wg0 + (int64_t)f * d, wd0 = e * (int64_t)d * f;
      for (int n = 0; n < f; ++n) {
        double g = 0.0, u = 0.0, dh = 0.0, qg = 0.0, qu = 0.0, qh = 0.0, sh = 0.0;
        for (int c = 0; c < d; ++c) {
          const double tg = xr[c] * orc_ld(w_gate_up, wg0 + (int64_t)n * d + c, is_bf16);
          const double tu = xr[c] * orc_ld(w_gate_up, wu0 + (int64_t)n * d + c, is_bf16);
          g += tg;
          u += tu;
          qg += tg * tg;
          qu += tu * tu;
        }
        for (int m = 0; m < d; ++m) {
          const double wd = orc_ld(w_down, wd0 + (int64_t)m * f + n, is_bf16), th = dy[m] * wd;
          dh += th;
          qh += th * th;
          sh += fabs(wd) * wdy[m];
        }
        const double s = 1.0 / (1.0 + exp(-g)), silu = g * s, dsilu = s * (1.0 + g * (1.0 - s));
        const double hv = silu * u, duv = dh * silu, dgv = dh * u * dsilu;
        h[n] = is_bf16 ? orc_round_bf16(hv) : hv;
        du[n] = is_bf16 ? orc_round_bf16(duv) : duv;
        dg[n] = is_bf16 ? orc_round_bf16(dgv) : dgv;
        if (adm_out != NULL && is_bf16) {
          const double eg = ldexp(sqrt((double)d * qg), -21), eu = ldexp(sqrt((double)d * qu), -21);
          const double eh = ldexp(sqrt((double)d * qh), -21) + sh;
          const double d2silu = s * (1.0 - s) * (2.0 + g * (1.0 - 2.0 * s)); /* silu''(g) */
          const double bound[3] = {
              fabs(dsilu * u) * eg + fabs(silu) * eu + ldexp(fabs(hv), -20),
              fabs(u * dsilu) * eh + fabs(dh * dsilu) * eu + fabs(dh * u * d2silu) * eg + ldexp(fabs(dgv), -20),
              fabs(silu) * eh + fabs(dh * dsilu) * eg + ldexp(fabs(duv), -20)};
          const double exact[3] = {hv, dgv, duv};
          for (int q = 0; q < 3; ++q) {
            adm_out[((i * 3 + q) * 2 + 0) * (int64_t)f + n] = orc_round_bf16(exact[q] - bound[q]);
            adm_out[((i * 3 + q) * 2 + 1) * (int64_t)f + n] = orc_round_bf16(exact[q] + bound[q]);
          }
        }
      }
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int n = 0; n < f; ++n)
          acc += dg[n] * orc_ld(w_gate_up, wg0 + (int64_t)n * d + c, is_bf16) +
                 du[n] * orc_ld(w_gate_up, wu0 + (int64_t)n * d + c, is_bf16);
        dx_row[i * d + c] = is_bf16 ? orc_round_bf16(acc) : acc;
      }
      if (y_out != NULL)
        for (int m = 0; m < d; ++m) {
          double acc = 0.0;
          for (int n = 0; n < f; ++n) acc += h[n] * orc_ld(w_down, wd0 + (int64_t)m * f + n, is_bf16);
          y_out[i * d + m] = is_bf16 ? orc_round_bf16(acc) : acc;
        }
      if (dy_out != NULL) memcpy(dy_out + i * (int64_t)d, dy, sizeof(double) * (size_t)d);
      if (h_out != NULL) memcpy(h_out + i * (int64_t)f, h, sizeof(double) * (size_t)f);
      if (dgu_out != NULL) {
        memcpy(dgu_out + i * 2 * (int64_t)f, dg, sizeof(double) * (size_t)f);
        memcpy(dgu_out + i * 2 * (int64_t)f + f, du, sizeof(double) * (size_t)f);
      }
    }
    free(xr);
    free(dy);
    free(wdy);
    free(h);
    free(dg);
    free(du);
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Delivery: owner r receives, at row recv_off_{e,r} + i of its buffer, row padded_off_{e,r} + i of    */
/* the expert output, for the n_{e,r} real rows of each group only.                                    */

int orc_deliver(int R, int E, int d, const int32_t* counts, const int32_t* padded_off,
                const int32_t* recv_off, const double* y_pad, double* const* recv) {
  for (int e = 0; e < E; ++e)
    for (int r = 0; r < R; ++r) {
      int g = e * R + r;
      for (int i = 0; i < counts[g]; ++i)
        memcpy(recv[r] + ((int64_t)recv_off[g] + i) * d, y_pad + ((int64_t)padded_off[g] + i) * d,
               sizeof(double) * (size_t)d);
    }
  return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Combine: out[r*T_o+t] = sum over slots j (ascending) with plan >= 0 of w_j * recv[r][plan]; tokens */
/* with no local expert get zeros.  Rounded to bf16 in bf16 mode.                                      */

int orc_combine(int R, int T_o, int k, int d, int is_bf16, const int32_t* plan, const float* topk_w,
                const double* const* recv, double* out) {
  for (int r = 0; r < R; ++r)
    for (int t = 0; t < T_o; ++t) {
      int64_t tok = (int64_t)r * T_o + t;
      double* o = out + tok * d;
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      for (int j = 0; j < k; ++j) {
        int32_t p = plan[tok * k + j];
        if (p < 0) continue;
        double w = topk_w[tok * k + j];
        const double* src = recv[r] + (int64_t)p * d;
        for (int c = 0; c < d; ++c) o[c] += w * src[c];
      }
      if (is_bf16)
        for (int c = 0; c < d; ++c) o[c] = orc_round_bf16(o[c]);
    }
  return 0;
}

/* out[i] = bf16 rounding of in[i], i < n */
void orc_round_bf16_n(int64_t n, const double* in, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_round_bf16(in[i]);
}

/* Neighbouring bf16 value of bf16 value h toward v (h itself if v == h). */
void orc_bf16_toward_n(int64_t n, const double* h, const double* v, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = v[i] == h[i] ? h[i] : orc_bf16_step(h[i], v[i] > h[i]);
}

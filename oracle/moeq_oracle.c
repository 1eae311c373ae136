/*
 * fp64 CPU oracle for the quantized Mixture-of-Experts expert forward.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The product path (the HIP
 * library and its Python binding) never calls it, and the two share no
 * source: this file includes no product header and defines its own view of
 * the blob layout from the written specification.
 *
 * What it computes, per token and layer, all in fp64, one plain loop per
 * definition (no blocking, no fusion, no reordering):
 *   - optional unit-weight RMS norm of the layer input (the Flash-MoE page,
 *     fr.news.hada.io, "Deferred GPU Expert Compute": combine + norm +
 *     residual are done on the GPU and handed straight to the next layer);
 *   - router logits l_e = sum_j Wr[e,j] * xhat_j, then the K experts with the
 *     largest logits, ties to the lower index (Flash-MoE "Architecture du
 *     modèle": 512 experts, K active per token; the tie rule is this
 *     oracle's reading, the pages are silent);
 *   - softmax of the selected logits (renormalised over the selection);
 *   - per selected expert and the shared expert: explicit dequantisation
 *     w = q * scale + bias of every row (Flash-MoE "Noyau de
 *     déquantification optimisé FMA"), g = Wg xhat, u = Wu xhat,
 *     a = silu(g) * u (SwiGLU, Flash-MoE "Shaders de calcul Metal"),
 *     d = Wd a;
 *   - y = h + sum_k w_k d_k + gamma * d_shared (MoE combine + residual +
 *     gate, same section), gamma = 1 unless a shared-gate vector is given,
 *     then gamma = sigmoid(gvec . xhat).
 *
 * Blob layout read here (one blob per expert):
 *   [gate.q | up.q | down.q | gate.sb | up.sb | down.sb]
 *   q sections hold rows of packed unsigned values, 32/bits per
 *   little-endian u32, value j of a row at bit bits*(j mod (32/bits)) of
 *   word j/(32/bits); gate/up rows run over hidden, down rows over inter.
 *   3-bit rows (values 0..7, 3*cols/8 bytes) hold two planes: first the
 *   low two bits of every value, packed as a 2-bit row (value j at bit
 *   2*(j mod 16) of word j/16), then the high bit: value j at bit
 *   2*(j mod 16) + ((j/16) mod 2) of word j/32 of the plane.
 *   sb sections hold one u32 per (row, group of 64 inputs): bf16 scale in
 *   the low half, bf16 bias in the high half.
 *
 * Plain C99, OpenMP only across tokens (each token's arithmetic is a fixed
 * sequential loop, so results do not depend on the thread count).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t hidden, inter, n_experts, n_shared, bits, group;
} oracle_shape;

enum { ORACLE_NO_RENORM = 1, ORACLE_RMSNORM = 2 };

static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static int64_t qbytes(const oracle_shape* s) {
  return (int64_t)s->hidden * s->inter * s->bits / 8;
}

static int64_t sbbytes(const oracle_shape* s) {
  return (int64_t)s->hidden * s->inter / s->group * 4;
}

int64_t oracle_expert_bytes(const oracle_shape* s) {
  return 3 * (qbytes(s) + sbbytes(s));
}

/* Dequantise row `row` of section sec (0 gate, 1 up, 2 down) into out[cols]. */
void oracle_dequant_row(const oracle_shape* s, const uint8_t* blob, int sec,
                        int row, double* out) {
  int cols = (sec == 2) ? s->inter : s->hidden;
  int per_word = 32 / s->bits;
  uint32_t mask = (1u << s->bits) - 1u;
  const uint8_t* q = blob + sec * qbytes(s);
  const uint8_t* sb = blob + 3 * qbytes(s) + sec * sbbytes(s);
  int64_t words_per_row = cols / per_word;
  int64_t groups_per_row = cols / s->group;
  const int64_t row_bytes = (int64_t)cols * s->bits / 8;
  for (int j = 0; j < cols; ++j) {
    uint32_t word, v;
    if (s->bits == 3) {   /* low-bits plane, then high-bit plane */
      const uint8_t* r = q + (int64_t)row * row_bytes;
      uint32_t hw;
      memcpy(&word, r + 4 * (j / 16), 4);
      memcpy(&hw, r + cols / 4 + 4 * (j / 32), 4);
      v = ((word >> (2 * (j % 16))) & 3u) + 4u * ((hw >> (2 * (j % 16) + (j / 16) % 2)) & 1u);
    } else {
      memcpy(&word, q + 4 * ((int64_t)row * words_per_row + j / per_word), 4);
      v = (word >> (s->bits * (j % per_word))) & mask;
    }
    uint32_t pair;
    memcpy(&pair, sb + 4 * ((int64_t)row * groups_per_row + j / s->group), 4);
    double scale = bf16_value((uint16_t)(pair & 0xFFFFu));
    double bias = bf16_value((uint16_t)(pair >> 16));
    out[j] = (double)v * scale + bias;
  }
}

/* y[r] = sum_j W[r,j] * x[j] for every row of section sec. */
void oracle_section_matvec(const oracle_shape* s, const uint8_t* blob, int sec,
                           const double* x, double* y) {
  int rows = (sec == 2) ? s->hidden : s->inter;
  int cols = (sec == 2) ? s->inter : s->hidden;
  double* w = (double*)malloc(sizeof(double) * (size_t)cols);
  for (int r = 0; r < rows; ++r) {
    oracle_dequant_row(s, blob, sec, r, w);
    double acc = 0.0;
    for (int j = 0; j < cols; ++j) acc += w[j] * x[j];
    y[r] = acc;
  }
  free(w);
}

double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert on one input: g, u [inter], a [inter], d [hidden]. */
void oracle_expert_ffn(const oracle_shape* s, const uint8_t* blob,
                       const double* xhat, double* g, double* u, double* a,
                       double* d) {
  oracle_section_matvec(s, blob, 0, xhat, g);
  oracle_section_matvec(s, blob, 1, xhat, u);
  for (int r = 0; r < s->inter; ++r) a[r] = oracle_silu(g[r]) * u[r];
  oracle_section_matvec(s, blob, 2, a, d);
}

void oracle_rmsnorm(const double* h, int n, double eps, double* xhat) {
  double ss = 0.0;
  for (int j = 0; j < n; ++j) ss += h[j] * h[j];
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int j = 0; j < n; ++j) xhat[j] = h[j] * inv;
}

void oracle_router_logits(const oracle_shape* s, const uint16_t* wr,
                          const double* xhat, double* logits) {
  for (int e = 0; e < s->n_experts; ++e) {
    double acc = 0.0;
    for (int j = 0; j < s->hidden; ++j)
      acc += bf16_value(wr[(int64_t)e * s->hidden + j]) * xhat[j];
    logits[e] = acc;
  }
}

typedef struct { double v; int32_t i; } ranked;

static int by_logit_desc_index_asc(const void* pa, const void* pb) {
  const ranked* a = (const ranked*)pa;
  const ranked* b = (const ranked*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->i > b->i) - (a->i < b->i);
}

/* Full sort of all E experts by (logit descending, index ascending). */
void oracle_topk(const double* logits, int E, int K, int32_t* idx) {
  ranked* r = (ranked*)malloc(sizeof(ranked) * (size_t)E);
  for (int e = 0; e < E; ++e) { r[e].v = logits[e]; r[e].i = e; }
  qsort(r, (size_t)E, sizeof(ranked), by_logit_desc_index_asc);
  for (int k = 0; k < K; ++k) idx[k] = r[k].i;
  free(r);
}

/* Softmax weights of the selected experts.  renorm != 0: softmax over the
 * K selected logits; renorm == 0: full softmax over all E, read at the
 * selected experts. */
void oracle_softmax_selected(const double* logits, int E, const int32_t* idx,
                             int K, int renorm, double* w) {
  if (K == 0) return;
  double m = logits[idx[0]];
  for (int k = 1; k < K; ++k) if (logits[idx[k]] > m) m = logits[idx[k]];
  double z = 0.0;
  if (renorm) {
    for (int k = 0; k < K; ++k) z += exp(logits[idx[k]] - m);
  } else {
    for (int e = 0; e < E; ++e) if (logits[e] > m) m = logits[e];
    for (int e = 0; e < E; ++e) z += exp(logits[e] - m);
  }
  for (int k = 0; k < K; ++k) w[k] = exp(logits[idx[k]] - m) / z;
}

/* Routing of T tokens: logits [T][E] (may be NULL), idx [T][K], w [T][K],
 * gamma [T] (shared-expert weight).  h [T][H] is the layer input. */
void oracle_route(const oracle_shape* s, const uint16_t* wr,
                  const uint16_t* shared_gate_or_null, const double* h, int T,
                  int K, int flags, double* logits_or_null, int32_t* idx,
                  double* w, double* gamma) {
  int H = s->hidden, E = s->n_experts;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t) {
    double* xhat = (double*)malloc(sizeof(double) * (size_t)H);
    double* lg = (double*)malloc(sizeof(double) * (size_t)E);
    if (flags & ORACLE_RMSNORM) oracle_rmsnorm(h + (int64_t)t * H, H, 1e-6, xhat);
    else memcpy(xhat, h + (int64_t)t * H, sizeof(double) * (size_t)H);
    oracle_router_logits(s, wr, xhat, lg);
    oracle_topk(lg, E, K, idx + (int64_t)t * K);
    oracle_softmax_selected(lg, E, idx + (int64_t)t * K, K,
                            !(flags & ORACLE_NO_RENORM), w + (int64_t)t * K);
    if (shared_gate_or_null) {
      double acc = 0.0;
      for (int j = 0; j < H; ++j) acc += bf16_value(shared_gate_or_null[j]) * xhat[j];
      gamma[t] = 1.0 / (1.0 + exp(-acc));
    } else {
      gamma[t] = 1.0;
    }
    if (logits_or_null) memcpy(logits_or_null + (int64_t)t * E, lg, sizeof(double) * (size_t)E);
    free(lg);
    free(xhat);
  }
}

/* One MoE layer for T tokens.
 *   blobs  : n_experts + n_shared host pointers; only the experts some
 *            token selects (and the shared ones) are read, others may be NULL
 *   h      : [T][H] layer input (the residual)
 *   outputs: logits [T][E] (optional), idx/w [T][K], gamma [T],
 *            gu [T][K+S][2][I] (optional), a [T][K+S][I] (optional),
 *            d [T][K+S][H] (optional), y [T][H]
 * Expert slot k < K is the k-th routed expert, slot K the shared one.
 * Returns 0, or -1 if a needed blob pointer is NULL. */
int oracle_moe_layer(const oracle_shape* s, const uint8_t* const* blobs,
                     const uint16_t* wr, const uint16_t* shared_gate_or_null,
                     const double* h, int T, int K, int flags,
                     double* logits_or_null, int32_t* idx, double* w,
                     double* gamma, double* gu_or_null, double* a_or_null,
                     double* d_or_null, double* y) {
  int H = s->hidden, I = s->inter, E = s->n_experts, S = s->n_shared;
  int KS = K + S;
  oracle_route(s, wr, shared_gate_or_null, h, T, K, flags, logits_or_null, idx, w, gamma);
  for (int t = 0; t < T; ++t) {
    for (int k = 0; k < K; ++k) if (!blobs[idx[(int64_t)t * K + k]]) return -1;
  }
  for (int e = 0; e < S; ++e) if (!blobs[E + e]) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t) {
    const double* ht = h + (int64_t)t * H;
    double* xhat = (double*)malloc(sizeof(double) * (size_t)H);
    double* g = (double*)malloc(sizeof(double) * (size_t)I);
    double* u = (double*)malloc(sizeof(double) * (size_t)I);
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    double* d = (double*)malloc(sizeof(double) * (size_t)H);
    if (flags & ORACLE_RMSNORM) oracle_rmsnorm(ht, H, 1e-6, xhat);
    else memcpy(xhat, ht, sizeof(double) * (size_t)H);
    double* yt = y + (int64_t)t * H;
    for (int j = 0; j < H; ++j) yt[j] = ht[j];
    for (int k = 0; k < KS; ++k) {
      int expert = (k < K) ? idx[(int64_t)t * K + k] : E + (k - K);
      double weight = (k < K) ? w[(int64_t)t * K + k] : gamma[t];
      oracle_expert_ffn(s, blobs[expert], xhat, g, u, a, d);
      for (int j = 0; j < H; ++j) yt[j] += weight * d[j];
      int64_t slot = (int64_t)t * KS + k;
      if (gu_or_null) {
        memcpy(gu_or_null + (slot * 2 + 0) * I, g, sizeof(double) * (size_t)I);
        memcpy(gu_or_null + (slot * 2 + 1) * I, u, sizeof(double) * (size_t)I);
      }
      if (a_or_null) memcpy(a_or_null + slot * I, a, sizeof(double) * (size_t)I);
      if (d_or_null) memcpy(d_or_null + slot * H, d, sizeof(double) * (size_t)H);
    }
    free(d); free(a); free(u); free(g); free(xhat);
  }
  return 0;
}

/*
 * Seeded synthetic inputs for the quantized MoE expert path (host side).
 *
 * This file holds input generation only: no step of the expert path's
 * arithmetic (dequantisation, dot products, routing, activation, combine)
 * lives here.  Both the fp64 oracle and the HIP library are fed from these
 * streams; neither links against the other.
 *
 * Random source: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), used as a
 * counter-based generator: element i of a stream with key k is
 * mix64(k + (i + 1) * GAMMA), which is the (i+1)-th output of a SplitMix64
 * generator seeded with k.  The device twin (synth_device.hip) implements
 * the same definition so that a 218 GB expert pool can be filled in HBM and
 * checked byte for byte against this file.
 *
 * Expert blob layout (one contiguous blob per expert; sizes for hidden H,
 * intermediate I, bits b in {2,4}, group G = 64):
 *   [gate.q | up.q | down.q | gate.sb | up.sb | down.sb]
 *   gate.q, up.q : I rows x (H*b/32) little-endian u32 words
 *   down.q       : H rows x (I*b/32) u32 words
 *   value j of a row sits in word j/(32/b) at bit offset b*(j mod (32/b))
 *   *.sb         : rows x (cols/G) u32, low half = bf16 scale,
 *                  high half = bf16 bias, one pair per group of G
 *                  consecutive input-dim elements
 * Flash-MoE (fr.news.hada.io, "Noyau de déquantification optimisé FMA")
 * gives the dequantised weight as nibble*scale + bias; the page is silent
 * on packing, which is fixed here.
 *
 * Compiled with -ffp-contract=off: the scale formula below is a multiply
 * followed by an add, each rounded, exactly as the device twin does it.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint32_t layer, uint32_t unit,
                          uint32_t tensor, uint32_t bits) {
  uint64_t k = mix64(seed ^ 0x6D6F65715F736565ULL);
  k = mix64(k + (((uint64_t)layer << 32) | (uint64_t)unit));
  k = mix64(k + (((uint64_t)tensor << 8) | (uint64_t)bits));
  return k;
}

uint64_t synth_hash(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GAMMA);
}

/* Round-to-nearest-even fp32 -> bf16 (inputs here are finite). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

typedef struct {
  int32_t hidden, inter, bits, group;
  float s_lo, s_hi;    /* scale ~ U(s_lo, s_hi), rounded to bf16 */
  float bias_mult;     /* bias = bf16(bias_mult * scale) */
  uint64_t seed;
} synth_expert_spec;

enum { T_GATE_Q = 0, T_UP_Q, T_DOWN_Q, T_GATE_SB, T_UP_SB, T_DOWN_SB,
       T_ROUTER = 6, T_TOKEN = 7, T_SHARED_GATE = 8 };

int64_t synth_expert_bytes(const synth_expert_spec* s) {
  int64_t q = (int64_t)s->hidden * s->inter * s->bits / 8;
  int64_t sb = (int64_t)s->hidden * s->inter / s->group * 4;
  return 3 * (q + sb);
}

/* Byte offsets of the six sections, in blob order. */
void synth_expert_offsets(const synth_expert_spec* s, int64_t off[7]) {
  int64_t q = (int64_t)s->hidden * s->inter * s->bits / 8;
  int64_t sb = (int64_t)s->hidden * s->inter / s->group * 4;
  off[0] = 0; off[1] = q; off[2] = 2 * q;
  off[3] = 3 * q; off[4] = 3 * q + sb; off[5] = 3 * q + 2 * sb;
  off[6] = 3 * q + 3 * sb;
}

static uint32_t scale_bias_word(const synth_expert_spec* s, uint64_t h) {
  uint64_t u24 = h >> 40;
  double u = (double)u24 * (1.0 / 16777216.0);          /* exact */
  double span = (double)s->s_hi - (double)s->s_lo;
  double prod = span * u;                                /* rounded */
  double sd = (double)s->s_lo + prod;                    /* rounded */
  uint16_t sc = f32_to_bf16_rne((float)sd);
  float bias = s->bias_mult * bf16_to_f32(sc);          /* exact for -8, -1.5 */
  uint16_t bi = f32_to_bf16_rne(bias);
  return (uint32_t)sc | ((uint32_t)bi << 16);
}

/* Fill one expert blob (synth_expert_bytes(s) bytes, 4-byte aligned). */
void synth_fill_expert(const synth_expert_spec* s, uint32_t layer,
                       uint32_t expert, uint8_t* blob) {
  int64_t off[7];
  synth_expert_offsets(s, off);
  for (int t = 0; t < 6; ++t) {
    uint64_t key = synth_stream_key(s->seed, layer, expert, (uint32_t)t,
                                    (uint32_t)s->bits);
    uint32_t* w = (uint32_t*)(blob + off[t]);
    int64_t n = (off[t + 1] - off[t]) / 4;
    if (t < 3) {
      for (int64_t i = 0; i < n; ++i) w[i] = (uint32_t)synth_hash(key, (uint64_t)i);
    } else {
      for (int64_t i = 0; i < n; ++i) w[i] = scale_bias_word(s, synth_hash(key, (uint64_t)i));
    }
  }
}

/* Fill `count` consecutive expert blobs of one layer, blob i at
 * out + i * stride (stride >= synth_expert_bytes). */
void synth_fill_experts(const synth_expert_spec* s, uint32_t layer,
                        uint32_t first_expert, int32_t count, int64_t stride,
                        uint8_t* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < count; ++i)
    synth_fill_expert(s, layer, first_expert + (uint32_t)i, out + (int64_t)i * stride);
}

/* n iid N(0, sigma^2) values rounded to bf16: Box-Muller from hashes 2i and
 * 2i+1 of the stream (host only; value i depends on i alone, so the
 * blocked parallel loop gives the same bytes as a serial one). */
void synth_fill_gaussian_bf16(uint64_t key, int64_t n, double sigma,
                                  uint16_t* out) {
  const int64_t blk = 1 << 16;
  int64_t nb = (n + blk - 1) / blk;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    int64_t lo = b * blk, hi = lo + blk < n ? lo + blk : n;
    const double two_pi = 6.283185307179586476925286766559;
    for (int64_t i = lo; i < hi; ++i) {
      uint64_t h1 = synth_hash(key, (uint64_t)(2 * i));
      uint64_t h2 = synth_hash(key, (uint64_t)(2 * i + 1));
      double u1 = ((double)(h1 >> 11) + 1.0) * (1.0 / 9007199254740992.0);
      double u2 = (double)(h2 >> 11) * (1.0 / 9007199254740992.0);
      double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
      out[i] = f32_to_bf16_rne((float)(z * sigma));
    }
  }
}

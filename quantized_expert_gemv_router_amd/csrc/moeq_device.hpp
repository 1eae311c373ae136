// Device building blocks shared by the moeq kernels (gfx950, wave64).
//
// Dequantised dot products use the fp16 "magic exponent" form.  A packed
// unsigned field q placed at mantissa bit 2^k of fp16 1024.0 (k = 0 for a
// nibble at bits 0-3, k = 4 at bits 4-7; for 2-bit fields k = 0, 2, .., 8)
// reads as the fp16 number 1024 + 2^k q exactly.  So each pair of values
// costs one v_and_or (mask the two fields of a 32-bit word in place and OR
// in the exponent) and one v_dot2_f32_f16, with one shift per word to bring
// the upper fields into the mantissa.  The activation staged for a field
// at 2^k is pre-divided by 2^k (exact), so the product is (1024 + 2^k q)
// x / 2^k = 1024 x' + q x, with x' the stored value.  Per chunk of
// consecutive inputs sharing a scale s and bias b (Flash-MoE, "Noyau de
// déquantification optimisé FMA": w = q*s + b):
//     sum_j (q_j s + b) x_j = s * (dot - 1024 X') + b * X
// with dot the magic-exponent sum, X the sum of the chunk's inputs and X'
// the sum of the stored (pre-divided) values, both precomputed once per
// input vector in LDS.  Activations are staged in LDS as fp16 pairs laid
// out to match the pair order the masks produce, after a power-of-two
// rescale per vector (exact) that puts max|x| in [2^14, 2^15) so no input
// overflows or loses precision to fp16 subnormals.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moeq.h"

namespace moeq {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kMagic = 1024.0f;

// status bits written to the workspace status word
constexpr int32_t kStatusBadExpert = 1;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c,
                                false);
}

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
  half2v h;
  h.x = (_Float16)a;
  h.y = (_Float16)b;
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float half_lo(uint32_t p) {
  return (float)__builtin_bit_cast(half2v, p).x;
}
__device__ __forceinline__ float half_hi(uint32_t p) {
  return (float)__builtin_bit_cast(half2v, p).y;
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ double shfl_xor_f64(double v, int o) {
  int2 p = __builtin_bit_cast(int2, v);
  p.x = __shfl_xor(p.x, o, 64);
  p.y = __shfl_xor(p.y, o, 64);
  return __builtin_bit_cast(double, p);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += shfl_xor_f64(v, o);
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64);
// every lane of a group receives its group's sum.
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ----------------------------------------------------------- packed layout

// Values per u32 word, fp16 pairs per word, values per 16-byte chunk.
// Pair slot m of a word holds values (m, m + kPerWord/2) of the word, one
// in each 16-bit half; kSlotDiv[m] is the power of two its field sits at
// once masked (the staged activation is divided by it).
template <int BITS> struct Pack;
template <> struct Pack<4> {
  static constexpr int kPerWord = 8, kPairsPerWord = 4, kPerChunk = 32, kUnitsPerChunk = 4;
  static constexpr float kSlotDiv[4] = {1.0f, 16.0f, 1.0f, 16.0f};
};
template <> struct Pack<2> {
  static constexpr int kPerWord = 16, kPairsPerWord = 8, kPerChunk = 64, kUnitsPerChunk = 8;
  static constexpr float kSlotDiv[8] = {1.0f, 4.0f, 16.0f, 64.0f, 256.0f, 1.0f, 4.0f, 16.0f};
};
// 3-bit experts: a row holds a low-bits plane (the values' two low bits,
// packed as a 2-bit row) followed by a high-bit plane of cols/32 words in
// which word w holds the high bit of value 32w + m at bit 2m and of value
// 32w + 16 + m at bit 2m + 1 (m < 16).  A chunk of 64 values is one 16-byte
// unit of the low plane plus 8 bytes of the high plane, and the activations
// are staged exactly as for 2-bit values.
template <> struct Pack<3> : Pack<2> {};
// Bits of packed values per staged chunk's low plane (the 16-byte unit).
template <int BITS> constexpr int kPlaneBits = BITS == 3 ? 2 : BITS;
// Floats of precomputed sums per staged chunk: X and 1024 * X'.
constexpr int kChunkSums = 2;

// Two fp16 1024.0 in a vector register: as an operand of v_and_or_b32 it
// cannot be a literal, and a register keeps the compiler from splitting the
// and/or pair.
__device__ __forceinline__ uint32_t magic_pair() {
  uint32_t m;
  asm("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

// The staged fp16 pairs of one chunk, in registers.
template <int BITS> struct XChunk {
  uint4 u[Pack<BITS>::kUnitsPerChunk];
};

// Chunk cc of a staged vector (vec, nch chunks: the stride between a
// chunk's 16-byte units).
template <int BITS>
__device__ __forceinline__ XChunk<BITS> load_xchunk(const uint32_t* __restrict__ vec, int cc, int nch) {
  XChunk<BITS> x;
  const uint4* xv = reinterpret_cast<const uint4*>(vec) + cc;
#pragma unroll
  for (int u = 0; u < Pack<BITS>::kUnitsPerChunk; ++u) x.u[u] = xv[u * nch];
  return x;
}

// Magic-exponent dot of one 16-byte chunk of packed values against the
// staged fp16 pairs of the same chunk.
template <int BITS>
__device__ __forceinline__ float chunk_dot(u32x4 q, const XChunk<BITS>& x) {
  float acc = 0.0f;
  const uint32_t mg = magic_pair();
  if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = q[i], t = w >> 8;
      acc = dot2((w & 0x000F000Fu) | mg, x.u[i].x, acc);
      acc = dot2((w & 0x00F000F0u) | mg, x.u[i].y, acc);
      acc = dot2((t & 0x000F000Fu) | mg, x.u[i].z, acc);
      acc = dot2((t & 0x00F000F0u) | mg, x.u[i].w, acc);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 xa = x.u[2 * i], xb = x.u[2 * i + 1];
      const uint32_t w = q[i], t = w >> 10;
      acc = dot2((w & 0x00030003u) | mg, xa.x, acc);
      acc = dot2((w & 0x000C000Cu) | mg, xa.y, acc);
      acc = dot2((w & 0x00300030u) | mg, xa.z, acc);
      acc = dot2((w & 0x00C000C0u) | mg, xa.w, acc);
      acc = dot2((w & 0x03000300u) | mg, xb.x, acc);
      acc = dot2((t & 0x00030003u) | mg, xb.y, acc);
      acc = dot2((t & 0x000C000Cu) | mg, xb.z, acc);
      acc = dot2((t & 0x00300030u) | mg, xb.w, acc);
    }
  }
  return acc;
}

template <int BITS>
__device__ __forceinline__ float chunk_dot(u32x4 q, const uint32_t* __restrict__ vec, int cc, int nch) {
  return chunk_dot<BITS>(q, load_xchunk<BITS>(vec, cc, nch));
}

// The high-bit plane of a 3-bit chunk against the chunk's staged pairs: for
// low-plane word i the high bits sit at the even (i even) or odd (i odd) bits
// of plane word i/2; shifted down by that parity each sits at the low bit of
// its value's 2-bit field, so the 2-bit staging (pair slot m divided by 4^m)
// serves them and the sum is 1024 X' + sum(high * x).
template <int BITS>
__device__ __forceinline__ float chunk_dot_hi(uint2 h, const XChunk<BITS>& x) {
  float acc = 0.0f;
  const uint32_t mg = magic_pair();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 xa = x.u[2 * i], xb = x.u[2 * i + 1];
    const uint32_t hw = (i >> 1) ? h.y : h.x;
    const uint32_t w = (i & 1) ? hw >> 1 : hw, t = w >> 10;
    acc = dot2((w & 0x00010001u) | mg, xa.x, acc);
    acc = dot2((w & 0x00040004u) | mg, xa.y, acc);
    acc = dot2((w & 0x00100010u) | mg, xa.z, acc);
    acc = dot2((w & 0x00400040u) | mg, xa.w, acc);
    acc = dot2((w & 0x01000100u) | mg, xb.x, acc);
    acc = dot2((t & 0x00010001u) | mg, xb.y, acc);
    acc = dot2((t & 0x00040004u) | mg, xb.z, acc);
    acc = dot2((t & 0x00100010u) | mg, xb.w, acc);
  }
  return acc;
}

// Magic-exponent sum of one chunk of BITS-bit values: the low plane (or the
// whole value) from q, at 3 bits plus 4 times the high plane from qh.
template <int BITS>
__device__ __forceinline__ float chunk_dot_q(u32x4 q, uint2 qh, const XChunk<BITS>& x) {
  if constexpr (BITS == 3) return chunk_dot<BITS>(q, x) + 4.0f * chunk_dot_hi<BITS>(qh, x);
  else return chunk_dot<BITS>(q, x);
}

// One chunk's contribution s * (dot - n 1024 X') + b * X, n being the number
// of 1024 X' offsets the sum carries (5 at 3 bits: one from the low plane,
// four from the high plane's weight of 4).
template <int BITS>
__device__ __forceinline__ float chunk_term(float dot, uint32_t sb, float2 x) {
  constexpr float kOffsets = BITS == 3 ? 5.0f : 1.0f;
  return fmaf(bf16_lo(sb), dot - kOffsets * x.y, bf16_hi(sb) * x.x);
}

// One chunk's contribution: s * (dot - 1024 X') + b * X, with x the
// chunk's two precomputed sums {X, 1024 X'}.
__device__ __forceinline__ float chunk_affine(float dot, uint32_t sb, float2 x) {
  return fmaf(bf16_lo(sb), dot - x.y, bf16_hi(sb) * x.x);
}
__device__ __forceinline__ float chunk_affine(float dot, uint32_t sb, const float* xs) {
  return chunk_affine(dot, sb, *reinterpret_cast<const float2*>(xs));
}

// Rounds the PW values v[] * f to fp16, divides each pair slot by its
// power of two (exact) and packs the pairs into pr[]; adds the chunk
// sums' share of this word to X (the rounded values) and Xs (1024 times
// the stored values).  The fp32 products and packed pairs are pinned so the
// sums add exactly the values the dot products read: the 1024 X' term
// must cancel the magic offsets inside the dot.
template <int BITS>
__device__ __forceinline__ void pack_word(const float* v, float f, uint32_t* pr, float& X, float& Xs) {
  constexpr int HP = Pack<BITS>::kPairsPerWord;
#pragma unroll
  for (int j = 0; j < HP; ++j) {
    float lo = v[j] * f, hi = v[j + HP] * f;
    asm volatile("" : "+v"(lo), "+v"(hi));
    const float d = Pack<BITS>::kSlotDiv[j];
    // round to fp16 first, then the exact division by a power of two
    const float lr = (float)(_Float16)lo, hr = (float)(_Float16)hi;
    pr[j] = pack_half2(lr * (1.0f / d), hr * (1.0f / d));
    asm volatile("" : "+v"(pr[j]));
    const float sl = half_lo(pr[j]), sh = half_hi(pr[j]);
    Xs += (sl + sh) * kMagic;
    X += (sl + sh) * d;
  }
}

// ------------------------------------------------------------- LDS staging
//
// A staged vector of n values (n a multiple of 64, nch = n / kPerChunk
// chunks) occupies
//   pairs : n/2 u32, in 16-byte units: unit u of chunk c at unit index
//           u * nch + c, so lanes reading consecutive chunks read
//           consecutive LDS addresses (no bank conflicts).  Word i of a
//           chunk fills units kUnitsPerChunk/4 * i ..; pair m of a word
//           = (v[w*PW + m], v[w*PW + m + PW/2]), each divided by the slot's
//           power of two.
//   sums  : kChunkSums * nch floats ({X, 1024 X'} per chunk)
// plus one float per vector: the power of two that undoes the rescale.

// Writes the pr[] pairs of word w of a staged vector (base vec, nch chunks).
template <int BITS>
__device__ __forceinline__ void store_word(uint32_t* vec, int w, int nch, const uint32_t* pr) {
  constexpr int UPW = Pack<BITS>::kUnitsPerChunk / 4;   // 16-byte units per word
  uint4* dst = reinterpret_cast<uint4*>(vec);
  const int c = w >> 2, i = w & 3;
#pragma unroll
  for (int u = 0; u < UPW; ++u)
    dst[(UPW * i + u) * nch + c] = make_uint4(pr[4 * u], pr[4 * u + 1], pr[4 * u + 2], pr[4 * u + 3]);
}

// Power-of-two factor p with max_abs * p in [2^14, 2^15) (1 if max_abs == 0
// or not finite).
__device__ __forceinline__ float pow2_stage_factor(float max_abs) {
  if (!(max_abs > 0.0f) || !isfinite(max_abs)) return 1.0f;
  int e = ilogbf(max_abs);          // max_abs in [2^e, 2^(e+1))
  return ldexpf(1.0f, min(14 - e, 126));   // 2^126 keeps 1/p a normal float
}

// ----------------------------------------------------------- memory access

template <class T>
__device__ __forceinline__ T load_stream(const T* p) {
  // A global (not flat) load: flat loads also count against the LDS
  // counter, so every later wait on LDS traffic would wait for them too.
  using GlobalT = __attribute__((address_space(1))) const T;
  return __builtin_nontemporal_load((GlobalT*)p);
}

// Eight bytes at p (8-byte aligned), streamed.
__device__ __forceinline__ uint2 load_stream_u2(const void* p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = load_stream(static_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

// A global load with the default (temporal) cache policy: the L2 keeps the
// line.  For data whose line is consumed by more than one request (a row
// read in 64-byte halves a chunk apart, activation rows re-read by the
// weight tiles of one XCD), a non-temporal load would let the line go
// before its second use and fetch it again.
template <class T>
__device__ __forceinline__ T load_keep(const T* p) {
  using GlobalT = __attribute__((address_space(1))) const T;
  return *(GlobalT*)p;
}

// Range-checked streaming loads through a buffer resource (base address in
// scalar registers, byte size).  A load whose offset lies outside [0, size)
// returns zeros without touching memory, so a wave can issue its loads
// unconditionally and let the range check drop the ones it does not need.
// Loads issued under a branch are a poor fit for the compiler's wait-count
// placement: the first use of any of them then waits for every load in
// flight.  `base` and `bytes` must be wave-uniform.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // 32-bit data format, untyped access
constexpr int kCpolNonTemporal = 2;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 load_rsrc_b128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCpolNonTemporal));
}
__device__ __forceinline__ uint32_t load_rsrc_b32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kCpolNonTemporal);
}
__device__ __forceinline__ uint2 load_rsrc_b64(rsrc_t r, uint32_t off) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kCpolNonTemporal));
  return make_uint2(v.x, v.y);
}
// Keeps the compiler from sinking loads issued above it into the branches
// that use them (no wait is implied).
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// Cross-workgroup hand-off without cache-wide flushes.  Data that another
// workgroup (possibly on another XCD, with its own L2) will read is written
// with agent-scope atomic stores (write-through) and read with agent-scope
// atomic loads; the producer then waits for its stores to complete before
// bumping an arrival counter.  Because every shared access is itself an
// agent-scope atomic, no L2 write-back or invalidate (which an agent-scope
// fence would issue per wave) is needed.
template <class T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this wave's outstanding memory operations have completed.
__device__ __forceinline__ void drain_memory() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
}

// A pointer that is the same in every lane, made scalar so that loads from
// it take a scalar base address.
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Block barrier that orders LDS traffic only: waits for this wave's LDS
// operations, not for its global loads in flight.  (__syncthreads carries a
// release fence that also waits for every outstanding vector memory
// operation whenever a global store may be pending.)  The memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void set_status(int32_t* status, int32_t bits) {
  if (status) __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moeq

namespace moeq {

// ------------------------------------------------- DPP wave reductions
// Full-wave reductions with DPP lane moves (no LDS crossbar round trip):
// xor-1 and xor-2 within quads, half-row and row mirrors, then row
// broadcasts 15 and 31 fold the four rows; lane 63 ends with the result,
// which v_readlane makes uniform.  Fixed combination order, so a sum is
// bit-identical run to run.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_move(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_move_f64(double old, double v) {
  const int2 o = __builtin_bit_cast(int2, old), x = __builtin_bit_cast(int2, v);
  int2 r;
  r.x = dpp_move<CTRL, ROW_MASK>(o.x, x.x);
  r.y = dpp_move<CTRL, ROW_MASK>(o.y, x.y);
  return __builtin_bit_cast(double, r);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const int2 x = __builtin_bit_cast(int2, v);
  int2 r;
  r.x = __builtin_amdgcn_readlane(x.x, lane);
  r.y = __builtin_amdgcn_readlane(x.y, lane);
  return __builtin_bit_cast(double, r);
}

// Sum over the wave, returned in every lane (uniform).
__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
  v += dpp_move_f64<kDppQuadXor1>(0.0, v);
  v += dpp_move_f64<kDppQuadXor2>(0.0, v);
  v += dpp_move_f64<kDppHalfMirror>(0.0, v);
  v += dpp_move_f64<kDppMirror>(0.0, v);
  v += dpp_move_f64<kDppBcast15, 0xA>(0.0, v);
  v += dpp_move_f64<kDppBcast31, 0xC>(0.0, v);
  return readlane_f64(v, 63);
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __int_as_float(dpp_move<kDppQuadXor1>(0, __float_as_int(v)));
  v += __int_as_float(dpp_move<kDppQuadXor2>(0, __float_as_int(v)));
  v += __int_as_float(dpp_move<kDppHalfMirror>(0, __float_as_int(v)));
  v += __int_as_float(dpp_move<kDppMirror>(0, __float_as_int(v)));
  v += __int_as_float(dpp_move<kDppBcast15, 0xA>(0, __float_as_int(v)));
  v += __int_as_float(dpp_move<kDppBcast31, 0xC>(0, __float_as_int(v)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over aligned groups of W lanes (W a power of two <= 64) with DPP lane
// moves, no LDS crossbar round trips.  The sum is valid in lane W - 1 of
// each group (in every lane of the group for W <= 16).
template <int W>
__device__ __forceinline__ float group_sum_dpp(float v) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
  if constexpr (W >= 2) v += __int_as_float(dpp_move<kDppQuadXor1>(0, __float_as_int(v)));
  if constexpr (W >= 4) v += __int_as_float(dpp_move<kDppQuadXor2>(0, __float_as_int(v)));
  if constexpr (W >= 8) v += __int_as_float(dpp_move<kDppHalfMirror>(0, __float_as_int(v)));
  if constexpr (W >= 16) v += __int_as_float(dpp_move<kDppMirror>(0, __float_as_int(v)));
  if constexpr (W >= 32) v += __int_as_float(dpp_move<kDppBcast15, 0xA>(0, __float_as_int(v)));
  if constexpr (W >= 64) v += __int_as_float(dpp_move<kDppBcast31, 0xC>(0, __float_as_int(v)));
  return v;
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, __int_as_float(dpp_move<kDppQuadXor1>(__float_as_int(v), __float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<kDppQuadXor2>(__float_as_int(v), __float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<kDppHalfMirror>(__float_as_int(v), __float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<kDppMirror>(__float_as_int(v), __float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<kDppBcast15, 0xA>(__float_as_int(v), __float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<kDppBcast31, 0xC>(__float_as_int(v), __float_as_int(v))));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

}  // namespace moeq

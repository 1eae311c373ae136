// Prefill: T tokens through L stacked MoE layers at once (the same layer as
// decode, token by token; tokens are independent, there is no attention).
// fr.news.hada.io, Flash-MoE, "Architecture du modèle" (512 experts, K
// routed + one shared per token, 60 layers), "Noyau de déquantification
// optimisé FMA" (w = value * scale + bias), "Shaders de calcul Metal"
// (dequantised mat-vec, SwiGLU, combine + residual); openclawradar.com/fr
// (top-10 routing over 512 experts).
//
// Per layer, all on the device:
//   norm     x = h / sqrt(mean(h^2) + 1e-6) -> fp16, stored permuted
//   router   logits[t][e] = (Wr[e] . h[t]) / rms[t] in fp64 (tiled GEMM)
//   top-K    per token, ties to the lower index, softmax of the selection
//   group    (token, slot) pairs sorted by expert, token order kept
//   gate/up  per expert: [pairs x H] fp16 times the dequantised [2I x H]
//            weights on MFMA (fp16 in, fp32 accumulation), SwiGLU fused,
//            activations stored fp16
//   down     per expert: [pairs x I] times the dequantised [H x I] weights
//            -> per-pair fp32 rows
//   combine  h[t] += sum_s w[t][s] d[t][s] + d[t][shared], in slot order
//
// Weights are dequantised in registers to fp16 (exact nibble, one fp16
// rounding of s*q + b) just before they enter the MFMA; each expert's rows
// are streamed from memory once per tile of up to 64 pairs.  Within an MFMA
// the K order of a lane's eight values is the nibble order of a packed word
// (0,4,1,5,2,6,3,7); the activations are stored in that order so both
// operands agree.  The results do not depend on the launch geometry (no
// atomics on floating-point values; grouping keeps token order).
#include <hip/hip_runtime.h>

#include <climits>
#include <vector>

#include "moeq.h"
#include "moeq_device.hpp"
#include "moeq_internal.hpp"
#include "topk.hpp"

namespace moeq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kPThreads = 256;          // four waves
constexpr int kMB = 4;                  // row blocks of 16 per tile
constexpr int kMT = 16 * kMB;           // pairs per tile
constexpr int kNBW = 2;                 // blocks of 16 weight rows per wave
constexpr int kNT = 4 * 16 * kNBW;      // weight rows per tile
constexpr int kKC = 128;                // K per chunk (two groups of 64)
constexpr int kPitch = kKC + 8;         // LDS row pitch in halves (bank spread)
constexpr int kSbWin = 8;               // chunks per scale/bias window (16 groups)
constexpr int kSbPitch = 2 * kSbWin + 4; // LDS words per row of a window: 16 rows read at one
                                         // group offset fall in distinct banks

// position of value j of a packed word in the stored (MFMA) order
__device__ __forceinline__ int perm_pos(int r) {
  const int j = r & 7;
  return (r & ~7) | (j < 4 ? 2 * j : 2 * (j - 4) + 1);
}

// ------------------------------------------------------------------ norm
// One block per token: fp64 sum of squares, 1/rms, and x in fp16 (permuted
// within each 8-block).  Block 0 also clears the per-expert counters.
__global__ __launch_bounds__(kPThreads) void norm_kernel(const float* __restrict__ h, int H,
                                                          double* __restrict__ inv_rms,
                                                          _Float16* __restrict__ xh, int32_t* counts,
                                                          int n_counts) {
  __shared__ double part[kPThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (t == 0)
    for (int i = tid; i < n_counts; i += kPThreads) counts[i] = 0;
  const float* row = h + (int64_t)t * H;
  double ss = 0.0;
  for (int j = tid; j < H; j += kPThreads) ss = fma((double)row[j], (double)row[j], ss);
  ss = wave_sum_f64_dpp(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < kPThreads / 64; ++w) tot += part[w];
  const double inv = 1.0 / sqrt(tot / (double)H + 1e-6);
  if (tid == 0) inv_rms[t] = inv;
  for (int b = tid; b < H / 8; b += kPThreads) {
    const float4 v0 = *reinterpret_cast<const float4*>(row + 8 * b);
    const float4 v1 = *reinterpret_cast<const float4*>(row + 8 * b + 4);
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    half8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j < 4 ? 2 * j : 2 * (j - 4) + 1] = (_Float16)(float)((double)v[j] * inv);
    *reinterpret_cast<half8*>(xh + (int64_t)t * H + 8 * b) = o;
  }
}

// ---------------------------------------------------------------- router
// logits[t][e] = (sum_j Wr[e][j] h[t][j]) * inv_rms[t] in fp64 (bf16 and
// fp32 inputs are exact in fp64) on fp64 MFMA (16x16x4).  A block computes a
// 64-token x 64-expert tile, each wave a 32 x 32 quarter (2 x 2 MFMA
// blocks); K advances in chunks of 16 staged in LDS as fp64, the next
// chunk's inputs loaded into registers while the current one is consumed.
// Lane layout of v_mfma_f64_16x16x4_f64: A lane l = (row l%16, k l/16),
// B lane l = (k l/16, col l%16), D element i of lane l = (row 4i + l/16,
// col l%16).
constexpr int kRT = 64, kRK = 16;
typedef double double4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kPThreads) void router_kernel(const float* __restrict__ h,
                                                            const uint16_t* const* __restrict__ routers,
                                                            int layer, int T, int H, int E,
                                                            const double* __restrict__ inv_rms,
                                                            double* __restrict__ logits) {
  __shared__ double As[kRK][kRT + 2];
  __shared__ double Bs[kRK][kRT + 2];
  const uint16_t* wr = uniform_ptr(routers[layer]);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * kRT, e0 = blockIdx.y * kRT;
  // staging: thread -> (row r, four consecutive k)
  const int sr = tid / 4, sk = (tid % 4) * 4;
  const bool tok_ok = t0 + sr < T, exp_ok = e0 + sr < E;
  const float* hrow = h + (int64_t)(tok_ok ? t0 + sr : 0) * H + sk;
  const uint16_t* wrow = wr + (int64_t)(exp_ok ? e0 + sr : 0) * H + sk;
  float4 hv = tok_ok ? *reinterpret_cast<const float4*>(hrow) : make_float4(0.f, 0.f, 0.f, 0.f);
  uint2 wv = exp_ok ? *reinterpret_cast<const uint2*>(wrow) : make_uint2(0u, 0u);
  double4v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = double4v{0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < H; k0 += kRK) {
    As[sk + 0][sr] = hv.x;
    As[sk + 1][sr] = hv.y;
    As[sk + 2][sr] = hv.z;
    As[sk + 3][sr] = hv.w;
    Bs[sk + 0][sr] = (double)__uint_as_float(wv.x << 16);
    Bs[sk + 1][sr] = (double)__uint_as_float(wv.x & 0xFFFF0000u);
    Bs[sk + 2][sr] = (double)__uint_as_float(wv.y << 16);
    Bs[sk + 3][sr] = (double)__uint_as_float(wv.y & 0xFFFF0000u);
    __syncthreads();
    if (k0 + kRK < H) {   // uniform: next chunk's inputs in flight during the MFMAs
      hv = tok_ok ? *reinterpret_cast<const float4*>(hrow + k0 + kRK) : make_float4(0.f, 0.f, 0.f, 0.f);
      wv = exp_ok ? *reinterpret_cast<const uint2*>(wrow + k0 + kRK) : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int ks = 0; ks < kRK / 4; ++ks) {
      const int kk = ks * 4 + (lane >> 4);
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = As[kk][wm * 32 + i * 16 + (lane & 15)];
        b[i] = Bs[kk][wn * 32 + i * 16 + (lane & 15)];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + wm * 32 + i * 16 + 4 * r + (lane >> 4);
      if (t >= T) continue;
      const double inv = inv_rms[t];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = e0 + wn * 32 + j * 16 + (lane & 15);
        if (e < E) logits[(int64_t)t * E + e] = acc[i][j][r] * inv;
      }
    }
}

// ----------------------------------------------------------------- top-K
template <int M>
__global__ __launch_bounds__(kPThreads) void topk_kernel(const double* __restrict__ logits, int E, int K,
                                                          int no_renorm, int32_t* __restrict__ idx,
                                                          float* __restrict__ w, int32_t* trace) {
  __shared__ double lg[64 * 4 * M];
  __shared__ int64_t ck[64];
  __shared__ int ci[64];
  __shared__ int sel[MOEQ_MAX_TOPK];
  __shared__ double selv[MOEQ_MAX_TOPK];
  const int t = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < E; e += kPThreads) lg[e] = logits[(int64_t)t * E + e];
  __syncthreads();
  block_topk_keys<4, M, 1>(lg, E, K, ck, ci, sel, selv);
  if (tid < 64) {
    const float wt = no_renorm ? wave_softmax_weight(lg, E, K, selv, true) : wave_softmax_selected(selv, K);
    if (tid < K) {
      idx[(int64_t)t * K + tid] = sel[tid];
      w[(int64_t)t * K + tid] = wt;
      if (trace) trace[(int64_t)t * K + tid] = sel[tid];
    }
  }
}

// -------------------------------------------------------------- grouping
__global__ void count_kernel(const int32_t* __restrict__ idx, int n, int E, int32_t* counts, int32_t* status) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= n) return;
  const int e = idx[p];
  if (e >= 0 && e < E) atomicAdd(&counts[e], 1);
  else set_status(status, 1);
}

// One block: offsets of each expert's pair list (shared experts hold every
// token), the prefix of its tile count, and per row tile (expert, first
// list entry, rows).
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts, int E, int S, int T,
                                                     int32_t* __restrict__ offs, int32_t* __restrict__ mtoff,
                                                     int4* __restrict__ tiles) {
  __shared__ int32_t sc[1024], sm[1024];
  const int n = E + S, tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  int c_sum = 0, m_sum = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < n) {
      const int c = e < E ? counts[e] : T;
      c_sum += c;
      m_sum += (c + kMT - 1) / kMT;
    }
  }
  sc[tid] = c_sum;
  sm[tid] = m_sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {   // inclusive scan (Hillis-Steele)
    const int a = tid >= o ? sc[tid - o] : 0, b = tid >= o ? sm[tid - o] : 0;
    __syncthreads();
    sc[tid] += a;
    sm[tid] += b;
    __syncthreads();
  }
  int co = sc[tid] - c_sum, mo = sm[tid] - m_sum;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < n) {
      const int c = e < E ? counts[e] : T;
      offs[e] = co;
      mtoff[e] = mo;
      for (int mi = 0; mi * kMT < c; ++mi)   // the expert's row tiles
        tiles[mo + mi] = make_int4(e, co + mi * kMT, min(kMT, c - mi * kMT), 0);
      co += c;
      mo += (c + kMT - 1) / kMT;
    }
  }
  if (tid == 1023) {
    offs[n] = sc[1023];
    mtoff[n] = sm[1023];
  }
}

// One block per expert: its pairs in token order (p = t*K + slot ascending),
// stored as row ids t*(K+S) + slot.
__global__ __launch_bounds__(kPThreads) void compact_kernel(const int32_t* __restrict__ idx, int T, int K, int S,
                                                             int E, const int32_t* __restrict__ offs,
                                                             int32_t* __restrict__ lists) {
  __shared__ int wc[kPThreads / 64];
  __shared__ int running;
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = offs[e], KS = K + S;
  if (e >= E) {
    for (int t = tid; t < T; t += kPThreads) lists[base + t] = t * KS + K + (e - E);
    return;
  }
  if (tid == 0) running = 0;
  __syncthreads();
  const int n = T * K;
  for (int p0 = 0; p0 < n; p0 += kPThreads) {
    const int p = p0 + tid;
    const bool hit = p < n && idx[p] == e;
    const uint64_t mask = __ballot(hit);
    if (lane == 0) wc[wave] = __popcll(mask);
    __syncthreads();
    int before = running;
    for (int w2 = 0; w2 < wave; ++w2) before += wc[w2];
    if (hit) {
      const int r = before + __popcll(mask & ((1ull << lane) - 1));
      lists[base + r] = (p / K) * KS + p % K;
    }
    __syncthreads();
    if (tid == 0)
      for (int w2 = 0; w2 < kPThreads / 64; ++w2) running += wc[w2];
    __syncthreads();
  }
}

// ---------------------------------------------------------- expert GEMMs
struct GemmArgs {
  const void* const* blobs;   // this layer's table row [E + S]
  int E, S, K, H, I;
  const int32_t* offs;        // [E + S + 1]
  const int32_t* mtoff;       // [E + S + 1]
  const int4* tiles;          // per row tile: expert, first list entry, rows
  const int32_t* lists;       // pair rows grouped by expert
  const _Float16* xh;         // [T][H] permuted fp16 (gate/up input)
  _Float16* abuf;             // [T*(K+S)][I] permuted fp16 (gate/up out, down in)
  float* dbuf;                // [T*(K+S)][H] fp32 (down out)
  int32_t* status;
};

// Eight fp16 weights of one packed word, dequantised: w = q*s + b.  Each
// pair (q_i, q_{i+4}) is masked in place and OR-ed into an fp16 exponent
// whose mantissa unit is the field's own: a nibble at bits 0-3 of a half
// reads as 1024 + q, one at bits 4-7 as 64 + q (one v_and_or per pair,
// one shift per word), then the exact subtract and one fma.
__device__ __forceinline__ half8 dequant_word(uint32_t word, half2v s2, half2v b2) {
  uint32_t m1024, m64;   // in registers: v_and_or_b32 takes no literal
  asm("v_mov_b32 %0, 0x64006400" : "=v"(m1024));
  asm("v_mov_b32 %0, 0x54005400" : "=v"(m64));
  const half2v k1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f}, k64 = {(_Float16)-64.0f, (_Float16)-64.0f};
  const uint32_t hi = word >> 8;
  const uint32_t t[4] = {(word & 0x000F000Fu) | m1024, (word & 0x00F000F0u) | m64, (hi & 0x000F000Fu) | m1024,
                         (hi & 0x00F000F0u) | m64};
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v q = __builtin_bit_cast(half2v, t[i]) + ((i & 1) ? k64 : k1024);
    const half2v v = q * s2 + b2;
    r[2 * i] = v[0];
    r[2 * i + 1] = v[1];
  }
  return r;
}

__device__ __forceinline__ void sb_halves(uint32_t sb, half2v& s2, half2v& b2) {
  const _Float16 s = (_Float16)__uint_as_float(sb << 16), b = (_Float16)__uint_as_float(sb & 0xFFFF0000u);
  s2 = half2v{s, s};
  b2 = half2v{b, b};
}

// GU: gate and up rows (2 matrices), SwiGLU into abuf.  Otherwise down rows
// into dbuf.  NPF chunks of weights are in flight per wave; it divides the
// chunk count.
template <bool GU, int NPF, int NW>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : 2) void gemm_kernel(GemmArgs a) {
  constexpr int NMAT = GU ? 2 : 1;
  constexpr int NTH = 64 * NW;              // threads
  constexpr int NTR = NW * 16 * kNBW;       // weight rows per tile
  __shared__ __align__(16) _Float16 As[2][kMT * kPitch];
  // scale/bias words of the tile's rows, windows of 2*kSbWin groups,
  // double-buffered: [buffer][matrix][row][group in window]
  __shared__ __align__(16) uint32_t Sb[2][NMAT][NTR][kSbPitch];
  __shared__ int32_t src_row[kMT], dst_row[kMT];
  __shared__ int s_e, s_row0, s_n;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = a.E, S = a.S, KS = a.K + S;
  const int KD = GU ? a.H : a.I;            // reduction length
  const int NR = GU ? a.I : a.H;            // weight rows per matrix
  const int NC = KD / kKC;                  // chunks
  const int NT = NR / NTR;                  // tiles along the weight rows
  const int n_mt = a.mtoff[E + S];
  const int total = (n_mt + 7) / 8 * 8 * NT;
  const int64_t qsec = (int64_t)a.H * a.I / 2;   // bytes of one q section
  const int64_t ssec = (int64_t)a.H * a.I / 64 * 4;

  for (int wi = blockIdx.x; wi < total; wi += gridDim.x) {
    // the NT tiles of one row tile land on one XCD (wi mod 8)
    const int grp = wi / (8 * NT), r8 = wi % (8 * NT);
    const int nt = r8 / 8, mt = grp * 8 + r8 % 8;
    if (mt >= n_mt) continue;   // uniform over the block
    if (tid == 0) {
      const int4 tl = a.tiles[mt];
      s_e = tl.x;
      s_row0 = tl.y;
      s_n = tl.z;
    }
    __syncthreads();
    const int e = s_e, nrows = s_n;
    if (tid < kMT) {
      const int p = a.lists[s_row0 + min(tid, nrows - 1)];   // padding rows repeat a real row
      src_row[tid] = GU ? p / KS : p;
      dst_row[tid] = p;
    }
    const uint8_t* blob = uniform_ptr(static_cast<const uint8_t*>(a.blobs[e]));
    __syncthreads();
    if (blob == nullptr) {   // missing expert: flag it, leave its outputs unwritten
      if (tid == 0) set_status(a.status, 1);
      continue;
    }

    // this lane's weight rows, matrices and packed-word offsets
    const int q4 = lane >> 4;                     // k quarter of the MFMA operand
    const uint32_t* qrow[NMAT][kNBW];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nb = 0; nb < kNBW; ++nb) {
        const int n = nt * NTR + wave * (16 * kNBW) + nb * 16 + (lane & 15);
        const int sec = GU ? m : 2;
        qrow[m][nb] = reinterpret_cast<const uint32_t*>(blob + sec * qsec + (int64_t)n * (KD / 2)) + 4 * q4;
      }
    // scale/bias windows: thread -> (matrix, row, quarter of the window's 16
    // words); piece p of NPIECE covers rows [p*PR, (p+1)*PR) of every matrix
    const int gpr = KD / 64;
    constexpr int PR = NTH / 4 / NMAT;             // rows per piece and matrix
    constexpr int NPIECE = NTR / PR;               // pieces per window
    const int sb_m = tid / (NTH / NMAT), sb_r = (tid / 4) % PR, sb_qt = tid & 3;
    const uint32_t* sb_src = reinterpret_cast<const uint32_t*>(blob + 3 * qsec + (GU ? sb_m : 2) * ssec) +
                             (int64_t)(nt * NTR + sb_r) * gpr + 4 * sb_qt;
    auto load_sb = [&](int win, int piece) -> u32x4 {   // window win, piece piece
      const int w = min(win, (NC - 1) / kSbWin);
      const int g0 = w * 2 * kSbWin + 4 * sb_qt;          // first group of this thread's four
      const uint32_t* p = sb_src + (int64_t)piece * PR * gpr + w * 2 * kSbWin;
      if (g0 + 4 <= gpr) return load_keep(reinterpret_cast<const u32x4*>(p));
      u32x4 v = {0u, 0u, 0u, 0u};                          // rows shorter than a window
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (g0 + e < gpr) v[e] = load_keep(p + e);
      return v;
    };
    auto store_sb = [&](int buf, int piece, u32x4 v) {
      *reinterpret_cast<u32x4*>(&Sb[buf][sb_m][piece * PR + sb_r][4 * sb_qt]) = v;
    };

    // activation rows: thread -> (row, part of a 128-K chunk)
    constexpr int APR = NTH / kMT;                 // threads per row
    constexpr int AV = kKC / APR / 8;              // 16-byte vectors per thread
    const int arow = tid / APR, apart = tid % APR;
    const _Float16* asrc = GU ? a.xh + (int64_t)src_row[arow] * KD : a.abuf + (int64_t)src_row[arow] * KD;
    auto load_a = [&](int c, u32x4 (&v)[AV]) {
      const u32x4* p = reinterpret_cast<const u32x4*>(asrc + c * kKC + apart * (8 * AV));
#pragma unroll
      for (int i = 0; i < AV; ++i) v[i] = load_keep(p + i);
    };
    auto store_a = [&](int buf, const u32x4 (&v)[AV]) {
      u32x4* d = reinterpret_cast<u32x4*>(&As[buf][arow * kPitch + apart * (8 * AV)]);
#pragma unroll
      for (int i = 0; i < AV; ++i) d[i] = v[i];
    };

    // raw weights of one chunk: lane quarter q4 holds the four contiguous
    // words 4*q4 .. 4*q4+3 of the chunk's 16 (all in group 2c + q4/2, so one
    // scale/bias pair); MFMA k-step h takes word 4*q4 + h.  The weights are
    // fully dequantised, so a k-step may span two groups.
    struct Raw {
      u32x4 q[NMAT][kNBW];
    };
    Raw raw[NPF];
    auto load_w = [&](int c, Raw& r) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nb = 0; nb < kNBW; ++nb) r.q[m][nb] = load_keep(reinterpret_cast<const u32x4*>(qrow[m][nb] + 16 * c));
    };

    float4v acc[NMAT][kNBW][kMB];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nb = 0; nb < kNBW; ++nb)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) acc[m][nb][mb] = float4v{0.f, 0.f, 0.f, 0.f};

    // prologue: NPF chunks of weights and two chunks of activations in
    // flight, chunk 0 of activations in LDS.  Activations of chunk c+1 are
    // loaded a full chunk before they are stored, so waiting for them never
    // waits for the weight loads issued after them (loads complete in order).
    u32x4 an[2][AV];
#pragma unroll
    for (int j = 0; j < NPF; ++j) load_w(min(j, NC - 1), raw[j]);
    load_a(0, an[0]);
    load_a(min(1, NC - 1), an[1]);
    {
      u32x4 v[NPIECE];
#pragma unroll
      for (int p = 0; p < NPIECE; ++p) v[p] = load_sb(0, p);
#pragma unroll
      for (int p = 0; p < NPIECE; ++p) store_sb(0, p, v[p]);
    }
    store_a(0, an[0]);
    block_sync_lds();
    // the next window's pieces are loaded one per chunk (piece = chunk mod
    // NPIECE) and stored one chunk later; every piece is in place before
    // the window starts
    u32x4 sbn = load_sb(1, 0);

    for (int c0 = 0; c0 < NC; c0 += NPF) {
#pragma unroll
      for (int j = 0; j < NPF; ++j) {
        const int c = c0 + j;
        const int buf = c & 1;
        if (NPF % 2 == 0 ? (j & 1) == 0 : buf == 0) load_a(min(c + 2, NC - 1), an[0]);
        else load_a(min(c + 2, NC - 1), an[1]);
        const _Float16* A = &As[buf][0];
        const int wbuf = (c / kSbWin) & 1, wg = (2 * c + (q4 >> 1)) % (2 * kSbWin);
        half2v s2[NMAT][kNBW], b2[NMAT][kNBW];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int nb = 0; nb < kNBW; ++nb)
            sb_halves(Sb[wbuf][m][wave * (16 * kNBW) + nb * 16 + (lane & 15)][wg], s2[m][nb], b2[m][nb]);
        // dequantise one k-step at a time (fewer live registers)
#pragma unroll
        for (int hk = 0; hk < 4; ++hk) {
          half8 bw[NMAT][kNBW];
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int nb = 0; nb < kNBW; ++nb) bw[m][nb] = dequant_word(raw[j].q[m][nb][hk], s2[m][nb], b2[m][nb]);
          // every row block, padding rows included (they repeat a real
          // row and are not stored): no branch between the MFMAs, so the
          // independent accumulators hide each other's latency
          half8 af[kMB];   // all row blocks' fragments read before the first MFMA
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
            af[mb] = *reinterpret_cast<const half8*>(A + (mb * 16 + (lane & 15)) * kPitch + 8 * (4 * q4 + hk));
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int nb = 0; nb < kNBW; ++nb)
                acc[m][nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mb], bw[m][nb], acc[m][nb][mb], 0, 0, 0);
          }
        }
        load_w(min(c + NPF, NC - 1), raw[j]);
        // scale/bias: store the piece loaded last chunk, load the next one
        store_sb(((c / kSbWin) + 1) & 1, c % NPIECE, sbn);
        sbn = load_sb((c + 1) / kSbWin + 1, (c + 1) % NPIECE);
        if (NPF % 2 == 0 ? (j & 1) == 0 : buf == 0) store_a(buf ^ 1, an[1]);
        else store_a(buf ^ 1, an[0]);
        block_sync_lds();
      }
    }

    // epilogue: lane holds weight row n = ... + (lane & 15), rows 4*(lane>>4)+i of each block
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb) {
      const int n = nt * NTR + wave * (16 * kNBW) + nb * 16 + (lane & 15);
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mb * 16 + 4 * q4 + i;
          if (r < nrows) {
            const int p = dst_row[r];
            if constexpr (GU) {
              const float gv = acc[0][nb][mb][i], uv = acc[1 % NMAT][nb][mb][i];
              a.abuf[(int64_t)p * a.I + perm_pos(n)] = (_Float16)(gv / (1.0f + __expf(-gv)) * uv);
            } else {
              a.dbuf[(int64_t)p * a.H + n] = acc[0][nb][mb][i];
            }
          }
        }
      }
    }
    __syncthreads();   // row tables and LDS reused by the next tile
  }
}

// ------------------------------------------------- down GEMM, resident A
// The down GEMM with the pairs' activation tile resident in LDS: a block
// takes one row tile (up to 64 pairs of one expert) and a run of TG weight
// tiles of 256 rows; the tile's activations (64 x I fp16) are read once and
// every weight tile of the run streams against them, with no block barrier
// in the K loop.  Weights and their scale/bias words are prefetched NPF
// chunks ahead, across the weight tiles of the run.  I <= kResMaxI.
constexpr int kResMaxI = 1024;
constexpr int kResThreads = 512;
constexpr int kResUnits = kMT * kResMaxI / 8 / kResThreads;   // 16-byte activation units per thread

template <int NPF, int TG>
__global__ __launch_bounds__(kResThreads, 1) void down_resident_kernel(GemmArgs a) {
  constexpr int NTR = (kResThreads / 64) * 16 * kNBW;   // weight rows per tile: 256
  extern __shared__ __align__(16) _Float16 Ar[];        // [kMT][I + 8]
  __shared__ int32_t src_row[kMT];
  __shared__ int s_e, s_row0, s_n;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4;
  const int E = a.E, S = a.S, H = a.H, I = a.I;
  const int pitch = I + 8;
  const int NC = I / kKC;                  // chunks per weight tile
  const int NT = H / NTR;                  // weight tiles
  const int NG = (NT + TG - 1) / TG;       // runs per row tile
  const int n_mt = a.mtoff[E + S];
  const int total = n_mt * NG;
  const int64_t qsec = (int64_t)H * I / 2, ssec = (int64_t)H * I / 64 * 4;

  for (int wi = blockIdx.x; wi < total; wi += gridDim.x) {
    const int mt = wi / NG, nt0 = (wi % NG) * TG;
    const int ntn = min(TG, NT - nt0);
    if (tid == 0) {
      const int4 tl = a.tiles[mt];
      s_e = tl.x;
      s_row0 = tl.y;
      s_n = tl.z;
    }
    __syncthreads();
    const int e = s_e, nrows = s_n, row0 = s_row0;
    if (tid < kMT) src_row[tid] = a.lists[row0 + min(tid, nrows - 1)];   // padding rows repeat a real row
    const uint8_t* blob = uniform_ptr(static_cast<const uint8_t*>(a.blobs[e]));
    __syncthreads();
    if (blob == nullptr) {   // missing expert: flag it, leave its outputs unwritten
      if (tid == 0) set_status(a.status, 1);
      continue;
    }
    // activation tile: every 16-byte unit requested before any is stored
    const int upr = I / 8;   // units per row
    u32x4 av[kResUnits];
#pragma unroll
    for (int i = 0; i < kResUnits; ++i) {
      const int x = min(tid + i * kResThreads, kMT * upr - 1);
      const int r = x / upr, u = x - r * upr;
      av[i] = load_keep(reinterpret_cast<const u32x4*>(a.abuf + (int64_t)src_row[r] * I) + u);
    }

    // weights: flat chunk f = t * NC + c over the run's tiles; lane quarter
    // q4 holds words 4*q4 .. 4*q4+3 of the chunk's 16 (group 2c + q4/2)
    struct Raw {
      u32x4 q[kNBW];
      uint32_t sb[kNBW];
    };
    Raw raw[NPF];
    const int nf = ntn * NC;
    const uint8_t* dq = blob + 2 * qsec;
    const uint32_t* dsb = reinterpret_cast<const uint32_t*>(blob + 3 * qsec + 2 * ssec);
    auto load_w = [&](int f, Raw& r) {
      f = min(f, nf - 1);
      const int t = f / NC, c = f - t * NC;
#pragma unroll
      for (int nb = 0; nb < kNBW; ++nb) {
        const int n = (nt0 + t) * NTR + wave * (16 * kNBW) + nb * 16 + (lane & 15);
        r.q[nb] = load_keep(reinterpret_cast<const u32x4*>(dq + (int64_t)n * (I / 2)) + 4 * c + q4);
        r.sb[nb] = load_keep(dsb + (int64_t)n * (I / 64) + 2 * c + (q4 >> 1));
      }
    };
#pragma unroll
    for (int j = 0; j < NPF; ++j) load_w(j, raw[j]);
#pragma unroll
    for (int i = 0; i < kResUnits; ++i) {
      const int x = tid + i * kResThreads;
      if (x < kMT * upr) {
        const int r = x / upr, u = x - r * upr;
        *reinterpret_cast<u32x4*>(&Ar[r * pitch + 8 * u]) = av[i];
      }
    }
    block_sync_lds();

    float4v acc[kNBW][kMB];
#pragma unroll
    for (int nb = 0; nb < kNBW; ++nb)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) acc[nb][mb] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int f0 = 0; f0 < nf; f0 += NPF) {   // NPF divides NC
#pragma unroll
      for (int j = 0; j < NPF; ++j) {
        const int f = f0 + j;
        const int t = f / NC, c = f - t * NC;
        half2v s2[kNBW], b2[kNBW];
#pragma unroll
        for (int nb = 0; nb < kNBW; ++nb) sb_halves(raw[j].sb[nb], s2[nb], b2[nb]);
        // activation fragments of every row block (see gemm_kernel), one
        // k-step ahead: the reads of step hk+1 are in flight while step hk's
        // MFMAs run, and one wait covers a step's four reads
        const _Float16* arow = &Ar[(lane & 15) * pitch + c * kKC + 8 * (4 * q4)];
        half8 af[2][kMB];
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) af[0][mb] = *reinterpret_cast<const half8*>(arow + mb * 16 * pitch);
#pragma unroll
        for (int hk = 0; hk < 4; ++hk) {
          if (hk < 3) {
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
              af[(hk + 1) & 1][mb] = *reinterpret_cast<const half8*>(arow + mb * 16 * pitch + 8 * (hk + 1));
          }
          half8 bw[kNBW];
#pragma unroll
          for (int nb = 0; nb < kNBW; ++nb) bw[nb] = dequant_word(raw[j].q[nb][hk], s2[nb], b2[nb]);
          const half8 (&cur)[kMB] = af[hk & 1];
          asm volatile("" ::"v"(cur[0]), "v"(cur[1]), "v"(cur[2]), "v"(cur[3]) : "memory");
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int nb = 0; nb < kNBW; ++nb)
              acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur[mb], bw[nb], acc[nb][mb], 0, 0, 0);
        }
        load_w(f + NPF, raw[j]);
        if (c == NC - 1) {   // tile t done: lane holds weight row n, pairs 4*(lane>>4)+i of each block
#pragma unroll
          for (int nb = 0; nb < kNBW; ++nb) {
            const int n = (nt0 + t) * NTR + wave * (16 * kNBW) + nb * 16 + (lane & 15);
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int r = mb * 16 + 4 * q4 + i;
                if (r < nrows) a.dbuf[(int64_t)src_row[r] * H + n] = acc[nb][mb][i];
              }
              acc[nb][mb] = float4v{0.f, 0.f, 0.f, 0.f};
            }
          }
        }
      }
    }
    __syncthreads();   // row table and LDS reused by the next item
  }
}

// --------------------------------------------------------------- combine
// h[t][i] += sum_{s<K} w[t][s] d[t][s][i] + sum_shared d[t][K+j][i], in
// slot order, one fma per term.
__global__ __launch_bounds__(kPThreads) void combine_kernel(float* __restrict__ h, const float* __restrict__ dbuf,
                                                             const float* __restrict__ w, int K, int S, int H) {
  const int t = blockIdx.x, KS = K + S;
  const float* d = dbuf + (int64_t)t * KS * H;
  for (int i = threadIdx.x; i < H; i += kPThreads) {
    float acc = h[(int64_t)t * H + i];
    for (int s = 0; s < K; ++s) acc = fmaf(w[(int64_t)t * K + s], d[(int64_t)s * H + i], acc);
    for (int s = K; s < KS; ++s) acc = fmaf(1.0f, d[(int64_t)s * H + i], acc);
    h[(int64_t)t * H + i] = acc;
  }
}

// Tiles of 256 weight rows (eight waves) when the rows divide into them: one
// activation chunk then feeds twice the weights.  Gate/up keeps two chunks
// of weights in flight (it holds two matrices per chunk), down four.
template <bool GU, int NW>
void launch_gemm_w(const GemmArgs& g, int nc, int grid, hipStream_t st) {
  constexpr int NPF_MAX = GU ? 2 : 4;
  if (NPF_MAX >= 4 && nc % 4 == 0)
    hipLaunchKernelGGL((gemm_kernel<GU, NPF_MAX, NW>), dim3(grid), dim3(64 * NW), 0, st, g);
  else if (nc % 2 == 0) hipLaunchKernelGGL((gemm_kernel<GU, 2, NW>), dim3(grid), dim3(64 * NW), 0, st, g);
  else hipLaunchKernelGGL((gemm_kernel<GU, 1, NW>), dim3(grid), dim3(64 * NW), 0, st, g);
}

template <bool GU>
hipError_t launch_gemm(const GemmArgs& g, int nc, int cus, hipStream_t st) {
  const int nr = GU ? g.I : g.H;
  const int xcd_cus = max(8, cus / 8 * 8);
  if (nr % (8 * 16 * kNBW) == 0) launch_gemm_w<GU, 8>(g, nc, xcd_cus, st);
  else launch_gemm_w<GU, 4>(g, nc, 2 * xcd_cus, st);
  return hipGetLastError();
}

// Down GEMM: resident activation tiles where the tile fits in LDS and the
// weight rows divide into 256-row tiles; otherwise the streamed form.
hipError_t launch_down(const GemmArgs& g, int cus, hipStream_t st) {
  constexpr int TG = 4, NPF = 4;
  const int NC = g.I / kKC;
  if (g.I <= kResMaxI && g.H % 256 == 0 && NC % NPF == 0) {
    const size_t lds = sizeof(_Float16) * (size_t)kMT * (g.I + 8);
    static const bool lds_ok =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&down_resident_kernel<NPF, TG>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(sizeof(_Float16) * kMT * (kResMaxI + 8))) == hipSuccess;
    if (lds_ok) {
      hipLaunchKernelGGL((down_resident_kernel<NPF, TG>), dim3(max(1, cus)), dim3(kResThreads), lds, st, g);
      return hipGetLastError();
    }
    (void)hipGetLastError();
  }
  return launch_gemm<false>(g, NC, cus, st);
}

int device_cus_prefill() {
  static int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
  }();
  return n;
}

// Optional per-kernel-class event pairs on the launch stream (diagnostic
// timing of the prefill kernels).
enum { kTNorm, kTRouter, kTTopk, kTGroup, kTGateUp, kTDown, kTCombine, kTClasses };
struct PrefillTimer {
  bool on = false;
  std::vector<hipEvent_t> start[kTClasses], stop[kTClasses];
  void mark(std::vector<hipEvent_t>* v, hipStream_t st) {
    if (!on) return;
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return;
    if (hipEventRecord(e, st) != hipSuccess) {
      (void)hipEventDestroy(e);
      return;
    }
    v->push_back(e);
  }
  void begin(int c, hipStream_t st) { mark(&start[c], st); }
  void end(int c, hipStream_t st) { mark(&stop[c], st); }
  void clear() {
    for (int c = 0; c < kTClasses; ++c) {
      for (hipEvent_t e : start[c]) (void)hipEventDestroy(e);
      for (hipEvent_t e : stop[c]) (void)hipEventDestroy(e);
      start[c].clear();
      stop[c].clear();
    }
  }
};
PrefillTimer g_timer;

}  // namespace

PrefillLayout prefill_layout(const moeq_shape& s, int T, int k) {
  PrefillLayout p;
  const int64_t KS = (int64_t)k + s.n_shared, P = (int64_t)T * KS, n = s.n_experts + s.n_shared;
  p.status = 0;
  p.inv = 256;
  p.xh = p.inv + align_up((int64_t)T * 8);
  p.logits = p.xh + align_up((int64_t)T * s.hidden * 2);
  p.idx = p.logits + align_up((int64_t)T * s.n_experts * 8);
  p.w = p.idx + align_up((int64_t)T * k * 4);
  p.counts = p.w + align_up((int64_t)T * k * 4);
  p.offs = p.counts + align_up(n * 4);
  p.mtoff = p.offs + align_up((n + 1) * 4);
  p.tiles = p.mtoff + align_up((n + 1) * 4);
  p.lists = p.tiles + align_up((P / kMT + n + 1) * 16);
  p.abuf = p.lists + align_up(P * 4);
  p.dbuf = p.abuf + align_up(P * s.inter * 2);
  p.total = p.dbuf + align_up(P * s.hidden * 4);
  return p;
}

hipError_t launch_prefill_layer(const moeq_shape& s, const void* const* blobs, const uint16_t* const* routers,
                                int layer, int T, int k, uint32_t flags, float* h, int32_t* trace,
                                char* ws, hipStream_t st) {
  const PrefillLayout W = prefill_layout(s, T, k);
  const int E = s.n_experts, S = s.n_shared, H = s.hidden, I = s.inter, KS = k + S;
  double* inv = reinterpret_cast<double*>(ws + W.inv);
  _Float16* xh = reinterpret_cast<_Float16*>(ws + W.xh);
  double* logits = reinterpret_cast<double*>(ws + W.logits);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + W.idx);
  float* w = reinterpret_cast<float*>(ws + W.w);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + W.counts);
  int32_t* offs = reinterpret_cast<int32_t*>(ws + W.offs);
  int32_t* mtoff = reinterpret_cast<int32_t*>(ws + W.mtoff);
  int4* tiles = reinterpret_cast<int4*>(ws + W.tiles);
  int32_t* lists = reinterpret_cast<int32_t*>(ws + W.lists);
  int32_t* status = reinterpret_cast<int32_t*>(ws + W.status);

  PrefillTimer& tm = g_timer;
  tm.begin(kTNorm, st);
  hipLaunchKernelGGL(norm_kernel, dim3(T), dim3(kPThreads), 0, st, h, H, inv, xh, counts, E);
  tm.end(kTNorm, st);
  tm.begin(kTRouter, st);
  hipLaunchKernelGGL(router_kernel, dim3((T + kRT - 1) / kRT, (E + kRT - 1) / kRT), dim3(kPThreads), 0, st, h,
                     routers, layer, T, H, E, inv, logits);
  tm.end(kTRouter, st);
  const int nr = (flags & MOEQ_F_NO_RENORM) ? 1 : 0;
  tm.begin(kTTopk, st);
  if (E <= 512)
    hipLaunchKernelGGL(topk_kernel<2>, dim3(T), dim3(kPThreads), 0, st, logits, E, k, nr, idx, w, trace);
  else
    hipLaunchKernelGGL(topk_kernel<16>, dim3(T), dim3(kPThreads), 0, st, logits, E, k, nr, idx, w, trace);
  tm.end(kTTopk, st);
  tm.begin(kTGroup, st);
  hipLaunchKernelGGL(count_kernel, dim3((T * k + 255) / 256), dim3(256), 0, st, idx, T * k, E, counts, status);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, E, S, T, offs, mtoff, tiles);
  hipLaunchKernelGGL(compact_kernel, dim3(E + S), dim3(kPThreads), 0, st, idx, T, k, S, E, offs, lists);
  tm.end(kTGroup, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  GemmArgs g{};
  g.blobs = blobs + (int64_t)layer * (E + S);
  g.E = E; g.S = S; g.K = k; g.H = H; g.I = I;
  g.offs = offs; g.mtoff = mtoff; g.tiles = tiles; g.lists = lists;
  g.xh = xh;
  g.abuf = reinterpret_cast<_Float16*>(ws + W.abuf);
  g.dbuf = reinterpret_cast<float*>(ws + W.dbuf);
  g.status = status;
  const int cus = device_cus_prefill();
  tm.begin(kTGateUp, st);
  if ((e = launch_gemm<true>(g, H / kKC, cus, st)) != hipSuccess) return e;
  tm.end(kTGateUp, st);
  tm.begin(kTDown, st);
  if ((e = launch_down(g, cus, st)) != hipSuccess) return e;
  tm.end(kTDown, st);
  tm.begin(kTCombine, st);
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(kPThreads), 0, st, h, g.dbuf, w, k, S, H);
  tm.end(kTCombine, st);
  (void)KS;
  return hipGetLastError();
}

}  // namespace moeq

using namespace moeq;

extern "C" {

int moeq_prefill_timing(int enable) {
  g_timer.clear();
  g_timer.on = enable != 0;
  return ok();
}

int moeq_prefill_timing_read(double* ms, int32_t* launches) {
  if (!ms || !launches) return fail(MOEQ_E_INVALID, "ms and launches must be non-NULL");
  for (int c = 0; c < kTClasses; ++c) {
    ms[c] = 0.0;
    launches[c] = 0;
    const size_t n = g_timer.start[c].size() < g_timer.stop[c].size() ? g_timer.start[c].size()
                                                                        : g_timer.stop[c].size();
    for (size_t i = 0; i < n; ++i) {
      hipError_t e = hipEventSynchronize(g_timer.stop[c][i]);
      if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize (prefill timing)");
      float t = 0.f;
      e = hipEventElapsedTime(&t, g_timer.start[c][i], g_timer.stop[c][i]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime (prefill timing)");
      ms[c] += t;
      ++launches[c];
    }
  }
  g_timer.clear();
  return ok();
}

int moeq_prefill_workspace_bytes(const moeq_shape* s, int T, int k, int64_t* bytes) {
  if (int rc = check_shape(s)) return rc;
  if (!bytes) return fail(MOEQ_E_INVALID, "bytes is NULL");
  if (T < 0 || k < 0) return fail(MOEQ_E_INVALID, "T=%d k=%d must be non-negative", T, k);
  *bytes = prefill_layout(*s, T, k).total;
  return ok();
}

int moe_expert_stack_prefill(const moeq_shape* s, const moeq_experts* ex, const uint16_t* const* w_router,
                             int layer0, int L, int T, int k, uint32_t flags, float* h, int32_t* topk_trace,
                             void* workspace, void* stream) {
  if (int rc = check_shape(s)) return rc;
  if (s->bits != 4) return fail(MOEQ_E_UNSUPPORTED, "prefill is implemented for 4-bit experts (bits=%d)", s->bits);
  if (s->hidden % kKC || s->inter % kNT || s->hidden % kNT)
    return fail(MOEQ_E_UNSUPPORTED, "prefill needs hidden and inter multiples of %d (hidden=%d inter=%d)", kNT,
                s->hidden, s->inter);
  if (T < 0 || L < 0 || layer0 < 0) return fail(MOEQ_E_INVALID, "T=%d L=%d layer0=%d must be >= 0", T, L, layer0);
  if (k < 1 || k > s->n_experts || k > MOEQ_MAX_TOPK)
    return fail(k > MOEQ_MAX_TOPK ? MOEQ_E_UNSUPPORTED : MOEQ_E_INVALID, "k=%d outside [1, min(E, %d)]", k,
                MOEQ_MAX_TOPK);
  if ((int64_t)T * (k + s->n_shared) > INT_MAX / 2 || (int64_t)T * s->n_experts > INT_MAX / 2)
    return fail(MOEQ_E_UNSUPPORTED, "T=%d too large", T);
  if (flags & ~(uint32_t)MOEQ_F_NO_RENORM) return fail(MOEQ_E_UNSUPPORTED, "flags 0x%x: only MOEQ_F_NO_RENORM", flags);
  if (T == 0 || L == 0) return ok();
  if (!ex || !ex->blobs || !w_router || !h || !workspace)
    return fail(MOEQ_E_INVALID, "experts, w_router, h and workspace must be non-NULL");
  if (layer0 + L > ex->n_layers)
    return fail(MOEQ_E_INVALID, "layers [%d, %d) exceed the table's %d", layer0, layer0 + L, ex->n_layers);
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int l = 0; l < L; ++l) {
    int32_t* tr = topk_trace ? topk_trace + (int64_t)l * T * k : nullptr;
    const hipError_t e = launch_prefill_layer(*s, ex->blobs, w_router, layer0 + l, T, k, flags, h, tr,
                                              static_cast<char*>(workspace), st);
    if (e != hipSuccess) return hip_fail(e, "prefill layer launch");
  }
  return ok();
}

}  // extern "C"

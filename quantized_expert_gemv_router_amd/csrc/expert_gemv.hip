// Gate and up projections of the selected experts and the shared expert:
// group-wise affine 4-bit / 3-bit / 2-bit dequantised mat-vec (Flash-MoE,
// fr.news.hada.io, "Noyau de déquantification optimisé FMA" and "Shaders de
// calcul Metal").  For row r of [gate; up] and token t:
//   y[r] = sum_g ( s[r,g] * sum_{j in g} q[r,j] x[t,j] + b[r,g] * sum_{j in g} x[t,j] )
//
// Gate rows and up rows are contiguous in the blob, so the [gate; up] block
// is addressed as 2I rows of one matrix.  Every selected expert of the batch
// and the shared expert are handled in one launch; two grid shapes:
//  - one token: one workgroup per (slot, block of 4*RPW rows).  Each wave
//    requests its RPW rows with 16-byte non-temporal loads into registers
//    as soon as its slot's expert is known (no grouping: one token's slots
//    are separate outputs), stages the token into LDS as
//    fp16 pairs while those loads are in flight, then produces one
//    wave-wide sum per row;
//  - several tokens: one workgroup per (chunk of 4 of the expert's tokens,
//    expert item, range of rows), sized so the first chunks give a few
//    workgroups per CU; an expert that many tokens chose (the shared one,
//    or a popular routed one) thus spreads over as many more workgroups.
//    The workgroup finds its expert and stages its tokens once, then
//    streams its rows in tiles of 16 rows, double-buffered in registers:
//    the loads of tile j + 1 are in flight while tile j is applied to every
//    staged token (4-bit: each row's chunk dequantised once for all of
//    them).  Loads are range-checked buffer loads, so rows past the range
//    read as zeros without touching memory.
#include <cstdlib>

#include "grouping.hpp"
#include "moeq_internal.hpp"
#include "staging.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTokensPerStage = 4;

template <int BITS, int CPL, int RPW, int WMAX, int MMAX>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a, int n_rb, int list_words) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ GroupLds g;
  __shared__ float red[2 * kTokensPerStage * kWaves];
  __shared__ float undo[kTokensPerStage];
  constexpr int PC = Pack<BITS>::kPerChunk;
  constexpr int RPB = kWaves * RPW;
  const int item = blockIdx.x / n_rb, rb = blockIdx.x - item * n_rb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I, KS = a.k + a.S;
  const int nch = H / PC;
  const int P = a.T * a.k;
  // dynamic LDS: pairs [4][H/2] | xsum [4][kChunkSums * nch] | list | ids | ptrs
  uint32_t* pairs = smem;
  float* xsum = reinterpret_cast<float*>(pairs + kTokensPerStage * (H / 2));
  uint32_t* list = reinterpret_cast<uint32_t*>(xsum + kTokensPerStage * kChunkSums * nch);
  int* ids = reinterpret_cast<int*>(list + list_words);
  const uint8_t** ptrs = reinterpret_cast<const uint8_t**>(ids + list_words);

  if constexpr (MMAX == 1) group_single(item, a.topk_idx, a.blobs, a.k, a.E, a.S, g, list, a.status);
  else group_item(item, a.topk_idx, a.blobs, a.T, a.k, a.E, a.S, g, list, ids, ptrs, a.status);
  if (g.expert < 0) return;
  const uint8_t* blob = g.blob;
  (void)P;

  const int64_t row_bytes = (int64_t)H * BITS / 8;
  const int gpr = H / 64;   // scale/bias groups per row
  const uint32_t* sb = reinterpret_cast<const uint32_t*>(blob + 3 * (int64_t)H * I * BITS / 8);
  const int row0 = rb * RPB + wave * RPW;

  u32x4 q[RPW][CPL];
  uint2 qh[RPW][CPL];   // 3-bit: the chunk's high-bit plane
  uint32_t sbw[RPW][CPL];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int r = row0 + i;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int cc = lane + 64 * c;
      qh[i][c] = make_uint2(0u, 0u);
      if (r < 2 * I && cc < nch) {
        q[i][c] = load_stream(reinterpret_cast<const u32x4*>(blob + r * row_bytes) + cc);
        if constexpr (BITS == 3) qh[i][c] = load_stream_u2(blob + r * row_bytes + H / 4 + 8 * cc);
        sbw[i][c] = load_stream(sb + (int64_t)r * gpr + (cc * PC) / 64);
      } else {
        q[i][c] = u32x4{0u, 0u, 0u, 0u};
        sbw[i][c] = 0u;
      }
    }
  }

  for (int m0 = 0; m0 < g.count; m0 += MMAX) {
    const int nv = min(MMAX, g.count - m0);
    auto loader = [&](int m, int64_t o, float* v) {
      const int t = (int)(list[m0 + m] >> 8);
      load_act<Pack<BITS>::kPerWord>(a.x, a.x_f32, (int64_t)t * H + o, v);
    };
    stage_batch<BITS, WMAX, MMAX>(nv, H, loader, a.rmsnorm != 0, pairs, xsum, undo, red);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = row0 + i;
      if (r >= 2 * I) break;
      for (int m = 0; m < nv; ++m) {
        const uint32_t* xp = pairs + (int64_t)m * (H / 2);
        const float* xs = xsum + (int64_t)m * kChunkSums * nch;
        float part = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int cc = lane + 64 * c;
          if (cc < nch)
            part += chunk_term<BITS>(chunk_dot_q<BITS>(q[i][c], qh[i][c], load_xchunk<BITS>(xp, cc, nch)), sbw[i][c],
                                     *reinterpret_cast<const float2*>(xs + kChunkSums * cc));
        }
        const float v = wave_sum_dpp(part) * undo[m];
        if (lane == 0) {
          const uint32_t e = list[m0 + m];
          const int t = (int)(e >> 8), slot = (int)(e & 255u);
          const int sec = r >= I ? 1 : 0;
          a.gate_up[(((int64_t)t * KS + slot) * 2 + sec) * I + (r - sec * I)] = v;
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------ several tokens
constexpr int kBatchRPW = 4;                      // rows per wave per tile
constexpr int kTileRows = kWaves * kBatchRPW;     // rows per tile

template <int BITS, int CPL>
struct GuTile {
  u32x4 q[kBatchRPW][CPL];
  uint2 qh[kBatchRPW][CPL];   // 3-bit: the chunk's high-bit plane
  uint32_t sb[kBatchRPW][CPL];
};

// Tile `j` of this wave's rows: row = r_lo + j * kTileRows + wave * kBatchRPW + i.
// Rows at or past r_hi (and lanes past the last chunk) read at offset
// q_bytes / s_bytes, the end of the buffer's range: zeros, and no memory
// request.
template <int BITS, int CPL>
__device__ __forceinline__ void issue_gu_tile(GuTile<BITS, CPL>& t, rsrc_t rq, rsrc_t rs, uint32_t q_bytes,
                                              uint32_t s_bytes, int j, int r_lo, int r_hi, int row_bytes,
                                              int gpr, int nch, int wave, int lane_in) {
  constexpr int PC = Pack<BITS>::kPerChunk;
  int lane;   // re-derived per tile: its offsets are not kept live across the loop
  asm volatile("v_mov_b32 %0, %1" : "=v"(lane) : "v"(lane_in));
#pragma unroll
  for (int i = 0; i < kBatchRPW; ++i) {
    const int r = r_lo + j * kTileRows + wave * kBatchRPW + i;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int cc = lane + 64 * c;
      const bool ok = r < r_hi && cc < nch;
      const uint32_t qo = ok ? (uint32_t)r * (uint32_t)row_bytes + 16u * (uint32_t)cc : q_bytes;
      const uint32_t so = ok ? 4u * ((uint32_t)r * (uint32_t)gpr + (uint32_t)(cc * PC / 64)) : s_bytes;
      t.q[i][c] = load_rsrc_b128(rq, qo);
      if constexpr (BITS == 3) {
        // the high-bit plane follows the low plane (2/3 of the row's bytes)
        const uint32_t ho = ok ? (uint32_t)r * (uint32_t)row_bytes + (uint32_t)(2 * row_bytes / 3) + 8u * (uint32_t)cc
                               : q_bytes;
        t.qh[i][c] = load_rsrc_b64(rq, ho);
      } else {
        t.qh[i][c] = make_uint2(0u, 0u);
      }
      t.sb[i][c] = load_rsrc_b32(rs, so);
    }
  }
  issue_fence();
}

// 4-bit chunk dequantised once into its 16 magic-exponent fp16 pairs (the
// operands chunk_dot forms, in the same order), then dotted with any number
// of staged chunks: the dequant is paid once per row, not once per token.
struct DqChunk4 {
  uint32_t p[16];
};
__device__ __forceinline__ DqChunk4 dequant_chunk4(u32x4 q) {
  DqChunk4 d;
  const uint32_t mg = magic_pair();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = q[i], t = w >> 8;
    d.p[4 * i + 0] = (w & 0x000F000Fu) | mg;
    d.p[4 * i + 1] = (w & 0x00F000F0u) | mg;
    d.p[4 * i + 2] = (t & 0x000F000Fu) | mg;
    d.p[4 * i + 3] = (t & 0x00F000F0u) | mg;
  }
  return d;
}
__device__ __forceinline__ float dot_chunk4(const DqChunk4& d, const XChunk<4>& x) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = dot2(d.p[4 * i + 0], x.u[i].x, acc);
    acc = dot2(d.p[4 * i + 1], x.u[i].y, acc);
    acc = dot2(d.p[4 * i + 2], x.u[i].z, acc);
    acc = dot2(d.p[4 * i + 3], x.u[i].w, acc);
  }
  return acc;
}

// Applies tile j to the nv staged tokens (list entries m0..m0+nv).
template <int BITS, int CPL, int MMAX>
__device__ __forceinline__ void apply_gu_tile(const GuTile<BITS, CPL>& t, const GemvArgs& a, int j, int r_lo,
                                              int r_hi, int nv, int m0, const uint32_t* pairs,
                                              const float* xsum, const float* undo, const uint32_t* list,
                                              int nch, int wave, int lane_in) {
  const int H = a.H, I = a.I, KS = a.k + a.S;
  // the lane index re-derived per tile, so the LDS addresses built from it
  // are recomputed here rather than hoisted out of the tile loop, where
  // they would hold dozens of registers for the kernel's lifetime
  int lane;
  asm volatile("v_mov_b32 %0, %1" : "=v"(lane) : "v"(lane_in));
  float part[kBatchRPW][MMAX];
#pragma unroll
  for (int i = 0; i < kBatchRPW; ++i)
#pragma unroll
    for (int m = 0; m < MMAX; ++m) part[i][m] = 0.0f;
  if constexpr (BITS == 4) {
    // chunk-major: every staged token's chunk c, then each row's chunk c
    // dequantised once and applied to all of them
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int cc = lane + 64 * c;
      if (cc < nch) {
        XChunk<4> xc[MMAX];
        float2 x2[MMAX];
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
          if (m < nv) {
            xc[m] = load_xchunk<4>(pairs + (int64_t)m * (H / 2), cc, nch);
            x2[m] = *reinterpret_cast<const float2*>(xsum + (int64_t)m * kChunkSums * nch + kChunkSums * cc);
          }
        }
#pragma unroll
        for (int i = 0; i < kBatchRPW; ++i) {
          const DqChunk4 d = dequant_chunk4(t.q[i][c]);
#pragma unroll
          for (int m = 0; m < MMAX; ++m)
            if (m < nv) part[i][m] += chunk_affine(dot_chunk4(d, xc[m]), t.sb[i][c], x2[m]);
        }
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < MMAX; ++m) {
      if (m < nv) {
        const uint32_t* xp = pairs + (int64_t)m * (H / 2);
        const float* xs = xsum + (int64_t)m * kChunkSums * nch;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int cc = lane + 64 * c;
          if (cc < nch) {
            const XChunk<BITS> xc = load_xchunk<BITS>(xp, cc, nch);
            const float2 x2 = *reinterpret_cast<const float2*>(xs + kChunkSums * cc);
#pragma unroll
            for (int i = 0; i < kBatchRPW; ++i)
              part[i][m] += chunk_term<BITS>(chunk_dot_q<BITS>(t.q[i][c], t.qh[i][c], xc), t.sb[i][c], x2);
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MMAX; ++m) {
    if (m < nv) {
      const uint32_t e = list[m0 + m];
      const int tk = (int)(e >> 8), slot = (int)(e & 255u);
      const float u = undo[m];
#pragma unroll
      for (int i = 0; i < kBatchRPW; ++i) {
        const float v = wave_sum_dpp(part[i][m]) * u;
        const int r = r_lo + j * kTileRows + wave * kBatchRPW + i;
        if (lane == 0 && r < r_hi) {
          const int sec = r >= I ? 1 : 0;
          a.gate_up[(((int64_t)tk * KS + slot) * 2 + sec) * I + (r - sec * I)] = v;
        }
      }
    }
  }
}

// Grid, NS row ranges per unit: first the n_extra units that may hold a
// later token chunk (tokens 4c.. of an item's list, c >= 1; group_extra
// finds which, the rest exit), then chunk 0 of the n_routed routed items
// and the S shared experts (items missing from this batch exit).
template <int BITS, int CPL, int WMAX>
__global__ __launch_bounds__(kThreads) void gemv_batch_kernel(GemvArgs a, int NS, int n_routed, int n_extra,
                                                                                     int list_words) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ GroupLds g;
  __shared__ float red[2 * kTokensPerStage * kWaves];
  __shared__ float undo[kTokensPerStage];
  constexpr int MMAX = kTokensPerStage;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I;
  const int nch = H / Pack<BITS>::kPerChunk;
  uint32_t* pairs = smem;
  float* xsum = reinterpret_cast<float*>(pairs + kTokensPerStage * (H / 2));
  uint32_t* list = reinterpret_cast<uint32_t*>(xsum + kTokensPerStage * kChunkSums * nch);
  int* ids = reinterpret_cast<int*>(list + list_words);
  const uint8_t** ptrs = reinterpret_cast<const uint8_t**>(ids + list_words);

  uint32_t* hist = reinterpret_cast<uint32_t*>(ptrs + list_words);
  int split;
  if ((int)blockIdx.x < n_extra * NS) {   // later token chunks first: they run long
    const int u = blockIdx.x / NS;
    split = blockIdx.x - u * NS;
    group_extra<MMAX>(u, a.topk_idx, a.blobs, a.T, a.k, a.E, a.S, g, list, ids, ptrs, hist, a.status);
  } else {
    const int b = blockIdx.x - n_extra * NS;
    const int it = b / NS;
    split = b - it * NS;
    const int item = it < n_routed ? it : -1 - (it - n_routed);
    group_item(item, a.topk_idx, a.blobs, a.T, a.k, a.E, a.S, g, list, ids, ptrs, a.status);
  }
  if (g.expert < 0) return;
  const int m0 = g.chunk * MMAX;
  if (m0 >= g.count) return;
  const int nv = min(MMAX, g.count - m0);

  // this workgroup's rows: whole tiles, split as evenly as the tiles allow
  const int rows = 2 * I;
  const int ntiles = (rows + kTileRows - 1) / kTileRows;
  const int t_lo = (int)((int64_t)ntiles * split / NS), t_hi = (int)((int64_t)ntiles * (split + 1) / NS);
  if (t_lo >= t_hi) return;
  const int r_lo = t_lo * kTileRows, r_hi = min(rows, t_hi * kTileRows);
  const int nt = t_hi - t_lo;

  const int row_bytes = H * BITS / 8;
  const int gpr = H / 64;
  const uint8_t* blob = g.blob;
  const uint32_t q_bytes = (uint32_t)rows * (uint32_t)row_bytes, s_bytes = (uint32_t)rows * (uint32_t)gpr * 4u;
  const rsrc_t rq = make_rsrc(blob, q_bytes);
  const rsrc_t rs = make_rsrc(blob + 3 * (int64_t)H * I * BITS / 8, s_bytes);

  auto loader = [&](int m, int64_t o, float* v) {
    const int t = (int)(list[m0 + m] >> 8);
    load_act<Pack<BITS>::kPerWord>(a.x, a.x_f32, (int64_t)t * H + o, v);
  };
  stage_batch<BITS, WMAX, MMAX>(nv, H, loader, a.rmsnorm != 0, pairs, xsum, undo, red);

  GuTile<BITS, CPL> ta, tb;
  issue_gu_tile<BITS, CPL>(ta, rq, rs, q_bytes, s_bytes, 0, r_lo, r_hi, row_bytes, gpr, nch, wave, lane);
  for (int j = 0; j < nt; j += 2) {
    issue_gu_tile<BITS, CPL>(tb, rq, rs, q_bytes, s_bytes, j + 1, r_lo, r_hi, row_bytes, gpr, nch, wave, lane);
    apply_gu_tile<BITS, CPL, MMAX>(ta, a, j, r_lo, r_hi, nv, m0, pairs, xsum, undo, list, nch, wave, lane);
    issue_gu_tile<BITS, CPL>(ta, rq, rs, q_bytes, s_bytes, j + 2, r_lo, r_hi, row_bytes, gpr, nch, wave, lane);
    if (j + 1 < nt)
      apply_gu_tile<BITS, CPL, MMAX>(tb, a, j + 1, r_lo, r_hi, nv, m0, pairs, xsum, undo, list, nch, wave, lane);
  }
}

template <int BITS, int CPL, int WMAX>
hipError_t launch_batch(const GemvArgs& a, hipStream_t stream, int cus) {
  const int n_routed = min(a.E, a.T * a.k);
  const int list_words = (max(a.T * a.k, a.T) + 3) & ~3;
  const int nch = a.H / Pack<BITS>::kPerChunk;
  const int ntiles = (2 * a.I + kTileRows - 1) / kTileRows;
  // about eight workgroups per CU over the items' first token chunks
  const int n_items = n_routed + a.S;
  const int NS = max(1, min((8 * cus + n_items - 1) / max(n_items, 1), ntiles));
  const int NTC = (a.T + kTokensPerStage - 1) / kTokensPerStage;
  const int n_extra = a.T * a.k / kTokensPerStage + a.S * (NTC - 1);   // bound on later token chunks
  const size_t lds = sizeof(uint32_t) * ((size_t)kTokensPerStage * (a.H / 2) +
                                         (size_t)kTokensPerStage * kChunkSums * nch +
                                         2 * (size_t)list_words + (size_t)a.E) +
                     sizeof(void*) * (size_t)list_words;
  const int64_t grid = (int64_t)(n_extra + n_items) * NS;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((gemv_batch_kernel<BITS, CPL, WMAX>), dim3((unsigned)grid), dim3(kThreads), lds, stream, a,
                     NS, n_routed, n_extra, list_words);
  return hipGetLastError();
}

int cu_count() {
  static int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
    return v;
  }();
  return n;
}

int rows_per_wave_setting() {
  static int v = [] {
    const char* s = std::getenv("MOEQ_GEMV_ROWS_PER_WAVE");
    int r = s ? std::atoi(s) : 0;
    return (r == 2 || r == 4 || r == 8) ? r : 0;
  }();
  return v;
}

template <int BITS, int CPL, int RPW, int WMAX>
hipError_t launch_t(const GemvArgs& a, hipStream_t stream) {
  constexpr int RPB = kWaves * RPW;
  const int n_rb = (2 * a.I + RPB - 1) / RPB;
  const int items = min(a.E, a.T * a.k) + a.S;
  const int list_words = (max(a.T * a.k, a.T) + 3) & ~3;
  const int nch = a.H / Pack<BITS>::kPerChunk;
  const size_t lds = sizeof(uint32_t) * ((size_t)kTokensPerStage * (a.H / 2) +
                                         (size_t)kTokensPerStage * kChunkSums * nch +
                                         2 * (size_t)list_words) +
                     sizeof(void*) * (size_t)list_words;
  hipLaunchKernelGGL((gemv_kernel<BITS, CPL, RPW, WMAX, 1>), dim3(items * n_rb), dim3(kThreads), lds, stream, a,
                     n_rb, list_words);
  return hipGetLastError();
}

template <int BITS, int CPL, int WMAX>
hipError_t launch_rpw(const GemvArgs& a, hipStream_t stream) {
  int rpw = rows_per_wave_setting();
  if (rpw == 0) {
    // enough workgroups to cover every CU twice with 8-row waves, else 4
    const int items = min(a.E, a.T * a.k) + a.S;
    rpw = (items * ((2 * a.I + 31) / 32) >= 512) ? 8 : 4;
  }
  if (rpw == 8) return launch_t<BITS, CPL, 8, WMAX>(a, stream);
  if (rpw == 2) return launch_t<BITS, CPL, 2, WMAX>(a, stream);
  return launch_t<BITS, CPL, 4, WMAX>(a, stream);
}

}  // namespace

hipError_t launch_expert_gemv(const GemvArgs& a, hipStream_t stream) {
  const int pbits = a.bits == 3 ? 2 : a.bits;         // the staged layout's (low plane's) bits
  const int nch = a.H * pbits / 128;                  // 16-byte (low-plane) chunks per row
  const int cpl = (nch + 63) / 64;
  const int nwords = a.H * pbits / 32;                // staged words per input vector
  const int wmax = (nwords + kThreads - 1) / kThreads;
  if (a.T > 1) {
    const int cus = cu_count();
    if (a.bits == 4) {
      if (cpl <= 1) return wmax <= 1 ? launch_batch<4, 1, 1>(a, stream, cus) : launch_batch<4, 1, 2>(a, stream, cus);
      if (cpl <= 2) return wmax <= 2 ? launch_batch<4, 2, 2>(a, stream, cus) : launch_batch<4, 2, 4>(a, stream, cus);
      return launch_batch<4, 4, 4>(a, stream, cus);
    }
    if (a.bits == 3) {
      if (cpl <= 1) return launch_batch<3, 1, 1>(a, stream, cus);
      return launch_batch<3, 2, 2>(a, stream, cus);
    }
    if (cpl <= 1) return launch_batch<2, 1, 1>(a, stream, cus);
    return launch_batch<2, 2, 2>(a, stream, cus);
  }
  if (a.bits == 4) {
    if (cpl <= 1) return wmax <= 1 ? launch_rpw<4, 1, 1>(a, stream) : launch_rpw<4, 1, 2>(a, stream);
    if (cpl <= 2) return wmax <= 2 ? launch_rpw<4, 2, 2>(a, stream) : launch_rpw<4, 2, 4>(a, stream);
    return launch_rpw<4, 4, 4>(a, stream);
  }
  if (a.bits == 3) {
    if (cpl <= 1) return launch_rpw<3, 1, 1>(a, stream);
    return launch_rpw<3, 2, 2>(a, stream);
  }
  if (cpl <= 1) return launch_rpw<2, 1, 1>(a, stream);
  return launch_rpw<2, 2, 2>(a, stream);
}

}  // namespace moeq

// Gate and up projections of the selected experts and the shared expert:
// group-wise affine 4-bit / 2-bit dequantised mat-vec (Flash-MoE,
// fr.news.hada.io, "Noyau de déquantification optimisé FMA" and "Shaders de
// calcul Metal").  For row r of [gate; up] and token t:
//   y[r] = sum_g ( s[r,g] * sum_{j in g} q[r,j] x[t,j] + b[r,g] * sum_{j in g} x[t,j] )
//
// Grid: one workgroup per (expert item, block of 4*RPW rows of [gate; up]),
// every selected expert of the batch and the shared expert in one launch.
// Each wave requests its RPW rows with 16-byte non-temporal loads into
// registers as soon as its expert is known, stages the tokens routed to the
// expert (up to 4 at a time) into LDS as fp16 pairs while those loads are
// in flight, then applies the rows to every token: one wave-wide sum per
// (row, token).  Gate rows and up rows are contiguous in the blob, so the
// [gate; up] block is addressed as 2I rows of one matrix.
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

  group_item(item, a.topk_idx, a.blobs, a.T, a.k, a.E, a.S, g, list, ids, ptrs, a.status);
  if (g.expert < 0) return;
  const uint8_t* blob = g.blob;
  (void)P;

  const int64_t row_bytes = (int64_t)H * BITS / 8;
  const int gpr = H / 64;   // scale/bias groups per row
  const uint32_t* sb = reinterpret_cast<const uint32_t*>(blob + 3 * (int64_t)H * I * BITS / 8);
  const int row0 = rb * RPB + wave * RPW;

  u32x4 q[RPW][CPL];
  uint32_t sbw[RPW][CPL];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int r = row0 + i;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int cc = lane + 64 * c;
      if (r < 2 * I && cc < nch) {
        q[i][c] = load_stream(reinterpret_cast<const u32x4*>(blob + r * row_bytes) + cc);
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
          if (cc < nch) part += chunk_affine(chunk_dot<BITS>(q[i][c], xp, cc, nch), sbw[i][c], xs + kChunkSums * cc);
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
  if (a.T == 1)
    hipLaunchKernelGGL((gemv_kernel<BITS, CPL, RPW, WMAX, 1>), dim3(items * n_rb), dim3(kThreads), lds,
                       stream, a, n_rb, list_words);
  else
    hipLaunchKernelGGL((gemv_kernel<BITS, CPL, RPW, WMAX, kTokensPerStage>), dim3(items * n_rb),
                       dim3(kThreads), lds, stream, a, n_rb, list_words);
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
  const int nch = a.H * a.bits / 128;                 // 16-byte chunks per row
  const int cpl = (nch + 63) / 64;
  const int nwords = a.H * a.bits / 32;               // packed words per input vector
  const int wmax = (nwords + kThreads - 1) / kThreads;
  if (a.bits == 4) {
    if (cpl <= 1) return wmax <= 1 ? launch_rpw<4, 1, 1>(a, stream) : launch_rpw<4, 1, 2>(a, stream);
    if (cpl <= 2) return wmax <= 2 ? launch_rpw<4, 2, 2>(a, stream) : launch_rpw<4, 2, 4>(a, stream);
    return launch_rpw<4, 4, 4>(a, stream);
  }
  if (cpl <= 1) return launch_rpw<2, 1, 1>(a, stream);
  return launch_rpw<2, 2, 2>(a, stream);
}

}  // namespace moeq

// Gate and up projections of the selected experts and the shared expert:
// group-wise affine 4-bit / 2-bit dequantised mat-vec (Flash-MoE,
// fr.news.hada.io, "Noyau de déquantification optimisé FMA" and "Shaders de
// calcul Metal").  For row r of [gate; up] and token t:
//   y[r] = sum_g ( s[r,g] * sum_{j in g} q[r,j] x[t,j] + b[r,g] * sum_{j in g} x[t,j] )
//
// Grid: one workgroup per (expert item, block of 16 rows of [gate; up]),
// every selected expert of the batch and the shared expert in one launch.
// Each wave streams its 4 rows once with 16-byte non-temporal loads kept in
// registers, then applies them to every token routed to the expert (tokens
// staged 4 at a time in LDS as fp16 pairs); one wave-wide sum per (row,
// token).  Gate rows and up rows are contiguous in the blob, so the
// [gate; up] block is addressed as 2I rows of one matrix.
#include "grouping.hpp"
#include "moeq_internal.hpp"
#include "staging.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 4;
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;
constexpr int kTokensPerStage = 4;

__device__ __forceinline__ float x_value(const void* x, int x_f32, int64_t i) {
  return x_f32 ? static_cast<const float*>(x)[i]
               : __uint_as_float((uint32_t) static_cast<const uint16_t*>(x)[i] << 16);
}

template <int BITS, int CPL>
__global__ __launch_bounds__(64 * kWaves) void gemv_kernel(GemvArgs a, int n_rb, int list_words,
                                                           int mc) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ GroupLds g;
  __shared__ float red[2 * kMaxStage * kWaves];
  __shared__ float undo[kMaxStage];
  constexpr int PC = Pack<BITS>::kPerChunk;
  constexpr int PPC = PC / 2;
  const int item = blockIdx.x / n_rb, rb = blockIdx.x - item * n_rb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I, KS = a.k + a.S;
  const int nch = H / PC;
  uint32_t* list = smem;
  uint32_t* pairs = smem + list_words;
  float* xsum = reinterpret_cast<float*>(pairs + (int64_t)mc * (H / 2));

  group_item(item, a.topk_idx, a.T, a.k, a.E, a.S, g, list, a.status);
  if (g.expert < 0 || g.count == 0) return;
  const uint8_t* blob = static_cast<const uint8_t*>(a.blobs[g.expert]);
  if (blob == nullptr) return;

  const int64_t row_bytes = (int64_t)H * BITS / 8;
  const int gpr = H / 64;   // scale/bias groups per row
  const uint32_t* sb = reinterpret_cast<const uint32_t*>(blob + 3 * (int64_t)H * I * BITS / 8);
  const int row0 = rb * kRowsPerBlock + wave * kRowsPerWave;

  u32x4 q[kRowsPerWave][CPL];
  uint32_t sbw[kRowsPerWave][CPL];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
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

  for (int m0 = 0; m0 < g.count; m0 += mc) {
    const int nv = min(mc, g.count - m0);
    auto src = [&](int m, int j) -> float {
      const int t = (int)(list[m0 + m] >> 8);
      return x_value(a.x, a.x_f32, (int64_t)t * H + j);
    };
    stage_many<BITS>(nv, H, src, a.rmsnorm != 0, pairs, xsum, undo, red);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int r = row0 + i;
      if (r >= 2 * I) break;
      for (int m = 0; m < nv; ++m) {
        const uint32_t* xp = pairs + (int64_t)m * (H / 2);
        const float* xs = xsum + (int64_t)m * nch;
        float part = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int cc = lane + 64 * c;
          if (cc < nch) part += chunk_affine(chunk_dot<BITS>(q[i][c], xp + cc * PPC), sbw[i][c], xs[cc]);
        }
        const float v = wave_sum(part) * undo[m];
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

template <int BITS, int CPL>
hipError_t launch_t(const GemvArgs& a, hipStream_t stream) {
  const int n_rb = (2 * a.I + kRowsPerBlock - 1) / kRowsPerBlock;
  const int items = min(a.E, a.T * a.k) + a.S;
  const int list_words = ((a.T * (a.k > 0 ? a.k : 1)) + 3) & ~3;
  const int mc = min(kTokensPerStage, a.T);
  const int nch = a.H / Pack<BITS>::kPerChunk;
  const size_t lds = sizeof(uint32_t) * ((size_t)list_words + (size_t)mc * (a.H / 2) + (size_t)mc * nch);
  hipLaunchKernelGGL((gemv_kernel<BITS, CPL>), dim3(items * n_rb), dim3(64 * kWaves), lds, stream,
                     a, n_rb, list_words, mc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_gemv(const GemvArgs& a, hipStream_t stream) {
  const int nch = a.H * a.bits / 128;   // 16-byte chunks per row
  const int cpl = (nch + 63) / 64;
  if (a.bits == 4) {
    if (cpl <= 1) return launch_t<4, 1>(a, stream);
    if (cpl <= 2) return launch_t<4, 2>(a, stream);
    return launch_t<4, 4>(a, stream);
  }
  if (cpl <= 1) return launch_t<2, 1>(a, stream);
  return launch_t<2, 2>(a, stream);
}

}  // namespace moeq

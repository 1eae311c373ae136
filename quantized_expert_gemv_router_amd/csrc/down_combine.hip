// SwiGLU, down projection and weighted combine (Flash-MoE,
// fr.news.hada.io, "Shaders de calcul Metal": SwiGLU and MoE combine +
// residual + gate; "Deferred GPU Expert Compute": the combined output stays
// on the GPU for the next layer):
//   a   = silu(g) * u                         per (token, slot)
//   d_i = sum_g ( s[i,g] sum_{r in g} q[i,r] a_r + b[i,g] sum_{r in g} a_r )
//   out[t] = residual[t] + sum_{s<k} w[t,s] d_s + gamma[t] d_shared
//
// Grid: one workgroup per (expert item, block of 32 output rows), all
// selected experts and the shared expert in one launch.  a is built from
// gate_up while staging it into LDS (fp16 pairs, per-vector power-of-two
// rescale).  Per-slot down outputs go to the workspace; the last workgroup
// to finish a row block (agent-scope arrival counter) sums them per token
// in slot order, so the result does not depend on arrival order and a
// token's output is the same whatever else is in the batch.
#include "grouping.hpp"
#include "moeq_internal.hpp"
#include "staging.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerBlock = 32;
constexpr int kRowsPerWave = kRowsPerBlock / kWaves;   // 8
constexpr int kTokensPerStage = 8;

// LPR lanes per row, each handling chunks sl, sl + LPR, ... (CPL per lane);
// 64 / LPR rows per step, kRowsPerWave / (64 / LPR) steps (at least 1).
template <int BITS, int LPR, int CPL>
__global__ __launch_bounds__(64 * kWaves) void down_kernel(DownArgs a, int n_rb, int list_words,
                                                           int mc) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ GroupLds g;
  __shared__ float red[2 * kMaxStage * kWaves];
  __shared__ float undo[kMaxStage];
  __shared__ int is_last;
  constexpr int PC = Pack<BITS>::kPerChunk;
  constexpr int PPC = PC / 2;
  constexpr int RPS = 64 / LPR;                       // rows per step
  constexpr int STEPS = (kRowsPerWave + RPS - 1) / RPS;
  const int item = blockIdx.x / n_rb, rb = blockIdx.x - item * n_rb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I, KS = a.k + a.S;
  const int nch = I / PC;                             // chunks per down row
  uint32_t* list = smem;
  uint32_t* pairs = smem + list_words;
  float* xsum = reinterpret_cast<float*>(pairs + (int64_t)mc * (I / 2));

  group_item(item, a.topk_idx, a.T, a.k, a.E, a.S, g, list, a.status);
  const int n_items = g.n_distinct + a.S;
  if (g.expert >= 0 && g.count > 0) {
    const uint8_t* blob = static_cast<const uint8_t*>(a.blobs[g.expert]);
    if (blob != nullptr) {
      const int64_t qoff = 2 * (int64_t)H * I * BITS / 8;            // down.q
      const int64_t row_bytes = (int64_t)I * BITS / 8;
      const uint32_t* sb = reinterpret_cast<const uint32_t*>(
          blob + 3 * (int64_t)H * I * BITS / 8 + 2 * (int64_t)H * I / 64 * 4);  // down.sb
      const int gpr = I / 64;
      const int sub = lane % LPR, rsub = lane / LPR;
      const int wrow0 = rb * kRowsPerBlock + wave * kRowsPerWave;

      u32x4 q[STEPS][CPL];
      uint32_t sbw[STEPS][CPL];
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        const int r = wrow0 + s * RPS + rsub;
        const bool row_ok = (s * RPS + rsub) < kRowsPerWave && r < H;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int cc = sub + LPR * c;
          if (row_ok && cc < nch) {
            q[s][c] = load_stream(reinterpret_cast<const u32x4*>(blob + qoff + r * row_bytes) + cc);
            sbw[s][c] = load_stream(sb + (int64_t)r * gpr + (cc * PC) / 64);
          } else {
            q[s][c] = u32x4{0u, 0u, 0u, 0u};
            sbw[s][c] = 0u;
          }
        }
      }

      for (int m0 = 0; m0 < g.count; m0 += mc) {
        const int nv = min(mc, g.count - m0);
        auto src = [&](int m, int j) -> float {
          const uint32_t e = list[m0 + m];
          const int t = (int)(e >> 8), slot = (int)(e & 255u);
          const float* gu = a.gate_up + ((int64_t)t * KS + slot) * 2 * I;
          const float gv = gu[j], uv = gu[I + j];
          return gv / (1.0f + __expf(-gv)) * uv;
        };
        stage_many<BITS>(nv, I, src, false, pairs, xsum, undo, red);
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
          const int r = wrow0 + s * RPS + rsub;
          const bool row_ok = (s * RPS + rsub) < kRowsPerWave && r < H;
          for (int m = 0; m < nv; ++m) {
            const uint32_t* xp = pairs + (int64_t)m * (I / 2);
            const float* xs = xsum + (int64_t)m * nch;
            float part = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              const int cc = sub + LPR * c;
              if (row_ok && cc < nch)
                part += chunk_affine(chunk_dot<BITS>(q[s][c], xp + cc * PPC), sbw[s][c], xs[cc]);
            }
            const float v = group_sum(part, LPR) * undo[m];
            if (sub == 0 && row_ok) {
              const uint32_t e = list[m0 + m];
              const int t = (int)(e >> 8), slot = (int)(e & 255u);
              a.dbuf[((int64_t)t * KS + slot) * H + r] = v;
            }
          }
        }
        __syncthreads();
      }
    }
  }
  if (g.expert < 0) return;   // no item for this workgroup: not counted

  // arrival; the last of the row block's n_items workgroups combines
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    uint32_t old = atomic_add_acq_rel(a.rb_counters + rb, 1u);
    is_last = (old == (uint32_t)(n_items - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  if (tid == 0) atomic_store_relaxed(a.rb_counters + rb, 0u);
  const int rows = min(kRowsPerBlock, H - rb * kRowsPerBlock);
  for (int idx = tid; idx < a.T * rows; idx += blockDim.x) {
    const int t = idx / rows, r = rb * kRowsPerBlock + (idx - t * rows);
    float acc = a.res_f32 ? static_cast<const float*>(a.residual)[(int64_t)t * H + r]
                          : __uint_as_float((uint32_t) static_cast<const uint16_t*>(a.residual)[(int64_t)t * H + r] << 16);
    for (int s = 0; s < a.k; ++s) {
      const int e = a.topk_idx[(int64_t)t * a.k + s];
      if (e < 0 || e >= a.E) continue;
      acc = fmaf(a.topk_w[(int64_t)t * a.k + s], a.dbuf[((int64_t)t * KS + s) * H + r], acc);
    }
    for (int s = 0; s < a.S; ++s) {
      const float gam = a.shared_w ? a.shared_w[t] : 1.0f;
      acc = fmaf(gam, a.dbuf[((int64_t)t * KS + a.k + s) * H + r], acc);
    }
    a.out[(int64_t)t * H + r] = acc;
  }
}

template <int BITS, int LPR, int CPL>
hipError_t launch_t(const DownArgs& a, int n_rb, hipStream_t stream) {
  const int items = min(a.E, a.T * a.k) + a.S;
  const int list_words = ((a.T * (a.k > 0 ? a.k : 1)) + 3) & ~3;
  const int mc = min(kTokensPerStage, max(a.T, 1));
  const int nch = a.I / Pack<BITS>::kPerChunk;
  const size_t lds = sizeof(uint32_t) * ((size_t)list_words + (size_t)mc * (a.I / 2) + (size_t)mc * nch);
  hipLaunchKernelGGL((down_kernel<BITS, LPR, CPL>), dim3(items * n_rb), dim3(64 * kWaves), lds,
                     stream, a, n_rb, list_words, mc);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const DownArgs& a, int n_rb, hipStream_t stream) {
  const int nch = a.I / Pack<BITS>::kPerChunk;
  if (nch <= 1) return launch_t<BITS, 1, 1>(a, n_rb, stream);
  if (nch <= 2) return launch_t<BITS, 2, 1>(a, n_rb, stream);
  if (nch <= 4) return launch_t<BITS, 4, 1>(a, n_rb, stream);
  if (nch <= 8) return launch_t<BITS, 8, 1>(a, n_rb, stream);
  if (nch <= 16) return launch_t<BITS, 16, 1>(a, n_rb, stream);
  if (nch <= 32) return launch_t<BITS, 32, 1>(a, n_rb, stream);
  if (nch <= 64) return launch_t<BITS, 64, 1>(a, n_rb, stream);
  if (nch <= 128) return launch_t<BITS, 64, 2>(a, n_rb, stream);
  return launch_t<BITS, 64, 4>(a, n_rb, stream);
}

}  // namespace

int down_row_blocks(int H) { return (H + kRowsPerBlock - 1) / kRowsPerBlock; }

hipError_t launch_down_combine(const DownArgs& a, hipStream_t stream) {
  const int n_rb = down_row_blocks(a.H);
  return a.bits == 4 ? launch_bits<4>(a, n_rb, stream) : launch_bits<2>(a, n_rb, stream);
}

}  // namespace moeq

// Router logits, top-K selection and softmax weights for decode batches.
//
// Flash-MoE (fr.news.hada.io, "Architecture du modèle") routes each token
// to K of 512 experts (one more is shared and always active);
// openclawradar.com/fr uses top-10 of 512.  Logits are l_e = Wr[e,:] . xhat
// with xhat the layer input (optionally RMS-normalised); the selection is
// the K largest logits, ties to the lower expert index, and the weights are
// the softmax of the selected logits.
//
// One wave per router row: the row (bf16, H/8 16-byte chunks) is streamed
// once and dotted with every token in fp64 (bf16 x bf16 and bf16 x fp32
// products are exact in fp64).  With RMS norm the same pass accumulates
// sum(x^2) (the lanes of a wave cover every column exactly once), and the
// logit is inv_rms * sum(W x).  The last workgroup to finish (arrival
// counter, agent-scope acquire/release) selects top-K for every token from
// the fp64 logits staged in LDS and writes indices, weights and the shared
// expert's weight.
#include "moeq_device.hpp"
#include "moeq_internal.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 2;            // router rows per workgroup
constexpr int kTokGroup = 8;         // tokens dotted per pass over a row

__device__ __forceinline__ void load_x8(const void* x, int x_f32, int64_t off, double v[8]) {
  if (x_f32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
  }
}

// (value desc, index asc) total order: does (va, ia) rank before (vb, ib)?
__device__ __forceinline__ bool ranks_before(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__device__ void select_token(const RouterArgs& a, int t, double* lg, int* sel, double* selv) {
  const int lane = threadIdx.x & 63;
  const int E = a.E;
  const double* src = a.logits + (int64_t)t * (E + 1);
  for (int e = lane; e < E; e += 64) lg[e] = src[e];
  if (a.logits_out)
    for (int e = lane; e < E; e += 64) a.logits_out[(int64_t)t * E + e] = src[e];
  __builtin_amdgcn_wave_barrier();
  uint64_t taken = 0;
  for (int r = 0; r < a.k; ++r) {
    double bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int m = 0, e = lane; e < E; ++m, e += 64) {
      double v = lg[e];
      if (!((taken >> m) & 1) && ranks_before(v, e, bv, bi)) { bv = v; bi = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      double ov = shfl_xor_f64(bv, o);
      int oi = __shfl_xor(bi, o, 64);
      if (ranks_before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (lane == 0) { sel[r] = bi; selv[r] = bv; }
  }
  __builtin_amdgcn_wave_barrier();
  const double m = selv[0];   // the top-ranked logit is the maximum
  double z = 0.0;
  if (a.no_renorm) {
    double part = 0.0;
    for (int e = lane; e < E; e += 64) part += exp(lg[e] - m);
    z = wave_sum_f64(part);
  } else {
    for (int r = 0; r < a.k; ++r) z += exp(selv[r] - m);
  }
  if (lane < a.k) {
    a.topk_idx[(int64_t)t * a.k + lane] = sel[lane];
    a.topk_w[(int64_t)t * a.k + lane] = (float)(exp(selv[lane] - m) / z);
  }
  if (lane == 0 && a.shared_w) {
    a.shared_w[t] = a.shared_gate ? (float)(1.0 / (1.0 + exp(-src[E]))) : 1.0f;
  }
  __builtin_amdgcn_wave_barrier();
}

__global__ __launch_bounds__(64 * kWaves) void router_kernel(RouterArgs a) {
  extern __shared__ double lds_lg[];   // [kWaves][E]
  __shared__ int sel[kWaves][MOEQ_MAX_TOPK];
  __shared__ double selv[kWaves][MOEQ_MAX_TOPK];
  __shared__ int is_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rows = a.E + (a.shared_gate ? 1 : 0);
  const int row = blockIdx.x * kWaves + wave;
  const int nch = a.H / 8;

  if (row < rows) {
    const uint16_t* wrow = row < a.E ? a.w_router + (int64_t)row * a.H : a.shared_gate;
    for (int t0 = 0; t0 < a.T; t0 += kTokGroup) {
      const int nt = min(kTokGroup, a.T - t0);
      double acc[kTokGroup], ss[kTokGroup];
#pragma unroll
      for (int i = 0; i < kTokGroup; ++i) { acc[i] = 0.0; ss[i] = 0.0; }
      for (int c = lane; c < nch; c += 64) {
        u32x4 u = load_stream(reinterpret_cast<const u32x4*>(wrow) + c);
        double w[8] = {bf16_lo(u[0]), bf16_hi(u[0]), bf16_lo(u[1]), bf16_hi(u[1]),
                       bf16_lo(u[2]), bf16_hi(u[2]), bf16_lo(u[3]), bf16_hi(u[3])};
#pragma unroll
        for (int i = 0; i < kTokGroup; ++i) {
          if (i < nt) {
            double xv[8];
            load_x8(a.x, a.x_f32, (int64_t)(t0 + i) * a.H + 8 * c, xv);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              acc[i] = fma(w[j], xv[j], acc[i]);
              ss[i] = fma(xv[j], xv[j], ss[i]);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kTokGroup; ++i) {
        if (i < nt) {
          double d = wave_sum_f64(acc[i]);
          if (a.rmsnorm) {
            double s2 = wave_sum_f64(ss[i]);
            d = d * (1.0 / sqrt(s2 / (double)a.H + 1e-6));
          }
          if (lane == 0) a.logits[(int64_t)(t0 + i) * (a.E + 1) + row] = d;
        }
      }
    }
  }

  // last workgroup to arrive selects top-K for every token
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t old = atomic_add_acq_rel(a.counter, 1u);
    is_last = (old == gridDim.x - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  if (threadIdx.x == 0) atomic_store_relaxed(a.counter, 0u);
  for (int t = wave; t < a.T; t += kWaves)
    select_token(a, t, lds_lg + (int64_t)wave * a.E, sel[wave], selv[wave]);
}

}  // namespace

hipError_t launch_router_topk(const RouterArgs& a, hipStream_t stream) {
  const int rows = a.E + (a.shared_gate ? 1 : 0);
  const int grid = (rows + kWaves - 1) / kWaves;
  const size_t lds = sizeof(double) * (size_t)kWaves * (size_t)a.E;
  hipLaunchKernelGGL(router_kernel, dim3(grid), dim3(64 * kWaves), lds, stream, a);
  return hipGetLastError();
}

}  // namespace moeq

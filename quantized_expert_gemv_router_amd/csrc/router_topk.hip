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
// logit is inv_rms * sum(W x).  Logits are written with agent-scope
// write-through stores; the last workgroup to bump the arrival counter
// selects top-K for every token from the fp64 logits staged in LDS and
// writes indices, weights and the shared expert's weight.
#include "moeq_device.hpp"
#include "moeq_internal.hpp"
#include "topk.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 2;            // router rows per workgroup (one per wave)
constexpr int kThreads = 64 * kWaves;
constexpr int kStageVec = 16;        // 16-byte loads in flight per thread while staging x

__host__ __device__ inline int token_group(int H) {
  const int tg = 16384 / H;
  return tg < 1 ? 1 : (tg > 4 ? 4 : tg);
}

// Last-workgroup selection for token t by one wave: stage its fp64 logits
// in LDS (all loads in flight together), pick top-K, write the outputs.
__device__ void select_token(const RouterArgs& a, int t, double* lg, int* sel, double* selv) {
  const int lane = threadIdx.x & 63;
  const int E = a.E;
  const double* src = a.logits + (int64_t)t * (E + 1);
  for (int base = 0; base < E; base += 64 * 8) {
    double b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = base + 64 * i + lane;
      b[i] = e < E ? ld_agent(src + e) : 0.0;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = base + 64 * i + lane;
      if (e < E) lg[e] = b[i];
    }
  }
  if (a.logits_out)
    for (int e = lane; e < E; e += 64) a.logits_out[(int64_t)t * E + e] = lg[e];
  __builtin_amdgcn_wave_barrier();
  wave_topk(lg, E, a.k, sel, selv);
  const float w = wave_softmax_weight(lg, E, a.k, selv, a.no_renorm != 0);
  if (lane < a.k) {
    a.topk_idx[(int64_t)t * a.k + lane] = sel[lane];
    a.topk_w[(int64_t)t * a.k + lane] = w;
  }
  if (lane == 0 && a.shared_w) {
    a.shared_w[t] = a.shared_gate ? (float)(1.0 / (1.0 + exp(-ld_agent(src + E)))) : 1.0f;
  }
  __builtin_amdgcn_wave_barrier();
}

// One wave per router row (rows E.. hold the optional shared-gate vector).
// The row's bf16 chunks (CPL per lane) are loaded once into registers; the
// tokens are staged TG at a time into LDS as fp32 with all loads of a group
// in flight together.
template <int CPL>
__global__ __launch_bounds__(kThreads) void router_kernel(RouterArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int sel[kWaves][MOEQ_MAX_TOPK];
  __shared__ double selv[kWaves][MOEQ_MAX_TOPK];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, E = a.E;
  const int TG = token_group(H);
  float* xs = reinterpret_cast<float*>(smem_raw);                          // [TG][H]
  double* lds_lg = reinterpret_cast<double*>(smem_raw + sizeof(float) * (size_t)TG * H);  // [kWaves][E]
  const int rows = E + (a.shared_gate ? 1 : 0);
  const int row = blockIdx.x * kWaves + wave;
  const bool has_row = row < rows;
  const int nch = H / 8;

  u32x4 wv[CPL];
  {
    const uint16_t* wmat = a.w_table ? a.w_table[a.w_layer] : a.w_router;
    const uint16_t* wrow = row < E ? wmat + (int64_t)row * H : a.shared_gate;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int cc = lane + 64 * c;
      wv[c] = (has_row && cc < nch) ? load_stream(reinterpret_cast<const u32x4*>(wrow) + cc)
                                    : u32x4{0u, 0u, 0u, 0u};
    }
  }

  for (int t0 = 0; t0 < a.T; t0 += TG) {
    const int nt = min(TG, a.T - t0);
    // stage nt tokens (contiguous rows of x) into xs as fp32
    const int esz = a.x_f32 ? 4 : 2;
    const int n16 = nt * H * esz / 16;
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(a.x) + (int64_t)t0 * H * esz);
    __syncthreads();
    for (int base = 0; base < n16; base += kThreads * kStageVec) {
      uint4 buf[kStageVec];
#pragma unroll
      for (int i = 0; i < kStageVec; ++i) {
        const int v = base + i * kThreads + tid;
        if (v < n16) buf[i] = src[v];
      }
#pragma unroll
      for (int i = 0; i < kStageVec; ++i) {
        const int v = base + i * kThreads + tid;
        if (v < n16) {
          float4* d = reinterpret_cast<float4*>(xs);
          const uint4 u = buf[i];
          if (a.x_f32) {
            d[v] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                               __uint_as_float(u.w));
          } else {
            d[2 * v] = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
            d[2 * v + 1] = make_float4(bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w));
          }
        }
      }
    }
    __syncthreads();
    if (has_row) {
      for (int i = 0; i < nt; ++i) {
        const float4* xt = reinterpret_cast<const float4*>(xs + (int64_t)i * H);
        double acc = 0.0, ss = 0.0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int cc = lane + 64 * c;
          if (cc < nch) {
            const float4 xa = xt[2 * cc], xb = xt[2 * cc + 1];
            const double xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
            const double w[8] = {bf16_lo(wv[c][0]), bf16_hi(wv[c][0]), bf16_lo(wv[c][1]),
                                 bf16_hi(wv[c][1]), bf16_lo(wv[c][2]), bf16_hi(wv[c][2]),
                                 bf16_lo(wv[c][3]), bf16_hi(wv[c][3])};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              acc = fma(w[j], xv[j], acc);
              ss = fma(xv[j], xv[j], ss);
            }
          }
        }
        double d = wave_sum_f64(acc);
        if (a.rmsnorm) {
          const double s2 = wave_sum_f64(ss);
          d = d * (1.0 / sqrt(s2 / (double)H + 1e-6));
        }
        if (lane == 0) st_agent(a.logits + (int64_t)(t0 + i) * (E + 1) + row, d);
      }
    }
  }

  // the last workgroup to arrive selects top-K for every token
  drain_memory();
  __syncthreads();
  if (tid == 0) is_last = atomic_add_agent(a.counter, 1u) == gridDim.x - 1;
  __syncthreads();
  if (!is_last) return;
  if (tid == 0) st_agent(a.counter, 0u);
  for (int t = wave; t < a.T; t += kWaves)
    select_token(a, t, lds_lg + (int64_t)wave * E, sel[wave], selv[wave]);
}

}  // namespace

hipError_t launch_router_topk(const RouterArgs& a, hipStream_t stream) {
  const int rows = a.E + (a.shared_gate ? 1 : 0);
  const int grid = (rows + kWaves - 1) / kWaves;
  const size_t lds = sizeof(float) * (size_t)token_group(a.H) * a.H +
                     sizeof(double) * (size_t)kWaves * (size_t)a.E;
  const int cpl = (a.H / 8 + 63) / 64;
  if (cpl <= 1)
    hipLaunchKernelGGL(router_kernel<1>, dim3(grid), dim3(kThreads), lds, stream, a);
  else if (cpl <= 2)
    hipLaunchKernelGGL(router_kernel<2>, dim3(grid), dim3(kThreads), lds, stream, a);
  else if (cpl <= 4)
    hipLaunchKernelGGL(router_kernel<4>, dim3(grid), dim3(kThreads), lds, stream, a);
  else if (cpl <= 8)
    hipLaunchKernelGGL(router_kernel<8>, dim3(grid), dim3(kThreads), lds, stream, a);
  else
    hipLaunchKernelGGL(router_kernel<16>, dim3(grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace moeq

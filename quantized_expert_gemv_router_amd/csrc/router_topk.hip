// Router logits, top-K selection and softmax weights for decode batches.
//
// Flash-MoE (fr.news.hada.io, "Architecture du modèle") routes each token
// to K of 512 experts (one more is shared and always active);
// openclawradar.com/fr uses top-10 of 512.  Logits are l_e = Wr[e,:] . xhat
// with xhat the layer input (optionally RMS-normalised); the selection is
// the K largest logits, ties to the lower expert index, and the weights are
// the softmax of the selected logits.
//
// One wave per router row: the row (bf16, H/8 16-byte chunks) is loaded
// once into registers and dotted with every token in fp64 (bf16 x bf16 and
// bf16 x fp32 products are exact in fp64).  Tokens are staged into LDS as
// fp32 a group at a time; the dots of a group's tokens are interleaved and
// their wave sums are DPP reductions, so one token's latency hides behind
// the next.  With RMS norm, sum(x^2) of each token is accumulated (fp64)
// while it is staged, and the logit is inv_rms * sum(W x).  Logits are
// written with agent-scope write-through stores; the last workgroup to bump
// the arrival counter selects top-K for every token, one token per wave at a
// time (keys in registers for E <= 512, else the logits staged in LDS), and
// writes indices, weights and the shared expert's weight.
#include "moeq_device.hpp"
#include "moeq_internal.hpp"
#include "topk.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 8;            // router rows per workgroup (one per wave)
constexpr int kThreads = 64 * kWaves;
constexpr int kTokenGroup = 4;       // tokens per staging pass (upper bound)
constexpr int kStageVec = 4;         // 16-byte loads in flight per thread while staging x
constexpr int kLdsWaves = 2;         // waves that select from LDS when E > 64 * kKeySlots
constexpr int kKeySlots = 8;         // logits per lane in the register selection

__host__ __device__ inline int token_group(int H) {
  const int tg = 16384 / H;
  return tg < 1 ? 1 : (tg > kTokenGroup ? kTokenGroup : tg);
}

// Selection for token t by one wave, E <= 64 * M: lane l holds logits
// l, l + 64, ... as order keys (ascending slot = ascending id).
template <int M>
__device__ void select_token_keys(const RouterArgs& a, int t, int* sel) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, K = a.k;
  const double* src = a.logits + (int64_t)t * (E + 1);
  double v[M];
  int64_t key[M];
  int id[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = lane + 64 * m;
    v[m] = e < E ? ld_agent(src + e) : 0.0;
  }
  const double sg = (lane == 0 && a.shared_w && a.shared_gate) ? ld_agent(src + E) : 0.0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = lane + 64 * m;
    key[m] = e < E ? order_key(v[m]) : kNoKey;
    id[m] = e;
    if (a.logits_out && e < E) a.logits_out[(int64_t)t * E + e] = v[m];
  }
  wave_select<M, true>(key, id, K, [&](int r, int64_t, int win) {
    sel[r] = win;
  });
  __builtin_amdgcn_wave_barrier();
  // the selected logits, read back from the registers of their owner lanes
  const int mine = lane < K ? sel[lane] : -1;
  double sv = 0.0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    // lane l fetches logit `mine` = owner (mine & 63), slot (mine >> 6)
    const int2 p = __builtin_bit_cast(int2, v[m]);
    const double got = __builtin_bit_cast(
        double, make_int2(__shfl(p.x, mine & 63, 64), __shfl(p.y, mine & 63, 64)));
    if (mine >= 0 && (mine >> 6) == m) sv = got;
  }
  const double top = readlane_f64(sv, 0);   // rank 0 is the maximum
  double z;
  if (a.no_renorm) {
    double part = 0.0;
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (lane + 64 * m < E) part += exp(v[m] - top);
    z = wave_sum_f64_dpp(part);
  } else {
    z = wave_sum_f64_dpp(lane < K ? exp(sv - top) : 0.0);
  }
  if (lane < K) {
    a.topk_idx[(int64_t)t * K + lane] = mine;
    a.topk_w[(int64_t)t * K + lane] = (float)(exp(sv - top) / z);
  }
  if (lane == 0 && a.shared_w)
    a.shared_w[t] = a.shared_gate ? (float)(1.0 / (1.0 + exp(-sg))) : 1.0f;
  __builtin_amdgcn_wave_barrier();
}

// Selection for token t by one wave from the logits staged in LDS (any E).
__device__ void select_token_lds(const RouterArgs& a, int t, double* lg, int* sel, double* selv) {
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
template <int CPL>
__global__ __launch_bounds__(kThreads) void router_kernel(RouterArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int sel[kWaves][MOEQ_MAX_TOPK];
  __shared__ double selv[kWaves][MOEQ_MAX_TOPK];
  __shared__ double red[kTokenGroup][kWaves];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, E = a.E;
  const int TG = token_group(H);
  float* xs = reinterpret_cast<float*>(smem_raw);                                      // [TG][H]
  double* lds_lg = reinterpret_cast<double*>(smem_raw + sizeof(float) * (size_t)TG * H);  // [kLdsWaves][E]
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

  const int esz = a.x_f32 ? 4 : 2;
  const int per16 = 16 / esz;            // elements per 16-byte load
  for (int t0 = 0; t0 < a.T; t0 += TG) {
    const int nt = min(TG, a.T - t0);
    // stage nt tokens (contiguous rows of x) into xs as fp32
    const int n16 = nt * H / per16;
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(a.x) + (int64_t)t0 * H * esz);
    double ss[kTokenGroup] = {};
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
          float f[8];
          float4* d = reinterpret_cast<float4*>(xs);
          const uint4 u = buf[i];
          double part = 0.0;
          if (a.x_f32) {
            f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
            f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
            d[v] = make_float4(f[0], f[1], f[2], f[3]);
#pragma unroll
            for (int j = 0; j < 4; ++j) part = fma((double)f[j], (double)f[j], part);
          } else {
            f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
            f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
            d[2 * v] = make_float4(f[0], f[1], f[2], f[3]);
            d[2 * v + 1] = make_float4(f[4], f[5], f[6], f[7]);
#pragma unroll
            for (int j = 0; j < 8; ++j) part = fma((double)f[j], (double)f[j], part);
          }
          if (a.rmsnorm) {
            const int ti = v * per16 / H;
#pragma unroll
            for (int j = 0; j < kTokenGroup; ++j)
              if (j == ti) ss[j] += part;
          }
        }
      }
    }
    if (a.rmsnorm) {
#pragma unroll
      for (int j = 0; j < kTokenGroup; ++j) {
        const double s2 = wave_sum_f64_dpp(ss[j]);
        if (lane == 0) red[j][wave] = s2;
      }
    }
    __syncthreads();
    if (has_row) {
      double acc[kTokenGroup] = {};
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int cc = lane + 64 * c;
        if (cc < nch) {
          const double w[8] = {bf16_lo(wv[c][0]), bf16_hi(wv[c][0]), bf16_lo(wv[c][1]),
                               bf16_hi(wv[c][1]), bf16_lo(wv[c][2]), bf16_hi(wv[c][2]),
                               bf16_lo(wv[c][3]), bf16_hi(wv[c][3])};
#pragma unroll
          for (int i = 0; i < kTokenGroup; ++i) {
            if (i < nt) {
              const float4* xt = reinterpret_cast<const float4*>(xs + (int64_t)i * H);
              const float4 xa = xt[2 * cc], xb = xt[2 * cc + 1];
              const double xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
              for (int j = 0; j < 8; ++j) acc[i] = fma(w[j], xv[j], acc[i]);
            }
          }
        }
      }
      double d[kTokenGroup];
#pragma unroll
      for (int i = 0; i < kTokenGroup; ++i) d[i] = wave_sum_f64_dpp(acc[i]);
      if (lane == 0) {
#pragma unroll
        for (int i = 0; i < kTokenGroup; ++i) {
          if (i < nt) {
            double di = d[i];
            if (a.rmsnorm) {
              double s2 = 0.0;
              for (int w = 0; w < kWaves; ++w) s2 += red[i][w];
              di = di * (1.0 / sqrt(s2 / (double)H + 1e-6));
            }
            st_agent(a.logits + (int64_t)(t0 + i) * (E + 1) + row, di);
          }
        }
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
  if (E <= 64) {
    for (int t = wave; t < a.T; t += kWaves) select_token_keys<1>(a, t, sel[wave]);
  } else if (E <= 128) {
    for (int t = wave; t < a.T; t += kWaves) select_token_keys<2>(a, t, sel[wave]);
  } else if (E <= 256) {
    for (int t = wave; t < a.T; t += kWaves) select_token_keys<4>(a, t, sel[wave]);
  } else if (E <= 64 * kKeySlots) {
    for (int t = wave; t < a.T; t += kWaves) select_token_keys<kKeySlots>(a, t, sel[wave]);
  } else if (wave < kLdsWaves) {
    for (int t = wave; t < a.T; t += kLdsWaves)
      select_token_lds(a, t, lds_lg + (int64_t)wave * E, sel[wave], selv[wave]);
  }
}

}  // namespace

hipError_t launch_router_topk(const RouterArgs& a, hipStream_t stream) {
  const int rows = a.E + (a.shared_gate ? 1 : 0);
  const int grid = (rows + kWaves - 1) / kWaves;
  const size_t lds = sizeof(float) * (size_t)token_group(a.H) * a.H +
                     (a.E > 64 * kKeySlots ? sizeof(double) * (size_t)kLdsWaves * (size_t)a.E : 0);
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

// Router logits, top-K selection and softmax weights for decode batches.
//
// Flash-MoE (fr.news.hada.io, "Architecture du modèle") routes each token
// to K of 512 experts (one more is shared and always active);
// openclawradar.com/fr uses top-10 of 512.  Logits are l_e = Wr[e,:] . xhat
// with xhat the layer input (optionally RMS-normalised); the selection is
// the K largest logits, ties to the lower expert index, and the weights are
// the softmax of the selected logits.
//
// Up to 8 tokens (router_kernel): one wave per router row.  The row (bf16,
// H/8 16-byte chunks) is loaded once into registers and dotted with every
// token in fp64 (bf16 x bf16 and bf16 x fp32 products are exact in fp64).
// Up to 16 tokens are copied into LDS in their own type (bf16 or fp32) per
// pass; the dots of four tokens at a time are interleaved and their wave
// sums are DPP reductions, so one token's latency hides behind the next.
// With RMS norm, sum(x^2) of each staged token is taken once (fp64, one
// wave per token) and the logit is inv_rms * sum(W x).  Logits are written
// with agent-scope write-through stores, and the last workgroup to bump the
// arrival counter selects top-K: one token with the whole workgroup (E <=
// 512), else one token per wave.
//
// More tokens: the logits of 16 tokens x 16 rows per workgroup on the fp64
// MFMA (router_mfma_kernel, unscaled; H <= 4096 and E <= 512, else the
// vector kernel without its selection), then a second launch selects for
// all tokens at once, applying 1/rms itself: one workgroup per token with
// the threshold top-K over one logit per thread (E <= 512), else one wave
// per token.
//
// Either way the logits are held as keys in registers for E <= 512 (else
// staged in LDS), and the indices, weights and the shared expert's weight
// are written.
#include "moeq_device.hpp"
#include "moeq_internal.hpp"
#include "topk.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 8;            // router rows per workgroup (one per wave)
constexpr int kThreads = 64 * kWaves;
constexpr int kTokenGroup = 4;       // tokens whose dots are interleaved
constexpr int kMaxStaged = 16;       // tokens per staging pass (upper bound)
constexpr int kStageVec = 8;         // 16-byte loads in flight per thread while staging x
constexpr int kLdsWaves = 2;         // waves that select from LDS when E > 64 * kKeySlots
constexpr int kKeySlots = 8;         // logits per lane in the register selection
constexpr int kStageBudget = 128 * 1024;   // LDS bytes for staged tokens and LDS selection

// Tokens staged per pass: x in its own type (esz bytes per value), within
// the LDS budget left after the LDS selection's logits.
__host__ __device__ inline int token_group(int H, int esz, int E) {
  const int budget = kStageBudget - (E > 64 * kKeySlots ? kLdsWaves * E * 8 : 0);
  const int tg = budget / (H * esz);
  return tg < 1 ? 1 : (tg > kMaxStaged ? kMaxStaged : tg);
}

// 8 consecutive staged values of x as fp64 (bf16 or fp32 in LDS).
__device__ __forceinline__ void staged_x8(const unsigned char* xs, int x_f32, int64_t elem, double* xv) {
  if (x_f32) {
    const float4* p = reinterpret_cast<const float4*>(xs + elem * 4);
    const float4 xa = p[0], xb = p[1];
    xv[0] = xa.x; xv[1] = xa.y; xv[2] = xa.z; xv[3] = xa.w;
    xv[4] = xb.x; xv[5] = xb.y; xv[6] = xb.z; xv[7] = xb.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(xs + elem * 2);
    xv[0] = bf16_lo(u.x); xv[1] = bf16_hi(u.x); xv[2] = bf16_lo(u.y); xv[3] = bf16_hi(u.y);
    xv[4] = bf16_lo(u.z); xv[5] = bf16_hi(u.z); xv[6] = bf16_lo(u.w); xv[7] = bf16_hi(u.w);
  }
}

// Selection for tokens t0, t0 + step, ... by one wave, E <= 64 * M: lane l
// holds logits l, l + 64, ... as order keys (ascending slot = ascending id).  The next token's logits are requested before the current one is
// selected.  sel/selv (this wave's LDS) receive the ranked ids and logits.
template <int M>
__device__ void select_tokens_keys(const RouterArgs& a, int t0, int step, int* sel, double* selv) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, K = a.k, T = a.T;
  auto fetch = [&](int t, double (&d)[M], double& g) {
    const double* src = a.logits + (int64_t)t * (E + 1);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int e = lane + 64 * m;
      d[m] = (t < T && e < E) ? ld_agent(src + e) : 0.0;
    }
    g = (t < T && lane == 0 && a.shared_w && a.shared_gate) ? ld_agent(src + E) : 0.0;
  };
  double v[M], sg;
  fetch(t0, v, sg);
  for (int t = t0; t < T; t += step) {
    double nv[M], nsg;
    fetch(t + step, nv, nsg);
    int64_t key[M];
    int id[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int e = lane + 64 * m;
      key[m] = e < E ? order_key(v[m]) : kNoKey;
      id[m] = e;
      if (a.logits_out && e < E) a.logits_out[(int64_t)t * E + e] = v[m];
    }
    wave_select<M, true>(key, id, K, [&](int r, int64_t kk, int win) {
      sel[r] = win;
      // the logit back from its key (a -0 logit comes back as +0)
      selv[r] = __longlong_as_double(kk >= 0 ? kk : (kk ^ 0x7FFFFFFFFFFFFFFFll));
    });
    __builtin_amdgcn_wave_barrier();
    const double top = selv[0];   // rank 0 is the maximum
    const double ex = lane < K ? exp(selv[lane] - top) : 0.0;
    double z;
    if (a.no_renorm) {
      double part = 0.0;
#pragma unroll
      for (int m = 0; m < M; ++m)
        if (lane + 64 * m < E) part += exp(v[m] - top);
      z = wave_sum_f64_dpp(part);
    } else {
      z = wave_sum_f64_dpp(ex);
    }
    if (lane < K) {
      a.topk_idx[(int64_t)t * K + lane] = sel[lane];
      a.topk_w[(int64_t)t * K + lane] = (float)(ex / z);
    }
    if (lane == 0 && a.shared_w)
      a.shared_w[t] = a.shared_gate ? (float)(1.0 / (1.0 + exp(-sg))) : 1.0f;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int m = 0; m < M; ++m) v[m] = nv[m];
    sg = nsg;
  }
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
// LDS of the workgroup selection.
struct BlockSelLds {
  double lg[64 * kWaves];
  double red[kWaves];
  int wk[2 * kWaves];
  int64_t ck[64 * kWaves];
  int ci[64 * kWaves];
  int cnt[kWaves];
  int sel[MOEQ_MAX_TOPK];
  double selv[MOEQ_MAX_TOPK];
};

// Selection for token t by the whole workgroup (kWaves waves), E <= 64 *
// kWaves: thread i holds logit v of expert i as an order key; the
// threshold top-K over the workgroup (samples, candidates, ranking by
// counting; the two-level wave selection when more than 64 candidates
// pass), then wave 0 takes the softmax weights.  g: the shared-gate logit
// (thread 0).
__device__ void block_select(const RouterArgs& a, int t, double v, double g, BlockSelLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, K = a.k;
  const int64_t key = tid < E ? order_key(v) : kNoKey;
  if (tid < E) {
    L.lg[tid] = v;
    if (a.logits_out) a.logits_out[(int64_t)t * E + tid] = v;
  }
  topk_samples<kWaves>(key, K, L.wk);
  __syncthreads();
  topk_candidates<kWaves>(key, tid, K, L.wk, L.ck, L.ci, L.cnt);
  __syncthreads();
  const bool fast = topk_select<kWaves>(K, L.ck, L.ci, L.cnt, [&](int r, int win) {
    if (wave == 0) L.sel[r] = win;
  });
  if (!fast) block_topk_keys<kWaves, 1, 2>(L.lg, E, K, L.ck, L.ci, L.sel, L.selv);   // block-uniform
  __syncthreads();
  if (wave == 0) {
    const int mine = lane < K ? L.sel[lane] : 0;
    const double top = L.lg[L.sel[0]];   // rank 0 is the maximum
    const double ex = lane < K ? exp(L.lg[mine] - top) : 0.0;
    double z;
    if (a.no_renorm) {
      double part = 0.0;
      for (int e = lane; e < E; e += 64) part += exp(L.lg[e] - top);
      z = wave_sum_f64_dpp(part);
    } else {
      z = wave_sum_f64_dpp(ex);
    }
    if (lane < K) {
      a.topk_idx[(int64_t)t * K + lane] = mine;
      a.topk_w[(int64_t)t * K + lane] = (float)(ex / z);
    }
    if (lane == 0 && a.shared_w) a.shared_w[t] = a.shared_gate ? (float)(1.0 / (1.0 + exp(-g))) : 1.0f;
  }
}

// SELECT: the last workgroup to arrive selects for every token (small
// batches); otherwise select_kernel does, one wave per token, in a second
// launch.
template <int CPL, bool SELECT>
__global__ __launch_bounds__(kThreads) void router_kernel(RouterArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int sel[kWaves][MOEQ_MAX_TOPK];
  __shared__ double selv[kWaves][MOEQ_MAX_TOPK];
  __shared__ double inv_rms[kMaxStaged];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, E = a.E;
  const int esz = a.x_f32 ? 4 : 2;
  const int TG = token_group(H, esz, E);
  unsigned char* xs = smem_raw;                                                      // [TG][H] x
  double* lds_lg = reinterpret_cast<double*>(smem_raw + (size_t)TG * H * esz);       // [kLdsWaves][E]
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
    // copy nt tokens (contiguous rows of x) into LDS as they are
    const int n16 = nt * H * esz / 16;
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.x) + (int64_t)t0 * H * esz);
    u32x4* dst = reinterpret_cast<u32x4*>(xs);
    __syncthreads();
    for (int base = 0; base < n16; base += kThreads * kStageVec) {
      u32x4 buf[kStageVec];
#pragma unroll
      for (int i = 0; i < kStageVec; ++i) {
        const int v = base + i * kThreads + tid;
        if (v < n16) buf[i] = src[v];
      }
#pragma unroll
      for (int i = 0; i < kStageVec; ++i) {
        const int v = base + i * kThreads + tid;
        if (v < n16) dst[v] = buf[i];
      }
    }
    __syncthreads();
    if (a.rmsnorm) {
      // sum(x^2) per token (fp64), one wave per token
      for (int i = wave; i < nt; i += kWaves) {
        double ss = 0.0;
        for (int c = lane; c < nch; c += 64) {
          double xv[8];
          staged_x8(xs, a.x_f32, (int64_t)i * H + 8 * c, xv);
#pragma unroll
          for (int j = 0; j < 8; ++j) ss = fma(xv[j], xv[j], ss);
        }
        ss = wave_sum_f64_dpp(ss);
        if (lane == 0) inv_rms[i] = 1.0 / sqrt(ss / (double)H + 1e-6);
      }
      __syncthreads();
    }
    if (has_row) {
      for (int g0 = 0; g0 < nt; g0 += kTokenGroup) {
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
              if (g0 + i < nt) {
                double xv[8];
                staged_x8(xs, a.x_f32, (int64_t)(g0 + i) * H + 8 * cc, xv);
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
            if (g0 + i < nt) {
              const double di = a.rmsnorm ? d[i] * inv_rms[g0 + i] : d[i];
              st_agent(a.logits + (int64_t)(t0 + g0 + i) * (E + 1) + row, di);
            }
          }
        }
      }
    }
  }

  if constexpr (!SELECT) return;
  // the last workgroup to arrive selects top-K for every token
  drain_memory();
  __syncthreads();
  if (tid == 0) is_last = atomic_add_agent(a.counter, 1u) == gridDim.x - 1;
  __syncthreads();
  if (!is_last) return;
  if (tid == 0) st_agent(a.counter, 0u);
  if (a.T == 1 && E <= 64 * kWaves) {   // one token: the whole workgroup selects it
    __shared__ BlockSelLds L;
    const double v = tid < E ? ld_agent(a.logits + tid) : 0.0;
    const double g = (tid == 0 && a.shared_w && a.shared_gate) ? ld_agent(a.logits + E) : 0.0;
    block_select(a, 0, v, g, L);
  } else if (E <= 64) {
    select_tokens_keys<1>(a, wave, kWaves, sel[wave], selv[wave]);
  } else if (E <= 128) {
    select_tokens_keys<2>(a, wave, kWaves, sel[wave], selv[wave]);
  } else if (E <= 256) {
    select_tokens_keys<4>(a, wave, kWaves, sel[wave], selv[wave]);
  } else if (E <= 64 * kKeySlots) {
    select_tokens_keys<kKeySlots>(a, wave, kWaves, sel[wave], selv[wave]);
  } else if (wave < kLdsWaves) {
    for (int t = wave; t < a.T; t += kLdsWaves)
      select_token_lds(a, t, lds_lg + (int64_t)wave * E, sel[wave], selv[wave]);
  }
}

// ------------------------------------------------ batches on the fp64 MFMA
// Unscaled logits sum_j W[e,j] x[t,j] of a tile of 16 tokens x 16 router
// rows on v_mfma_f64_16x16x4f64, whose lane layout is: A lane l = (row
// l%16, k slot l/16), B lane l = (k slot l/16, column l%16), D element i of
// lane l = (row 4i + l/16, column l%16); rows are tokens, columns router
// rows.  H is cut into 32-value chunks, wave w taking an eighth of them.
// In a chunk, lane (r, q) holds values 8q .. 8q+7 of its token and of its
// router row (one 16-byte load each), and MFMA j pairs value 8q + j of
// both, so the four k slots of MFMA j are 8 apart and the chunk's 8 MFMAs
// cover its 32 values.  All of a wave's chunks are requested before the
// first MFMA.  The eight waves' tiles are summed in wave order through LDS.
// bf16 x bf16 and bf16 x fp32 products are exact in fp64, as in the
// vector kernel; only the order of the fp64 sum differs.
constexpr int kMfmaWaves = 8;
constexpr int kMfmaChunks = 16;   // chunks per wave: H <= 32 * 8 * 16 = 4096
typedef double double4v __attribute__((ext_vector_type(4)));

template <bool F32>
__global__ __launch_bounds__(64 * kMfmaWaves) void router_mfma_kernel(RouterArgs a) {
  __shared__ double part[kMfmaWaves][16][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, E = a.E, T = a.T;
  const int rows = E + (a.shared_gate ? 1 : 0);
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  const int r = lane & 15, q = lane >> 4;
  const uint16_t* wmat = a.w_table ? a.w_table[a.w_layer] : a.w_router;
  const int e = e0 + r, t = t0 + r;
  const uint16_t* wrow = e < E ? wmat + (int64_t)e * H : (e < rows ? a.shared_gate : nullptr);
  const bool tok_ok = t < T;
  const int nch = H / 32;
  const int c_lo = nch * wave / kMfmaWaves, c_hi = nch * (wave + 1) / kMfmaWaves;
  u32x4 wq[kMfmaChunks], xq[kMfmaChunks][F32 ? 2 : 1];
#pragma unroll
  for (int i = 0; i < kMfmaChunks; ++i) {
    const int c = c_lo + i;
    const int k = c * 32 + q * 8;
    const bool ok = c < c_hi;
    wq[i] = (ok && wrow) ? load_stream(reinterpret_cast<const u32x4*>(wrow + k)) : u32x4{0u, 0u, 0u, 0u};
    if constexpr (F32) {
      const u32x4* xp = reinterpret_cast<const u32x4*>(static_cast<const float*>(a.x) + (int64_t)t * H + k);
      xq[i][0] = (ok && tok_ok) ? xp[0] : u32x4{0u, 0u, 0u, 0u};
      xq[i][1] = (ok && tok_ok) ? xp[1] : u32x4{0u, 0u, 0u, 0u};
    } else {
      const u32x4* xp = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) + (int64_t)t * H + k);
      xq[i][0] = (ok && tok_ok) ? xp[0] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  double4v acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int i = 0; i < kMfmaChunks; ++i) {
    if (c_lo + i < c_hi) {
      double wv[8], xv[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wv[2 * j] = bf16_lo(wq[i][j]);
        wv[2 * j + 1] = bf16_hi(wq[i][j]);
      }
      if constexpr (F32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xv[j] = __uint_as_float(xq[i][0][j]);
          xv[4 + j] = __uint_as_float(xq[i][1][j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xv[2 * j] = bf16_lo(xq[i][0][j]);
          xv[2 * j + 1] = bf16_hi(xq[i][0][j]);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(xv[j], wv[j], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(xv[j + 1], wv[j + 1], acc1, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][4 * i + q][r] = acc0[i] + acc1[i];
  __syncthreads();
  if (tid < 256) {
    const int tt = tid >> 4, rr = tid & 15;
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < kMfmaWaves; ++w) sum += part[w][tt][rr];
    if (t0 + tt < T && e0 + rr < rows) a.logits[(int64_t)(t0 + tt) * (E + 1) + e0 + rr] = sum;
  }
}

// One wave per token (token blockIdx.x), E > 64 * kWaves: top-K from the
// (scaled) logits staged in LDS, softmax weights, shared weight.
__global__ __launch_bounds__(64) void select_kernel(RouterArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int sel[MOEQ_MAX_TOPK];
  __shared__ double selv[MOEQ_MAX_TOPK];
  select_token_lds(a, blockIdx.x, reinterpret_cast<double*>(smem_raw), sel, selv);
}

// One workgroup per token (token blockIdx.x), E <= 64 * kWaves: the
// workgroup selection.  `raw`: the logits are unscaled sums, and with RMS
// norm the workgroup takes the token's 1/rms first.
__global__ __launch_bounds__(kThreads) void select_block_kernel(RouterArgs a, int raw) {
  __shared__ BlockSelLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x, E = a.E, H = a.H;
  const double* src = a.logits + (int64_t)t * (E + 1);
  // the logit first: its load is in flight during the sum of squares
  const double raw_v = tid < E ? ld_agent(src + tid) : 0.0;
  const double raw_g = (tid == 0 && a.shared_w && a.shared_gate) ? ld_agent(src + E) : 0.0;
  double scale = 1.0;
  if (raw && a.rmsnorm) {
    double ss = 0.0;
    for (int c = tid; c < H / 8; c += kThreads) {
      double xv[8];
      if (a.x_f32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + (int64_t)t * H + 8 * c);
        const float4 u0 = p[0], u1 = p[1];
        xv[0] = u0.x; xv[1] = u0.y; xv[2] = u0.z; xv[3] = u0.w;
        xv[4] = u1.x; xv[5] = u1.y; xv[6] = u1.z; xv[7] = u1.w;
      } else {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (int64_t)t * H + 8 * c);
        xv[0] = bf16_lo(u.x); xv[1] = bf16_hi(u.x); xv[2] = bf16_lo(u.y); xv[3] = bf16_hi(u.y);
        xv[4] = bf16_lo(u.z); xv[5] = bf16_hi(u.z); xv[6] = bf16_lo(u.w); xv[7] = bf16_hi(u.w);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fma(xv[j], xv[j], ss);
    }
    ss = wave_sum_f64_dpp(ss);
    if (lane == 0) L.red[wave] = ss;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += L.red[w];
    scale = 1.0 / sqrt(tot / (double)H + 1e-6);
  }
  block_select(a, t, raw_v * scale, raw_g * scale, L);
}

template <int CPL>
hipError_t launch_cpl(const RouterArgs& a, hipStream_t stream, int grid, size_t lds) {
  const bool split = a.T > kWaves;   // more tokens than the last workgroup has waves
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&router_kernel<CPL, false>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kStageBudget) == hipSuccess
          ? hipFuncSetAttribute(reinterpret_cast<const void*>(&router_kernel<CPL, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kStageBudget)
          : hipErrorInvalidValue;
  if (attr != hipSuccess) return attr;
  if (!split) {
    hipLaunchKernelGGL((router_kernel<CPL, true>), dim3(grid), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
  }
  // logits on the fp64 MFMA where a wave's share of H fits its registers
  // and the selection reads them in registers (E <= 512), else the vector
  // kernel
  const int rows = a.E + (a.shared_gate ? 1 : 0);
  const bool mfma = a.H % 32 == 0 && a.H / 32 <= kMfmaWaves * kMfmaChunks && a.E <= 64 * kKeySlots;
  if (mfma) {
    const dim3 g((rows + 15) / 16, (a.T + 15) / 16);
    if (a.x_f32) hipLaunchKernelGGL(router_mfma_kernel<true>, g, dim3(64 * kMfmaWaves), 0, stream, a);
    else hipLaunchKernelGGL(router_mfma_kernel<false>, g, dim3(64 * kMfmaWaves), 0, stream, a);
  } else {
    hipLaunchKernelGGL((router_kernel<CPL, false>), dim3(grid), dim3(kThreads), lds, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.E <= 64 * kWaves) {
    hipLaunchKernelGGL(select_block_kernel, dim3(a.T), dim3(kThreads), 0, stream, a, mfma ? 1 : 0);
  } else {   // the vector kernel wrote scaled logits (mfma needs E <= 512)
    const size_t sel_lds = sizeof(double) * (size_t)a.E;
    hipLaunchKernelGGL(select_kernel, dim3(a.T), dim3(64), sel_lds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_topk(const RouterArgs& a, hipStream_t stream) {
  const int rows = a.E + (a.shared_gate ? 1 : 0);
  const int grid = (rows + kWaves - 1) / kWaves;
  const int esz = a.x_f32 ? 4 : 2;
  const size_t lds = (size_t)token_group(a.H, esz, a.E) * a.H * esz +
                     (a.E > 64 * kKeySlots ? sizeof(double) * (size_t)kLdsWaves * (size_t)a.E : 0);
  const int cpl = (a.H / 8 + 63) / 64;
  if (cpl <= 1) return launch_cpl<1>(a, stream, grid, lds);
  if (cpl <= 2) return launch_cpl<2>(a, stream, grid, lds);
  if (cpl <= 4) return launch_cpl<4>(a, stream, grid, lds);
  if (cpl <= 8) return launch_cpl<8>(a, stream, grid, lds);
  return launch_cpl<16>(a, stream, grid, lds);
}

}  // namespace moeq

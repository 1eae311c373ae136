// One decode token through L stacked MoE layers in a single persistent
// launch (Flash-MoE, fr.news.hada.io, "Deferred GPU Expert Compute": the
// combined output, norm and residual stay on the GPU and feed the next
// layer; the measured ~30 us per-layer submission cost that pre-encoding
// removed on the openclawradar.com/ru page, "CMD2", is what a single
// launch avoids here).
//
// Per layer l, with h the residual stream (fp32, resident):
//   xhat = h / sqrt(mean(h^2) + 1e-6)           unit-weight RMS norm
//   logits = Wr_l xhat (fp64), top-K, softmax   router
//   for each selected expert and the shared one: g, u (dequant mat-vec),
//   a = silu(g) u, d = Wd a;  h <- h + sum_k w_k d_k + d_shared
//
// Grid: one workgroup of 8 waves per CU, all co-resident (cooperative
// launch).  Three grid barriers per layer separate the all-to-all steps:
// h complete -> router rows; logits complete -> top-K and gate/up;
// activations complete -> down and combine.  Everything whose address is
// known early is requested before the barrier that precedes its use: the
// next layer's router rows and shared-expert gate/up rows during the
// previous layer's last barrier, and the down rows of every selected expert
// right after top-K.  Each workgroup keeps its own copy of h in LDS for
// the norm, the router dots and the gate/up staging, and owns a fixed set
// of rows in every matrix:
//   router rows  e = b + NB*i, split into 8/RW segments across waves;
//   gate/up rows r = b + NB*i of every selected expert (so a = silu(g)*u
//   is formed locally);
//   down rows    r = b + NB*i of every selected expert (so the combine is
//   a per-row sum in registers, in slot order, no atomics).
// Cross-workgroup data (logits, activations, h) moves with agent-scope
// write-through stores and loads; each barrier waits for the caller's
// stores to complete before arriving.  Barriers are two-level counter trees
// with a bounded spin: on time-out a workgroup sets the status word and an
// abort flag and every workgroup leaves the kernel.
#include "moeq_device.hpp"
#include "moeq_internal.hpp"
#include "staging.hpp"
#include "topk.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroups = 8;                 // barrier tree: groups of workgroups
constexpr int kBarWords = 32 * (kGroups + 2);
constexpr int kSpinLimit = 1 << 18;        // polls before a barrier gives up
constexpr int kMaxKS = 8;                  // selected + shared experts per layer

// ------------------------------------------------------------------ barrier
struct GridBarrier {
  uint32_t* base;       // [0]: top counter, [32*(1+g)]: group g, [32*(1+kGroups)]: abort
  int group, gsize, ngroups;
  uint32_t epoch;

  // Whole block.  Returns false if the grid is aborting.
  __device__ __forceinline__ bool sync(int32_t* status, int* flag) {
    drain_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
      ++epoch;
      uint32_t* gc = base + 32 * (1 + group);
      uint32_t* top = base;
      uint32_t* abort = base + 32 * (1 + kGroups);
      const uint32_t old = atomic_add_agent(gc, 1u);
      if (old == epoch * (uint32_t)gsize - 1u) atomic_add_agent(top, 1u);
      const uint32_t target = epoch * (uint32_t)ngroups;
      int ok = 1;
      for (int spins = 0; ld_agent(top) < target; ++spins) {
        if ((spins & 63) == 63 && ld_agent(abort) != 0u) { ok = 0; break; }
        if (spins > kSpinLimit) {
          set_status(status, kStatusTimeout);
          st_agent(abort, 1u);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      *flag = ok;
    }
    __syncthreads();
    return *flag != 0;
  }
};

// --------------------------------------------------------------- geometry
template <int BITS, int CPLR, int CPLG, int RPWG, int LPRD, int CPLD, int STEPSD>
struct StackCfg {
  static constexpr int PC = Pack<BITS>::kPerChunk;
  static constexpr int PPC = PC / 2;
  static constexpr int RPSD = 64 / LPRD;   // down rows per wave step
};

struct StackLds {
  int hs, xp, xs, ap, as, gres, dres, lg, total;
};

__host__ __device__ inline int al16(int v) { return (v + 15) & ~15; }

__host__ __device__ inline StackLds stack_lds_layout(int H, int I, int E, int KS, int PC, int RG, int RD) {
  StackLds L;
  L.hs = 0;
  L.xp = al16(L.hs + 4 * H);
  L.xs = al16(L.xp + 2 * H);
  L.ap = al16(L.xs + 4 * (H / PC));
  L.as = al16(L.ap + KS * 2 * I);
  L.gres = al16(L.as + 4 * KS * (I / PC));
  L.dres = al16(L.gres + 4 * KS * 2 * RG);
  L.lg = al16(L.dres + 4 * KS * RD);
  L.total = al16(L.lg + 8 * E);
  return L;
}

__device__ __forceinline__ const uint8_t* blob_of(const StackArgs& a, int layer, int e) {
  return static_cast<const uint8_t*>(a.blobs[(int64_t)layer * (a.E + a.S) + e]);
}

template <int BITS, int CPLR, int CPLG, int RPWG, int LPRD, int CPLD, int STEPSD, int KSMAX>
__global__ __launch_bounds__(kThreads) void stack_kernel(StackArgs a) {
  using C = StackCfg<BITS, CPLR, CPLG, RPWG, LPRD, CPLD, STEPSD>;
  constexpr int PC = C::PC, PPC = C::PPC, RPSD = C::RPSD;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ double rpart[kWaves];
  __shared__ float red[2 * kMaxKS * kWaves];
  __shared__ float undo_x[1], undo_a[kMaxKS];
  __shared__ int sel[MOEQ_MAX_TOPK];
  __shared__ double selv[MOEQ_MAX_TOPK];
  __shared__ float selw[MOEQ_MAX_TOPK];
  __shared__ const uint8_t* eblob[kMaxKS];
  __shared__ double ssum[kWaves];
  __shared__ int bar_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NB = gridDim.x, b = blockIdx.x;
  const int H = a.H, I = a.I, E = a.E, K = a.K, S = a.S, KS = K + S;
  const int nchG = H / PC, nchD = I / PC;

  // LDS carve-up (byte offsets, 16-byte aligned; see stack_lds_layout)
  const int RG = (I + NB - 1) / NB, RD = (H + NB - 1) / NB;
  const StackLds L_ = stack_lds_layout(H, I, E, KS, PC, RG, RD);
  float* hs = reinterpret_cast<float*>(smem + L_.hs);          // [H]
  uint32_t* xp = reinterpret_cast<uint32_t*>(smem + L_.xp);    // [H/2]
  float* xs = reinterpret_cast<float*>(smem + L_.xs);          // [H/PC]
  uint32_t* ap = reinterpret_cast<uint32_t*>(smem + L_.ap);    // [KS][I/2]
  float* as = reinterpret_cast<float*>(smem + L_.as);          // [KS][I/PC]
  float* gres = reinterpret_cast<float*>(smem + L_.gres);      // [KS][2][RG]
  float* dres = reinterpret_cast<float*>(smem + L_.dres);      // [KS][RD]
  double* lg = reinterpret_cast<double*>(smem + L_.lg);        // [E]

  GridBarrier bar;
  bar.base = a.bar;
  bar.ngroups = min(kGroups, NB);
  bar.group = b % bar.ngroups;
  bar.gsize = (NB - bar.group + bar.ngroups - 1) / bar.ngroups;
  bar.epoch = 0;

  // router geometry: RW rows per block, 8/RW segments per row
  const int RW = a.router_rows;                 // power of two <= 8
  const int NSEG = kWaves / RW;
  const int r_row = b + NB * (wave / NSEG);
  const int r_seg = wave % NSEG;
  const int seg_len = H / NSEG;                 // bf16 elements per segment
  const int seg_ch = seg_len / 8;               // 16-byte chunks per segment

  // gate/up tasks of this wave: t = wave*RPWG + m -> (slot j, section, row i)
  // down tasks: u = (wave*STEPSD + s)*RPSD + lane/LPRD -> (slot j, row i)
  u32x4 wr[CPLR];
  u32x4 qg[RPWG][CPLG];
  uint32_t sg[RPWG][CPLG];
  u32x4 qd[STEPSD][CPLD];
  uint32_t sd[STEPSD][CPLD];

  auto gu_task = [&](int m, int& j, int& sec, int& row) -> bool {
    const int t = wave * RPWG + m;
    j = t / (2 * RG);
    sec = (t / RG) % 2;
    row = b + NB * (t % RG);
    return j < KS && row < I;
  };
  auto load_router = [&](int layer) {
    const bool ok = r_row < E;
    const uint16_t* w = ok ? a.routers[layer] + (int64_t)r_row * H + (int64_t)r_seg * seg_len : nullptr;
#pragma unroll
    for (int c = 0; c < CPLR; ++c) {
      const int cc = lane + 64 * c;
      wr[c] = (ok && cc < seg_ch) ? load_stream(reinterpret_cast<const u32x4*>(w) + cc)
                                  : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // gate/up rows of slots in [jlo, jhi) (the shared slots are known early)
  auto load_gu = [&](int layer, int jlo, int jhi, const uint8_t* const* blobs_by_slot) {
    const int64_t row_bytes = (int64_t)H * BITS / 8;
    const int gpr = H / 64;
#pragma unroll
    for (int m = 0; m < RPWG; ++m) {
      int j, sec, row;
      const bool ok = gu_task(m, j, sec, row);
      if (!(ok && j >= jlo && j < jhi)) continue;
      const uint8_t* blob = blobs_by_slot[j];
      if (blob == nullptr) {   // missing table entry: contribute nothing
#pragma unroll
        for (int c = 0; c < CPLG; ++c) { qg[m][c] = u32x4{0u, 0u, 0u, 0u}; sg[m][c] = 0u; }
        continue;
      }
      const uint32_t* sb = reinterpret_cast<const uint32_t*>(blob + 3 * (int64_t)H * I * BITS / 8);
      const int r = sec * I + row;   // row of [gate; up]
#pragma unroll
      for (int c = 0; c < CPLG; ++c) {
        const int cc = lane + 64 * c;
        if (cc < nchG) {
          qg[m][c] = load_stream(reinterpret_cast<const u32x4*>(blob + r * row_bytes) + cc);
          sg[m][c] = load_stream(sb + (int64_t)r * gpr + (cc * PC) / 64);
        } else {
          qg[m][c] = u32x4{0u, 0u, 0u, 0u};
          sg[m][c] = 0u;
        }
      }
    }
    (void)layer;
  };
  auto load_down = [&](const uint8_t* const* blobs_by_slot) {
    const int64_t row_bytes = (int64_t)I * BITS / 8;
    const int gpr = I / 64;
    const int sub = lane % LPRD;
#pragma unroll
    for (int s = 0; s < STEPSD; ++s) {
      const int u = (wave * STEPSD + s) * RPSD + lane / LPRD;
      const int j = u / RD, row = b + NB * (u % RD);
      const bool ok = j < KS && row < H && blobs_by_slot[j < KS ? j : 0] != nullptr;
#pragma unroll
      for (int c = 0; c < CPLD; ++c) {
        const int cc = sub + LPRD * c;
        if (ok && cc < nchD) {
          const uint8_t* blob = blobs_by_slot[j];
          const int64_t qoff = 2 * (int64_t)H * I * BITS / 8;
          const uint32_t* sb = reinterpret_cast<const uint32_t*>(
              blob + 3 * (int64_t)H * I * BITS / 8 + 2 * (int64_t)H * I / 64 * 4);
          qd[s][c] = load_stream(reinterpret_cast<const u32x4*>(blob + qoff + row * row_bytes) + cc);
          sd[s][c] = load_stream(sb + (int64_t)row * gpr + (cc * PC) / 64);
        } else {
          qd[s][c] = u32x4{0u, 0u, 0u, 0u};
          sd[s][c] = 0u;
        }
      }
    }
  };

  // diagnostic phase stamps (block 0, after a block-wide barrier)
  auto stamp = [&](int li, int ev) {
    if (a.clocks && b == 0) {
      __syncthreads();
      if (tid == 0) a.clocks[(int64_t)li * kStackClockEvents + ev] = (int64_t)wall_clock64();
    }
  };

  // prologue: first layer's router rows and shared-expert gate/up rows
  const int l0 = a.layer0;
  if (tid < S) eblob[K + tid] = blob_of(a, l0, E + tid);
  __syncthreads();
  load_router(l0);
  load_gu(l0, K, KS, eblob);

  for (int li = 0; li < a.L; ++li) {
    const int layer = l0 + li;
    stamp(li, 0);
    // ---------------------------------------------------------- phase R
    // h -> LDS (agent-scope loads: h was written by every block)
    {
      constexpr int kMaxPer = MOEQ_MAX_HIDDEN / 2 / kThreads;   // u64 per thread
      uint64_t hv[kMaxPer];
      const uint64_t* src = reinterpret_cast<const uint64_t*>(a.h);
#pragma unroll
      for (int i = 0; i < kMaxPer; ++i) {
        const int p = tid + i * kThreads;
        hv[i] = (2 * p < H) ? ld_agent(src + p) : 0ull;
      }
      double ss = 0.0;
#pragma unroll
      for (int i = 0; i < kMaxPer; ++i) {
        const int p = tid + i * kThreads;
        if (2 * p < H) {
          const float lo = __uint_as_float((uint32_t)hv[i]), hi = __uint_as_float((uint32_t)(hv[i] >> 32));
          hs[2 * p] = lo;
          hs[2 * p + 1] = hi;
          ss = fma((double)lo, (double)lo, ss);
          ss = fma((double)hi, (double)hi, ss);
        }
      }
      ss = wave_sum_f64(ss);
      if (lane == 0) ssum[wave] = ss;
    }
    __syncthreads();
    stamp(li, 1);
    double ss = 0.0;
    for (int i = 0; i < kWaves; ++i) ss += ssum[i];
    const double inv = 1.0 / sqrt(ss / (double)H + 1e-6);

    // router: fp64 partial dot of this wave's segment
    {
      double acc = 0.0;
      if (r_row < E) {
#pragma unroll
        for (int c = 0; c < CPLR; ++c) {
          const int cc = lane + 64 * c;
          if (cc < seg_ch) {
            const float* hp = hs + r_seg * seg_len + 8 * cc;
            const float4 x0 = *reinterpret_cast<const float4*>(hp);
            const float4 x1 = *reinterpret_cast<const float4*>(hp + 4);
            acc = fma((double)bf16_lo(wr[c][0]), (double)x0.x, acc);
            acc = fma((double)bf16_hi(wr[c][0]), (double)x0.y, acc);
            acc = fma((double)bf16_lo(wr[c][1]), (double)x0.z, acc);
            acc = fma((double)bf16_hi(wr[c][1]), (double)x0.w, acc);
            acc = fma((double)bf16_lo(wr[c][2]), (double)x1.x, acc);
            acc = fma((double)bf16_hi(wr[c][2]), (double)x1.y, acc);
            acc = fma((double)bf16_lo(wr[c][3]), (double)x1.z, acc);
            acc = fma((double)bf16_hi(wr[c][3]), (double)x1.w, acc);
          }
        }
      }
      acc = wave_sum_f64(acc);
      if (lane == 0) rpart[wave] = acc;
    }
    __syncthreads();
    if (lane == 0 && r_seg == 0 && r_row < E) {
      double d = 0.0;
      for (int sgi = 0; sgi < NSEG; ++sgi) d += rpart[wave + sgi];
      st_agent(a.logits + r_row, d * inv);
    }
    stamp(li, 2);
    // stage xhat (fp16 pairs) from the LDS copy of h while others finish
    {
      auto loader = [&](int, int64_t o, float* v) {
#pragma unroll
        for (int j = 0; j < Pack<BITS>::kPerWord; ++j) v[j] = hs[o + j];
      };
      stage_batch<BITS, 1, 1>(1, H, loader, true, xp, xs, undo_x, red);
    }
    stamp(li, 3);
    if (!bar.sync(a.status, &bar_flag)) return;
    stamp(li, 4);

    // ---------------------------------------------------------- phase G
    if (wave == 0) {
      for (int base = 0; base < E; base += 64 * 8) {
        double v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = base + 64 * i + lane;
          v[i] = e < E ? ld_agent(a.logits + e) : 0.0;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = base + 64 * i + lane;
          if (e < E) lg[e] = v[i];
        }
      }
      __builtin_amdgcn_wave_barrier();
      wave_topk(lg, E, K, sel, selv);
      const float w = wave_softmax_weight(lg, E, K, selv, a.no_renorm != 0);
      if (lane < K) {
        selw[lane] = w;
        eblob[lane] = blob_of(a, layer, sel[lane]);
        if (eblob[lane] == nullptr) set_status(a.status, kStatusBadExpert);
        if (b == 0 && a.topk_trace) a.topk_trace[(int64_t)li * K + lane] = sel[lane];
      }
    }
    __syncthreads();
    stamp(li, 5);
    load_gu(layer, 0, K, eblob);     // routed gate/up rows
    load_down(eblob);                // down rows of every slot
    {
      const float ux = undo_x[0];
#pragma unroll
      for (int m = 0; m < RPWG; ++m) {
        int j, sec, row;
        const bool ok = gu_task(m, j, sec, row);
        if (!ok) continue;
        float part = 0.0f;
#pragma unroll
        for (int c = 0; c < CPLG; ++c) {
          const int cc = lane + 64 * c;
          if (cc < nchG) part += chunk_affine(chunk_dot<BITS>(qg[m][c], xp + cc * PPC), sg[m][c], xs[cc]);
        }
        const float v = wave_sum(part) * ux;
        if (lane == 0) gres[(j * 2 + sec) * RG + (row - b) / NB] = v;
      }
    }
    __syncthreads();
    stamp(li, 6);
    for (int t = tid; t < KS * RG; t += kThreads) {
      const int j = t / RG, i = t - j * RG, row = b + NB * i;
      if (row < I) {
        const float g = gres[(j * 2) * RG + i], u = gres[(j * 2 + 1) * RG + i];
        st_agent(a.abuf + (int64_t)j * I + row, g / (1.0f + __expf(-g)) * u);
      }
    }
    stamp(li, 7);
    if (!bar.sync(a.status, &bar_flag)) return;
    stamp(li, 8);

    // ---------------------------------------------------------- phase D
    {
      auto loader = [&](int m, int64_t o, float* v) {
        const float* src = a.abuf + (int64_t)m * I + o;
#pragma unroll
        for (int j = 0; j < Pack<BITS>::kPerWord; j += 2) {
          const uint64_t p = ld_agent(reinterpret_cast<const uint64_t*>(src + j));
          v[j] = __uint_as_float((uint32_t)p);
          v[j + 1] = __uint_as_float((uint32_t)(p >> 32));
        }
      };
      stage_batch<BITS, 1, KSMAX>(KS, I, loader, false, ap, as, undo_a, red);
    }
    stamp(li, 9);
    {
      const int sub = lane % LPRD;
#pragma unroll
      for (int s = 0; s < STEPSD; ++s) {
        const int u = (wave * STEPSD + s) * RPSD + lane / LPRD;
        const int j = u / RD, i = u % RD;
        const bool ok = j < KS && b + NB * i < H;
        const int jj = ok ? j : 0;
        float part = 0.0f;
#pragma unroll
        for (int c = 0; c < CPLD; ++c) {
          const int cc = sub + LPRD * c;
          if (ok && cc < nchD)
            part += chunk_affine(chunk_dot<BITS>(qd[s][c], ap + (int64_t)jj * (I / 2) + cc * PPC), sd[s][c],
                                 as[jj * nchD + cc]);
        }
        const float d = group_sum(part, LPRD) * undo_a[jj];
        if (ok && sub == 0) dres[j * RD + i] = d;
      }
    }
    __syncthreads();
    const bool last = li + 1 == a.L;
    for (int i = tid; i < RD; i += kThreads) {
      const int row = b + NB * i;
      if (row < H) {
        float acc = hs[row];
        for (int j = 0; j < K; ++j) acc = fmaf(selw[j], dres[j * RD + i], acc);
        for (int j = K; j < KS; ++j) acc = fmaf(1.0f, dres[j * RD + i], acc);
        if (a.h_trace) a.h_trace[(int64_t)li * H + row] = hs[row];
        st_agent(a.h + row, acc);
      }
    }
    stamp(li, 10);
    if (last) break;   // h of the last layer is complete when the launch ends
    {
      const int next = layer + 1;
      if (tid < S) eblob[K + tid] = blob_of(a, next, E + tid);
      __syncthreads();
      load_router(next);
      load_gu(next, K, KS, eblob);
    }
    stamp(li, 11);
    if (!bar.sync(a.status, &bar_flag)) return;
  }
}

__global__ void reset_barrier_kernel(uint32_t* bar) {
  for (int i = threadIdx.x; i < kBarWords; i += blockDim.x) bar[i] = 0u;
}

template <int BITS, int CPLR, int CPLG, int RPWG, int LPRD, int CPLD, int STEPSD, int KSMAX>
hipError_t launch_t(const StackArgs& a, int nb, size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL(reset_barrier_kernel, dim3(1), dim3(256), 0, stream, a.bar);
  StackArgs args = a;
  void* params[] = {&args};
  return hipLaunchCooperativeKernel(
      reinterpret_cast<const void*>(&stack_kernel<BITS, CPLR, CPLG, RPWG, LPRD, CPLD, STEPSD, KSMAX>),
      dim3(nb), dim3(kThreads), params, (unsigned int)lds, stream);
}

int device_cus() {
  static int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
  }();
  return n;
}

// Does instantiation <BITS, CPLR, CPLG, RPWG, LPRD, CPLD, STEPSD, KSMAX>
// cover this shape on nb blocks?
struct Geometry {
  int nb, rw, H, I, E, KS, bits;
  bool fits(int BITS, int CPLR, int CPLG, int RPWG, int LPRD, int CPLD, int STEPSD, int KSMAX) const {
    if (bits != BITS || KS > KSMAX) return false;
    const int PC = 128 / BITS;
    const int seg_ch = H / (kWaves / rw) / 8;
    if (seg_ch > 64 * CPLR || (H / (kWaves / rw)) % 8) return false;
    if (H / PC > 64 * CPLG) return false;
    const int RG = (I + nb - 1) / nb, RD = (H + nb - 1) / nb;
    if (KS * 2 * RG > kWaves * RPWG) return false;
    const int nchd = I / PC;
    if (nchd > LPRD * CPLD) return false;
    if (KS * RD > kWaves * STEPSD * (64 / LPRD)) return false;
    if (H * BITS / 32 > kThreads || I * BITS / 32 > kThreads) return false;   // one staged word per thread
    return true;
  }
};

}  // namespace

int stack_barrier_words() { return kBarWords; }

// Geometry check and dispatch.  Returns hipErrorNotSupported (without
// launching) when no persistent instantiation covers the shape; the caller
// then runs the layers one launch at a time.
hipError_t launch_stack_decode(StackArgs& a, hipStream_t stream) {
  const int nb = device_cus();
  if (nb < 1) return hipErrorNoDevice;
  const int KS = a.K + a.S;
  if (a.K < 1 || KS > kMaxKS) return hipErrorNotSupported;
  const int rw_need = (a.E + nb - 1) / nb;
  int rw = 1;
  while (rw < rw_need) rw <<= 1;
  if (rw > kWaves) return hipErrorNotSupported;
  a.router_rows = rw;
  const int PC = 128 / a.bits;
  const int RG = (a.I + nb - 1) / nb, RD = (a.H + nb - 1) / nb;
  const size_t lds = (size_t)stack_lds_layout(a.H, a.I, a.E, KS, PC, RG, RD).total;
  if (lds > 96 * 1024) return hipErrorNotSupported;
  const Geometry g{nb, rw, a.H, a.I, a.E, KS, a.bits};
  // hidden 4096, intermediate 1024, 512 experts on 256 CUs, 4-bit K+S <= 4
  // or 2-bit K+S <= 5; a small shape for tests; else the per-layer path.
  if (g.fits(4, 2, 2, 4, 32, 1, 4, 4)) return launch_t<4, 2, 2, 4, 32, 1, 4, 4>(a, nb, lds, stream);
  if (g.fits(2, 2, 1, 5, 16, 1, 3, 5)) return launch_t<2, 2, 1, 5, 16, 1, 3, 5>(a, nb, lds, stream);
  if (g.fits(4, 1, 1, 1, 4, 1, 1, 4)) return launch_t<4, 1, 1, 1, 4, 1, 1, 4>(a, nb, lds, stream);
  return hipErrorNotSupported;
}

}  // namespace moeq

// Block-cooperative staging of several activation vectors into LDS in the
// fp16 pair layout the dequantised dot products read (see moeq_device.hpp).
#pragma once

#include "moeq_device.hpp"

namespace moeq {

constexpr int kMaxStage = 8;   // vectors staged at once

// Stage nvec vectors of n values.  src(m, j) gives the raw value j of vector
// m; with `rmsnorm` each vector is first scaled by 1/sqrt(mean(v^2) + 1e-6).
// pairs: [nvec][n/2] u32, xsum: [nvec][n / chunk] f32, undo: [nvec] f32,
// red: 2 * kMaxStage * nwaves floats of scratch.  Whole block; ends synced.
template <int BITS, class Src>
__device__ __forceinline__ void stage_many(int nvec, int n, Src src, bool rmsnorm,
                                           uint32_t* __restrict__ pairs,
                                           float* __restrict__ xsum, float* __restrict__ undo,
                                           float* __restrict__ red) {
  constexpr int PW = Pack<BITS>::kPerWord;
  constexpr int HP = PW / 2;
  constexpr int PPC = 4 * HP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  // pass 1: sum of squares and max |v| per vector
  for (int m = 0; m < nvec; ++m) {
    float ss = 0.0f, mx = 0.0f;
    for (int j = tid; j < n; j += blockDim.x) {
      float v = src(m, j);
      ss = fmaf(v, v, ss);
      mx = fmaxf(mx, fabsf(v));
    }
    ss = wave_sum(ss);
    mx = wave_max(mx);
    if (lane == 0) { red[(2 * m) * nw + wave] = ss; red[(2 * m + 1) * nw + wave] = mx; }
  }
  __syncthreads();
  // pass 2: fp16 pairs, after the per-vector norm and power-of-two rescale
  const int np = n / 2;
  for (int m = 0; m < nvec; ++m) {
    float ss = 0.0f, mx = 0.0f;
    for (int i = 0; i < nw; ++i) { ss += red[(2 * m) * nw + i]; mx = fmaxf(mx, red[(2 * m + 1) * nw + i]); }
    const float mul = rmsnorm ? 1.0f / sqrtf(ss / (float)n + 1e-6f) : 1.0f;
    const float p = pow2_stage_factor(mx * mul);
    const float f = mul * p;
    if (tid == 0) undo[m] = 1.0f / p;
    uint32_t* dst = pairs + (int64_t)m * np;
    for (int i = tid; i < np; i += blockDim.x) {
      int w = i / HP, mm = i - w * HP;
      int j = w * PW + mm;
      dst[i] = pack_half2(src(m, j) * f, src(m, j + HP) * f);
    }
  }
  __syncthreads();
  // pass 3: per-chunk sums of the rounded values
  const int nch = n / Pack<BITS>::kPerChunk;
  for (int idx = tid; idx < nvec * nch; idx += blockDim.x) {
    int m = idx / nch, c = idx - m * nch;
    const uint32_t* p = pairs + (int64_t)m * np + c * PPC;
    float s = 0.0f;
    for (int i = 0; i < PPC; ++i) s += half_lo(p[i]) + half_hi(p[i]);
    xsum[idx] = s;
  }
  __syncthreads();
}

}  // namespace moeq

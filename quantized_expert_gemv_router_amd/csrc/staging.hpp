// Block-cooperative staging of activation vectors into LDS in the fp16 pair
// layout the dequantised dot products read (see moeq_device.hpp).
//
// Work unit: one packed word's worth of inputs (8 values at 4-bit, 16 at
// 2-bit).  Thread i owns words i, i + blockDim, ... of every vector; all
// its global loads are issued before any use, so a staging pass costs one
// memory latency.  Each thread then writes its words' fp16 pairs and sums
// them; the four words of a 16-byte chunk belong to four consecutive
// threads, whose sums are combined with two lane shuffles.
#pragma once

#include "moeq_device.hpp"

namespace moeq {

// Loads PW consecutive activation values starting at element o of x
// (bf16 or fp32, 16-byte aligned runs).
template <int PW>
__device__ __forceinline__ void load_act(const void* x, int x_f32, int64_t o, float* v) {
  if (x_f32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + o);
#pragma unroll
    for (int i = 0; i < PW / 4; ++i) {
      float4 f = p[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + o);
#pragma unroll
    for (int i = 0; i < PW / 8; ++i) {
      uint4 u = p[i];
      v[8 * i + 0] = bf16_lo(u.x); v[8 * i + 1] = bf16_hi(u.x);
      v[8 * i + 2] = bf16_lo(u.y); v[8 * i + 3] = bf16_hi(u.y);
      v[8 * i + 4] = bf16_lo(u.z); v[8 * i + 5] = bf16_hi(u.z);
      v[8 * i + 6] = bf16_lo(u.w); v[8 * i + 7] = bf16_hi(u.w);
    }
  }
}

// SwiGLU of PW consecutive intermediate values: silu(g) * u, reading
// g at gu[o..] and u at gu[I + o..] (fp32).
template <int PW>
__device__ __forceinline__ void load_swiglu(const float* gu, int I, int64_t o, float* v) {
  const float4* pg = reinterpret_cast<const float4*>(gu + o);
  const float4* pu = reinterpret_cast<const float4*>(gu + I + o);
#pragma unroll
  for (int i = 0; i < PW / 4; ++i) {
    float4 g = pg[i], u = pu[i];
    v[4 * i + 0] = g.x / (1.0f + __expf(-g.x)) * u.x;
    v[4 * i + 1] = g.y / (1.0f + __expf(-g.y)) * u.y;
    v[4 * i + 2] = g.z / (1.0f + __expf(-g.z)) * u.z;
    v[4 * i + 3] = g.w / (1.0f + __expf(-g.w)) * u.w;
  }
}

// Stage nvec (<= MMAX) vectors of n values (n a multiple of 64, n / PW <=
// WMAX * blockDim).  load(m, o, v) fills v[0..PW) with values o..o+PW of
// vector m.  With `rmsnorm` each vector is scaled by 1/sqrt(mean(v^2)+1e-6)
// first.  Then each vector is rescaled by a power of two p (max|v| * p in
// [2^14, 2^15)), rounded to fp16 pairs in the slot layout chunk_dot reads,
// and summed per 16-byte chunk.
// pairs: [nvec][n/2] u32 (16-byte aligned), xsum: [nvec][kChunkSums * n /
// chunk] f32 (8-byte aligned), undo: [nvec] f32 (= 1/p), red: 2 * MMAX *
// nwaves floats.  Whole block; returns after a barrier.
template <int BITS, int WMAX, int MMAX, class Loader>
__device__ __forceinline__ void stage_batch(int nvec, int n, Loader load, bool rmsnorm,
                                            uint32_t* __restrict__ pairs,
                                            float* __restrict__ xsum, float* __restrict__ undo,
                                            float* __restrict__ red) {
  constexpr int PW = Pack<BITS>::kPerWord;
  constexpr int HP = PW / 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int nwords = n / PW;
  const int np = n / 2;
  const int nch = n / Pack<BITS>::kPerChunk;
  float v[MMAX][WMAX][PW];
#pragma unroll
  for (int m = 0; m < MMAX; ++m) {
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      const int w = tid + i * blockDim.x;
      if (m < nvec && w < nwords) {
        load(m, (int64_t)w * PW, v[m][i]);
      } else {
#pragma unroll
        for (int j = 0; j < PW; ++j) v[m][i][j] = 0.0f;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MMAX; ++m) {
    if (m < nvec) {
      float ss = 0.0f, mx = 0.0f;
#pragma unroll
      for (int i = 0; i < WMAX; ++i)
#pragma unroll
        for (int j = 0; j < PW; ++j) {
          ss = fmaf(v[m][i][j], v[m][i][j], ss);
          mx = fmaxf(mx, fabsf(v[m][i][j]));
        }
      ss = wave_sum(ss);
      mx = wave_max(mx);
      if (lane == 0) { red[(2 * m) * nw + wave] = ss; red[(2 * m + 1) * nw + wave] = mx; }
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < MMAX; ++m) {
    if (m < nvec) {
      float ss = 0.0f, mx = 0.0f;
      for (int i = 0; i < nw; ++i) {
        ss += red[(2 * m) * nw + i];
        mx = fmaxf(mx, red[(2 * m + 1) * nw + i]);
      }
      const float mul = rmsnorm ? 1.0f / sqrtf(ss / (float)n + 1e-6f) : 1.0f;
      const float p = pow2_stage_factor(mx * mul);
      const float f = mul * p;
      if (tid == 0) undo[m] = 1.0f / p;
#pragma unroll
      for (int i = 0; i < WMAX; ++i) {
        const int w = tid + i * blockDim.x;
        float X = 0.0f, Xs = 0.0f;
        if (w < nwords) {
          uint32_t pr[HP];
          pack_word<BITS>(v[m][i], f, pr, X, Xs);
          store_word<BITS>(pairs + (int64_t)m * np, w, nch, pr);
        }
        // words 4c..4c+3 of chunk c sit in four consecutive lanes
        X += __shfl_xor(X, 1, 64);
        X += __shfl_xor(X, 2, 64);
        Xs += __shfl_xor(Xs, 1, 64);
        Xs += __shfl_xor(Xs, 2, 64);
        if ((tid & 3) == 0 && w < nwords)
          *reinterpret_cast<float2*>(xsum + (int64_t)m * kChunkSums * nch + kChunkSums * (w >> 2)) =
              make_float2(X, Xs);
      }
    }
  }
  __syncthreads();
}

}  // namespace moeq

// Device twin of synth_host.c: fills expert blobs in HBM from the same
// counter-based SplitMix64 streams (Steele, Lea, Flood, OOPSLA 2014), byte
// for byte identical to the host generator.  Input generation only; no step
// of the expert path's arithmetic lives here.
//
// The scale formula is a separately rounded fp64 multiply then add
// (__dmul_rn / __dadd_rn, so no fused multiply-add can form), matching the
// host build's -ffp-contract=off.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint32_t layer, uint32_t unit,
                                               uint32_t tensor, uint32_t bits) {
  uint64_t k = mix64(seed ^ 0x6D6F65715F736565ULL);
  k = mix64(k + (((uint64_t)layer << 32) | (uint64_t)unit));
  k = mix64(k + (((uint64_t)tensor << 8) | (uint64_t)bits));
  return k;
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct Spec {
  int32_t hidden, inter, bits, group;
  float s_lo, s_hi, bias_mult;
  uint64_t seed;
};

// grid: (blocks over words, experts); each thread writes u32 words.
__global__ void fill_experts_kernel(Spec s, uint32_t layer, uint32_t first_expert,
                                    int64_t stride, uint8_t* out) {
  const uint32_t expert = first_expert + blockIdx.y;
  const int64_t qw = (int64_t)s.hidden * s.inter * s.bits / 32;     // words per q section
  const int64_t sbw = (int64_t)s.hidden * s.inter / s.group;        // words per sb section
  const int64_t total = 3 * (qw + sbw);
  uint32_t* blob = reinterpret_cast<uint32_t*>(out + (int64_t)blockIdx.y * stride);
  uint64_t keys[6];
#pragma unroll
  for (int t = 0; t < 6; ++t) keys[t] = stream_key(s.seed, layer, expert, (uint32_t)t, (uint32_t)s.bits);
  const double span = (double)s.s_hi - (double)s.s_lo;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total;
       w += (int64_t)gridDim.x * blockDim.x) {
    int t;
    int64_t i;
    if (w < 3 * qw) { t = (int)(w / qw); i = w - t * qw; }
    else { int64_t r = w - 3 * qw; t = 3 + (int)(r / sbw); i = r - (t - 3) * sbw; }
    const uint64_t h = mix64(keys[t] + ((uint64_t)i + 1) * kGamma);
    uint32_t v;
    if (t < 3) {
      v = (uint32_t)h;
    } else {
      const double u = (double)(h >> 40) * (1.0 / 16777216.0);
      const double sd = __dadd_rn((double)s.s_lo, __dmul_rn(span, u));
      const uint16_t sc = f32_to_bf16_rne((float)sd);
      const float bias = s.bias_mult * __uint_as_float((uint32_t)sc << 16);
      v = (uint32_t)sc | ((uint32_t)f32_to_bf16_rne(bias) << 16);
    }
    blob[w] = v;
  }
}

}  // namespace

extern "C" {

// Fill `count` blobs of one layer at out + i*stride (device memory, stride a
// multiple of 4).  Asynchronous on `stream`; returns a hipError_t code.
int synth_device_fill_experts(const Spec* spec, uint32_t layer, uint32_t first_expert,
                              int32_t count, int64_t stride, void* out, void* stream) {
  if (count <= 0) return 0;
  const int threads = 256;
  const int blocks_x = 1024;
  hipLaunchKernelGGL(fill_experts_kernel, dim3(blocks_x, count), dim3(threads), 0,
                     static_cast<hipStream_t>(stream), *spec, layer, first_expert, stride,
                     static_cast<uint8_t*>(out));
  return (int)hipGetLastError();
}

}  // extern "C"

// Device fill for the seeded synthetic inputs: the counter-mode SplitMix64
// generator and the Irwin-Hall(4) draw defined in engram_synth/__init__.py,
// written out again here so that multi-gigabyte arrays (embedding tables,
// hidden states) are produced in HBM without a host round trip.  Holds no step
// of the Engram method.  Built with -ffp-contract=off: the value is one exact
// int->float conversion, one IEEE multiply and one IEEE add, as on the host.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float ih4(uint64_t key, uint64_t counter, float scale, float bias) {
  const uint64_t z = mix64(key + (counter + 1ull) * kGolden);
  const int32_t s = (int32_t)((z & 0xFFFFull) + ((z >> 16) & 0xFFFFull) + ((z >> 32) & 0xFFFFull) + (z >> 48));
  return __fadd_rn(__fmul_rn((float)(s - 131070), scale), bias);
}

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ void __launch_bounds__(256) fill_ih4_bf16(uint16_t* __restrict__ out, int64_t n, uint64_t key,
                                                     int64_t base, float scale, float bias) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = bf16_rne(ih4(key, (uint64_t)(base + i), scale, bias));
}

__global__ void __launch_bounds__(256) fill_ih4_f32(float* __restrict__ out, int64_t n, uint64_t key,
                                                    int64_t base, float scale, float bias) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = ih4(key, (uint64_t)(base + i), scale, bias);
}

}  // namespace

// Fill out[0..n) with stream elements base..base+n-1.  dtype 0 = float32,
// 1 = bfloat16 bits.  Returns 0 or a hipError_t code.
extern "C" int synth_fill_ih4(void* out, int64_t n, uint64_t key, int64_t base, float scale, float bias,
                              int dtype, hipStream_t stream) {
  if (n <= 0) return 0;
  if (out == nullptr || base < 0) return (int)hipErrorInvalidValue;
  const int64_t blocks64 = (n + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 262144 ? blocks64 : 262144);
  if (dtype == 1)
    fill_ih4_bf16<<<blocks, 256, 0, stream>>>((uint16_t*)out, n, key, base, scale, bias);
  else
    fill_ih4_f32<<<blocks, 256, 0, stream>>>((float*)out, n, key, base, scale, bias);
  return (int)hipGetLastError();
}

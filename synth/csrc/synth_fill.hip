// Device fills for the seeded synthetic inputs.  Same definition as the host
// generator in synth/__init__.py (SplitMix64 stream per tensor, Irwin-Hall(4)
// of its 16-bit fields scaled by one float32 multiply, bf16 by round to
// nearest even), so host and device draw bit-identical values.
// Holds no arithmetic of the model.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float normal_at(uint64_t key, uint64_t i, float scale) {
  const uint64_t z = mix64(key + (i + 1) * 0x9E3779B97F4A7C15ull);
  const int64_t s = (int64_t)(z & 0xFFFF) + (int64_t)((z >> 16) & 0xFFFF) + (int64_t)((z >> 32) & 0xFFFF) +
                    (int64_t)(z >> 48);
  return __fmul_rn((float)(s - 131070), scale);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct Fill4 {
  int64_t n0, n1, n2, n3;     // logical dims
  int64_t s0, s1, s2, s3;     // destination strides (elements)
  uint64_t key, start;
  float scale;
  int dtype;                  // 0 = float32, 1 = bf16
  int absval;
};

__global__ void fill_normal4(void* dst, Fill4 f) {
  const int64_t total = f.n0 * f.n1 * f.n2 * f.n3;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = i;
    const int64_t i3 = r % f.n3; r /= f.n3;
    const int64_t i2 = r % f.n2; r /= f.n2;
    const int64_t i1 = r % f.n1;
    const int64_t i0 = r / f.n1;
    const int64_t off = i0 * f.s0 + i1 * f.s1 + i2 * f.s2 + i3 * f.s3;
    float v = normal_at(f.key, f.start + (uint64_t)i, f.scale);
    if (f.absval) v = fabsf(v);
    if (f.dtype == 1) ((uint16_t*)dst)[off] = to_bf16(v);
    else ((float*)dst)[off] = v;
  }
}

__global__ void fill_uniform_int(int32_t* dst, int64_t n, uint64_t key, uint64_t start, uint32_t range) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t z = mix64(key + (start + (uint64_t)i + 1) * 0x9E3779B97F4A7C15ull);
    dst[i] = (int32_t)(((z >> 32) * (uint64_t)range) >> 32);
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

// Logical tensor [n0][n1][n2][n3] with generator index ((i0*n1+i1)*n2+i2)*n3+i3
// (offset by `start`) written at dst[i0*s0 + i1*s1 + i2*s2 + i3*s3].
int synth_fill_normal4(void* dst, int dtype, int64_t n0, int64_t n1, int64_t n2, int64_t n3, int64_t s0, int64_t s1,
                       int64_t s2, int64_t s3, uint64_t key, uint64_t start, float scale, int absval, void* stream) {
  if (!dst || n0 <= 0 || n1 <= 0 || n2 <= 0 || n3 <= 0) return -1;
  Fill4 f{n0, n1, n2, n3, s0, s1, s2, s3, key, start, scale, dtype, absval};
  fill_normal4<<<grid_for(n0 * n1 * n2 * n3), 256, 0, (hipStream_t)stream>>>(dst, f);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int synth_fill_uniform_int(int32_t* dst, int64_t n, uint64_t key, uint64_t start, uint32_t range, void* stream) {
  if (!dst || n <= 0 || range == 0) return -1;
  fill_uniform_int<<<grid_for(n), 256, 0, (hipStream_t)stream>>>(dst, n, key, start, range);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"

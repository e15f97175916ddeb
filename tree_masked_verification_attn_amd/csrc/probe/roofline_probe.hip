// Measured ceilings of the MI355X this library runs on, for the benchmark's "fraction of
// achievable" figures beside the published peaks: a streaming-read kernel (the HBM bandwidth a
// read-only kernel reaches) and a matrix-core kernel (the bf16 MFMA rate at the clock the chip
// holds under load).  Not part of the scoring pass; built into its own library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 8;   // sixteen-byte loads in flight per thread

// Every 16-byte unit of src read once (grid-stride over groups of kReadUnroll units per thread);
// an XOR of the words goes to sink[block] so the loads are not removed.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* src, size_t units, uint32_t* sink) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * kReadThreads * kReadUnroll;
  for (size_t base = (size_t)blockIdx.x * kReadThreads * kReadUnroll + threadIdx.x; base < units; base += stride) {
    uint4 r[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) {
      const size_t u = base + (size_t)k * kReadThreads;
      r[k] = u < units ? src[u] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) x ^= r[k].x ^ r[k].y ^ r[k].z ^ r[k].w;
  }
  for (int d = 32; d > 0; d >>= 1) x ^= (uint32_t)__shfl_xor((int)x, d);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, x);
}

// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave, iters rounds; the
// accumulators go to sink so the chain is not removed.
__global__ __launch_bounds__(256) void mfma_kernel(float* sink, int iters) {
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (float)(i + 1));
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from src once; sink must hold `grid` zeroed words.  Returns the
// HIP error of the launch.
int tavprobe_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, void* stream) {
  stream_read_kernel<<<grid, kReadThreads, 0, (hipStream_t)stream>>>((const uint4*)src, bytes / 16, sink);
  return (int)hipGetLastError();
}

// grid x 256 threads, 4 * iters MFMAs of 32 x 32 x 16 per wave (32768 flops each); sink holds
// grid * 256 floats.
int tavprobe_mfma(float* sink, int iters, int grid, void* stream) {
  mfma_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(sink, iters);
  return (int)hipGetLastError();
}

}  // extern "C"

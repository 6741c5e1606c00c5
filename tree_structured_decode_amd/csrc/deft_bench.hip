// Streaming-read calibration kernel (measurement aid beside libdeft): reads a
// buffer once with 16-byte vector loads and reduces it per work-group, so the
// benchmark can time the HBM read bandwidth the device actually reaches.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "deft_bench.h"

namespace {

constexpr int kThreads = 512;
constexpr int kBlocks = 256 * 8;   // eight 512-thread work-groups per compute unit of an MI355X

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each thread keeps four loads in flight per iteration (64 bytes), summed
// into registers; work-group sums go to `sink`.
__global__ __launch_bounds__(kThreads) void stream_read(const f32x4* src, size_t n16, float* sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const f32x4 a = __builtin_nontemporal_load(src + i);
    const f32x4 b = __builtin_nontemporal_load(src + i + stride);
    const f32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const f32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc += a + b + c + d;
  }
  for (; i < n16; i += stride) acc += __builtin_nontemporal_load(src + i);
  float v = acc[0] + acc[1] + acc[2] + acc[3];
  __shared__ float part[kThreads / 64];
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) s += part[w];
    sink[blockIdx.x] = s;
  }
}

}  // namespace

extern "C" {

size_t deft_bench_stream_read_sink_floats(void) { return kBlocks; }

int deft_bench_stream_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (!src || !sink || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0) return -1;
  hipLaunchKernelGGL(stream_read, dim3(kBlocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const f32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"

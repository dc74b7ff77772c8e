// Measurement helper, not part of the denoise path: a stream of independent
// v_mfma_f32_16x16x32 (fp16 or bf16) instructions with no memory traffic, to
// measure what the matrix cores sustain on this device (the ceiling the
// convolution kernels are compared with next to the published peak).
#include "internal.h"
#include "mfma_common.h"

namespace oidn {
namespace {

constexpr int kCalThreads = 256;
constexpr int kCalChains = 8;   // independent accumulators per wave

template <bool BF>
__global__ __launch_bounds__(kCalThreads) void mfma_stream(long iters, float* sink) {
  const int lane = threadIdx.x & 63;
  const uint4 a = make_uint4(0x3c003c00u ^ lane, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u);
  const uint4 b = make_uint4(0x3c003c00u, 0x3c003c00u ^ lane, 0x3c003c00u, 0x3c003c00u);
  // kCalChains independent accumulators, named one by one (an array of them
  // in the loop made the compiler shuffle registers between iterations)
  floatx4 c0{}, c1{}, c2{}, c3{}, c4{}, c5{}, c6{}, c7{};
  for (long i = 0; i < iters; ++i) {
    c0 = mfma16<BF>(a, b, c0);
    c1 = mfma16<BF>(a, b, c1);
    c2 = mfma16<BF>(a, b, c2);
    c3 = mfma16<BF>(a, b, c3);
    c4 = mfma16<BF>(a, b, c4);
    c5 = mfma16<BF>(a, b, c5);
    c6 = mfma16<BF>(a, b, c6);
    c7 = mfma16<BF>(a, b, c7);
  }
  const floatx4 s4 = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  const float s = s4[0] + s4[1] + s4[2] + s4[3];
  if (s == 1234.5f) sink[threadIdx.x] = s;   // never true for these operands; keeps the work
}

// A read stream: every lane loads 16-byte words, grid-strided over the
// buffer, streaming (non-temporal) so the lines are not kept.
__global__ __launch_bounds__(kCalThreads) void read_stream(const uint4* __restrict__ p, size_t n,
                                                           float* sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  unsigned acc = 0;
  const size_t stride = (size_t)gridDim.x * kCalThreads;
  for (size_t i = (size_t)blockIdx.x * kCalThreads + threadIdx.x; i < n; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = i + k * stride < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i + k * stride)
                                : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= v[k].x + v[k].y + v[k].z + v[k].w;
  }
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = (float)acc;   // keeps the loads
}

}  // namespace

hipError_t launch_read_stream(const void* p, size_t bytes, float* sink, hipStream_t stream) {
  const int blocks = 256 * 8;
  hipLaunchKernelGGL(read_stream, dim3(blocks), dim3(kCalThreads), 0, stream,
                     static_cast<const uint4*>(p), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_stream(int bf16, long iters, int blocks, float* sink, hipStream_t stream) {
  if (bf16)
    hipLaunchKernelGGL(mfma_stream<true>, dim3(blocks), dim3(kCalThreads), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_stream<false>, dim3(blocks), dim3(kCalThreads), 0, stream, iters, sink);
  return hipGetLastError();
}

long mfma_stream_flops(long iters, int blocks) {
  // 4 waves per block, kCalChains MFMAs of 16 x 16 x 32 per iteration
  return (long)blocks * 4 * kCalChains * iters * 2L * 16 * 16 * 32;
}

}  // namespace oidn

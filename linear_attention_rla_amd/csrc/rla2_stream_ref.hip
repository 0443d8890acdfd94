// Plain streaming kernels: the practical HBM reference for a given read/write mix.
//
// Measurement infrastructure for the benchmark, not part of the method: each kernel reads R
// input streams and writes W output streams of 16-byte vectors (R in 1..4, W in 0..2, or one
// stream read and written back in place), with the same non-temporal load and store policy as
// the library's kernels, four vectors per lane in flight, in one of two access patterns: a
// grid-stride loop over a fixed grid, or one 16 KB block of every stream per workgroup (all of
// its loads issued before its stores) over as many workgroups as there are blocks. Which one
// moves a mix faster depends on the mix, so the benchmark times both on 1 GiB streams and
// keeps the faster: the rate a kernel of the library reaches can then be set beside what a
// kernel that does nothing but move the same mix of bytes reaches on the same part (a
// reference, not a bound). Built into its own library (libstream_ref.so), loaded only by the
// benchmark.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

struct Streams {
  const f32x4* in[4];
  f32x4* out[2];
};

// BLOCKS: one block of kThreads * kUnroll vectors per workgroup (the grid covers the streams
// once); otherwise a grid-stride loop.
template <int R, int W, bool BLOCKS>
__global__ __launch_bounds__(kThreads) void stream_kernel(Streams s, size_t n, float* __restrict__ sink) {
  const size_t stride = BLOCKS ? n : (size_t)gridDim.x * kThreads * kUnroll;
  f32x4 keep = {0.f, 0.f, 0.f, 0.f};
  for (size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n; base += stride) {
    f32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i < n) {
#pragma unroll
        for (int r = 0; r < R; ++r) x[u] += __builtin_nontemporal_load(s.in[r] + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      if (i < n) {
#pragma unroll
        for (int w = 0; w < W; ++w) __builtin_nontemporal_store(x[u], s.out[w] + i);
      }
      keep += x[u];
    }
  }
  // read-only mixes keep their loads by storing one word per workgroup
  if (W == 0 && threadIdx.x == 0) sink[blockIdx.x] = keep.x + keep.y + keep.z + keep.w;
}

// one stream read and written back to the same place (the decode step's in-place state update)
template <bool BLOCKS>
__global__ __launch_bounds__(kThreads) void stream_inplace_kernel(f32x4* __restrict__ a, size_t n) {
  const size_t stride = BLOCKS ? n : (size_t)gridDim.x * kThreads * kUnroll;
  for (size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n; base += stride) {
    f32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      if (i < n) x[u] = a[i];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      if (i < n) __builtin_nontemporal_store(x[u] + 1.0f, a + i);
    }
  }
}

template <int R, int W>
hipError_t launch(const Streams& s, size_t n, float* sink, int grid, bool blocks, hipStream_t st) {
  if (blocks)
    hipLaunchKernelGGL((stream_kernel<R, W, true>), dim3(grid), dim3(kThreads), 0, st, s, n, sink);
  else
    hipLaunchKernelGGL((stream_kernel<R, W, false>), dim3(grid), dim3(kThreads), 0, st, s, n, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Streams `reads` inputs and `writes` outputs of `n_vec` 16-byte vectors each (reads 1..4,
// writes 0..2), or with in_place = 1 the single stream in[0] read and written back (reads = 1,
// writes = 1, out unused). All pointers are device pointers to at least n_vec * 16 bytes,
// 16-byte aligned. pattern 0: a grid-stride loop over `grid` workgroups of 256 threads (0
// chooses 2048); pattern 1: one 16 KB block per workgroup, ceil(n_vec / 1024) workgroups
// (`grid` ignored). `sink` receives one float per workgroup for read-only mixes (as many
// floats as workgroups). Asynchronous on `stream`. Returns the HIP error code of the launch
// (hipSuccess = 0), or hipErrorInvalidValue for an unsupported mix, pattern or size.
int rla2_stream_ref(int reads, int writes, int in_place, int pattern, const void* const* in, void* const* out,
                    size_t n_vec, float* sink, int grid, hipStream_t stream) {
  if (pattern != 0 && pattern != 1) return (int)hipErrorInvalidValue;
  const bool blocks = pattern == 1;
  if (blocks) {
    const size_t nb = (n_vec + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    if (nb == 0 || nb > 0x7fffffffu) return (int)hipErrorInvalidValue;
    grid = (int)nb;
  } else if (grid <= 0) {
    grid = 2048;
  }
  if (in == nullptr || in[0] == nullptr) return (int)hipErrorInvalidValue;
  if (in_place) {
    if (reads != 1 || writes != 1) return (int)hipErrorInvalidValue;
    f32x4* a = static_cast<f32x4*>(const_cast<void*>(in[0]));
    if (blocks)
      hipLaunchKernelGGL(stream_inplace_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, a, n_vec);
    else
      hipLaunchKernelGGL(stream_inplace_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, a, n_vec);
    return (int)hipGetLastError();
  }
  if (reads < 1 || reads > 4 || writes < 0 || writes > 2) return (int)hipErrorInvalidValue;
  if (writes == 0 && sink == nullptr) return (int)hipErrorInvalidValue;
  Streams s{};
  for (int r = 0; r < reads; ++r) {
    if (in[r] == nullptr) return (int)hipErrorInvalidValue;
    s.in[r] = static_cast<const f32x4*>(in[r]);
  }
  for (int w = 0; w < writes; ++w) {
    if (out == nullptr || out[w] == nullptr) return (int)hipErrorInvalidValue;
    s.out[w] = static_cast<f32x4*>(out[w]);
  }
  hipError_t e = hipErrorInvalidValue;
  switch (reads * 3 + writes) {
    case 1 * 3 + 0: e = launch<1, 0>(s, n_vec, sink, grid, blocks, stream); break;
    case 1 * 3 + 1: e = launch<1, 1>(s, n_vec, sink, grid, blocks, stream); break;
    case 1 * 3 + 2: e = launch<1, 2>(s, n_vec, sink, grid, blocks, stream); break;
    case 2 * 3 + 0: e = launch<2, 0>(s, n_vec, sink, grid, blocks, stream); break;
    case 2 * 3 + 1: e = launch<2, 1>(s, n_vec, sink, grid, blocks, stream); break;
    case 2 * 3 + 2: e = launch<2, 2>(s, n_vec, sink, grid, blocks, stream); break;
    case 3 * 3 + 0: e = launch<3, 0>(s, n_vec, sink, grid, blocks, stream); break;
    case 3 * 3 + 1: e = launch<3, 1>(s, n_vec, sink, grid, blocks, stream); break;
    case 3 * 3 + 2: e = launch<3, 2>(s, n_vec, sink, grid, blocks, stream); break;
    case 4 * 3 + 0: e = launch<4, 0>(s, n_vec, sink, grid, blocks, stream); break;
    case 4 * 3 + 1: e = launch<4, 1>(s, n_vec, sink, grid, blocks, stream); break;
    case 4 * 3 + 2: e = launch<4, 2>(s, n_vec, sink, grid, blocks, stream); break;
    default: break;
  }
  return (int)e;
}

}  // extern "C"

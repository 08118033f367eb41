// mlaq_diag.hip -- measurement floors for the benchmark (libmlaq_diag.so).
// Not part of the fused path. Two kernels give the cost of the launch shape
// itself in a hipGraph: one that does nothing, and one that streams the same
// bytes as the fused kernel's weight read (each 256-thread block reads 8 KiB,
// 16 bytes per lane per load) and writes nothing, so their per-node times are
// the floors the fused kernel's time is compared against.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void empty_kernel(uint32_t* sink) {
  if (threadIdx.x == 0xffffu) sink[0] = 1u; // never true: keeps the kernel non-empty for the compiler
}

// Block b reads bytes [8 KiB * b, 8 KiB * (b + 1)) of p.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* p, uint32_t* sink) {
  const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p + size_t(blockIdx.x) * 8192) + threadIdx.x;
  const u32x4_t a = q[0];
  const u32x4_t b = q[256];
  const uint32_t x = a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
  if (x == 0x9e3779b9u && threadIdx.x == 0) sink[0] = x; // data-dependent, practically never taken
}

} // namespace

extern "C" {

// Enqueue the empty kernel with `grid` blocks of 256 threads. `sink`: device
// uint32[1]. Returns 0 or a hipError_t value.
int mlaqdiag_empty(int grid, void* sink, void* stream) {
  if (grid < 1 || !sink) return int(hipErrorInvalidValue);
  void* args[] = {&sink};
  return int(hipLaunchKernel(reinterpret_cast<const void*>(&empty_kernel), dim3(grid), dim3(256), args, 0,
                             static_cast<hipStream_t>(stream)));
}

// Enqueue a read of `bytes` bytes at `p` (16-byte aligned, bytes a positive
// multiple of 8192): bytes / 8192 blocks of 256 threads. Returns 0 or a
// hipError_t value.
int mlaqdiag_stream_read(const void* p, size_t bytes, void* sink, void* stream) {
  if (!p || !sink || bytes == 0 || bytes % 8192 != 0 || (reinterpret_cast<uintptr_t>(p) & 15) != 0)
    return int(hipErrorInvalidValue);
  const uint8_t* pp = static_cast<const uint8_t*>(p);
  void* args[] = {&pp, &sink};
  return int(hipLaunchKernel(reinterpret_cast<const void*>(&stream_read_kernel), dim3(unsigned(bytes / 8192)),
                             dim3(256), args, 0, static_cast<hipStream_t>(stream)));
}

} // extern "C"

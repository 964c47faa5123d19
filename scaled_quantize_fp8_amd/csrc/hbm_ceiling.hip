// Measurement kernels for bench.py (not part of the library's boundary):
// plain HBM streams with the access pattern and launch shape of the cast and
// amax kernels but no arithmetic, so that each cast can be reported against
// what the memory system delivers for its own mix of reads and writes.
//   read   16-byte non-temporal loads, 8 in flight per lane, at most one
//          workgroup per compute unit (the amax pass's shape, grid-stride
//          over the rest); the loaded words are folded into one
//          value that is stored only if it equals a sentinel, so the loads
//          cannot be removed and nothing is written in practice;
//   r2w1   16 bytes read, 8 bytes written per lane-chunk (bf16 in, one byte
//          per element out: the per-tensor cast's 2:1 mix), 4 chunks in flight,
//          one iteration per lane (the cast's shape);
//   copy   16 bytes read and written per lane-chunk (1:1).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int kT = 256;

template <int U, int MODE>
__global__ __launch_bounds__(kT) void stream_ceiling_kernel(const v4u* __restrict__ x, int64_t n16,
                                                            void* __restrict__ y, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kT;
  int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(x + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (MODE == 0) {
        acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
      } else if constexpr (MODE == 1) {
        const v2u o = {v[u][0] ^ v[u][1], v[u][2] ^ v[u][3]};
        __builtin_nontemporal_store(o, reinterpret_cast<v2u*>(y) + i + u * stride);
      } else {
        __builtin_nontemporal_store(v[u], reinterpret_cast<v4u*>(y) + i + u * stride);
      }
    }
  }
  for (; i < n16; i += stride) {
    const v4u v = __builtin_nontemporal_load(x + i);
    if constexpr (MODE == 0) {
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    } else if constexpr (MODE == 1) {
      const v2u o = {v[0] ^ v[1], v[2] ^ v[3]};
      __builtin_nontemporal_store(o, reinterpret_cast<v2u*>(y) + i);
    } else {
      __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(y) + i);
    }
  }
  if constexpr (MODE == 0) {
    if (acc == 0x9e3779b9u) sink[0] = acc;
  }
}

unsigned blocks_for(int64_t n16, int64_t per_block) {
  int64_t b = (n16 + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > (1 << 20)) b = 1 << 20;
  return (unsigned)b;
}

}  // namespace

extern "C" {

// Returns 0, or -1 for a bad argument (x 16-byte aligned, bytes a multiple of
// 16; y sized bytes / 2 for r2w1 and bytes for copy, 16-byte aligned).
int sfp8_ceiling_read(const void* x, int64_t bytes, uint32_t* sink, hipStream_t s) {
  if (!x || !sink || bytes <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(x) % 16) return -1;
  const int64_t n16 = bytes / 16;
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || ncu <= 0)
    ncu = 256;
  unsigned nb = blocks_for(n16, (int64_t)kT * 8 * 8);
  if (nb > (unsigned)ncu) nb = (unsigned)ncu;
  hipLaunchKernelGGL((stream_ceiling_kernel<8, 0>), dim3(nb), dim3(kT), 0, s, static_cast<const v4u*>(x), n16,
                     nullptr, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int sfp8_ceiling_r2w1(const void* x, int64_t bytes, void* y, hipStream_t s) {
  if (!x || !y || bytes <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(x) % 16 ||
      reinterpret_cast<uintptr_t>(y) % 16)
    return -1;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL((stream_ceiling_kernel<4, 1>), dim3(blocks_for(n16, (int64_t)kT * 4)), dim3(kT), 0, s,
                     static_cast<const v4u*>(x), n16, y, nullptr);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int sfp8_ceiling_copy(const void* x, int64_t bytes, void* y, hipStream_t s) {
  if (!x || !y || bytes <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(x) % 16 ||
      reinterpret_cast<uintptr_t>(y) % 16)
    return -1;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL((stream_ceiling_kernel<4, 2>), dim3(blocks_for(n16, (int64_t)kT * 4)), dim3(kT), 0, s,
                     static_cast<const v4u*>(x), n16, y, nullptr);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"

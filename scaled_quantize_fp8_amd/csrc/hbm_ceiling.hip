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
//   copy   16 bytes read and written per lane-chunk (1:1);
//   t2w1   the transposed MX cast's pattern: bf16 [rows x cols] read in
//          128 x 64 or 128 x 128 tiles, one tile per workgroup (consecutive
//          lanes on consecutive 16-byte pieces of a row), and one byte per
//          element written at the transposed position, qT [cols x rows], as
//          whole 128-byte lines of qT (8 lanes per line); the written words
//          are the lane's loaded words folded together, not a transpose.
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

template <int TC, bool NT>
__global__ __launch_bounds__(kT) void transpose_ceiling_kernel(const uint8_t* __restrict__ x, int64_t ld_bytes,
                                                               uint8_t* __restrict__ q, int64_t ldq) {
  constexpr int RC = TC * 2 / 16;                   // 16-byte pieces per tile row
  constexpr int NR = 128 * RC / kT;                 // pieces read per lane
  constexpr int NW = TC * 8 / kT;                   // pieces written per lane (8 per qT line)
  const int64_t r0 = (int64_t)blockIdx.y * 128, c0 = (int64_t)blockIdx.x * TC;
  v4u v[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int idx = threadIdx.x + k * kT;
    v[k] = __builtin_nontemporal_load(
        reinterpret_cast<const v4u*>(x + (r0 + idx / RC) * ld_bytes + c0 * 2 + (idx % RC) * 16));
  }
  v4u f = v[0];
#pragma unroll
  for (int k = 1; k < NR; ++k) f ^= v[k];
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const int idx = threadIdx.x + k * kT;
    v4u* dst = reinterpret_cast<v4u*>(q + (c0 + idx / 8) * ldq + r0 + (idx % 8) * 16);
    const v4u o = f ^ (unsigned)k;
    if constexpr (NT) __builtin_nontemporal_store(o, dst);
    else *dst = o;
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

// x bf16 [rows x cols] with row stride ld elements, qT [cols x rows] bytes
// with row stride ldq; tiles of 128 x tc (tc 64 or 128); rows % 128 == 0,
// cols % tc == 0, x, qT, ld * 2 and ldq 16-byte aligned (else -1).  nt:
// non-temporal stores.
int sfp8_ceiling_t2w1(const void* x, int64_t rows, int64_t cols, int64_t ld, void* qT, int64_t ldq, int tc, int nt,
                      hipStream_t s) {
  if (!x || !qT || (tc != 64 && tc != 128) || rows <= 0 || cols <= 0 || rows % 128 || cols % tc || ld < cols ||
      ldq < rows || (ld * 2) % 16 || ldq % 16 || reinterpret_cast<uintptr_t>(x) % 16 ||
      reinterpret_cast<uintptr_t>(qT) % 16 || cols / tc > 0x7fffffff || rows / 128 > 65535)
    return -1;
  const dim3 grid((unsigned)(cols / tc), (unsigned)(rows / 128));
  const uint8_t* xp = static_cast<const uint8_t*>(x);
  uint8_t* qp = static_cast<uint8_t*>(qT);
  if (tc == 64 && nt) hipLaunchKernelGGL((transpose_ceiling_kernel<64, true>), grid, dim3(kT), 0, s, xp, ld * 2, qp, ldq);
  if (tc == 64 && !nt) hipLaunchKernelGGL((transpose_ceiling_kernel<64, false>), grid, dim3(kT), 0, s, xp, ld * 2, qp, ldq);
  if (tc == 128 && nt) hipLaunchKernelGGL((transpose_ceiling_kernel<128, true>), grid, dim3(kT), 0, s, xp, ld * 2, qp, ldq);
  if (tc == 128 && !nt) hipLaunchKernelGGL((transpose_ceiling_kernel<128, false>), grid, dim3(kT), 0, s, xp, ld * 2, qp, ldq);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"

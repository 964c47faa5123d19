// Host-side helpers for the C entry points: argument checks that run before
// any HIP call, launch-error mapping, and launch-shape choices.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "../../include/scaled_fp8.h"

namespace sfp8 {

inline bool valid_fmt(int f) { return f == FP8_E4M3 || f == FP8_E5M2; }
inline bool valid_mx_rule(int r) { return r == MX_RULE_FMAX || r == MX_RULE_OCP; }
inline bool valid_dtype(int d) { return d == FP8_DT_BF16 || d == FP8_DT_F32; }
inline int dtype_size(int d) { return d == FP8_DT_BF16 ? 2 : 4; }
inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Largest extent of one dimension or leading dimension, and largest element
// span of one matrix: every size product the host code forms afterwards
// (elements, bytes, tiles, scale blocks) then stays far inside int64.
constexpr int64_t kMaxExtent = int64_t(1) << 40;
constexpr int64_t kMaxSpan = int64_t(1) << 56;
inline bool extent_ok(int64_t v) { return v >= 0 && v <= kMaxExtent; }

// rows x cols matrix with leading dimension ld: sizes non-negative and within
// kMaxExtent, ld >= cols (ld is irrelevant when rows <= 1 but must still be
// >= cols if rows > 1), rows * max(ld, cols) within kMaxSpan.
inline int check_matrix(int64_t rows, int64_t cols, int64_t ld) {
  if (!extent_ok(rows) || !extent_ok(cols) || !extent_ok(ld)) return FP8_ERR_SHAPE;
  if (rows > 1 && ld < cols) return FP8_ERR_SHAPE;
  int64_t span;
  if (__builtin_mul_overflow(rows, ld > cols ? ld : cols, &span) || span > kMaxSpan) return FP8_ERR_SHAPE;
  return FP8_OK;
}

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? FP8_OK : FP8_ERR_LAUNCH;
}

// Workgroups for a streaming kernel over `units` work items of `per_block`
// items each, capped so that a grid-stride loop keeps each lane busy with a
// few iterations (256 CUs x 16 workgroups in flight).
// Compute units of the current device (the GEMM's small-grid threshold and
// persistent grid, the read-only passes' grid cap).  Cached per device
// (concurrent first calls store the same value).
inline int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

inline unsigned stream_blocks(int64_t units, int64_t per_block) {
  int64_t b = (units + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > (1 << 20)) b = 1 << 20;     // grid-stride loops cover the rest
  return (unsigned)b;
}

// Packed E8M0 scale layout (mx_pack_scales, mx_quantize_packed,
// mx_scaled_gemm_packed): per 256-row tile and group of 16 K-blocks, the
// tile's 256 x 16 codes as one contiguous 4 KiB block.
constexpr int kPackRows = 256, kPackBlocks = 16, kPackTile = kPackRows * kPackBlocks;
inline int64_t packed_scale_groups(int64_t kb) { return (kb + kPackBlocks - 1) / kPackBlocks; }
inline int64_t packed_bytes(int64_t rows, int64_t kb) {
  return ((rows + kPackRows - 1) / kPackRows) * packed_scale_groups(kb) * (int64_t)kPackTile;
}
// packed_bytes for caller-supplied sizes: -1 when they are out of range.
inline int64_t packed_bytes_checked(int64_t rows, int64_t kb) {
  if (!extent_ok(rows) || !extent_ok(kb)) return -1;
  int64_t t;
  if (__builtin_mul_overflow((rows + kPackRows - 1) / kPackRows, packed_scale_groups(kb), &t)) return -1;
  if (__builtin_mul_overflow(t, (int64_t)kPackTile, &t) || t > kMaxSpan) return -1;
  return t;
}

// Zero one float on `stream` with a tiny fill kernel (not hipMemsetAsync, so
// that the call sequence can be captured into a HIP graph safely).
void zero_float_async(float* p, hipStream_t stream);
// Zero an optional float and an optional 64-bit count with one fill kernel.
void zero_outputs_async(float* f, unsigned long long* n, hipStream_t stream);

}  // namespace sfp8

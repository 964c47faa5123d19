// Arguments of the streaming (one-read, optional-write) pass shared by
// fp8_amax and fp8_quantize.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfp8 {

struct StreamArgs {
  const void* x;           // [rows x cols] bf16 or f32, leading dimension ld (elements)
  int64_t rows, cols, ld;
  const int32_t* bias;     // device int32 exponent bias (quantize only)
  uint8_t* q;              // [rows x cols] FP8 codes, leading dimension ldq (quantize only)
  int64_t ldq;
  float* amax;             // device float, already zeroed (amax only)
  unsigned long long* sat; // device count of saturated elements, already zeroed (quantize; may be null)
};

// Enqueue one pass over x: cast to FP8 into q when write_q, max-reduce |x|
// into *amax when amax, count the elements the cast saturates into *a.sat
// when that pointer is set (casts only).  Picks the 16-byte vector kernel when the operands
// allow it and collapses contiguous matrices into one long row.
void launch_stream_pass(StreamArgs a, int dtype, int fmt, bool write_q, bool amax, hipStream_t stream);

}  // namespace sfp8

// Arguments of the streaming (one-read, optional-write) pass shared by
// fp8_amax and fp8_quantize.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfp8 {

// One step of delayed scaling in one launch (fp8_quantize_delayed): the
// amax window the bias comes from and is pushed into, the reduction state,
// and the step's outputs.
struct DelayedArgs {
  float* hist;                   // window of past amaxes (fp8_history_init)
  int32_t* state;                // [0] valid entries, [1] next slot
  int window, emax, margin;      // window length; bias rule of the format
  uint32_t* ws;                  // [0] ticket, [1] running max |x| bits, [2..3] saturated count (u64):
                                 // zero on entry, left zero
  int32_t* bias_out;
  float* amax_out;
  unsigned long long* sat_out;   // may be null
};

struct StreamArgs {
  const void* x;           // [rows x cols] bf16 or f32, leading dimension ld (elements)
  int64_t rows, cols, ld;
  const int32_t* bias;     // device int32 exponent bias (quantize only)
  uint8_t* q;              // [rows x cols] FP8 codes, leading dimension ldq (quantize only)
  int64_t ldq;
  float* amax;             // device float, already zeroed (amax only; written whole by the one-launch scale)
  unsigned long long* sat; // device count of saturated elements, already zeroed (quantize; may be null)
  // one-launch amax + scale (launch_amax_scale): reduction state and outputs
  uint32_t* ws;            // [0] ticket, [1] running max |x| bits (both 0 on entry, left 0)
  int emax, margin;        // bias rule of the format
  int32_t* bias_out;
  float* scale_out;        // optional
  float* scale_inv_out;    // optional
  DelayedArgs del;         // fp8_quantize_delayed only
};

// Reduction state of the one-launch amax + scale pass: a ticket and the
// running maximum, whatever the grid.
constexpr int64_t kAmaxScaleStateBytes = 8;
// ... and of the one-launch delayed step: ticket, running maximum, and a
// 64-bit saturation count.
constexpr int64_t kDelayedStateBytes = 16;

// One pass over x that reduces max |x| and derives the bias and scales from
// it in the same launch: each workgroup folds its maximum into a.ws[1] and
// takes a ticket in a.ws[0]; the last to finish writes *a.amax, *a.bias_out
// and the optional scales and resets both words.  a.ws must hold
// kAmaxScaleStateBytes, both words zero; launches sharing it must not overlap.
void launch_amax_scale(StreamArgs a, int dtype, hipStream_t stream);

// One step of delayed scaling over x in one launch: each workgroup takes the
// bias from the window (a.del), casts its share into a.q, and folds its
// maximum and saturation count into a.del.ws; the last to finish writes the
// bias, amax and count and pushes the amax into the window.
void launch_quantize_delayed(StreamArgs a, int dtype, int fmt, hipStream_t stream);

// Enqueue one pass over x: cast to FP8 into q when write_q, max-reduce |x|
// into *amax when amax, count the elements the cast saturates into *a.sat
// when that pointer is set (casts only).  Picks the 16-byte vector kernel when the operands
// allow it and collapses contiguous matrices into one long row.
void launch_stream_pass(StreamArgs a, int dtype, int fmt, bool write_q, bool amax, hipStream_t stream);

}  // namespace sfp8

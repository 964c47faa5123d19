// Per-tensor amax, exponent bias and delayed-scaling history for gfx950.
//
// "Training and inference of large language models using 8-bit floating
// point" (paper review), "Proposed method": per-tensor scaling biases come
// from each tensor's maximum absolute value through log2(format max / amax)
// with a configurable margin.  "Per-Tensor and Per-Block Scaling Strategies
// for Effective FP8 Training" (summary), "Key Questions Answered": delayed
// scaling takes the amax over a window of past iterations.
//
// The amax reduction itself shares the streaming kernel of quantize.hip
// (a pass that only reads); this file holds the scalar kernels and the
// entry points fp8_amax, fp8_amax_scale(_noalloc), fp8_compute_scale,
// fp8_history_*.
#include <mutex>

#include "common.hpp"
#include "host.hpp"
#include "stream_kernels.hpp"

namespace sfp8 {

static_assert(kAmaxScaleStateBytes <= FP8_AMAX_SCALE_WORKSPACE_BYTES && kDelayedStateBytes <= FP8_AMAX_SCALE_WORKSPACE_BYTES,
              "workspace holds the reduction state");

// Reduction state of fp8_amax_scale_noalloc: one copy per GPU, zeroed once
// when the library first uses it on that GPU; every call leaves its state
// words zero again.
constexpr int kScratchWords = FP8_AMAX_SCALE_WORKSPACE_BYTES / 4;
static __device__ __align__(256) uint32_t scratch[kScratchWords];

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// Device address of `scratch` on the current GPU (the host-side name is only
// a stand-in): looked up once per device with hipGetSymbolAddress, the array
// cleared on `stream` the first time; nullptr when the lookup fails.
static uint32_t* scratch_on_current_device(hipStream_t stream) {
  static std::mutex mu;
  static uint32_t* ptr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, stream, static_cast<uint32_t*>(p), kScratchWords);
    if (hipGetLastError() != hipSuccess) return nullptr;
    ptr[dev] = static_cast<uint32_t*>(p);
  }
  return ptr[dev];
}

__global__ void zero_float_kernel(float* p) { *p = 0.0f; }

void zero_float_async(float* p, hipStream_t stream) {
  hipLaunchKernelGGL(zero_float_kernel, dim3(1), dim3(1), 0, stream, p);
}

__global__ void zero_outputs_kernel(float* f, unsigned long long* n) {
  if (f) *f = 0.0f;
  if (n) *n = 0ull;
}

void zero_outputs_async(float* f, unsigned long long* n, hipStream_t stream) {
  if (f || n) hipLaunchKernelGGL(zero_outputs_kernel, dim3(1), dim3(1), 0, stream, f, n);
}

// One thread: bias and optional scales from one amax.
__global__ void compute_scale_kernel(const float* __restrict__ amax, int emax, int margin,
                                     int32_t* __restrict__ bias_out, float* __restrict__ scale_out,
                                     float* __restrict__ scale_inv_out) {
  const int b = bias_from_amax_bits(__float_as_uint(*amax), emax, margin, -126, 126);
  *bias_out = b;
  if (scale_out) *scale_out = pow2f(b);
  if (scale_inv_out) *scale_inv_out = pow2f(-b);
}

__global__ void history_init_kernel(float* __restrict__ hist, int32_t* __restrict__ state, int window) {
  for (int i = threadIdx.x; i < window; i += blockDim.x) hist[i] = 0.0f;
  if (threadIdx.x == 0) {
    state[0] = 0;
    state[1] = 0;
  }
}

__global__ void history_push_kernel(float* __restrict__ hist, int32_t* __restrict__ state, int window,
                                    const float* __restrict__ amax) {
  int count = state[0];
  int head = state[1];
  // a corrupted state is repaired into range rather than indexing outside hist
  head = (head < 0 || head >= window) ? 0 : head;
  count = count < 0 ? 0 : (count > window ? window : count);
  hist[head] = *amax;
  state[1] = (head + 1) % window;
  state[0] = count + 1 > window ? window : count + 1;
}

// Window maximum over the valid entries, then the bias rule.  The entries
// are amaxes (non-negative or NaN), so an unsigned compare of their bits is
// the float max with NaN on top.
__global__ void compute_scale_delayed_kernel(const float* __restrict__ hist, const int32_t* __restrict__ state,
                                             int window, int emax, int margin, int32_t* __restrict__ bias_out,
                                             float* __restrict__ scale_out, float* __restrict__ scale_inv_out) {
  __shared__ uint32_t red[4];
  int count = state[0];
  count = count < 0 ? 0 : (count > window ? window : count);
  uint32_t m = 0;
  for (int i = threadIdx.x; i < count; i += blockDim.x) {
    const uint32_t v = __float_as_uint(hist[i]) & 0x7fffffffu;
    m = m > v ? m : v;
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < (int)(blockDim.x / 64); ++i) m = m > red[i] ? m : red[i];
    m = m > red[0] ? m : red[0];
    const int b = bias_from_amax_bits(m, emax, margin, -126, 126);
    *bias_out = b;
    if (scale_out) *scale_out = pow2f(b);
    if (scale_inv_out) *scale_inv_out = pow2f(-b);
  }
}

}  // namespace sfp8

using namespace sfp8;

extern "C" {

const char* fp8_status_string(int status) {
  switch (status) {
    case FP8_OK: return "ok";
    case FP8_ERR_NULL: return "null pointer";
    case FP8_ERR_SHAPE: return "bad shape or leading dimension";
    case FP8_ERR_ALIGN: return "misaligned operand (16-byte base and leading dimension required)";
    case FP8_ERR_DTYPE: return "unknown data type";
    case FP8_ERR_FORMAT: return "unknown FP8 format";
    case FP8_ERR_LAUNCH: return "HIP launch failure";
    case FP8_ERR_UNSUPPORTED: return "unsupported combination";
    default: return "unknown status";
  }
}

int fp8_abi_version(void) { return 6; }

int fp8_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, float* amax_out,
             hipStream_t stream) {
  if (!amax_out) return FP8_ERR_NULL;
  if (!valid_dtype(dtype)) return FP8_ERR_DTYPE;
  int st = check_matrix(rows, cols, ld);
  if (st) return st;
  if (rows * cols > 0 && !x) return FP8_ERR_NULL;
  zero_float_async(amax_out, stream);
  if (rows * cols > 0) {
    StreamArgs a;
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld;
    a.bias = nullptr;
    a.q = nullptr;
    a.ldq = 0;
    a.amax = amax_out;
    a.sat = nullptr;
    launch_stream_pass(a, dtype, FP8_E4M3, /*write_q=*/false, /*amax=*/true, stream);
  }
  return launch_status();
}

// Checks and launch of fp8_amax_scale and fp8_amax_scale_noalloc.
static int amax_scale_impl(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int margin,
                           float* amax_out, int32_t* bias_out, float* scale_out, float* scale_inv_out,
                           uint32_t* state, hipStream_t stream) {
  StreamArgs a;
  a.x = x;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.bias = nullptr;
  a.q = nullptr;
  a.ldq = 0;
  a.amax = amax_out;
  a.sat = nullptr;
  a.ws = state;
  a.emax = fmt == FP8_E4M3 ? 8 : 15;
  a.margin = margin;
  a.bias_out = bias_out;
  a.scale_out = scale_out;
  a.scale_inv_out = scale_inv_out;
  launch_amax_scale(a, dtype, stream);
  return launch_status();
}

static int amax_scale_check(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                            const float* amax_out, const int32_t* bias_out) {
  if (!amax_out || !bias_out) return FP8_ERR_NULL;
  if (!valid_dtype(dtype)) return FP8_ERR_DTYPE;
  if (!valid_fmt(fmt)) return FP8_ERR_FORMAT;
  if (int st = check_matrix(rows, cols, ld)) return st;
  if (rows * cols > 0 && !x) return FP8_ERR_NULL;
  return FP8_OK;
}

int fp8_amax_scale(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int margin,
                   float* amax_out, int32_t* bias_out, float* scale_out, float* scale_inv_out, void* workspace,
                   hipStream_t stream) {
  if (int st = amax_scale_check(x, dtype, rows, cols, ld, fmt, amax_out, bias_out)) return st;
  if (!workspace) return FP8_ERR_NULL;
  if (!aligned(workspace, 4)) return FP8_ERR_ALIGN;
  return amax_scale_impl(x, dtype, rows, cols, ld, fmt, margin, amax_out, bias_out, scale_out, scale_inv_out,
                         static_cast<uint32_t*>(workspace), stream);
}

int fp8_amax_scale_noalloc(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int margin,
                           float* amax_out, int32_t* bias_out, float* scale_out, float* scale_inv_out,
                           hipStream_t stream) {
  if (int st = amax_scale_check(x, dtype, rows, cols, ld, fmt, amax_out, bias_out)) return st;
  uint32_t* state = scratch_on_current_device(stream);
  if (!state) return FP8_ERR_LAUNCH;
  return amax_scale_impl(x, dtype, rows, cols, ld, fmt, margin, amax_out, bias_out, scale_out, scale_inv_out, state,
                         stream);
}

int fp8_compute_scale(const float* amax, int fmt, int margin, int32_t* bias_out, float* scale_out,
                      float* scale_inv_out, hipStream_t stream) {
  if (!amax || !bias_out) return FP8_ERR_NULL;
  if (!valid_fmt(fmt)) return FP8_ERR_FORMAT;
  hipLaunchKernelGGL(compute_scale_kernel, dim3(1), dim3(1), 0, stream, amax, fmt == FP8_E4M3 ? 8 : 15,
                     margin, bias_out, scale_out, scale_inv_out);
  return launch_status();
}

int fp8_history_init(float* hist, int32_t* state, int window, hipStream_t stream) {
  if (!hist || !state) return FP8_ERR_NULL;
  if (window < 1 || window > 4096) return FP8_ERR_SHAPE;
  hipLaunchKernelGGL(history_init_kernel, dim3(1), dim3(256), 0, stream, hist, state, window);
  return launch_status();
}

int fp8_history_push(float* hist, int32_t* state, int window, const float* amax, hipStream_t stream) {
  if (!hist || !state || !amax) return FP8_ERR_NULL;
  if (window < 1 || window > 4096) return FP8_ERR_SHAPE;
  hipLaunchKernelGGL(history_push_kernel, dim3(1), dim3(1), 0, stream, hist, state, window, amax);
  return launch_status();
}

int fp8_compute_scale_delayed(const float* hist, const int32_t* state, int window, int fmt, int margin,
                              int32_t* bias_out, float* scale_out, float* scale_inv_out, hipStream_t stream) {
  if (!hist || !state || !bias_out) return FP8_ERR_NULL;
  if (window < 1 || window > 4096) return FP8_ERR_SHAPE;
  if (!valid_fmt(fmt)) return FP8_ERR_FORMAT;
  hipLaunchKernelGGL(compute_scale_delayed_kernel, dim3(1), dim3(256), 0, stream, hist, state, window,
                     fmt == FP8_E4M3 ? 8 : 15, margin, bias_out, scale_out, scale_inv_out);
  return launch_status();
}

}  // extern "C"

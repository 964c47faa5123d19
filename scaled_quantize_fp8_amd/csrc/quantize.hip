// Per-tensor and per-block (MX) FP8 casts for gfx950, plus the read-only amax
// pass, all HBM-bound streaming kernels.
//
// "Training and inference of large language models using 8-bit floating
// point" (paper review), "Proposed method": inputs are multiplied by their
// power-of-two scale, then cast to FP8 (E4 for weights/activations, E5 for
// gradients).  "Per-Tensor and Per-Block Scaling Strategies for Effective FP8
// Training" (summary), "Key Questions Answered": per-block scaling gives each
// block its own factor (here 1 x 32 along K with an E8M0 power of two).
//
// Design for CDNA4: each lane moves 16-byte chunks (global_load_dwordx4) with
// U chunks in flight, consecutive lanes own consecutive chunks so every wave
// instruction is one contiguous 1 KiB span, the cast is 4 VALU ops per
// element (unpack, v_ldexp, v_med3 clamp, half a v_cvt_pk), maxima are taken
// on integer bit patterns (packed u16 for bf16) and leave each workgroup as
// one atomicMax.  The per-block maximum of an MX block is a 4-lane (bf16) or
// 8-lane (f32) DPP reduction: no LDS, no barrier.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "host.hpp"
#include "stream_kernels.hpp"

namespace sfp8 {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;         // 16-byte loads in flight per lane (casts)
constexpr int kUnrollRead = 8;     // same for the read-only amax pass
constexpr int kUnrollElem = 8;     // element loads in flight per lane (unaligned rows)
// Unrolled iterations per lane the grid is sized for.  Casts run fastest as
// many short workgroups (one iteration each); a pass that reduces an amax
// ends every workgroup with a reduction and one atomic, so it wants fewer,
// longer ones (measured on the 70B-MLP W tensor: 6.15 TB/s cast, 6.27 TB/s amax).
constexpr int kItersCast = 1;
constexpr int kItersCastAmax = 4;
constexpr int kItersRead = 8;

// Streaming loads and stores with the non-temporal hint: every byte is
// touched once, and keeping it out of the caches measured 10-20% faster.
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const v4u_t v = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int DT> struct In;
template <> struct In<FP8_DT_BF16> {
  static constexpr int kEsz = 2;
  static constexpr int kEpc = 8;    // elements per 16-byte chunk
};
template <> struct In<FP8_DT_F32> {
  static constexpr int kEsz = 4;
  static constexpr int kEpc = 4;
};

// |x| bits of one element in float32 layout, and the element as a float.
template <int DT>
__device__ __forceinline__ uint32_t load_elem(const void* row, int64_t i, float* f) {
  if constexpr (DT == FP8_DT_BF16) {
    const uint32_t h = reinterpret_cast<const uint16_t*>(row)[i];
    *f = __uint_as_float(h << 16);
    return h << 16;
  } else {
    const uint32_t u = reinterpret_cast<const uint32_t*>(row)[i];
    *f = __uint_as_float(u);
    return u;
  }
}

// Cast of one element given its float32-layout bits (NaN handled here);
// *sat (when given) gains 1 if the scaled magnitude exceeds the format max.
template <int FMT>
__device__ __forceinline__ uint32_t cast_elem(uint32_t bits, int e, uint32_t* sat = nullptr) {
  if ((bits & 0x7fffffffu) > 0x7f800000u) return nan_code_f32(bits);
  const float v = __builtin_amdgcn_ldexpf(__uint_as_float(bits), e);
  if (sat) *sat += (uint32_t)(__builtin_fabsf(v) > Fmt<FMT>::kMax);
  return cvt1<FMT>(v);
}

// Cast of one 16-byte chunk; returns the packed codes (8 bytes for bf16, 4
// for f32) and the chunk's max |x| bits (float32 layout) in *amax_bits.
// With SAT, *nsat gains the number of the chunk's elements whose scaled
// magnitude exceeds the format maximum (NaN excluded).
template <int DT, int FMT, bool SAT = false>
__device__ __forceinline__ uint2 cast_chunk(uint4 v, int e, uint32_t* amax_bits, bool want_codes,
                                            uint32_t* nsat = nullptr) {
  uint2 o = make_uint2(0u, 0u);
  if constexpr (DT == FP8_DT_BF16) {
    const us2 m2 = max_us2(max_us2(abs_bf16x2(v.x), abs_bf16x2(v.y)),
                           max_us2(abs_bf16x2(v.z), abs_bf16x2(v.w)));
    const uint32_t m = hmax_us2(m2);
    *amax_bits = m << 16;
    if (want_codes) {
      const float f0 = __builtin_amdgcn_ldexpf(bf16_lo(v.x), e), f1 = __builtin_amdgcn_ldexpf(bf16_hi(v.x), e);
      const float f2 = __builtin_amdgcn_ldexpf(bf16_lo(v.y), e), f3 = __builtin_amdgcn_ldexpf(bf16_hi(v.y), e);
      const float f4 = __builtin_amdgcn_ldexpf(bf16_lo(v.z), e), f5 = __builtin_amdgcn_ldexpf(bf16_hi(v.z), e);
      const float f6 = __builtin_amdgcn_ldexpf(bf16_lo(v.w), e), f7 = __builtin_amdgcn_ldexpf(bf16_hi(v.w), e);
      o.x = cvt4<FMT>(f0, f1, f2, f3);
      o.y = cvt4<FMT>(f4, f5, f6, f7);
      if constexpr (SAT) *nsat += sat4<FMT>(f0, f1, f2, f3) + sat4<FMT>(f4, f5, f6, f7);
      if (__builtin_expect(m > 0x7f80u, 0)) {      // a NaN in the chunk: patch its bytes
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t h = (w[i >> 1] >> (16 * (i & 1))) & 0xffffu;
          if ((h & 0x7fffu) > 0x7f80u) {
            const int sh = 8 * (i & 3);
            uint32_t& dst = (i < 4) ? o.x : o.y;
            dst = (dst & ~(0xffu << sh)) | (nan_code_bf16(h) << sh);
          }
        }
      }
    }
  } else {
    const uint32_t a0 = v.x & 0x7fffffffu, a1 = v.y & 0x7fffffffu;
    const uint32_t a2 = v.z & 0x7fffffffu, a3 = v.w & 0x7fffffffu;
    const uint32_t m01 = a0 > a1 ? a0 : a1, m23 = a2 > a3 ? a2 : a3;
    const uint32_t m = m01 > m23 ? m01 : m23;
    *amax_bits = m;
    if (want_codes) {
      const float f0 = __builtin_amdgcn_ldexpf(__uint_as_float(v.x), e);
      const float f1 = __builtin_amdgcn_ldexpf(__uint_as_float(v.y), e);
      const float f2 = __builtin_amdgcn_ldexpf(__uint_as_float(v.z), e);
      const float f3 = __builtin_amdgcn_ldexpf(__uint_as_float(v.w), e);
      o.x = cvt4<FMT>(f0, f1, f2, f3);
      if constexpr (SAT) *nsat += sat4<FMT>(f0, f1, f2, f3);
      if (__builtin_expect(m > 0x7f800000u, 0)) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if ((w[i] & 0x7fffffffu) > 0x7f800000u) {
            const int sh = 8 * i;
            o.x = (o.x & ~(0xffu << sh)) | (nan_code_f32(w[i]) << sh);
          }
        }
      }
    }
  }
  return o;
}

template <int DT>
__device__ __forceinline__ void store_codes(uint8_t* qrow, int64_t chunk, uint2 o) {
  if constexpr (DT == FP8_DT_BF16) {
    const v2u_t v = {o.x, o.y};
    __builtin_nontemporal_store(v, reinterpret_cast<v2u_t*>(qrow) + chunk);
  } else {
    __builtin_nontemporal_store(o.x, reinterpret_cast<uint32_t*>(qrow) + chunk);
  }
}

// Streaming pass: rows are walked by gridDim.y, 16-byte chunks of a row by a
// grid-stride loop over x with U (kUnroll, or kUnrollRead for the amax-only
// pass) non-temporal loads in flight per lane.
// End of the one-launch amax + scale pass.  Thread 0 of each workgroup folds
// the workgroup's maximum into the running maximum ws[1] with a returning
// agent-scope atomic max, then takes a ticket ws[0]; the workgroup that takes
// the last ticket swaps the running maximum for zero and writes amax, bias and
// scales (the bias rule of fp8_compute_scale), then resets the ticket.
// Ordering without fences: the ticket's increment depends on the value the max
// returned, so it is issued only after that max has been performed at the
// word's coherence point; the last ticket thus follows every workgroup's max,
// and the final swap, issued after it, reads their combined result.  (An
// agent-scope release/acquire here costs an L2 write-back and invalidate per
// workgroup, which nearly doubled the pass.)  Increment: old <= 0x7fffffff
// (sign bits are cleared), so it is always 1.
__device__ __forceinline__ void amax_scale_finish(uint32_t v, uint32_t* red, const StreamArgs& a) {
  __shared__ uint32_t s_last;
  v = wave_max_u32(v);
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  const uint32_t nblk = gridDim.x * gridDim.y;
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int i = 0; i < nw; ++i) m = m > red[i] ? m : red[i];
    const uint32_t old = __hip_atomic_fetch_max(a.ws + 1, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t t = __hip_atomic_fetch_add(a.ws, 1u + (old >> 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = t == nblk - 1;
  }
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0) {
    const uint32_t m = __hip_atomic_exchange(a.ws + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *a.amax = __uint_as_float(m);
    const int bias = bias_from_amax_bits(m, a.emax, a.margin, -126, 126);
    *a.bias_out = bias;
    if (a.scale_out) *a.scale_out = pow2f(bias);
    if (a.scale_inv_out) *a.scale_inv_out = pow2f(-bias);
    __hip_atomic_store(a.ws, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One step of delayed scaling in one launch.  Start: the bias from the
// window, the rule of fp8_compute_scale_delayed (largest of the valid
// entries' magnitudes), computed by wave 0 and shared through LDS; every
// workgroup reads the window before it takes its ticket, so before the last
// one pushes.  End: the workgroup's maximum and saturation count fold into
// the workspace with returning atomics, the ticket's increment depends on
// both results (they are always 0 in it: the maximum's sign bit is clear,
// the count is below 2^63), and the workgroup that takes the last ticket
// swaps the state for zeros, writes bias, amax and count, and pushes the
// amax as fp8_history_push does.
__device__ __forceinline__ int window_bias(const DelayedArgs& d) {
  __shared__ int s_e;
  if (threadIdx.x < kWave) {
    int count = d.state[0];
    count = count < 0 ? 0 : (count > d.window ? d.window : count);
    uint32_t m = 0;
    for (int i = threadIdx.x; i < count; i += kWave) {
      const uint32_t v = __float_as_uint(d.hist[i]) & 0x7fffffffu;
      m = m > v ? m : v;
    }
    m = wave_max_u32(m);
    if (threadIdx.x == 0) s_e = bias_from_amax_bits(m, d.emax, d.margin, -126, 126);
  }
  __syncthreads();
  return s_e;
}

__device__ __forceinline__ void delayed_finish(uint32_t amax_bits, uint32_t nsat, int e, uint32_t* red,
                                               const DelayedArgs& d) {
  __shared__ uint32_t red_s[kThreads / kWave];
  __shared__ uint32_t s_last;
  amax_bits = wave_max_u32(amax_bits);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) nsat += (uint32_t)__shfl_xor((int)nsat, off, kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  if (lane == 0) {
    red[wid] = amax_bits;
    red_s[wid] = nsat;
  }
  __syncthreads();
  const uint32_t nblk = gridDim.x * gridDim.y;
  unsigned long long* ws_sat = reinterpret_cast<unsigned long long*>(d.ws + 2);
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    unsigned long long n = 0;
    for (int i = 0; i < nw; ++i) {
      m = m > red[i] ? m : red[i];
      n += red_s[i];
    }
    const uint32_t om = __hip_atomic_fetch_max(d.ws + 1, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long on = __hip_atomic_fetch_add(ws_sat, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t t = __hip_atomic_fetch_add(d.ws, 1u + (om >> 31) + (uint32_t)(on >> 63), __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    s_last = t == nblk - 1;
  }
  __syncthreads();
  if (threadIdx.x != 0 || !s_last) return;
  const uint32_t m = __hip_atomic_exchange(d.ws + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long n = __hip_atomic_exchange(ws_sat, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float amax = __uint_as_float(m);
  *d.amax_out = amax;
  *d.bias_out = e;
  if (d.sat_out) *d.sat_out = n;
  int count = d.state[0];
  int head = d.state[1];
  head = (head < 0 || head >= d.window) ? 0 : head;
  count = count < 0 ? 0 : (count > d.window ? d.window : count);
  d.hist[head] = amax;
  d.state[1] = (head + 1) % d.window;
  d.state[0] = count + 1 > d.window ? d.window : count + 1;
  __hip_atomic_store(d.ws, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT, int FMT, bool VEC, bool WQ, bool AMAX, bool SAT, bool SCALE = false, bool DEL = false>
__global__ __launch_bounds__(kThreads) void stream_kernel(StreamArgs a) {
  __shared__ uint32_t red[kThreads / kWave];
  __shared__ uint32_t red_sat[SAT ? kThreads / kWave : 1];
  uint32_t nsat = 0;
  constexpr int ESZ = In<DT>::kEsz;
  constexpr int EPC = In<DT>::kEpc;
  constexpr int U = WQ ? kUnroll : kUnrollRead;
  static_assert(!DEL || (WQ && AMAX && SAT && !SCALE), "the delayed step casts, reduces and counts");
  int e = 0;
  if constexpr (DEL) e = window_bias(a.del);
  else if constexpr (WQ) e = *a.bias;
  uint32_t amax_bits = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t r = blockIdx.y; r < a.rows; r += gridDim.y) {
    const char* xr = reinterpret_cast<const char*>(a.x) + r * a.ld * ESZ;
    uint8_t* qr = WQ ? a.q + r * a.ldq : nullptr;
    int64_t i0 = tid;            // this lane's first element for the element loop below
    if constexpr (VEC) {
      const int64_t cpr = a.cols / EPC;
      const uint4* x4 = reinterpret_cast<const uint4*>(xr);
      int64_t c = tid;
      for (; c + (U - 1) * stride < cpr; c += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = load_nt(x4 + c + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          uint32_t m;
          const uint2 o = cast_chunk<DT, FMT, SAT>(v[u], e, &m, WQ, &nsat);
          if (AMAX) amax_bits = amax_bits > m ? amax_bits : m;
          if (WQ) store_codes<DT>(qr, c + u * stride, o);
        }
      }
      for (; c < cpr; c += stride) {
        uint32_t m;
        const uint2 o = cast_chunk<DT, FMT, SAT>(load_nt(x4 + c), e, &m, WQ, &nsat);
        if (AMAX) amax_bits = amax_bits > m ? amax_bits : m;
        if (WQ) store_codes<DT>(qr, c, o);
      }
      i0 = cpr * EPC + tid;
    } else {
      // unaligned rows: element loads, kUnrollElem in flight per lane.  A
      // load past the row reads the row's last element instead (no branch
      // around the loads, which would wait on each one) and is then ignored.
      for (; i0 < a.cols; i0 += kUnrollElem * stride) {
        uint32_t bits[kUnrollElem];
#pragma unroll
        for (int u = 0; u < kUnrollElem; ++u) {
          const int64_t i = i0 + u * stride;
          float f;
          bits[u] = load_elem<DT>(xr, i < a.cols ? i : a.cols - 1, &f);
        }
#pragma unroll
        for (int u = 0; u < kUnrollElem; ++u) {
          const int64_t i = i0 + u * stride;
          if (i < a.cols) {
            const uint32_t ab = bits[u] & 0x7fffffffu;
            if (AMAX) amax_bits = amax_bits > ab ? amax_bits : ab;
            if (WQ) qr[i] = (uint8_t)cast_elem<FMT>(bits[u], e, SAT ? &nsat : nullptr);
          }
        }
      }
    }
    for (int64_t i = i0; i < a.cols; i += stride) {   // the tail of a vector row
      float f;
      const uint32_t bits = load_elem<DT>(xr, i, &f);
      const uint32_t ab = bits & 0x7fffffffu;
      if (AMAX) amax_bits = amax_bits > ab ? amax_bits : ab;
      if (WQ) qr[i] = (uint8_t)cast_elem<FMT>(bits, e, SAT ? &nsat : nullptr);
    }
  }
  if constexpr (DEL) {
    delayed_finish(amax_bits, nsat, e, red, a.del);
  } else {
    if (AMAX && !SCALE) block_max_to_global(amax_bits, red, a.amax);
    if (SCALE) amax_scale_finish(amax_bits, red, a);
    if (SAT) block_sum_to_global(nsat, red_sat, a.sat);
  }
}

template <int DT, int FMT, bool VEC, bool WQ, bool AMAX, bool SAT>
static void launch_t(const StreamArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((stream_kernel<DT, FMT, VEC, WQ, AMAX, SAT>), grid, dim3(kThreads), 0, s, a);
}

template <int DT, int FMT, bool VEC>
static void launch_mode(const StreamArgs& a, bool wq, bool am, bool sat, dim3 grid, hipStream_t s) {
  if (!wq) launch_t<DT, FMT, VEC, false, true, false>(a, grid, s);
  else if (sat && am) launch_t<DT, FMT, VEC, true, true, true>(a, grid, s);
  else if (sat) launch_t<DT, FMT, VEC, true, false, true>(a, grid, s);
  else if (am) launch_t<DT, FMT, VEC, true, true, false>(a, grid, s);
  else launch_t<DT, FMT, VEC, true, false, false>(a, grid, s);
}

template <int DT, int FMT>
static void launch_vec_mode(const StreamArgs& a, bool vec, bool wq, bool am, dim3 grid, hipStream_t s) {
  const bool sat = wq && a.sat != nullptr;
  if (vec) launch_mode<DT, FMT, true>(a, wq, am, sat, grid, s);
  else launch_mode<DT, FMT, false>(a, wq, am, sat, grid, s);
}

// Read-only passes (amax): at most one workgroup per compute unit, the
// grid-stride loop covering the rest.  Each workgroup ends in a reduction
// and atomics on one word, which many short workgroups queue on: one
// workgroup per CU reads the 70B-MLP X at 6.7 TB/s against 5.0 with 1024
// workgroups of 8 iterations per lane (W: 6.8 against 6.1).
// Casts that also reduce (fused amax, saturation count, the delayed step)
// end the same way: at most two workgroups per CU (one was slower: the
// writes want more memory parallelism; three or four were 5-10% slower).
// 70B-MLP X / W: cast with fused amax 83 -> 67 / 132 -> 116 us, one-launch
// delayed step 166 -> 79 / 275 -> 125 us.  Plain casts keep many short
// workgroups, measured fastest without atomics.
static void cap_grid(unsigned& gx, unsigned& gy, unsigned per_cu) {
  const unsigned ncu = per_cu * (unsigned)device_cu_count();
  if (gy > ncu) gy = ncu;
  const unsigned gxmax = ncu / gy > 0 ? ncu / gy : 1;
  if (gx > gxmax) gx = gxmax;
}
static void cap_read_grid(unsigned& gx, unsigned& gy) { cap_grid(gx, gy, 1); }


void launch_stream_pass(StreamArgs a, int dtype, int fmt, bool write_q, bool amax, hipStream_t stream) {
  const int esz = dtype_size(dtype);
  const int epc = 16 / esz;
  // contiguous matrix -> one long row
  if (a.rows > 1 && a.ld == a.cols && (!write_q || a.ldq == a.cols)) {
    a.cols *= a.rows;
    a.rows = 1;
    a.ld = a.cols;
    a.ldq = a.cols;
  }
  bool vec = aligned(a.x, 16) && (a.rows == 1 || (a.ld * esz) % 16 == 0);
  if (write_q) vec = vec && aligned(a.q, epc) && (a.rows == 1 || a.ldq % epc == 0);
  const int64_t units = vec ? (a.cols / epc) : a.cols;
  const int unroll = write_q ? kUnroll : kUnrollRead;
  const int iters = !write_q ? kItersRead : (amax ? kItersCastAmax : kItersCast);
  unsigned gx = stream_blocks(units, (int64_t)kThreads * (vec ? unroll : kUnrollElem) * iters);
  unsigned gy = (unsigned)(a.rows < 65535 ? a.rows : 65535);
  if (gy < 1) gy = 1;
  // bound the grid for many short rows
  while ((uint64_t)gx * gy > 32768 && gy > 1) gy = (gy + 1) / 2;
  if (!write_q) cap_read_grid(gx, gy);
  else if (amax || a.sat) cap_grid(gx, gy, 2);
  const dim3 grid(gx, gy);
  if (dtype == FP8_DT_BF16) {
    if (fmt == FP8_E4M3) launch_vec_mode<FP8_DT_BF16, FP8_E4M3>(a, vec, write_q, amax, grid, stream);
    else launch_vec_mode<FP8_DT_BF16, FP8_E5M2>(a, vec, write_q, amax, grid, stream);
  } else {
    if (fmt == FP8_E4M3) launch_vec_mode<FP8_DT_F32, FP8_E4M3>(a, vec, write_q, amax, grid, stream);
    else launch_vec_mode<FP8_DT_F32, FP8_E5M2>(a, vec, write_q, amax, grid, stream);
  }
}

void launch_amax_scale(StreamArgs a, int dtype, hipStream_t stream) {
  const int esz = dtype_size(dtype);
  const int epc = 16 / esz;
  if (a.rows > 1 && a.ld == a.cols) {              // contiguous matrix -> one long row
    a.cols *= a.rows;
    a.rows = 1;
    a.ld = a.cols;
  }
  const bool vec = aligned(a.x, 16) && (a.rows == 1 || (a.ld * esz) % 16 == 0);
  const int64_t units = vec ? (a.cols / epc) : a.cols;
  // the amax pass's grid (the reduction state does not depend on it)
  unsigned gx = stream_blocks(units, (int64_t)kThreads * (vec ? kUnrollRead : kUnrollElem) * kItersRead);
  unsigned gy = (unsigned)(a.rows < 65535 ? a.rows : 65535);
  if (gy < 1) gy = 1;
  while ((uint64_t)gx * gy > 32768 && gy > 1) gy = (gy + 1) / 2;
  cap_read_grid(gx, gy);
  const dim3 grid(gx, gy);
#define SFP8_AS(DT, V) \
  hipLaunchKernelGGL((stream_kernel<DT, FP8_E4M3, V, false, true, false, true>), grid, dim3(kThreads), 0, stream, a)
  if (dtype == FP8_DT_BF16) {
    if (vec) SFP8_AS(FP8_DT_BF16, true);
    else SFP8_AS(FP8_DT_BF16, false);
  } else {
    if (vec) SFP8_AS(FP8_DT_F32, true);
    else SFP8_AS(FP8_DT_F32, false);
  }
#undef SFP8_AS
}

void launch_quantize_delayed(StreamArgs a, int dtype, int fmt, hipStream_t stream) {
  const int esz = dtype_size(dtype);
  const int epc = 16 / esz;
  if (a.rows > 1 && a.ld == a.cols && a.ldq == a.cols) {   // contiguous matrices -> one long row
    a.cols *= a.rows;
    a.rows = 1;
    a.ld = a.cols;
    a.ldq = a.cols;
  }
  bool vec = aligned(a.x, 16) && (a.rows == 1 || (a.ld * esz) % 16 == 0);
  vec = vec && aligned(a.q, epc) && (a.rows == 1 || a.ldq % epc == 0);
  const int64_t units = vec ? (a.cols / epc) : a.cols;
  // the cast-with-amax grid of launch_stream_pass; one workgroup for an
  // empty tensor (it still takes the bias and pushes amax 0)
  unsigned gx = stream_blocks(units, (int64_t)kThreads * (vec ? kUnroll : kUnrollElem) * kItersCastAmax);
  unsigned gy = (unsigned)(a.rows < 65535 ? a.rows : 65535);
  if (gy < 1) gy = 1;
  while ((uint64_t)gx * gy > 32768 && gy > 1) gy = (gy + 1) / 2;
  cap_grid(gx, gy, 2);
  if (a.rows * a.cols == 0) gx = gy = 1;
  const dim3 grid(gx, gy);
#define SFP8_QD(DT, FMT, V)                                                                                  \
  hipLaunchKernelGGL((stream_kernel<DT, FMT, V, true, true, true, false, true>), grid, dim3(kThreads), 0, \
                     stream, a)
#define SFP8_QD2(DT, FMT)       \
  do {                          \
    if (vec) SFP8_QD(DT, FMT, true); \
    else SFP8_QD(DT, FMT, false);    \
  } while (0)
  if (dtype == FP8_DT_BF16) {
    if (fmt == FP8_E4M3) SFP8_QD2(FP8_DT_BF16, FP8_E4M3);
    else SFP8_QD2(FP8_DT_BF16, FP8_E5M2);
  } else {
    if (fmt == FP8_E4M3) SFP8_QD2(FP8_DT_F32, FP8_E4M3);
    else SFP8_QD2(FP8_DT_F32, FP8_E5M2);
  }
#undef SFP8_QD2
#undef SFP8_QD
}

// Workgroups of a cast-transpose launch over ntiles tiles: one per tile, or,
// when the kernel reduces (amax, saturation count, the delayed step),
// per_cu per CU (measured best: 2 for the vector kernel's 128 x 64 tiles, 8
// for the element kernel's 64 x 64 tiles) and at least 4 tiles each,
// walking the tiles.  Every
// workgroup ends in atomics on one word (three in the delayed step), which
// at one workgroup per tile cost the 70B-MLP X [16384 x 8192] 207 us with
// the amax and 584 us as the delayed step against 103 us for the plain cast.
static unsigned tile_blocks(int64_t ntiles, bool reduces, int per_cu) {
  int64_t n = ntiles;
  if (reduces) {
    n = (ntiles + 3) / 4;
    const int64_t cap = (int64_t)per_cu * device_cu_count();
    if (n > cap) n = cap;
  }
  if (n > 0x7fffffff) n = 0x7fffffff;
  return (unsigned)(n < 1 ? 1 : n);
}

// ---------------------------------------------------------------------------
// Cast-transpose, element form (any input the vector form does not take:
// fp32, unaligned rows or strides): 64 x 64 tiles; writes q [rows x cols]
// and qT [cols x rows] (the transposed copy a GEMM contracting over `rows`
// reads K-contiguous).  Wave w reads tile rows 16w .. 16w+15 one row per
// load, lane = column, so each load and each q store covers 64 consecutive
// elements; a lane packs its 16 codes into 4 dwords of a column-major LDS
// tile, and 4 lanes then write each 64-byte qT row, 16 bytes each (one
// vector store when qT rows are 16-byte aligned).
// ---------------------------------------------------------------------------
constexpr int kTT = 64;

template <int DT, int FMT, bool AMAX, bool SAT>
__global__ __launch_bounds__(kThreads) void cast_transpose_kernel(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, const int32_t* __restrict__ bias,
    uint8_t* __restrict__ q, int64_t ldq, uint8_t* __restrict__ qT, int64_t ldqT, float* __restrict__ amax,
    unsigned long long* __restrict__ sat) {
  static_assert(kThreads == 4 * kWave && kTT == kWave, "4 waves of 16 rows cover a 64 x 64 tile");
  // tT[16c + (k ^ (c/4 % 16))]: codes of tile column c (one qT row), tile
  // rows 4k .. 4k+3.  The XOR puts the 64 lanes of a column write and of a
  // row read on 64 distinct banks.
  __shared__ uint32_t tT[kTT * kTT / 4];
  __shared__ uint32_t red[kThreads / kWave];
  __shared__ uint32_t red_sat[SAT ? kThreads / kWave : 1];
  uint32_t nsat = 0;
  constexpr int ESZ = In<DT>::kEsz;
  const int e = *bias;
  const int lane = threadIdx.x % kWave;      // load phase: tile column
  const int w = threadIdx.x / kWave;         // load phase: tile rows 16w .. 16w+15
  const int tr = threadIdx.x / 4;            // store phase: qT row c0 + tr
  const int tq = (threadIdx.x % 4) * 16;     // store phase: its bytes tq .. tq+15
  const bool vec_out = reinterpret_cast<uintptr_t>(qT) % 16 == 0 && ldqT % 16 == 0;
  uint32_t amax_bits = 0;
  // Grid-stride over the tiles, so a reducing launch can be capped at a few
  // workgroups per CU and pay the end-of-kernel atomics only that often.
  const int64_t tiles_x = (cols + kTT - 1) / kTT;
  const int64_t ntiles = tiles_x * ((rows + kTT - 1) / kTT);
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t r0 = (t / tiles_x) * kTT;
    const int64_t c0 = (t % tiles_x) * kTT;
    const int64_t c = c0 + lane;
    const int64_t rw = r0 + 16 * w;
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
    if (c < cols) {
      const char* xc = reinterpret_cast<const char*>(x) + (rw * ld + c) * ESZ;
      uint8_t* qc = q + rw * ldq + c;
      // all 16 loads ahead of the casts and stores; in the last tile row a
      // row past the matrix reads its last row instead (no branch around
      // the loads) and is then ignored
      uint32_t bits[16];
      float f;
      if (rw + 16 <= rows) {
#pragma unroll
        for (int j = 0; j < 16; ++j) bits[j] = load_elem<DT>(xc + j * ld * ESZ, 0, &f);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int64_t dr = rw + j < rows ? j : rows - 1 - rw;
          bits[j] = load_elem<DT>(xc + dr * ld * ESZ, 0, &f);
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (rw + j < rows) {
          const uint32_t ab = bits[j] & 0x7fffffffu;
          if (AMAX) amax_bits = amax_bits > ab ? amax_bits : ab;
          const uint32_t code = cast_elem<FMT>(bits[j], e, SAT ? &nsat : nullptr);
          qc[j * ldq] = (uint8_t)code;
          packed[j / 4] |= code << (8 * (j % 4));
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) tT[16 * lane + ((4 * w + k) ^ ((lane >> 2) & 15))] = packed[k];
    __syncthreads();
    const int64_t cT = c0 + tr;
    if (cT < cols) {
      uint32_t d[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) d[k] = tT[16 * tr + ((tq / 4 + k) ^ ((tr >> 2) & 15))];
      uint8_t* dst = qT + cT * ldqT + r0 + tq;
      if (vec_out && r0 + tq + 16 <= rows) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(d[0], d[1], d[2], d[3]);
      } else {
#pragma unroll
        for (int b = 0; b < 16; ++b)
          if (r0 + tq + b < rows) dst[b] = (uint8_t)(d[b / 4] >> (8 * (b % 4)));
      }
    }
    if (t + gridDim.x < ntiles) __syncthreads();   // tT is rewritten by the next tile
  }
  if (AMAX) block_max_to_global(amax_bits, red, amax);
  if (SAT) block_sum_to_global(nsat, red_sat, sat);
}

// ---------------------------------------------------------------------------
// Cast-transpose, vector form (bf16 input): 128 x 64 tiles.  Lane (cg, rg)
// loads 16 bytes (8 columns) of 4 consecutive rows, casts them, stores the 4
// x 8 codes of q directly (8 bytes per row), transposes them 4 x 4 bytes at a
// time in registers and writes 8 dwords (4 rows each) into a column-major
// LDS tile; then 8 lanes write each 128-byte qT row (16 bytes each).  Tiles
// reaching past the matrix take a per-element path with the same exchange.
// ---------------------------------------------------------------------------
constexpr int kCtR = 128, kCtC = 64;

// Elements from which cast_transpose_vec_kernel stores qT through the cache.
constexpr int64_t kCtCachedMin = 32LL << 20;

// d_k = byte k of a0, a1, a2, a3 (a 4 x 4 byte transpose)
__device__ __forceinline__ void bytes_transpose4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                                 uint32_t (&d)[4]) {
  const uint32_t lo01 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);   // a0.0 a1.0 a0.1 a1.1
  const uint32_t hi01 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);   // a0.2 a1.2 a0.3 a1.3
  const uint32_t lo23 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
  d[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);             // a0.0 a1.0 a2.0 a3.0
  d[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  d[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  d[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// NTQT: non-temporal qT stores.  A store instruction writes 8 whole qT lines
// (8 lanes of 16 bytes each; 4 pieces 32 bytes apart into 16 lines was
// 1-6% slower).  Through the cache measures faster on large tensors (7B-MLP
// backward: dY and W, 45M elements, +9% / +11%) and slower on small ones
// (X, 16.7M elements, -11%: the dirty lines are still being written back
// when the kernel ends), so the host picks the kind by size.
// DEL: one step of delayed scaling (fp8_quantize_delayed): the bias from the
// window in del, the outputs and the push by the last workgroup, as in
// stream_kernel.
template <int FMT, bool AMAX, bool NTQT, bool SAT, bool DEL = false>
__global__ __launch_bounds__(kThreads) void cast_transpose_vec_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, const int32_t* __restrict__ bias,
    uint8_t* __restrict__ q, int64_t ldq, uint8_t* __restrict__ qT, int64_t ldqT, float* __restrict__ amax,
    unsigned long long* __restrict__ sat, DelayedArgs del) {
  static_assert(!DEL || (AMAX && SAT), "the delayed step reduces and counts");
  __shared__ uint32_t T[kCtC][kCtR / 4 + 1];       // codes, column-major, 4 rows per dword
  __shared__ uint32_t red[kThreads / kWave];
  __shared__ uint32_t red_sat[SAT ? kThreads / kWave : 1];
  uint32_t nsat = 0;
  int e;
  if constexpr (DEL) e = window_bias(del);
  else e = *bias;
  // one tile per workgroup, or (a grid capped for the reductions) a
  // grid-stride loop over the tiles, x fastest
  const int64_t tiles_x = (cols + kCtC - 1) / kCtC;
  const int64_t ntiles = tiles_x * ((rows + kCtR - 1) / kCtR);
  const int cg = threadIdx.x & 7, rg = threadIdx.x >> 3;
  uint32_t amax_bits = 0;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t r0 = (tile / tiles_x) * kCtR, c0 = (tile % tiles_x) * kCtC;
    const bool interior = r0 + kCtR <= rows && c0 + kCtC <= cols;
    uint2 o[4];
    if (interior) {
      // the lane's 4 rows loaded ahead of the tile's stores: all four in
      // flight at once (a prefetch of the next tile across the LDS phase
      // measured no faster)
      uint4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = load_nt(reinterpret_cast<const uint4*>(x + (r0 + 4 * rg + i) * ld + c0 + 8 * cg));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t m;
        o[i] = cast_chunk<FP8_DT_BF16, FMT, SAT>(v[i], e, &m, true, &nsat);
        if (AMAX) amax_bits = amax_bits > m ? amax_bits : m;
        const v2u_t ov = {o[i].x, o[i].y};
        __builtin_nontemporal_store(ov, reinterpret_cast<v2u_t*>(q + (r0 + 4 * rg + i) * ldq + c0 + 8 * cg));
      }
    } else {
      // per element, all 32 loads ahead of the casts and stores; an index
      // past the matrix reads its last row or column instead (no branch
      // around the loads) and is then ignored
      uint32_t bits[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + 4 * rg + i;
        const char* xr = reinterpret_cast<const char*>(x) + (r < rows ? r : rows - 1) * ld * 2;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int64_t c = c0 + 8 * cg + k;
          float f;
          bits[i][k] = load_elem<FP8_DT_BF16>(xr, c < cols ? c : cols - 1, &f);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + 4 * rg + i;
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int64_t c = c0 + 8 * cg + k;
          if (r < rows && c < cols) {
            const uint32_t ab = bits[i][k] & 0x7fffffffu;
            if (AMAX) amax_bits = amax_bits > ab ? amax_bits : ab;
            const uint32_t code = cast_elem<FMT>(bits[i][k], e, SAT ? &nsat : nullptr);
            q[r * ldq + c] = (uint8_t)code;
            w[k / 4] |= code << (8 * (k % 4));
          }
        }
        o[i] = make_uint2(w[0], w[1]);
      }
    }
    uint32_t d[8];
    {
      uint32_t t4[4];
      bytes_transpose4(o[0].x, o[1].x, o[2].x, o[3].x, t4);
      d[0] = t4[0]; d[1] = t4[1]; d[2] = t4[2]; d[3] = t4[3];
      bytes_transpose4(o[0].y, o[1].y, o[2].y, o[3].y, t4);
      d[4] = t4[0]; d[5] = t4[1]; d[6] = t4[2]; d[7] = t4[3];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) T[8 * cg + k][rg] = d[k];
    __syncthreads();
    // qT: each of the tile's 64 rows is one 128-byte line, 8 lanes of 16 bytes
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int idx = threadIdx.x + k * kThreads;
      const int j = idx >> 3, p = idx & 7;
      const int64_t cT = c0 + j;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = T[j][4 * p + i];
      if (interior) {
        v4u_t* dst = reinterpret_cast<v4u_t*>(qT + cT * ldqT + r0 + 16 * p);
        const v4u_t vv = {w[0], w[1], w[2], w[3]};
        if constexpr (NTQT) __builtin_nontemporal_store(vv, dst);
        else dst[0] = vv;
      } else if (cT < cols) {
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const int64_t r = r0 + 16 * p + b;
          if (r < rows) qT[cT * ldqT + r] = (uint8_t)(w[b / 4] >> (8 * (b % 4)));
        }
      }
    }
    if (tile + gridDim.x < ntiles) __syncthreads();   // T is rewritten by the next tile
  }
  if constexpr (DEL) {
    delayed_finish(amax_bits, nsat, e, red, del);
  } else {
    if (AMAX) block_max_to_global(amax_bits, red, amax);
    if (SAT) block_sum_to_global(nsat, red_sat, sat);
  }
}

// ---------------------------------------------------------------------------
// MX cast: 1 x 32 blocks along cols.  Vector kernel: a block is 4 lanes
// (bf16) or 8 lanes (f32) of 16-byte chunks; the block max is a DPP
// reduction inside the lane group, the group's first lane stores the E8M0
// code.  Element kernel (unaligned operands): one element per lane, a block
// being 32 lanes of a wave.
// ---------------------------------------------------------------------------
struct MxArgs {
  const void* x;
  int64_t rows, cols, ld;
  uint8_t* q;
  int64_t ldq;
  uint8_t* scales;
  int64_t lds;
  int packed;          // scales in the packed layout (host.hpp), sgroups groups per row tile
  int64_t sgroups;
  int64_t kb;          // packed: blocks per row of the code matrix (the last one pads its group)
  int collapsed;       // packed and the rows collapsed into one long row: block j of it is
                       // block j % kb of matrix row j / kb (fewer than 2^32 blocks)
  int nt;              // transposed cast: qT lines stored non-temporal
};

// Where the E8M0 code of (row r, block j) goes: row-major (scales + r lds + j)
// or the packed layout, ((r / 256) G + j / 16) 4096 + (r % 256) 16 + j % 16.
// The lane that stores a row's last code in the packed layout also writes
// code 127 over the rest of that 16-code group (blocks past the matrix).
__device__ __forceinline__ void store_scale(const MxArgs& a, int64_t r, int64_t j, uint32_t code) {
  if (a.packed) {
    if (a.collapsed) {
      const uint32_t rr = (uint32_t)j / (uint32_t)a.kb;
      j -= (int64_t)rr * a.kb;
      r = rr;
    }
    uint8_t* p = a.scales + ((r / kPackRows) * a.sgroups + j / kPackBlocks) * kPackTile +
                 (r % kPackRows) * kPackBlocks;
    p[j % kPackBlocks] = (uint8_t)code;
    if (j == a.kb - 1)
      for (int64_t t = j % kPackBlocks + 1; t < kPackBlocks; ++t) p[t] = 0x7fu;
  } else {
    a.scales[r * a.lds + j] = (uint8_t)code;
  }
}

// Fill n bytes (n % 16 == 0, p 16-byte aligned) with v: the padding of a
// packed scale buffer.
__global__ __launch_bounds__(256) void fill_u8_kernel(uint8_t* p, int64_t n16, uint32_t v4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) reinterpret_cast<uint4*>(p)[i] = make_uint4(v4, v4, v4, v4);
}

// Block exponent by the default rule (block max at or below the format
// maximum) or, with OCP, the OCP MX rule (block max in the top binade).
template <int FMT, bool OCP>
__device__ __forceinline__ void block_exponent(uint32_t bmax_bits, int* e, uint32_t* code) {
  if (bmax_bits > 0x7f800000u) {        // NaN in the block
    *e = 0;
    *code = 0xffu;
  } else {
    *e = bias_from_amax_bits(bmax_bits, Fmt<FMT>::kEmax, 0, -127, 127, OCP);
    *code = (uint32_t)(127 - *e);
  }
}

template <int DT, int FMT, bool OCP>
__global__ __launch_bounds__(kThreads) void mx_vec_kernel(MxArgs a) {
  constexpr int ESZ = In<DT>::kEsz;
  constexpr int EPC = In<DT>::kEpc;
  constexpr int L = 32 / EPC;           // lanes per block
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t cpr = a.cols / EPC;
  for (int64_t r = blockIdx.y; r < a.rows; r += gridDim.y) {
    const uint4* x4 = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.x) + r * a.ld * ESZ);
    uint8_t* qr = a.q + r * a.ldq;
    int64_t c = tid;
    // every lane of a block's group takes the same branch: stride and cpr
    // are multiples of L and the group's chunks share c / L
    for (; c + (kUnroll - 1) * stride < cpr; c += kUnroll * stride) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = load_nt(x4 + c + u * stride);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        uint32_t m;
        cast_chunk<DT, FMT>(v[u], 0, &m, false);
        const uint32_t bm = (L == 4) ? group4_max(m) : group8_max(m);
        int e;
        uint32_t code;
        block_exponent<FMT, OCP>(bm, &e, &code);
        const uint2 o = cast_chunk<DT, FMT>(v[u], e, &m, true);
        store_codes<DT>(qr, c + u * stride, o);
        if ((threadIdx.x % L) == 0) store_scale(a, r, (c + u * stride) / L, code);
      }
    }
    for (; c < cpr; c += stride) {
      uint32_t m;
      const uint4 v = load_nt(x4 + c);
      cast_chunk<DT, FMT>(v, 0, &m, false);
      const uint32_t bm = (L == 4) ? group4_max(m) : group8_max(m);
      int e;
      uint32_t code;
      block_exponent<FMT, OCP>(bm, &e, &code);
      const uint2 o = cast_chunk<DT, FMT>(v, e, &m, true);
      store_codes<DT>(qr, c, o);
      if ((threadIdx.x % L) == 0) store_scale(a, r, c / L, code);
    }
  }
}

// Max across aligned groups of 32 lanes: the group-of-8 DPP steps, the
// row mirror (16), then a swizzle exchanging lanes 16 apart in each 32.
__device__ __forceinline__ uint32_t group32_max(uint32_t v) {
  v = group8_max(v);
  uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);   // row mirror
  v = v > o ? v : o;
  o = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (0x10 << 10) | 0x1f);            // lane ^ 16
  return v > o ? v : o;
}

// Element kernel: a wave takes spans of kMxSpan consecutive elements of a
// row, 64 at a time (one element per lane, so each load and each code store
// covers 64 consecutive elements: two blocks); the block max is a reduction
// over the 32 lanes of a block.  The span's 16 E8M0 codes (one packed-layout
// group, since spans start at multiples of 512 elements) are gathered in
// every lane and stored by 16 lanes, one byte each.  Not for a packed layout
// whose rows were collapsed into one long row (a span could cross rows).
constexpr int kMxElemU = 8;                      // element loads in flight per lane
constexpr int kMxSpan = kMxElemU * kWave;        // 512 elements, 16 blocks

template <int DT, int FMT, bool OCP>
__global__ __launch_bounds__(kThreads) void mx_scalar_kernel(MxArgs a) {
  static_assert(kMxSpan / 32 == kPackBlocks, "a span is one packed-layout group");
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32;                    // block 2u + half of the span at step u
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / kWave);
  const int64_t spans = (a.cols + kMxSpan - 1) / kMxSpan;
  const int64_t kb = a.cols / 32;
  for (int64_t r = blockIdx.y; r < a.rows; r += gridDim.y) {
    const char* xr = reinterpret_cast<const char*>(a.x) + r * a.ld * In<DT>::kEsz;
    uint8_t* qr = a.q + r * a.ldq;
    for (int64_t sp = wave; sp < spans; sp += nwaves) {
      const int64_t i0 = sp * kMxSpan + lane;
      // all loads first; an index past the row reads its last element
      // instead (no branch around the loads).  cols % 32 == 0, so the 32
      // lanes of a block are past the row together or not at all.
      uint32_t bits[kMxElemU];
#pragma unroll
      for (int u = 0; u < kMxElemU; ++u) {
        const int64_t i = i0 + u * kWave;
        float f;
        bits[u] = load_elem<DT>(xr, i < a.cols ? i : a.cols - 1, &f);
      }
      uint32_t own[2] = {0u, 0u};                // codes of this half's blocks, step u in byte u % 4
#pragma unroll
      for (int u = 0; u < kMxElemU; ++u) {
        const int64_t i = i0 + u * kWave;
        const uint32_t m = group32_max(bits[u] & 0x7fffffffu);
        int e;
        uint32_t code;
        block_exponent<FMT, OCP>(m, &e, &code);
        own[u / 4] |= code << (8 * (u % 4));
        if (i < a.cols) qr[i] = (uint8_t)cast_elem<FMT>(bits[u], e);
      }
      // the other half's codes; even blocks come from half 0, odd from half 1
      const uint32_t oth0 = (uint32_t)__shfl_xor((int)own[0], 32), oth1 = (uint32_t)__shfl_xor((int)own[1], 32);
      const uint32_t ev0 = half ? oth0 : own[0], ev1 = half ? oth1 : own[1];
      const uint32_t od0 = half ? own[0] : oth0, od1 = half ? own[1] : oth1;
      if (lane < kPackBlocks) {
        const int64_t j = sp * kPackBlocks + lane;       // this lane's block of the row
        const uint32_t ev = lane < 8 ? ev0 : ev1, od = lane < 8 ? od0 : od1;
        const uint32_t code = (((lane & 1) ? od : ev) >> (8 * ((lane % 8) / 2))) & 0xffu;
        if (a.packed) {
          uint8_t* p = a.scales + ((r / kPackRows) * a.sgroups + sp) * kPackTile + (r % kPackRows) * kPackBlocks;
          p[lane] = j < kb ? (uint8_t)code : (uint8_t)0x7f;   // 127 pads the row's last group
        } else if (j < kb) {
          a.scales[r * a.lds + j] = (uint8_t)code;
        }
      }
    }
  }
}

template <int DT, int FMT, bool OCP>
static void launch_mx(const MxArgs& a, bool vec, hipStream_t s) {
  const int epc = 16 / In<DT>::kEsz;
  const int64_t units = vec ? a.cols / epc : a.cols;
  const int64_t per = vec ? (int64_t)kThreads * kUnroll * kItersCast : (int64_t)kThreads * kMxElemU;
  // one workgroup per `per` units of a row, rounded down when the matrix has
  // several rows: a second workgroup on a row's short remainder would run
  // only the non-unrolled tail (11008 columns: 1376 chunks, 5.4 per lane
  // from one workgroup beat 2.7 per lane from two)
  const unsigned gx = a.rows > 1 && units > per ? (unsigned)std::min<int64_t>(units / per, 1 << 20)
                                                 : stream_blocks(units, per);
  unsigned gy = (unsigned)(a.rows < 65535 ? a.rows : 65535);
  if (gy < 1) gy = 1;
  while ((uint64_t)gx * gy > 32768 && gy > 1) gy = (gy + 1) / 2;
  if (vec)
    hipLaunchKernelGGL((mx_vec_kernel<DT, FMT, OCP>), dim3(gx, gy), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((mx_scalar_kernel<DT, FMT, OCP>), dim3(gx, gy), dim3(kThreads), 0, s, a);
}

// ---------------------------------------------------------------------------
// Transposed MX cast: blocks of 32 consecutive ROWS of one column, written as
// qT [cols x rows] with scalesT [cols x rows/32], i.e. the MX cast of x^T
// (for a GEMM that contracts over `rows`, such as a weight gradient whose K
// is the token axis).  128 x 64 tiles (128 x 128 for large bf16 inputs: the
// longer row pieces read faster): the workgroup stages the tile in LDS
// (consecutive lanes load consecutive 16-byte chunks of a row), then lane
// (c, b) owns the whole 32-row block b of tile column c (two columns per
// lane on wide tiles): it reduces the
// block's maximum, casts its 32 elements and puts them, as 32 contiguous
// bytes of qT row c, back into LDS, from where the workgroup writes each of
// its qT rows as one full 128-byte line.
// ---------------------------------------------------------------------------
constexpr int kMtR = 128, kMtC = 64, kMtCWide = 128;
// Elements from which mx_transpose_kernel stores qT through the cache.
constexpr int64_t kMxtCachedMin = 64LL << 20;

template <int DT, int FMT, bool VEC, bool OCP, int TC = kMtC>
__global__ __launch_bounds__(kThreads) void mx_transpose_kernel(MxArgs a) {
  // The tile is staged in the input's own width (bf16 as 16-bit words, rows
  // of 72: 144 bytes; fp32 rows of 68 dwords): 16-byte aligned rows for the
  // staging writes, and a column read (64 lanes, one row) touches 64
  // consecutive elements.  16-bit staging halves the LDS of a bf16 tile,
  // so twice as many workgroups fit on a compute unit.
  using TT = std::conditional_t<DT == FP8_DT_BF16, uint16_t, uint32_t>;
  constexpr int PAD = DT == FP8_DT_BF16 ? 8 : 4;
  static_assert(TC == 64 || TC == 128, "tile columns");
  __shared__ __attribute__((aligned(16))) TT tile[kMtR][TC + PAD];
  constexpr int ESZ = In<DT>::kEsz;
  constexpr int EPC = In<DT>::kEpc;                // elements per 16-byte chunk
  constexpr int CPR = TC / EPC;                    // chunks per tile row
  const int64_t r0 = (int64_t)blockIdx.y * kMtR;
  const int64_t c0 = (int64_t)blockIdx.x * TC;
  const bool full_cols = c0 + TC <= a.cols;
  constexpr int LPL = kMtR * CPR / kThreads;       // 16-byte chunks per lane
  if (VEC && full_cols && r0 + kMtR <= a.rows) {
    // whole tile: a lane's loads all in flight before its LDS writes (a
    // branch per chunk made the compiler wait on each load)
    uint4 v[LPL];
#pragma unroll
    for (int k = 0; k < LPL; ++k) {
      const int idx = threadIdx.x + k * kThreads;
      const int64_t r = r0 + idx / CPR;
      v[k] = load_nt(reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.x) +
                                                    (r * a.ld + c0 + (idx % CPR) * EPC) * ESZ));
    }
#pragma unroll
    for (int k = 0; k < LPL; ++k) {
      const int idx = threadIdx.x + k * kThreads;
      *reinterpret_cast<uint4*>(&tile[idx / CPR][(idx % CPR) * EPC]) = v[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < LPL; ++k) {
      const int idx = threadIdx.x + k * kThreads;
      const int tr = idx / CPR, ch = idx % CPR;
      const int64_t r = r0 + tr;
      const char* xr = reinterpret_cast<const char*>(a.x) + r * a.ld * ESZ;
      uint4* trow = reinterpret_cast<uint4*>(&tile[tr][ch * EPC]);   // one 16-byte chunk of the row
      if (VEC && full_cols && r < a.rows) {
        trow[0] = load_nt(reinterpret_cast<const uint4*>(xr + (c0 + ch * EPC) * ESZ));
      } else {
        // element loads; an index past the matrix reads its last row or
        // column instead (no branch around the loads) and stores 0
        const char* xc = reinterpret_cast<const char*>(a.x) + (r < a.rows ? r : a.rows - 1) * a.ld * ESZ;
        TT w[EPC];
#pragma unroll
        for (int j = 0; j < EPC; ++j) {
          const int64_t c = c0 + ch * EPC + j;
          float f;
          const uint32_t bits = load_elem<DT>(xc, c < a.cols ? c : a.cols - 1, &f);
          w[j] = r < a.rows && c < a.cols ? (TT)(DT == FP8_DT_BF16 ? bits >> 16 : bits) : (TT)0;
        }
        trow[0] = *reinterpret_cast<const uint4*>(w);
      }
    }
  }
  __syncthreads();
  // lane (c, blk), c = lane + 64 h for each of the TC / 64 column halves h,
  // blk = the wave: tile rows 32 blk .. 32 blk + 31 of column c
  constexpr int NH = TC / 64;
  const int blk = threadIdx.x / 64;
  const int64_t rr = r0 + 32 * blk;                // first qT column of this block
  uint32_t w[NH][8];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int c = threadIdx.x % 64 + 64 * h;
    const int64_t col = c0 + c;                    // qT row
#pragma unroll
    for (int k = 0; k < 8; ++k) w[h][k] = 0;
    if (col < a.cols && rr < a.rows) {             // rows % 32 == 0: a block exists whole or not at all
      uint32_t v[32];
      uint32_t bm = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        v[i] = DT == FP8_DT_BF16 ? (uint32_t)tile[32 * blk + i][c] << 16 : (uint32_t)tile[32 * blk + i][c];
        const uint32_t ab = v[i] & 0x7fffffffu;
        bm = bm > ab ? bm : ab;
      }
      int e;
      uint32_t code;
      block_exponent<FMT, OCP>(bm, &e, &code);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        w[h][k] = cvt4<FMT>(__builtin_amdgcn_ldexpf(__uint_as_float(v[4 * k]), e),
                            __builtin_amdgcn_ldexpf(__uint_as_float(v[4 * k + 1]), e),
                            __builtin_amdgcn_ldexpf(__uint_as_float(v[4 * k + 2]), e),
                            __builtin_amdgcn_ldexpf(__uint_as_float(v[4 * k + 3]), e));
      if (__builtin_expect(bm > 0x7f800000u, 0)) {  // a NaN in the block: patch its codes
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if ((v[i] & 0x7fffffffu) > 0x7f800000u)
            w[h][i / 4] = (w[h][i / 4] & ~(0xffu << (8 * (i % 4)))) | (nan_code_f32(v[i]) << (8 * (i % 4)));
      }
      store_scale(a, col, rr / 32, code);          // qT row col, block rr / 32
    }
  }
  // The codes go out through LDS: the tile's TC qT rows of kMtR bytes
  // (row stride kMtR + 16: the 16-byte writes of 16 lanes hit 64 distinct
  // banks) are written back as whole 128-byte lines, 8 lanes per line, where
  // each lane had written 32 bytes into each of 64 rows.  Non-temporal
  // below kMxtCachedMin elements, through the cache above (the host's
  // choice, a.nt): measured on the 7B-MLP tensors (16.7M and 45M elements)
  // and the 70B-MLP X (134M).
  constexpr int OS = kMtR + 16;
  static_assert(TC * OS <= (int)sizeof(tile), "output staging fits in the tile");
  uint8_t* ost = reinterpret_cast<uint8_t*>(&tile[0][0]);
  __syncthreads();                                 // every column has been read
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int c = threadIdx.x % 64 + 64 * h;
    *reinterpret_cast<uint4*>(ost + c * OS + 32 * blk) = make_uint4(w[h][0], w[h][1], w[h][2], w[h][3]);
    *reinterpret_cast<uint4*>(ost + c * OS + 32 * blk + 16) = make_uint4(w[h][4], w[h][5], w[h][6], w[h][7]);
  }
  __syncthreads();
  constexpr int CH = kMtR / 16;                    // 16-byte chunks per qT row of the tile
#pragma unroll
  for (int k = 0; k < TC * CH / kThreads; ++k) {
    const int idx = threadIdx.x + k * kThreads;
    const int orow = idx / CH, ch = idx % CH;
    const int64_t ocol = c0 + orow, orr = r0 + 16 * ch;
    if (ocol < a.cols && orr < a.rows) {
      const uint4 d = *reinterpret_cast<const uint4*>(ost + orow * OS + 16 * ch);
      uint8_t* dst = a.q + ocol * a.ldq + orr;
      if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        if (a.nt) {
          const v4u_t dv = {d.x, d.y, d.z, d.w};
          __builtin_nontemporal_store(dv, reinterpret_cast<v4u_t*>(dst));
        } else {
          *reinterpret_cast<uint4*>(dst) = d;
        }
      } else {
        const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int b = 0; b < 16; ++b) dst[b] = (uint8_t)(dw[b / 4] >> (8 * (b % 4)));
      }
    }
  }
}

}  // namespace sfp8

using namespace sfp8;

// Per-tensor cast behind fp8_quantize and fp8_quantize_sat (sat_out: count
// of saturated elements, or null).
static int quantize_impl(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                         const int32_t* bias, uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT, float* amax_out,
                         unsigned long long* sat_out, hipStream_t stream) {
  if (!bias || !q) return FP8_ERR_NULL;
  if (!valid_dtype(dtype)) return FP8_ERR_DTYPE;
  if (!valid_fmt(fmt)) return FP8_ERR_FORMAT;
  int st = check_matrix(rows, cols, ld);
  if (st) return st;
  st = check_matrix(rows, cols, ldq);
  if (st) return st;
  if (qT && check_matrix(cols, rows, ldqT)) return FP8_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n > 0 && !x) return FP8_ERR_NULL;
  zero_outputs_async(amax_out, sat_out, stream);
  if (n == 0) return launch_status();
  const bool am = amax_out != nullptr, sc = sat_out != nullptr;
  if (qT && dtype == FP8_DT_BF16 && aligned(x, 16) && ld % 8 == 0 && aligned(q, 8) && ldq % 8 == 0 &&
      aligned(qT, 16) && ldqT % 16 == 0) {
    const dim3 grid(tile_blocks(((cols + kCtC - 1) / kCtC) * ((rows + kCtR - 1) / kCtR), am || sc, 2));
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const bool nt = n < kCtCachedMin;
#define SFP8_CTV4(FMT, AM, NT, SC)                                                                              \
  hipLaunchKernelGGL((cast_transpose_vec_kernel<FMT, AM, NT, SC>), grid, dim3(kThreads), 0, stream, xb, rows,   \
                     cols, ld, bias, q, ldq, qT, ldqT, amax_out, sat_out, DelayedArgs{})
#define SFP8_CTV3(FMT, AM, NT)                                                                                  \
  do {                                                                                                          \
    if (sc) SFP8_CTV4(FMT, AM, NT, true);                                                                       \
    else SFP8_CTV4(FMT, AM, NT, false);                                                                         \
  } while (0)
#define SFP8_CTV(FMT)                                                                                           \
  do {                                                                                                          \
    if (am) {                                                                                                   \
      if (nt) SFP8_CTV3(FMT, true, true);                                                                       \
      else SFP8_CTV3(FMT, true, false);                                                                         \
    } else {                                                                                                    \
      if (nt) SFP8_CTV3(FMT, false, true);                                                                      \
      else SFP8_CTV3(FMT, false, false);                                                                        \
    }                                                                                                           \
  } while (0)
    if (fmt == FP8_E4M3) SFP8_CTV(FP8_E4M3);
    else SFP8_CTV(FP8_E5M2);
#undef SFP8_CTV
#undef SFP8_CTV3
#undef SFP8_CTV4
    return launch_status();
  }
  if (qT) {
    const dim3 grid(tile_blocks(((cols + kTT - 1) / kTT) * ((rows + kTT - 1) / kTT), am || sc, 8));
#define SFP8_CT2(DT, FMT, AM, SC)                                                                                  \
  hipLaunchKernelGGL((cast_transpose_kernel<DT, FMT, AM, SC>), grid, dim3(kThreads), 0, stream, x, rows, cols, ld, \
                     bias, q, ldq, qT, ldqT, amax_out, sat_out)
#define SFP8_CT(DT, FMT)                                                                                           \
  do {                                                                                                             \
    if (am && sc) SFP8_CT2(DT, FMT, true, true);                                                                   \
    else if (am) SFP8_CT2(DT, FMT, true, false);                                                                   \
    else if (sc) SFP8_CT2(DT, FMT, false, true);                                                                   \
    else SFP8_CT2(DT, FMT, false, false);                                                                          \
  } while (0)
    if (dtype == FP8_DT_BF16) {
      if (fmt == FP8_E4M3) SFP8_CT(FP8_DT_BF16, FP8_E4M3);
      else SFP8_CT(FP8_DT_BF16, FP8_E5M2);
    } else {
      if (fmt == FP8_E4M3) SFP8_CT(FP8_DT_F32, FP8_E4M3);
      else SFP8_CT(FP8_DT_F32, FP8_E5M2);
    }
#undef SFP8_CT
#undef SFP8_CT2
    return launch_status();
  }
  StreamArgs a;
  a.x = x;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.bias = bias;
  a.q = q;
  a.ldq = ldq;
  a.amax = amax_out;
  a.sat = sat_out;
  launch_stream_pass(a, dtype, fmt, /*write_q=*/true, /*amax=*/am, stream);
  return launch_status();
}

extern "C" {

int fp8_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                 const int32_t* bias, uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT, float* amax_out,
                 hipStream_t stream) {
  return quantize_impl(x, dtype, rows, cols, ld, fmt, bias, q, ldq, qT, ldqT, amax_out, nullptr, stream);
}

int fp8_quantize_sat(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                     const int32_t* bias, uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT, float* amax_out,
                     uint64_t* sat_out, hipStream_t stream) {
  if (!sat_out) return FP8_ERR_NULL;
  static_assert(sizeof(unsigned long long) == sizeof(uint64_t), "64-bit count");
  return quantize_impl(x, dtype, rows, cols, ld, fmt, bias, q, ldq, qT, ldqT, amax_out,
                       reinterpret_cast<unsigned long long*>(sat_out), stream);
}

int fp8_quantize_delayed(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int margin,
                         float* hist, int32_t* state, int window, uint8_t* q, int64_t ldq, uint8_t* qT,
                         int64_t ldqT, int32_t* bias_out, float* amax_out, uint64_t* sat_out, void* workspace,
                         hipStream_t stream) {
  if (!hist || !state || !bias_out || !amax_out || !workspace) return FP8_ERR_NULL;
  if (window < 1 || window > 4096) return FP8_ERR_SHAPE;
  if (!valid_dtype(dtype)) return FP8_ERR_DTYPE;
  if (!valid_fmt(fmt)) return FP8_ERR_FORMAT;
  if (int st = check_matrix(rows, cols, ld)) return st;
  if (int st = check_matrix(rows, cols, ldq)) return st;
  if (qT && check_matrix(cols, rows, ldqT)) return FP8_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n > 0 && (!x || !q)) return FP8_ERR_NULL;     // an empty step writes no codes
  if (!aligned(workspace, 8)) return FP8_ERR_ALIGN;
  unsigned long long* sat = reinterpret_cast<unsigned long long*>(sat_out);
  DelayedArgs d;
  d.hist = hist;
  d.state = state;
  d.window = window;
  d.emax = fmt == FP8_E4M3 ? 8 : 15;
  d.margin = margin;
  d.ws = static_cast<uint32_t*>(workspace);
  d.bias_out = bias_out;
  d.amax_out = amax_out;
  d.sat_out = sat;
  if (qT && n > 0) {
    if (dtype == FP8_DT_BF16 && aligned(x, 16) && ld % 8 == 0 && aligned(q, 8) && ldq % 8 == 0 &&
        aligned(qT, 16) && ldqT % 16 == 0) {
      const dim3 grid(tile_blocks(((cols + kCtC - 1) / kCtC) * ((rows + kCtR - 1) / kCtR), true, 2));
      const uint16_t* xb = static_cast<const uint16_t*>(x);
      const bool nt = n < kCtCachedMin;
#define SFP8_CTD(FMT, NT)                                                                                     \
  hipLaunchKernelGGL((cast_transpose_vec_kernel<FMT, true, NT, true, true>), grid, dim3(kThreads), 0, stream, \
                     xb, rows, cols, ld, nullptr, q, ldq, qT, ldqT, nullptr, nullptr, d)
      if (fmt == FP8_E4M3) {
        if (nt) SFP8_CTD(FP8_E4M3, true);
        else SFP8_CTD(FP8_E4M3, false);
      } else {
        if (nt) SFP8_CTD(FP8_E5M2, true);
        else SFP8_CTD(FP8_E5M2, false);
      }
#undef SFP8_CTD
      return launch_status();
    }
    // other layouts with a transposed copy: the same step as three launches
    // (the workspace is not used and stays zero)
    if (int st = fp8_compute_scale_delayed(hist, state, window, fmt, margin, bias_out, nullptr, nullptr, stream))
      return st;
    if (int st = quantize_impl(x, dtype, rows, cols, ld, fmt, bias_out, q, ldq, qT, ldqT, amax_out, sat, stream))
      return st;
    return fp8_history_push(hist, state, window, amax_out, stream);
  }
  StreamArgs a{};
  a.x = x;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.q = q;
  a.ldq = ldq;
  a.del = d;
  launch_quantize_delayed(a, dtype, fmt, stream);
  return launch_status();
}

// Row-wise MX cast behind mx_quantize_rule (scales row-major, ld_scales) and
// mx_quantize_packed (scales in the packed layout).
static int mx_cast_rows(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int rule,
                        uint8_t* q, int64_t ldq, uint8_t* scales, int64_t ld_scales, bool packed,
                        hipStream_t stream) {
  if (!q || !scales) return FP8_ERR_NULL;
  if (!valid_dtype(dtype)) return FP8_ERR_DTYPE;
  if (!valid_fmt(fmt) || !valid_mx_rule(rule)) return FP8_ERR_FORMAT;
  if (cols % 32) return FP8_ERR_SHAPE;
  int st = check_matrix(rows, cols, ld);
  if (st) return st;
  st = check_matrix(rows, cols, ldq);
  if (st) return st;
  if (!packed) {
    st = check_matrix(rows, cols / 32, ld_scales);
    if (st) return st;
  } else if (!aligned(scales, 16)) {
    return FP8_ERR_ALIGN;
  }
  if (rows * cols == 0) return FP8_OK;
  if (!x) return FP8_ERR_NULL;
  MxArgs a;
  a.x = x;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.q = q;
  a.ldq = ldq;
  a.scales = scales;
  a.lds = ld_scales;
  a.packed = packed;
  a.sgroups = packed_scale_groups(cols / 32);
  a.kb = cols / 32;
  a.collapsed = 0;
  a.nt = 0;
  if (packed && (rows % kPackRows) != 0) {
    // rows past the matrix hold 127 (scale 1): fill the whole buffer first,
    // then the cast overwrites every code of the matrix (blocks past a row's
    // end are padded by the cast itself)
    const int64_t n16 = packed_bytes(rows, cols / 32) / 16;
    hipLaunchKernelGGL(fill_u8_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, stream, scales, n16,
                       0x7f7f7f7fu);
  }
  const int esz = dtype_size(dtype);
  const int epc = 16 / esz;
  // contiguous -> one long row (blocks never straddle rows since cols % 32 == 0).
  // Packed stores then recover a block's row by a division; one workgroup
  // per row is kept when a row is a whole number of workgroup iterations
  // (8192 bf16 columns: 6.0 TB/s per row against 5.7 collapsed), the long
  // row taken otherwise (11008 columns: 4.9 per row).
  const int64_t per_row = (int64_t)kThreads * kUnroll * kItersCast;
  const bool x_vec = aligned(x, 16) && (rows == 1 || (ld * esz) % 16 == 0) && aligned(q, epc) &&
                     (rows == 1 || ldq % epc == 0);
  const bool collapse = a.rows > 1 && a.ld == a.cols && a.ldq == a.cols &&
                        (packed ? x_vec && (a.cols / epc) % per_row != 0 && rows * (cols / 32) < (1LL << 32)
                                : a.lds == a.cols / 32);
  if (collapse) {
    a.collapsed = packed;
    a.cols *= a.rows;
    a.rows = 1;
    a.ld = a.cols;
    a.ldq = a.cols;
    a.lds = a.cols / 32;
  }
  const bool vec = aligned(a.x, 16) && (a.rows == 1 || (a.ld * esz) % 16 == 0) && aligned(a.q, epc) &&
                   (a.rows == 1 || a.ldq % epc == 0);
#define SFP8_MX(DT, FMT)                                       \
  do {                                                         \
    if (rule == MX_RULE_OCP) launch_mx<DT, FMT, true>(a, vec, stream); \
    else launch_mx<DT, FMT, false>(a, vec, stream);            \
  } while (0)
  if (dtype == FP8_DT_BF16) {
    if (fmt == FP8_E4M3) SFP8_MX(FP8_DT_BF16, FP8_E4M3);
    else SFP8_MX(FP8_DT_BF16, FP8_E5M2);
  } else {
    if (fmt == FP8_E4M3) SFP8_MX(FP8_DT_F32, FP8_E4M3);
    else SFP8_MX(FP8_DT_F32, FP8_E5M2);
  }
#undef SFP8_MX
  return launch_status();
}

int mx_quantize_rule(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int rule,
                     uint8_t* q, int64_t ldq, uint8_t* scales, int64_t ld_scales, hipStream_t stream) {
  return mx_cast_rows(x, dtype, rows, cols, ld, fmt, rule, q, ldq, scales, ld_scales, false, stream);
}

int mx_quantize_packed(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int rule,
                       uint8_t* q, int64_t ldq, uint8_t* packed, hipStream_t stream) {
  return mx_cast_rows(x, dtype, rows, cols, ld, fmt, rule, q, ldq, packed, 0, true, stream);
}

int mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, uint8_t* q,
                int64_t ldq, uint8_t* scales, int64_t ld_scales, hipStream_t stream) {
  return mx_quantize_rule(x, dtype, rows, cols, ld, fmt, MX_RULE_FMAX, q, ldq, scales, ld_scales, stream);
}

// Transposed MX cast behind mx_quantize_t_rule (scalesT row-major) and
// mx_quantize_t_packed (scalesT in the packed layout of the [cols x rows/32]
// code matrix).
static int mx_cast_t(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int rule,
                     uint8_t* qT, int64_t ldqT, uint8_t* scalesT, int64_t ld_scales, bool packed,
                     hipStream_t stream) {
  if (!qT || !scalesT) return FP8_ERR_NULL;
  if (!valid_dtype(dtype)) return FP8_ERR_DTYPE;
  if (!valid_fmt(fmt) || !valid_mx_rule(rule)) return FP8_ERR_FORMAT;
  if (rows % 32) return FP8_ERR_SHAPE;
  int st = check_matrix(rows, cols, ld);
  if (st) return st;
  st = check_matrix(cols, rows, ldqT);
  if (st) return st;
  if (!packed) {
    st = check_matrix(cols, rows / 32, ld_scales);
    if (st) return st;
  } else if (!aligned(scalesT, 16)) {
    return FP8_ERR_ALIGN;
  }
  if (rows * cols == 0) return FP8_OK;
  if (!x) return FP8_ERR_NULL;
  const int64_t gy = (rows + kMtR - 1) / kMtR;
  if (gy > 65535) return FP8_ERR_SHAPE;
  MxArgs a;
  a.x = x;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.q = qT;
  a.ldq = ldqT;
  a.scales = scalesT;
  a.lds = ld_scales;
  a.packed = packed;
  a.sgroups = packed_scale_groups(rows / 32);
  a.kb = rows / 32;
  a.collapsed = 0;
  a.nt = rows * cols < kMxtCachedMin;
  if (packed && (cols % kPackRows) != 0) {
    const int64_t n16 = packed_bytes(cols, rows / 32) / 16;        // 127 for the rows past the matrix
    hipLaunchKernelGGL(fill_u8_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, stream, scalesT, n16,
                       0x7f7f7f7fu);
  }
  // 16-byte loads when every row start is 16-byte aligned
  const bool vec = aligned(x, 16) && (ld * dtype_size(dtype)) % 16 == 0;
  // bf16 with 16-byte loads from kMxtCachedMin elements: tiles of 128 x 128
  // (70B-MLP X and W +6-13%; the 7B-MLP tensors gained on X, lost 4% on dY;
  // fp32 at 128 x 64 takes the same LDS; element loads ran 10-20% slower)
  const bool wide = dtype == FP8_DT_BF16 && vec && rows * cols >= kMxtCachedMin;
  const int tc = wide ? kMtCWide : kMtC;
  const dim3 grid((unsigned)((cols + tc - 1) / tc), (unsigned)gy);
#define SFP8_MXT(DT, FMT)                                                                              \
  do {                                                                                                 \
    constexpr int TW = DT == FP8_DT_BF16 ? kMtCWide : kMtC;                                            \
    if (rule == MX_RULE_OCP) {                                                                         \
      if (wide) hipLaunchKernelGGL((mx_transpose_kernel<DT, FMT, true, true, TW>), grid, dim3(kThreads), 0, stream, a); \
      else if (vec) hipLaunchKernelGGL((mx_transpose_kernel<DT, FMT, true, true>), grid, dim3(kThreads), 0, stream, a); \
      else hipLaunchKernelGGL((mx_transpose_kernel<DT, FMT, false, true>), grid, dim3(kThreads), 0, stream, a);   \
    } else {                                                                                           \
      if (wide) hipLaunchKernelGGL((mx_transpose_kernel<DT, FMT, true, false, TW>), grid, dim3(kThreads), 0, stream, a); \
      else if (vec) hipLaunchKernelGGL((mx_transpose_kernel<DT, FMT, true, false>), grid, dim3(kThreads), 0, stream, a); \
      else hipLaunchKernelGGL((mx_transpose_kernel<DT, FMT, false, false>), grid, dim3(kThreads), 0, stream, a);   \
    }                                                                                                  \
  } while (0)
  if (dtype == FP8_DT_BF16) {
    if (fmt == FP8_E4M3) SFP8_MXT(FP8_DT_BF16, FP8_E4M3);
    else SFP8_MXT(FP8_DT_BF16, FP8_E5M2);
  } else {
    if (fmt == FP8_E4M3) SFP8_MXT(FP8_DT_F32, FP8_E4M3);
    else SFP8_MXT(FP8_DT_F32, FP8_E5M2);
  }
#undef SFP8_MXT
  return launch_status();
}

int mx_quantize_t_rule(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int rule,
                       uint8_t* qT, int64_t ldqT, uint8_t* scalesT, int64_t ld_scales, hipStream_t stream) {
  return mx_cast_t(x, dtype, rows, cols, ld, fmt, rule, qT, ldqT, scalesT, ld_scales, false, stream);
}

int mx_quantize_t_packed(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int rule,
                         uint8_t* qT, int64_t ldqT, uint8_t* packed, hipStream_t stream) {
  return mx_cast_t(x, dtype, rows, cols, ld, fmt, rule, qT, ldqT, packed, 0, true, stream);
}

int mx_quantize_t(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, uint8_t* qT,
                  int64_t ldqT, uint8_t* scalesT, int64_t ld_scales, hipStream_t stream) {
  return mx_quantize_t_rule(x, dtype, rows, cols, ld, fmt, MX_RULE_FMAX, qT, ldqT, scalesT, ld_scales, stream);
}

}  // extern "C"

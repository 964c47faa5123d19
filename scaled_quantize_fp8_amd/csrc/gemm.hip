// Scaled FP8 GEMMs for gfx950: per-tensor (unscale in the epilogue) and
// block-scaled MX (E8M0 scales applied by the MFMA itself), both with fp32
// accumulation, bf16 or fp32 output and the output amax fused into the
// epilogue.
//
// "Training and inference of large language models using 8-bit floating
// point" (paper review), "Proposed method": the matrix multiplication runs on
// the FP8 operands and is unscaled afterwards; gradients (E5) meet weights
// or activations (E4) in the backward products.  "Per-Tensor and Per-Block
// Scaling Strategies for Effective FP8 Training" (summary), "Key Questions
// Answered": per-block scaling, each block with its own factor.
//
// Two kernels.
//   * gemm_fwd_kernel: every per-tensor product (both operands
//     K-contiguous, the forward product Y = X W^T, or either one MN-major,
//     [K x M] / [K x N] storage, the backward products dX = dY W and
//     dW = dY^T X; any K, a last partial K stage included) and every MX
//     product on packed scales, or on 4-byte aligned row-major scale rows
//     with K >= 512: 32x32x64 MFMAs fed from a
//     two-slot LDS pipeline (three slots for long per-tensor products on
//     small grids) with asynchronous global -> LDS copies; an MN-major
//     operand is copied as K rows and its fragments are read with the LDS
//     transpose read ds_read_b64_tr_b8.  Described where it is defined.
//   * gemm_kernel: every other case (MX on row-major scales with K < 512 or
//     rows that are not 4-byte aligned; K = 0) with the design below.
//
// gemm_kernel's CDNA4 mapping.
//   * Macro tile 256 (M) x 256 (N) x 128 (K bytes), 256 lanes = 4 waves in a
//     2 x 2 arrangement, each wave owning 128 x 128 of C as 8 x 8
//     v_mfma_f32_16x16x128_f8f6f4 blocks (256 fp32 accumulators per lane).
//   * Operands are staged in LDS, double-buffered (2 x 64 KiB of the 160 KiB),
//     K-contiguous: row r of a tile is 128 bytes, its 16-byte chunk c stored
//     at chunk c ^ ((r ^ (r >> 4)) & 7) so that the MFMA fragment reads
//     (16 rows, same chunk) and the staging writes are bank-conflict free.
//   * A lane's MFMA operand is two 16-byte K chunks of one row (lane group g
//     holds K [16g, 16g+16) and [64+16g, 64+16g+16)); the block-scaled MFMA
//     reads the E8M0 scale of (row, 32-wide K block j) from lane 16 j + row.
//   * The MFMA's first operand is a W (op(B)) fragment and its second an X
//     (op(A)) fragment, so a lane's four accumulators are four consecutive
//     n of one output row m: the epilogue stores 8 (bf16) or 16 (fp32)
//     contiguous bytes per lane.
//   * Transposed operands ([K x M] storage) are loaded 16 M-bytes at a time
//     for four consecutive k and transposed 4 x 4 bytes in registers
//     (v_perm_b32) on their way into the K-contiguous LDS layout.
//
// Both kernels map workgroups to tiles XCD-aware: consecutive workgroup ids
// land on different XCDs, so ids are remapped to give each XCD a contiguous
// range of tiles, walked in groups of 8 tile-rows for L2 reuse.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "host.hpp"

namespace sfp8 {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kGemmThreads = 256;
constexpr int kGroupM = 8;
constexpr int kTileBytes = BM * BK;          // 32 KiB per operand per stage
// The packed E8M0 layout (kPackRows x kPackBlocks codes per 4 KiB block,
// host.hpp): one group of 16 K-blocks is 4 K stages of this kernel.
// Forward kernel launch: persistent per-tensor grid (true) or one tile per
// workgroup (false, measured faster; see gemm_fwd_kernel).
constexpr bool kFwdPersistent = false;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 4)) & 7; }

// Offset of byte k (0..127) of tile row `row` in the swizzled layout.
__device__ __forceinline__ int lds_off(int row, int k) {
  return row * BK + ((((k >> 4) ^ swz(row)) << 4) | (k & 15));
}

struct GemmArgs {
  int64_t M, N, K;
  const uint8_t* A;
  int64_t lda;
  const uint8_t* B;
  int64_t ldb;
  const int32_t* bias_a;
  const int32_t* bias_b;
  const uint8_t* sa;       // MX scales of op(A) rows [M x K/32]
  int64_t lds_a;
  const uint8_t* sb;       // MX scales of op(B) rows [N x K/32]
  int64_t lds_b;
  void* C;
  int64_t ldc;
  float* out_amax;
  int out_f32;
  int vec_store;
  int row16;                 // C and every row start 16-byte aligned (full-line bf16 stores)
  int sa_dword;            // scale rows 4-byte aligned: one dword per stage
  int sb_dword;
  int scales_dma;          // forward kernel's scale copies: packed, or dword-aligned rows with K >= 512
  int scales_packed;       // sa / sb in the tiled layout of mx_pack_scales (forward kernel only)
  int64_t sgroups;         // packed layout: 16-block groups per row, ceil(K / 512)
};

// ---- buffer resources ------------------------------------------------------
// Raw buffer descriptors give range-checked loads: an offset at or past
// num_records reads zeros, which is how ragged tile edges are zero-filled.
constexpr uint32_t kOOB = 0x80000000u;       // offset that is always out of range
constexpr int kRsrcWord3 = 0x00020000;       // raw (untyped) buffer, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t rec = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)rec, kRsrcWord3);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// ---- K-contiguous operand: global -> LDS directly ----------------------------
// The tile is 32 blocks of 8 rows x 128 bytes (1 KiB).  Wave w fills blocks
// 8w .. 8w+7 with one buffer_load_dwordx4 ... lds each: lane L lands at byte
// 16 L of the block, i.e. row L/8, stored chunk L%8, so it fetches logical
// chunk (L%8) ^ swz(row) of that row (8 lanes = one 128-byte row segment).
__device__ __forceinline__ void dma_tile_k(uint8_t* S, __amdgpu_buffer_rsrc_t rsrc, int64_t ld, int64_t rows_left,
                                           int64_t k0, int64_t K) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = wave * 8 + i;
    const int row = blk * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    const int64_t gk = k0 + 16 * c;
    const uint32_t off = (row < rows_left && gk < K) ? (uint32_t)(row * ld + gk) : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(S + blk * 1024), 16, off, 0, 0, 0);
  }
}

// ---- transposed operand: global -> registers -> (transpose) -> LDS ---------
// Stored [K x R] (R contiguous): a lane loads 16 R-bytes for 4 consecutive k,
// twice (kg = lane/16 and lane/16 + 16).
__device__ __forceinline__ void load_tile_t(__amdgpu_buffer_rsrc_t rsrc, int64_t ld, int64_t rows_left,
                                            int64_t k0, int64_t K, uint4 (&reg)[8]) {
  const int t = threadIdx.x;
  const int r16 = t & 15;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int kg = (t >> 4) + 16 * u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gk = k0 + 4 * kg + j;
      const uint32_t off = (gk < K && 16 * r16 < rows_left) ? (uint32_t)(gk * ld + 16 * r16) : kOOB;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
      reg[4 * u + j] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
}

// 4 x 4 byte transpose: a_k holds bytes (r0..r3) of k-row k; d_j gets bytes
// (k0..k3) of row j.
__device__ __forceinline__ void transpose4x4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t& d0,
                                             uint32_t& d1, uint32_t& d2, uint32_t& d3) {
  const uint32_t x0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);   // a0b0 a1b0 a0b1 a1b1
  const uint32_t x1 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);   // a0b2 a1b2 a0b3 a1b3
  const uint32_t y0 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);   // a2b0 a3b0 a2b1 a3b1
  const uint32_t y1 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);   // a2b2 a3b2 a2b3 a3b3
  d0 = __builtin_amdgcn_perm(y0, x0, 0x05040100u);                  // a0b0 a1b0 a2b0 a3b0
  d1 = __builtin_amdgcn_perm(y0, x0, 0x07060302u);                  // a0b1 a1b1 a2b1 a3b1
  d2 = __builtin_amdgcn_perm(y1, x1, 0x05040100u);
  d3 = __builtin_amdgcn_perm(y1, x1, 0x07060302u);
}

__device__ __forceinline__ void store_tile_t(uint8_t* S, const uint4 (&reg)[8]) {
  const int t = threadIdx.x;
  const int r16 = t & 15;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int kg = (t >> 4) + 16 * u;
    const int k = 4 * kg;
    const uint4 a0 = reg[4 * u + 0], a1 = reg[4 * u + 1], a2 = reg[4 * u + 2], a3 = reg[4 * u + 3];
    const uint32_t w0[4] = {a0.x, a0.y, a0.z, a0.w};
    const uint32_t w1[4] = {a1.x, a1.y, a1.z, a1.w};
    const uint32_t w2[4] = {a2.x, a2.y, a2.z, a2.w};
    const uint32_t w3[4] = {a3.x, a3.y, a3.z, a3.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t d[4];
      transpose4x4(w0[w], w1[w], w2[w], w3[w], d[0], d[1], d[2], d[3]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * r16 + 4 * w + j;
        *reinterpret_cast<uint32_t*>(S + lds_off(row, k)) = d[j];
      }
    }
  }
}

// MX scales of a stage: lane t loads the four E8M0 codes of tile row t (one
// dword when the four blocks exist, bytes at the K tail); rows past the
// matrix and blocks past K get code 127 (scale 1) next to their zero data.
__device__ __forceinline__ uint32_t load_scales(const uint8_t* __restrict__ S, int64_t lds, int64_t row0,
                                                int64_t R, int64_t k0, int64_t K, bool dword_ok) {
  const int64_t gr = row0 + threadIdx.x;
  const int64_t kb0 = k0 / 32;
  const int64_t nkb = K / 32;
  if (gr >= R) return 0x7f7f7f7fu;
  const uint8_t* p = S + gr * lds + kb0;
  if (dword_ok && kb0 + 4 <= nkb) return *reinterpret_cast<const uint32_t*>(p);
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) v |= (uint32_t)(kb0 + j < nkb ? p[j] : 0x7fu) << (8 * j);
  return v;
}

// MFMA operand of v_mfma_*_16x16x128_f8f6f4 for tile rows row0 .. row0+15:
// lane l (g = l / 16) holds row row0 + l % 16, K bytes [16g, 16g + 16) in its
// first four registers and [64 + 16g, 64 + 16g + 16) in the last four.  The
// block-scaled form takes the E8M0 scale of (row l % 16, K block l / 16)
// from lane l, so the two chunks a lane holds need not share its block.
__device__ __forceinline__ v8i load_frag(const uint8_t* S, int row0, int lane) {
  const int row = row0 + (lane & 15);
  const int c = lane >> 4;
  const uint4 lo = *reinterpret_cast<const uint4*>(S + row * BK + ((c ^ swz(row)) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(S + row * BK + (((c + 4) ^ swz(row)) << 4));
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// Output tile mapping: XCD-aware remap, then groups of kGroupM tile-rows.
__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  const int64_t T = tiles_m * tiles_n;
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid % 8, local = bid / 8;
  const int64_t q = T / 8, r = T % 8;
  const int64_t lin = (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  const int64_t per_group = kGroupM * tiles_n;
  const int64_t group = lin / per_group;
  const int64_t first_m = group * kGroupM;
  const int64_t gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int64_t in_group = lin % per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

template <int FA, int FB, bool MX, bool TA, bool TB>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * kTileBytes];
  __shared__ uint32_t s_scale[MX ? 2 * 2 * BM : 1];
  __shared__ uint32_t red[kGemmThreads / kWave];

  const int64_t tiles_m = (g.M + BM - 1) / BM;
  const int64_t tiles_n = (g.N + BN - 1) / BN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // stage b: op(A) tile at smem + 2b * kTileBytes, op(B) tile right after it

  uint4 ra[TA ? 8 : 1], rb[TB ? 8 : 1];
  uint32_t rsa = 0, rsb = 0;
  const int64_t nk = (g.K + BK - 1) / BK;
  const int64_t rows_a = g.M - m0, rows_b = g.N - n0;
  // op(A) / op(B) tiles: K-contiguous ones read rows [m0, m0+256) x K,
  // transposed ones read columns [m0, m0+256) of a [K x M] matrix.
  const __amdgpu_buffer_rsrc_t rs_a =
      TA ? make_rsrc(g.A + m0, (g.K - 1) * g.lda + (rows_a < BM ? rows_a : BM))
         : make_rsrc(g.A + m0 * g.lda, ((rows_a < BM ? rows_a : BM) - 1) * g.lda + g.K);
  const __amdgpu_buffer_rsrc_t rs_b =
      TB ? make_rsrc(g.B + n0, (g.K - 1) * g.ldb + (rows_b < BN ? rows_b : BN))
         : make_rsrc(g.B + n0 * g.ldb, ((rows_b < BN ? rows_b : BN) - 1) * g.ldb + g.K);

  // issue the global reads of stage kt (DMA straight into buffer `buf` for
  // K-contiguous operands, registers for transposed ones and scales)
  auto gload = [&](int64_t kt, int buf) {
    const int64_t k0 = kt * BK;
    uint8_t* sa_ = smem + 2 * buf * kTileBytes;
    uint8_t* sb_ = sa_ + kTileBytes;
    if constexpr (TA) load_tile_t(rs_a, g.lda, rows_a, k0, g.K, ra);
    else dma_tile_k(sa_, rs_a, g.lda, rows_a, k0, g.K);
    if constexpr (TB) load_tile_t(rs_b, g.ldb, rows_b, k0, g.K, rb);
    else dma_tile_k(sb_, rs_b, g.ldb, rows_b, k0, g.K);
    if constexpr (MX) {
      rsa = load_scales(g.sa, g.lds_a, m0, g.M, k0, g.K, g.sa_dword);
      rsb = load_scales(g.sb, g.lds_b, n0, g.N, k0, g.K, g.sb_dword);
    }
  };
  // finish stage `buf` from registers (transposes, scales)
  auto sstore = [&](int buf) {
    uint8_t* sa_ = smem + 2 * buf * kTileBytes;
    uint8_t* sb_ = sa_ + kTileBytes;
    if constexpr (TA) store_tile_t(sa_, ra);
    if constexpr (TB) store_tile_t(sb_, rb);
    if constexpr (MX) {
      s_scale[buf * 2 * BM + threadIdx.x] = rsa;
      s_scale[buf * 2 * BM + BM + threadIdx.x] = rsb;
    }
  };

  if (nk > 0) {
    gload(0, 0);
    sstore(0);
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    // buffer cur^1 was last read in iteration kt-1, which every wave has
    // left (barrier below), so stage kt+1 may land in it now
    if (kt + 1 < nk) gload(kt + 1, cur ^ 1);

    const uint8_t* A_ = smem + 2 * cur * kTileBytes;
    const uint8_t* B_ = A_ + kTileBytes;
    v8i xf[8];
    // MX: this lane's E8M0 codes for the 8 op(A) fragments, 4 per register;
    // the MFMA's op_sel immediate picks the byte of fragment mb.
    int xs[2] = {0, 0};
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      xf[mb] = load_frag(A_, wm * 128 + mb * 16, lane);
      if constexpr (MX) {
        const uint32_t code =
            (s_scale[cur * 2 * BM + wm * 128 + mb * 16 + (lane & 15)] >> (8 * (lane >> 4))) & 0xffu;
        xs[mb >> 2] |= (int)(code << (8 * (mb & 3)));
      }
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const v8i wf = load_frag(B_, wn * 128 + nb * 16, lane);
      int ws = 0;
      if constexpr (MX)
        ws = (int)((s_scale[cur * 2 * BM + BM + wn * 128 + nb * 16 + (lane & 15)] >> (8 * (lane >> 4))) & 0xffu);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        if constexpr (MX) {
          if ((mb & 3) == 0)
            acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xf[mb], acc[nb][mb], FB, FA, 0, ws,
                                                                           0, xs[mb >> 2]);
          else if ((mb & 3) == 1)
            acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xf[mb], acc[nb][mb], FB, FA, 0, ws,
                                                                           1, xs[mb >> 2]);
          else if ((mb & 3) == 2)
            acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xf[mb], acc[nb][mb], FB, FA, 0, ws,
                                                                           2, xs[mb >> 2]);
          else
            acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xf[mb], acc[nb][mb], FB, FA, 0, ws,
                                                                           3, xs[mb >> 2]);
        } else {
          acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xf[mb], acc[nb][mb], FB, FA, 0, 0, 0, 0);
        }
      }
    }

    if (kt + 1 < nk) sstore(cur ^ 1);
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    __syncthreads();
  }

  // ---- epilogue: unscale, round, store, fused |C| max ----------------------
  // (for MX the exponent is 0, hidden from the compiler as in gemm_fwd_kernel)
  int e = MX ? 0 : -(*g.bias_a + *g.bias_b);
  if constexpr (MX) asm volatile("" : "+s"(e));
  uint32_t amax_bits = 0;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int64_t m = m0 + wm * 128 + mb * 16 + (lane & 15);
      const int64_t n = n0 + wn * 128 + nb * 16 + 4 * (lane >> 4);
      if (m >= g.M) continue;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = __builtin_amdgcn_ldexpf(acc[nb][mb][r], e);
      if (g.out_f32) {
        float* crow = reinterpret_cast<float*>(g.C) + m * g.ldc;
        if (g.vec_store && n + 3 < g.N) {
          *reinterpret_cast<float4*>(crow + n) = make_float4(v[0], v[1], v[2], v[3]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t ab = __float_as_uint(v[r]) & 0x7fffffffu;
            amax_bits = amax_bits > ab ? amax_bits : ab;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (n + r < g.N) {
              crow[n + r] = v[r];
              const uint32_t ab = __float_as_uint(v[r]) & 0x7fffffffu;
              amax_bits = amax_bits > ab ? amax_bits : ab;
            }
          }
        }
      } else {
        uint16_t h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = __builtin_bit_cast(uint16_t, (__bf16)v[r]);
        uint16_t* crow = reinterpret_cast<uint16_t*>(g.C) + m * g.ldc;
        if (g.vec_store && n + 3 < g.N) {
          *reinterpret_cast<uint2*>(crow + n) =
              make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t ab = ((uint32_t)h[r] & 0x7fffu) << 16;
            amax_bits = amax_bits > ab ? amax_bits : ab;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (n + r < g.N) {
              crow[n + r] = h[r];
              const uint32_t ab = ((uint32_t)h[r] & 0x7fffu) << 16;
              amax_bits = amax_bits > ab ? amax_bits : ab;
            }
          }
        }
      }
    }
  }
  if (g.out_amax) block_max_to_global(amax_bits, red, g.out_amax);
}


// ===========================================================================
// Forward kernel (32x32x64 MFMAs from LDS-DMA stages; K-contiguous or MN-major operands).
// ===========================================================================
// Global -> LDS copies are issued as inline assembly
// (buffer_load_dwordx4 ... lds): for the compiler's own LDS-DMA builtin, its
// waitcnt pass waits for every outstanding copy before any later LDS read,
// which would serialise the prefetch with the MFMAs.  Completion is tracked
// explicitly with s_waitcnt vmcnt (issued through the builtin, so that the
// pass knows about it and adds no waits of its own).
typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (base, stride 0, num_records, gfx9 raw format) in
// SGPRs for the inline-assembly loads below.
__device__ __forceinline__ v4i make_srd(const void* base, int64_t bytes) {
  const int64_t rec = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)rec);
  r[3] = kRsrcWord3;
  return r;
}

// 32-bit LDS byte offset of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// A descriptor held in SGPRs (its words are wave-uniform by construction).
__device__ __forceinline__ v4i uniform_srd(v4i r) {
  v4i u;
  u[0] = __builtin_amdgcn_readfirstlane(r[0]);
  u[1] = __builtin_amdgcn_readfirstlane(r[1]);
  u[2] = __builtin_amdgcn_readfirstlane(r[2]);
  u[3] = __builtin_amdgcn_readfirstlane(r[3]);
  return u;
}

// The compiler's hazard checks do not look inside inline assembly, so the
// copies below carry the wait states themselves: an LDS DMA needs one after
// the SALU write of M0, and a VMEM instruction needs five after a VALU
// (v_readfirstlane) wrote one of its SGPR operands.  W is the number of wait
// states placed between the M0 write and the load: 5 where the descriptor or
// soffset may have just come from v_readfirstlane (the first copy of each
// operand in a stage, where the compiler re-materialises descriptors it has
// moved to VGPRs; the scale copies; the prefetch), 1 elsewhere.
//
// 16 bytes per lane from buffer offset off + soff to LDS lds_addr + 16 * lane
// (lds_addr and soff wave-uniform).
template <int W>
__device__ __forceinline__ void dma_b128_so(v4i srd, uint32_t lds_addr, uint32_t off, uint32_t soff) {
  static_assert(W >= 1 && W <= 16, "wait states");
  asm volatile("s_mov_b32 m0, %1\n\ts_nop %4\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
               :: "v"(off), "s"(lds_addr), "s"(srd), "s"(soff), "i"(W - 1) : "memory", "m0");
}

// 4 bytes per lane from buffer offset off + soff to LDS lds_addr + 4 * lane.
template <int W>
__device__ __forceinline__ void dma_b32_so(v4i srd, uint32_t lds_addr, uint32_t off, uint32_t soff) {
  static_assert(W >= 1 && W <= 16, "wait states");
  asm volatile("s_mov_b32 m0, %1\n\ts_nop %4\n\tbuffer_load_dword %0, %2, %3 offen lds"
               :: "v"(off), "s"(lds_addr), "s"(srd), "s"(soff), "i"(W - 1) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N> __device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

typedef float v16f __attribute__((ext_vector_type(16)));

// The 16 bytes of v with the first s (uniform, 0..15) dropped: byte j of the
// result is byte j + s of v where j + s < 16; the rest repeat bytes of v.
__device__ __forceinline__ uint4 drop_bytes(uint4 v, int s) {
  const int q = s >> 2, b = s & 3;
  const bool h = (q & 2) != 0, o = (q & 1) != 0;
  const uint32_t u0 = h ? v.z : v.x, u1 = h ? v.w : v.y;
  const uint4 d = make_uint4(o ? u1 : u0, o ? v.z : u1, o ? v.w : v.z, v.w);   // dwords dropped
  // then bytes: dword k takes bytes b .. 3 of d[k] and 0 .. b - 1 of d[k + 1]
  return make_uint4(__builtin_amdgcn_alignbyte(d.y, d.x, b), __builtin_amdgcn_alignbyte(d.z, d.y, b),
                    __builtin_amdgcn_alignbyte(d.w, d.z, b), __builtin_amdgcn_alignbyte(d.w, d.w, b));
}

// 32x32x64 MFMA with E8M0 scales picked by byte (op_sel) from packed registers.
template <int FA_, int FB_>
__device__ __forceinline__ v16f mfma32(v8i a, v8i b, v16f c, int sa, int oa, int sb, int ob) {
#define SFP8_M(OA, OB) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA_, FB_, OA, sa, OB, sb)
  switch (oa * 4 + ob) {
    case 0: SFP8_M(0, 0); case 1: SFP8_M(0, 1); case 2: SFP8_M(0, 2); case 3: SFP8_M(0, 3);
    case 4: SFP8_M(1, 0); case 5: SFP8_M(1, 1); case 6: SFP8_M(1, 2); case 7: SFP8_M(1, 3);
    case 8: SFP8_M(2, 0); case 9: SFP8_M(2, 1); case 10: SFP8_M(2, 2); case 11: SFP8_M(2, 3);
    case 12: SFP8_M(3, 0); case 13: SFP8_M(3, 1); case 14: SFP8_M(3, 2); default: SFP8_M(3, 3);
  }
#undef SFP8_M
}

// ---------------------------------------------------------------------------
// Forward-layout kernel.
//   * Macro tile 256 x 256, K stages of 128 bytes, 4 waves in 2 x 2, each
//     wave owning 128 x 128 of C as 4 x 4 v_mfma_f32_32x32x64_f8f6f4 blocks
//     (256 fp32 accumulators per lane, all in AGPRs).
//   * LDS: op(A) stages at [0, 64K) (slot s at 32K s), op(B) stages at
//     [64K, 128K); a stage is 256 rows x 128 bytes, the 16-byte chunk c of
//     row r stored at chunk c ^ fswz(r), fswz(r) = (r & 7) ^ ((r >> 3) & 1).
//     A fragment read has 16 lanes on 16 consecutive rows and one logical
//     chunk; with 64 four-byte banks two 128-byte rows share a bank window,
//     so the 16 (row parity, stored chunk) pairs must differ: plain r & 7
//     repeats them at rows r and r + 8 (2-way conflicts on every read),
//     fswz does not (and stays a bijection within 8 rows).  Every fragment
//     read is a loop-invariant per-lane base plus an immediate (slot,
//     fragment).
//   * Pipeline, two slots: a stage is two 64-byte K sub-steps.  Phase A runs
//     sub-step 0's 16 MFMAs while reading sub-step 1's fragments; the wave
//     then waits for its own copies of stage kt+1 and the workgroup meets at
//     one barrier; phase B runs sub-step 1's MFMAs while reading stage kt+1's
//     sub-step 0 fragments and issuing stage kt+2's copies (one per MFMA) into
//     the slot stage kt has just released.
//   * The loop is unrolled by 2 (by 4 for MX, whose scale codes are copied
//     4 stages at a time) and always runs whole iterations: stages past nk
//     copy zeros through zero-sized buffer descriptors and add nothing, so
//     the loop body has no branches.  The workgroup's final wait covers
//     every copy; the C stores issued after them may drain after it ends.
//   * bf16 epilogue of an interior tile: a lane's accumulators are 4 n of
//     one row, so direct stores would write 16 bytes in each of 32 rows per
//     instruction; instead each 32 x 64 quarter of a wave's block row is
//     staged in 4 KiB of LDS and written back as whole 128-byte row segments
//     (measured +3% per-tensor, +5% MX on the 70B-MLP shape with every CU
//     writing its tile at once).
// ---------------------------------------------------------------------------
// 32x32x64 operand: K sub-step h (bytes 64h..64h+63) of rows row0 + (l % 32);
// lane l (g = l / 32) holds chunk 4h + g then 4h + 2 + g.  `base_lo/hi` are
// the lane's byte offsets for fragment 0 of slot 0; slot and fragment are
// immediates.
typedef unsigned short us2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (RNE), packed low / high.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  const f2v f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

template <int OFF>
__device__ __forceinline__ v8i frag_at(const uint8_t* lds, uint32_t base_lo, uint32_t base_hi) {
  const uint4 lo = *reinterpret_cast<const uint4*>(lds + base_lo + OFF);
  const uint4 hi = *reinterpret_cast<const uint4*>(lds + base_hi + OFF);
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// The same operand from an MN-major stage (K rows of RS = 256 or 128 bytes,
// MN contiguous, the 16-byte chunk c of K row k stored at chunk c ^ tswz(k):
// (k & 7) | ((k >> 4) & 1) << 3 for 256-byte rows, ((k >> 1) & 3) << 1 for
// 128-byte rows), by four LDS transpose reads.
// ds_read_b64_tr_b8 works on groups of 16 lanes: lane j of a group gives
// the address of 8 bytes, row j / 2 and half j % 2 of an 8 x 16-byte block,
// and receives column j of the block, its 8 rows.  Lane l (group q = l / 16,
// j = l % 16, g = l / 32) takes 8 K rows at 16 g + {0, 8, 32, 40} + 64 h of
// MN column 16 (q & 1) + j of the fragment: the 8-byte pieces of its
// operand in K order.  Its rows all have one tswz ((j >> 1) | g << 3 for
// 256-byte rows, ((j >> 2) & 3) << 1 for 128-byte rows), so `base` (per lane
// and fragment) plus an immediate (slot, sub-step, piece) addresses every
// read.
template <int OFF, int RS>
__device__ __forceinline__ v8i frag_tr(const uint8_t* lds, uint32_t base) {
  typedef int v2i_t __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) v2i_t* lds_v2i;
  const v2i_t p0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(lds + base + OFF));
  const v2i_t p1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(lds + base + OFF + 8 * RS));
  const v2i_t p2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(lds + base + OFF + 32 * RS));
  const v2i_t p3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(lds + base + OFF + 40 * RS));
  v8i f;
  f[0] = p0.x; f[1] = p0.y; f[2] = p1.x; f[3] = p1.y;
  f[4] = p2.x; f[5] = p2.y; f[6] = p3.x; f[7] = p3.y;
  return f;
}

template <int N> using IC = std::integral_constant<int, N>;

// Workgroup -> tile mapping of virtual block id vb (32-bit): XCD-aware remap,
// then groups of kGroupM tile-rows (the mapping tile_coords gives blockIdx).
__device__ __forceinline__ void tile_coords_vb(int vb, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int xcd = vb & 7, local = vb >> 3;
  const int q = T >> 3, r = T & 7;
  const int lin = (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  const int per_group = kGroupM * tiles_n;
  const int group = lin / per_group;
  const int first_m = group * kGroupM;
  const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int in_group = lin - group * per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// Buffer descriptors of one output tile's operand panels (and MX scale
// panels).  A panel's size ends at its last existing row, so rows past the
// matrix are out of range for tile-independent per-lane offsets; a tile
// past the end gets size-0 descriptors (every copy reads zeros).
struct TileSrd {
  v4i a, b, sa, sb;
};

template <int FA, int FB, bool MX, int BMX, int NSLOT, bool TA = false, bool TB = false, bool TL = false>
__global__ __launch_bounds__(kGemmThreads) void gemm_fwd_kernel(GemmArgs g) {
  // BMX: tile rows (256, or 128 for grids with fewer 256 x 256 tiles than
  // compute units).  A 256-row tile puts the 4 waves in 2 x 2, each 128 x
  // 128 of C; a 128-row tile in 1 x 4, each 128 x 64 (4 op(A) and 2 op(B)
  // fragments, 8 MFMAs per sub-step, 12 copies per stage).
  static_assert(BMX == 256 || BMX == 128, "tile rows");
  // TL (tail): the last K stage or scale group is partial.  K % 128 != 0:
  // the last stage's K-contiguous copies read zeros past K; MX on row-major
  // scales with K % 512 != 0: the last group of scale codes is copied from
  // 16 codes before the row's end and shifted into place.
  // Its own instantiation, so that the others carry none of its selects
  // (in every instantiation they had cost packed MX products 2-5%).
  constexpr int NI = BMX == 256 ? 4 : 2;            // op(B) fragments per wave
  constexpr int WN = NI * 32;                       // C columns per wave
  constexpr int NA = BMX / 32;                      // op(A) copies per stage per wave
  constexpr int NT = NI * 4;                        // MFMAs per sub-step
  // NSLOT: LDS slots (stages resident).  Two, or three for the per-tensor
  // 128-row tile at K >= 4096: its stages are half as long as a 256-row
  // tile's, too short to cover a copy's latency with one stage in flight
  // (2048 x 4096 x 4096: waves wait on copies 30% of their cycles against
  // 10% on the 70B-MLP shape).  With three, the L2 prefetch is off (no room
  // for its landing words) and the epilogue stages C in the slots, idle by
  // then.  Measured: 2048 x 4096 x 4096 +6%, 4096 x 2048 x 4096 +7%,
  // K = 8192 +17%; below K = 4096 two slots were 2-4% faster.
  constexpr int NS = NSLOT;
  static_assert(NS == 2 || (NS == 3 && BMX == 128 && !MX), "slot count");
  // TA / TB: op(A) / op(B) stored MN-major ([K x M] / [K x N], the
  // transposed layouts of the per-tensor product); their stages hold the
  // stage's 128 K rows of the tile's MN bytes (256, or BMX for op(A)), read
  // by LDS transposes (frag_tr)
  static_assert(!(TA || TB) || !MX, "MN-major operands: per-tensor products");

  constexpr int kSlotA = NS == 3 ? BMX * BK : kTileBytes;   // op(A) bytes per slot
  constexpr int kSlotB = kTileBytes;                        // op(B) bytes per slot
  constexpr bool PF = NS == 2;                              // L2 prefetch of op(B)
  __shared__ __attribute__((aligned(16))) uint8_t smem[NS * (kSlotA + kSlotB)];
  // MX scales, 4 stages per copy: [group slot][operand][tile row][4 dwords]
  __shared__ __attribute__((aligned(16))) uint32_t s_scale[MX ? 2 * 2 * BM * 4 : 1];
  __shared__ uint32_t red[kGemmThreads / kWave];
  __shared__ uint32_t pf_sink[PF ? 64 : 1];         // landing words of the L2 prefetch (never read)
  // bf16 epilogue staging, 4 KiB per wave (32 rows x 128 bytes of C).  MX
  // has room for two waves' areas only: waves 0 and 1 stage in the scale
  // slot the finished tile has released.
  constexpr int kStage = 32 * 128;
  __shared__ __attribute__((aligned(16))) uint8_t cstage[NS == 3 ? 16 : (MX ? 2 : 4) * kStage];
  constexpr int kRegB = NS * kSlotA;                // op(B) region offset
  constexpr int kFrag = 32 * BK;                    // 4 KiB between 32-row fragments
  constexpr int U = MX ? 4 : NS;                    // stages per loop iteration
  constexpr int LPS = NA + 8;                       // data copies per stage per wave
  // Launch shape (kFwdPersistent): one tile per workgroup, the dispatcher
  // refilling each compute unit as a workgroup ends.  The persistent form
  // (one workgroup per compute unit walking tiles, the last two stages of a
  // tile prefetching the next tile's first two) is kept for the per-tensor
  // product behind the switch; since a workgroup's final wait leaves its C
  // stores in flight it measures slower (70B-MLP shape: -2.1% at K = 8192,
  // -2.3% at K = 4096).  MX never runs persistent: its scale descriptors
  // leave no SGPRs for a second tile's.
  constexpr bool PERSIST = kFwdPersistent && !MX && BMX == 256;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: SGPR
  const int wm = BMX == 256 ? wave >> 1 : 0, wn = BMX == 256 ? wave & 1 : wave;
  const int tiles_m = (int)((g.M + BMX - 1) / BMX);
  const int tiles_n = (int)((g.N + BN - 1) / BN);
  const int tiles = tiles_m * tiles_n;
  const int P = gridDim.x;                          // persistent: tiles vb, vb + P, ...
  // stages (K % 128 == 0 unless TL), nk < 2^24
  const int nk = (int)(TL ? (g.K + BK - 1) / BK : g.K / BK);
  const int nkU = (nk + U - 1) / U * U;             // stages run per tile (zero stages past nk)
  const int ngroups = nkU / 4;                      // MX scale copies per tile
  const bool pk = MX && g.scales_packed;            // tiled scale layout (uniform)
  // Row-major scales with K % 512 != 0: the last group holds fewer than 16
  // real codes (K / 32 of a row in all).  Its copy is moved back to end at
  // the row's end (codes K/32 - 16 .. K/32 - 1, inside the row since
  // K >= 512), so code c of the group sits at byte c + gsb(G) of the 16;
  // blocks past K (zero operands) take whatever codes the other bytes hold.
  const int kbr = (int)(g.K / 32);                  // real 32-wide K blocks of a row
  auto gsb = [&](int G) {
    const int s = 16 * (G + 1) - kbr;
    return (!(TL && MX) || pk || G >= ngroups || s < 0) ? 0 : s;
  };

  auto make_tile = [&](int vb, TileSrd& T) {
    if (vb < tiles && (PERSIST || vb == (int)blockIdx.x)) {
      int tm, tn;
      tile_coords_vb(vb, tiles_m, tiles_n, tm, tn);
      const int64_t m0 = (int64_t)tm * BMX, n0 = (int64_t)tn * BN;
      const int64_t ra = g.M - m0 < BMX ? g.M - m0 : BMX, rb = g.N - n0 < BN ? g.N - n0 : BN;
      // MN-major: the panel is K rows from column m0 / n0; a ragged tile's
      // columns past the matrix end the last row's range (whole chunks:
      // M, N % 16 == 0) and elsewhere read bytes that only reach C rows or
      // columns past the matrix
      T.a = TA ? make_srd(g.A + m0, (g.K - 1) * g.lda + ra) : make_srd(g.A + m0 * g.lda, (ra - 1) * g.lda + g.K);
      T.b = TB ? make_srd(g.B + n0, (g.K - 1) * g.ldb + rb) : make_srd(g.B + n0 * g.ldb, (rb - 1) * g.ldb + g.K);
      if constexpr (MX) {
        if (g.scales_packed) {
          // one 256-row tile of the packed layout: sgroups x 4 KiB, rows past
          // the matrix padded with code 127 by mx_pack_scales
          const int64_t tb = g.sgroups * (int64_t)kPackTile;
          // a 128-row tile is one half of a packed 256-row tile: its rows
          // start 128 rows (2 KiB) into each 4 KiB group block
          const int64_t ah = BMX == 256 ? 0 : (int64_t)(tm & 1) * 128 * kPackBlocks;
          T.sa = make_srd(g.sa + (int64_t)(tm / (256 / BMX)) * tb + ah, tb - ah);
          T.sb = make_srd(g.sb + (int64_t)tn * tb, tb);
        } else {
          const int kb = TL ? kbr : 4 * nk;         // (the same when K % 128 == 0)
          T.sa = make_srd(g.sa + m0 * g.lds_a, (ra - 1) * g.lds_a + kb);
          T.sb = make_srd(g.sb + n0 * g.lds_b, (rb - 1) * g.lds_b + kb);
        }
      } else {
        T.sa = T.a;
        T.sb = T.b;
      }
    } else {
      T.a = make_srd(g.A, 0);
      T.b = make_srd(g.B, 0);
      T.sa = T.a;
      T.sb = T.b;
    }
  };

  // DMA: wave w fills 1 KiB blocks 8w..8w+7 (8 rows each) of each operand;
  // lane L lands at row 8 blk + L/8, stored chunk L%8, so it fetches logical
  // chunk (L%8) ^ fswz(row) = (L%8) ^ (L/8) ^ (blk & 1).  The stage's K
  // offset rides in soffset.  Offsets do not depend on the tile: a row past
  // the matrix has offset >= ra * ld >= (ra - 1) * ld + K, the panel's size.
  const int cl = (lane & 7) ^ (lane >> 3);          // ^ (blk & 1) = ^ (i & 1) below
  // K tail (K % 128 != 0; the missing blocks' scale codes are the packed
  // layout's padding, 127, or other codes of the row): in the last stage a
  // K-contiguous copy whose chunk
  // (cl ^ (i & 1)) starts at or past K % 128 gets an offset out of range
  // and reads zeros (it would read the next row's bytes).  An MN-major
  // operand's K rows past K are past its descriptor already: the range
  // check counts soffset, where the stage's K offset rides (measured with
  // an in-bounds probe: voffset + soffset >= num_records reads zero).
  const int krem = (int)(g.K % BK);
  const bool tail_e = TL && krem > 0 && 16 * cl >= krem;
  const bool tail_o = TL && krem > 0 && 16 * (cl ^ 1) >= krem;
  // MN-major: block b of the stage is K rows 4b .. 4b+3 (256 bytes each;
  // 8b .. 8b+7 of 128 bytes for op(A) of a 128-row tile); lane L lands at
  // row 4b + L/16, stored chunk L%16 (8b + L/8, L%8), so it fetches logical
  // chunk (L%16) ^ tswz(row); the stage's K offset (k0 rows) rides in
  // soffset as k0 * ld.
  uint32_t offa[8], offb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (wave * 8 + i) * 8 + (lane >> 3);
    const int rowa_c = (wave * NA + (i % NA)) * 8 + (lane >> 3);
    const int krow = (wave * 8 + i) * 4 + (lane >> 4);
    const int kc = (lane & 15) ^ ((krow & 7) | (((krow >> 4) & 1) << 3));
    // op(A) of a 128-row tile: K rows of 128 bytes, block b = rows 8b .. 8b+7
    const int krow_a = BMX == 256 ? krow : (wave * NA + (i % NA)) * 8 + (lane >> 3);
    const int kc_a = BMX == 256 ? kc : (lane & 7) ^ (((krow_a >> 1) & 3) << 1);
    offa[i] = TA ? (uint32_t)(krow_a * g.lda + 16 * kc_a) : (uint32_t)(rowa_c * g.lda + 16 * (cl ^ (i & 1)));
    offb[i] = TB ? (uint32_t)(krow * g.ldb + 16 * kc) : (uint32_t)(row * g.ldb + 16 * (cl ^ (i & 1)));
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
  // MX scales: lane L of wave w copies 16 bytes (the codes of 4 stages) of
  // tile row 64 w + L of each operand.  Group G covers stages 4G .. 4G+3:
  // bytes 16 G .. 16 G + 15 of a row-major scale row (a partial last group
  // from gsb(G) bytes earlier) or the 4 KiB block G of the packed layout
  // (padded with code 127 past the last block).
  // L2 prefetch of op(B) (the weight panel): every stage of a tile touches a
  // new K slice of it, and all XCDs walk the same panels in step, so its
  // copies are the ones that wait on HBM.  One workgroup per group of kGroupM
  // tile rows (the tiles that share the panel on an XCD) touches, 8 stages
  // ahead, one 128-byte line per panel row (lane L of wave w: row 64 w + L),
  // landing in pf_sink; the other workgroups issue the same load through a
  // size-0 descriptor.  Measured: +5% per-tensor, +7% MX (prefetching from
  // every workgroup, or both operands 2 stages ahead, was slower).
  // (MN-major op(B): the stage's 128 K rows of 256 bytes are 256 lines, one
  // per lane, and the K offset rides in soffset as k0 * ldb)
  const uint32_t pfb = TB ? (uint32_t)(((wave * 64 + lane) >> 1) * g.ldb + 128 * (lane & 1))
                          : (uint32_t)((wave * 64 + lane) * g.ldb);
  const uint32_t pf_lds = __builtin_amdgcn_readfirstlane(lds_offset(pf_sink));
  uint32_t offsa = 0, offsb = 0, ldss = 0;
  if constexpr (MX) {
    const int row = wave * 64 + lane;
    offsa = (uint32_t)(g.scales_packed ? row * 16 : row * g.lds_a);
    offsb = (uint32_t)(g.scales_packed ? row * 16 : row * g.lds_b);
    ldss = __builtin_amdgcn_readfirstlane(lds_offset(s_scale));
  }

  int vb = blockIdx.x;
  bool pf_owner = false;                            // this tile prefetches its B panel
  auto owner_of = [&](int v) {
    int tm, tn;
    tile_coords_vb(v, tiles_m, tiles_n, tm, tn);
    return (tm % kGroupM) == 0;
  };
  pf_owner = owner_of(vb);
  TileSrd cur, nxt;
  make_tile(vb, cur);
  if constexpr (PERSIST) make_tile(vb + P, nxt);
  int gbase = 0;                                    // scale groups of earlier tiles (slot parity)

  // Copies of stage s of the current tile, 0 <= s < nkU + 2: s < nk real,
  // nk <= s < nkU zeros (size-0 descriptor), s >= nkU the next tile's
  // stage s - nkU.  nkU is even, so slot parity runs on across tiles.
  auto dma = [&](int s, int t) {
    const int slot = s % NS;
    const bool nx = PERSIST && s >= nkU;
    const bool live = s < nk || nx;
    const uint32_t k0 = (uint32_t)((nx ? s - nkU : s) * BK);
    const bool isb = t >= NA;
    const int i = isb ? t - NA : t;
    uint32_t off = isb ? offb[i] : offa[i];
    if constexpr (TL) {
      if (!(isb ? TB : TA)) off = (!nx && s == nk - 1 && ((i & 1) ? tail_o : tail_e)) ? kOOB : off;
    }
    const uint32_t la = lds0 + (uint32_t)(isb ? kRegB + (wave * 8 + i) * 1024 + slot * kSlotB
                                              : (wave * NA + i) * 1024 + slot * kSlotA);
    v4i srd = isb ? cur.b : cur.a;
    if constexpr (PERSIST) srd = nx ? (isb ? nxt.b : nxt.a) : srd;
    srd[2] = live ? srd[2] : 0;
    const bool mn = isb ? TB : TA;
    const uint32_t so = mn ? k0 * (uint32_t)(isb ? g.ldb : g.lda) : k0;
    if (t == 0 || t == NA)
      dma_b128_so<5>(uniform_srd(srd), __builtin_amdgcn_readfirstlane(la), off, __builtin_amdgcn_readfirstlane(so));
    else
      dma_b128_so<1>(uniform_srd(srd), __builtin_amdgcn_readfirstlane(la), off, __builtin_amdgcn_readfirstlane(so));
  };
  // prefetch of op(B) stage s (descriptor choice as for the copies)
  auto prefetch_b = [&](int s, bool owner) {
    if constexpr (!PF) return;
    const bool nx = PERSIST && s >= nkU;
    const bool live = owner && (s < nk || nx);
    const uint32_t k0 = (uint32_t)((nx ? s - nkU : s) * BK);
    v4i srd = cur.b;
    if constexpr (PERSIST) srd = nx ? nxt.b : srd;
    srd[2] = live ? srd[2] : 0;
    dma_b32_so<5>(uniform_srd(srd), pf_lds, pfb, __builtin_amdgcn_readfirstlane(TB ? k0 * (uint32_t)g.ldb : k0));
  };
  // Scale group G of the current tile, 0 <= G <= ngroups (G == ngroups: the
  // next tile's group 0, whose copy starts at block 0).
  auto scale_dma = [&](int G) {
    if constexpr (MX) {
      const bool nx = G >= ngroups;
      // packed: group G is the 4 KiB block G of the tile (whole lines);
      // row-major: bytes 16 G .. 16 G + 15 of each row
      uint32_t so = (uint32_t)(nx ? 0 : (pk ? G * kPackTile : 16 * G));
      if constexpr (TL) so -= (uint32_t)gsb(G);
      const uint32_t la = ldss + (uint32_t)((((gbase + G) & 1) * 2 * BM + wave * 64) * 16);
      v4i sa = cur.sa, sb = cur.sb;
      if constexpr (PERSIST) {
        sa = nx ? nxt.sa : sa;
        sb = nx ? nxt.sb : sb;
      } else {
        sa[2] = nx ? 0 : sa[2];                     // no next tile: zeros
        sb[2] = nx ? 0 : sb[2];
      }
      dma_b128_so<5>(uniform_srd(sa), __builtin_amdgcn_readfirstlane(la), offsa, __builtin_amdgcn_readfirstlane(so));
      dma_b128_so<5>(uniform_srd(sb), __builtin_amdgcn_readfirstlane(la + BM * 16), offsb,
                  __builtin_amdgcn_readfirstlane(so));
    }
  };
  // E8M0 codes of one 4-stage group (16 per row) for this lane, two
  // registers per 32-row fragment (sc[0..3]: op(A) fragments j, sc[4..7]:
  // op(B) fragments i).  A 16-byte LDS read returns the row's 16 codes
  // (dword d = stage d of the group, byte b = its 32-wide K block b); lane
  // group g = lane / 32 scales K block 2h + g of sub-step h, so
  // v_perm packs bytes g, 2 + g of dwords (0, 1) into the register of stages
  // 0 and 1 and of dwords (2, 3) into that of stages 2 and 3: stage p,
  // sub-step h takes byte 2 (p & 1) + h (op_sel) of register p >> 1.  Rows
  // 16 bytes apart read as one contiguous span: no bank conflicts.  A
  // partial last group (TL) first drops its gsb(G) leading bytes (uniform
  // selects; the identity on whole groups).
  const uint32_t psel = (lane >> 5) ? 0x07050301u : 0x06040200u;
  auto read_group = [&](int G, int (&lo)[8], int (&hi)[8], int j0, int j1) {
    if constexpr (MX) {
      const int gs = (gbase + G) & 1;
      const int sh = gsb(G);
#pragma unroll
      for (int j = j0; j < j1; ++j) {
        uint4 da = *reinterpret_cast<const uint4*>(&s_scale[((gs * 2) * BM + wm * 128 + j * 32 + (lane & 31)) * 4]);
        uint4 db = *reinterpret_cast<const uint4*>(
            &s_scale[((gs * 2 + 1) * BM + wn * WN + (j % NI) * 32 + (lane & 31)) * 4]);
        if constexpr (TL) {
          da = drop_bytes(da, sh);
          db = drop_bytes(db, sh);
        }
        lo[j] = (int)__builtin_amdgcn_perm(da.y, da.x, psel);
        hi[j] = (int)__builtin_amdgcn_perm(da.w, da.z, psel);
        lo[4 + j] = (int)__builtin_amdgcn_perm(db.y, db.x, psel);
        hi[4 + j] = (int)__builtin_amdgcn_perm(db.w, db.z, psel);
      }
    }
  };

  // per-lane fragment bases (slot 0, fragment 0) for sub-steps 0 and 1
  const int s7 = (lane & 7) ^ ((lane >> 3) & 1), gq = lane >> 5;   // fswz of the lane's rows
  const uint32_t rowa = (uint32_t)((wm * 128 + (lane & 31)) * BK);
  const uint32_t rowb = (uint32_t)(kRegB + (wn * WN + (lane & 31)) * BK);
  const uint32_t a0lo = rowa + (((0 + gq) ^ s7) << 4), a0hi = rowa + (((2 + gq) ^ s7) << 4);
  const uint32_t a1lo = rowa + (((4 + gq) ^ s7) << 4), a1hi = rowa + (((6 + gq) ^ s7) << 4);
  const uint32_t b0lo = rowb + (((0 + gq) ^ s7) << 4), b0hi = rowb + (((2 + gq) ^ s7) << 4);
  const uint32_t b1lo = rowb + (((4 + gq) ^ s7) << 4), b1hi = rowb + (((6 + gq) ^ s7) << 4);
  // MN-major operands: per-lane base of fragment j (frag_tr), slot 0, sub-step 0
  const int tq = lane >> 4, tj = lane & 15;
  const int tsw = (tj >> 1) | (gq << 3);
  const int tsw_a = BMX == 256 ? tsw : ((tj >> 2) & 3) << 1;     // op(A) rows of BMX bytes
  uint32_t abase[4], bbase[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t kr = (uint32_t)((16 * gq + (tj >> 1)) * 256 + 8 * (tj & 1));
    const uint32_t kr_a = (uint32_t)((16 * gq + (tj >> 1)) * BMX + 8 * (tj & 1));
    abase[j] = kr_a + (uint32_t)(((((wm * 128 + 32 * j) >> 4) + (tq & 1)) ^ tsw_a) << 4);
    bbase[j] = kRegB + kr + (uint32_t)(((((wn * WN + 32 * j) >> 4) + (tq & 1)) ^ tsw) << 4);
  }
  // fragment j of sub-step H at slot offset OFF, in either layout
  auto frA = [&](auto off_c, auto h_c, auto j_c) -> v8i {
    constexpr int OFF = decltype(off_c)::value, H = decltype(h_c)::value, J = decltype(j_c)::value;
    if constexpr (TA) return frag_tr<OFF + H * 64 * BMX, BMX>(smem, abase[J]);
    else return frag_at<OFF + J * kFrag>(smem, H ? a1lo : a0lo, H ? a1hi : a0hi);
  };
  auto frB = [&](auto off_c, auto h_c, auto j_c) -> v8i {
    constexpr int OFF = decltype(off_c)::value, H = decltype(h_c)::value, J = decltype(j_c)::value;
    if constexpr (TB) return frag_tr<OFF + H * 64 * 256, 256>(smem, bbase[J]);
    else return frag_at<OFF + J * kFrag>(smem, H ? b1lo : b0lo, H ? b1hi : b0hi);
  };

  // prologue (first tile only; later tiles are prefetched by the previous
  // tile's last two stages): stages 0 and 1 in flight, stage 0 published,
  // its sub-step 0 fragments read
  scale_dma(0);
#pragma unroll
  for (int t = 0; t < LPS; ++t) dma(0, t);
#pragma unroll
  for (int t = 0; t < LPS; ++t) dma(1, t);
  if constexpr (NS == 3) {
#pragma unroll
    for (int t = 0; t < LPS; ++t) dma(2, t);
  }
  // Every stage's copy wait (wait_vm<1>) leaves one copy in flight: the L2
  // prefetch each stage issues last.  The prologue ends with one too (stage
  // 7's, which no stage prefetches), so that stage 0's wait covers all of
  // stage 1's copies; without it the last copy of stage 1 could still be in
  // flight when the barrier publishes the stage.  Three slots: no prefetch,
  // and each wait leaves the next stage's LPS copies in flight.
  prefetch_b(7, pf_owner);
  if constexpr (NS == 3) wait_vm<2 * LPS>();
  else if constexpr (PF) wait_vm<LPS + 1>();
  else wait_vm<LPS>();                               // no prefetch (MN-major op(B)): stage 1's copies
  __syncthreads();
  v8i x0[4], w0[4], x1[4], w1[4];
  int sc[2][8] = {};                                 // scale registers of stages 0-1 and 2-3 of the group
  int sc_next[8] = {};                               // the next group's stages 2-3, read with its 0-1
  x0[0] = frA(IC<0>{}, IC<0>{}, IC<0>{}); x0[1] = frA(IC<0>{}, IC<0>{}, IC<1>{});
  x0[2] = frA(IC<0>{}, IC<0>{}, IC<2>{}); x0[3] = frA(IC<0>{}, IC<0>{}, IC<3>{});
  w0[0] = frB(IC<0>{}, IC<0>{}, IC<0>{}); w0[1] = frB(IC<0>{}, IC<0>{}, IC<1>{});
  if constexpr (NI == 4) {
    w0[2] = frB(IC<0>{}, IC<0>{}, IC<2>{}); w0[3] = frB(IC<0>{}, IC<0>{}, IC<3>{});
  }
  read_group(0, sc[0], sc[1], 0, 4);

  v16f acc[NI][4];
  // One stage in slot SLOT: phase A = sub-step 0 MFMAs (set 0) while reading
  // sub-step 1 (set 1); publish stage kt+1 (wait own DMA, barrier); phase B =
  // sub-step 1 MFMAs while reading stage kt+1's sub-step 0 (set 0) and
  // issuing stage kt+2's DMA into the slot stage kt released.
  auto stage = [&](int kt, auto slot_c, auto scales_c, auto pos_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    constexpr int NSL = (SLOT + 1) % NS;
    constexpr bool SCALES = decltype(scales_c)::value;  // issue the next scale group
    constexpr int POS = decltype(pos_c)::value;         // stage within the 4-stage scale group (MX)
    constexpr int HB = POS >> 1;                        // scale register of this stage
    constexpr int OS = 2 * (POS & 1);                   // op_sel of sub-step 0
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int i = t >> 2, j = t & 3;
      switch (t) {
        case 0: x1[0] = frA(IC<SLOT * kSlotA>{}, IC<1>{}, IC<0>{}); break;
        case 1: x1[1] = frA(IC<SLOT * kSlotA>{}, IC<1>{}, IC<1>{}); break;
        case 2: x1[2] = frA(IC<SLOT * kSlotA>{}, IC<1>{}, IC<2>{}); break;
        case 3: x1[3] = frA(IC<SLOT * kSlotA>{}, IC<1>{}, IC<3>{}); break;
        case 4: w1[0] = frB(IC<SLOT * kSlotB>{}, IC<1>{}, IC<0>{}); break;
        case 5: w1[1] = frB(IC<SLOT * kSlotB>{}, IC<1>{}, IC<1>{}); break;
        case 6: if constexpr (NI == 4) w1[2] = frB(IC<SLOT * kSlotB>{}, IC<1>{}, IC<2>{}); break;
        case 7: if constexpr (NI == 4) w1[3] = frB(IC<SLOT * kSlotB>{}, IC<1>{}, IC<3>{}); break;
        default: break;
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MX)
        acc[i][j] = mfma32<FB, FA>(w0[i], x0[j], acc[i][j], sc[HB][4 + i], OS, sc[HB][j], OS);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w0[i], x0[j], acc[i][j], FB, FA, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NS == 3) wait_vm<LPS>();            // all but stage kt+2's copies
    else if constexpr (PF) wait_vm<1>();              // all but the prefetch, issued last
    else wait_vm<0>();                                // no prefetch: every copy
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int i = t >> 2, j = t & 3;
      {
        // the next group's codes at the group's third stage, after the last
        // use of its first registers: stages 0-1 straight into them, stages
        // 2-3 held until this group's last stage is done; one op(A) and one
        // op(B) fragment per MFMA slot
        constexpr int T0 = NT == 16 ? 8 : 4;
        if constexpr (MX && POS == 2)
          if (t >= T0 && t < T0 + 4) read_group((kt >> 2) + 1, sc[0], sc_next, t - T0, t - T0 + 1);
        switch (t) {
          case 0: x0[0] = frA(IC<NSL * kSlotA>{}, IC<0>{}, IC<0>{}); break;
          case 1: x0[1] = frA(IC<NSL * kSlotA>{}, IC<0>{}, IC<1>{}); break;
          case 2: x0[2] = frA(IC<NSL * kSlotA>{}, IC<0>{}, IC<2>{}); break;
          case 3: x0[3] = frA(IC<NSL * kSlotA>{}, IC<0>{}, IC<3>{}); break;
          case 4: w0[0] = frB(IC<NSL * kSlotB>{}, IC<0>{}, IC<0>{}); break;
          case 5: w0[1] = frB(IC<NSL * kSlotB>{}, IC<0>{}, IC<1>{}); break;
          case 6: if constexpr (NI == 4) w0[2] = frB(IC<NSL * kSlotB>{}, IC<0>{}, IC<2>{}); break;
          case 7: if constexpr (NI == 4) w0[3] = frB(IC<NSL * kSlotB>{}, IC<0>{}, IC<3>{}); break;
          default: break;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MX)
        acc[i][j] = mfma32<FB, FA>(w1[i], x1[j], acc[i][j], sc[HB][4 + i], OS + 1, sc[HB][j], OS + 1);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w1[i], x1[j], acc[i][j], FB, FA, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      // the stage's LPS copies spread over its NT MFMA slots
#pragma unroll
      for (int c = 0; c < LPS; ++c)
        if (c * NT / LPS == t) dma(kt + NS, c);
      if constexpr (SCALES)
        if (t == NT - 1) scale_dma((kt >> 2) + 1);
      if (t == NT - 1) prefetch_b(kt + 8, pf_owner);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // Global stores of an interior epilogue per wave (bf16: 4 block rows x NI/2
  // halves x 4 row groups; fp32: 4 x NI x 4), the ops issued after the last
  // copy of a workgroup's last tile; the final wait leaves them in flight.
  constexpr int kEpiStores = 4 * (NI / 2) * 4;
  // Output exponent: -(bias_a + bias_b), or 0 for MX (block scales are
  // applied inside the MFMA), applied to every accumulator by ldexp (exact at
  // 0).  For MX the 0 is hidden from the compiler: with the plain
  // accumulators as epilogue values it copied all 256 of them out of the
  // accumulation registers ahead of the interior/edge branch and spilled.
  int e = MX ? 0 : -(*g.bias_a + *g.bias_b);
  if constexpr (MX) asm volatile("" : "+s"(e));
  uint32_t amax_bits = 0;
  for (;;) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Unrolled by 2 (slot indices become immediates), by 4 for MX (the scale
    // group copy lands in a fixed stage).  The last two stages prefetch the
    // next tile's first two.
    for (int kt = 0; kt < nkU; kt += U) {
      using P0 = std::integral_constant<int, 0>;
      using P1 = std::integral_constant<int, 1>;
      using P2 = std::integral_constant<int, 2>;
      using P3 = std::integral_constant<int, 3>;
      stage(kt, S0{}, std::bool_constant<MX>{}, P0{});
      stage(kt + 1, S1{}, std::false_type{}, P1{});
      if constexpr (NS == 3) stage(kt + 2, std::integral_constant<int, 2>{}, std::false_type{}, P0{});
      if constexpr (MX) {
        stage(kt + 2, S0{}, std::false_type{}, P2{});
        stage(kt + 3, S1{}, std::false_type{}, P3{});
#pragma unroll
        for (int k = 0; k < 8; ++k) sc[1][k] = sc_next[k];
      }
    }

    if constexpr (NS == 3) {
      // the slots take the epilogue's staging: every copy (the zero copies
      // of stages past the last) has landed, every wave is out of the loop
      wait_vm<0>();
      __syncthreads();
    }
    int tm, tn;
    tile_coords_vb(vb, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BMX, n0 = (int64_t)tn * BN;
    // Epilogue.  Lane l of block (i, j) holds n = 8q + 4(l/32) + 0..3 of row
    // m = l%32.  An interior tile (all of it inside C, rows allowing vector
    // stores) takes a straight-line path: one row pointer per block row,
    // immediate column offsets, bf16 maxima as packed 16-bit maxima of |h|;
    // edge tiles check every element.
    const bool interior = m0 + BMX <= g.M && n0 + BN <= g.N && (g.out_f32 ? g.vec_store : g.row16);
    if (interior) {
      us2v pmax = {0, 0};
      uint8_t* stg = (NS == 3 ? smem : cstage) + (MX ? 0 : wave * kStage);
      if constexpr (MX) {
        const int fs = (gbase + ngroups - 1) & 1;     // scale slot of the tile's last group: free now
        stg = wave < 2 ? reinterpret_cast<uint8_t*>(s_scale) + fs * (2 * BM * 16) + wave * kStage
                       : cstage + (wave - 2) * kStage;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + wm * 128 + j * 32 + (lane & 31);
        const int64_t nb = n0 + wn * WN + 4 * (lane >> 5);
        if (g.out_f32) {
          float* crow = reinterpret_cast<float*>(g.C) + m * g.ldc + nb;
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float v[4];
#pragma unroll
              for (int r = 0; r < 4; ++r)
                v[r] = __builtin_amdgcn_ldexpf(acc[i][j][4 * q + r], e);
              *reinterpret_cast<float4*>(crow + i * 32 + 8 * q) = make_float4(v[0], v[1], v[2], v[3]);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const uint32_t ab = __float_as_uint(v[r]) & 0x7fffffffu;
                amax_bits = amax_bits > ab ? amax_bits : ab;
              }
            }
        } else {
          // bf16: each 32-row x 64-column quarter of the block row goes
          // through the wave's LDS staging area so that a store instruction
          // writes 8 whole 128-byte rows (one lane per 16 bytes) instead of
          // 16 bytes in each of 32 rows.  Staging row r holds its 16-byte
          // chunk c at chunk c ^ ((r >> 1) & 7): conflict-free for the 8-byte
          // writes (16 rows per access) and the 16-byte reads (2 rows).
          // lane-derived addresses are recomputed here: hoisted out of the
          // tile loop they would be spilled and reloaded from scratch
          int ln = lane;
          asm volatile("" : "+v"(ln));
          const uint32_t wr = (uint32_t)(ln & 31);
          const uint32_t wbase = wr * 128 + 8 * (ln >> 5);
          const uint32_t wsw = (wr >> 1) & 7;
          // stores: the wave's C block base (uniform) plus a 32-bit byte
          // offset (the host admits this path only if 128 rows span < 4 GiB)
          uint8_t* const cw = reinterpret_cast<uint8_t*>(g.C) + ((m0 + wm * 128) * g.ldc + n0 + wn * WN) * 2;
          const uint32_t ldcb = (uint32_t)g.ldc * 2u;
          const uint32_t lr = (uint32_t)(ln >> 3), ch = (uint32_t)(ln & 7);
          const uint32_t goff = lr * ldcb + 16u * ch;
          const uint32_t rsw0 = lr * 128 + 16 * (ch ^ (lr >> 1)), rsw1 = lr * 128 + 16 * (ch ^ (lr >> 1) ^ 4u);
#pragma unroll
          for (int p = 0; p < NI / 2; ++p) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int i = 2 * p + ii;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  v[r] = __builtin_amdgcn_ldexpf(acc[i][j][4 * q + r], e);
                const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2*>(stg + wbase + 16 * ((uint32_t)(4 * ii + q) ^ wsw)) = make_uint2(lo, hi);
                pmax = __builtin_elementwise_max(pmax, __builtin_bit_cast(us2v, lo & 0x7fff7fffu));
                pmax = __builtin_elementwise_max(pmax, __builtin_bit_cast(us2v, hi & 0x7fff7fffu));
              }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              // row 8k + lr, chunk ch; its swizzle (row >> 1) & 7 = (lr >> 1) ^ 4 (k & 1)
              const uint4 d = *reinterpret_cast<const uint4*>(stg + 8 * k * 128 + ((k & 1) ? rsw1 : rsw0));
              *reinterpret_cast<uint4*>(cw + goff + (uint32_t)(j * 32 + 8 * k) * ldcb + p * 128) = d;
            }
          }
        }
      }
      const uint32_t pm = ((uint32_t)(pmax[0] > pmax[1] ? pmax[0] : pmax[1])) << 16;
      amax_bits = amax_bits > pm ? amax_bits : pm;
    } else {
      // epilogue: lane l of block (i, j) holds n = 8q + 4(l/32) + 0..3 of column m = l%32
    #pragma unroll
      for (int i = 0; i < NI; ++i) {
    #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t m = m0 + wm * 128 + j * 32 + (lane & 31);
          if (m >= g.M) continue;
    #pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + wn * WN + i * 32 + 8 * q + 4 * (lane >> 5);
            float v[4];
    #pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = __builtin_amdgcn_ldexpf(acc[i][j][4 * q + r], e);
            if (g.out_f32) {
              float* crow = reinterpret_cast<float*>(g.C) + m * g.ldc;
              if (g.vec_store && n + 3 < g.N) {
                *reinterpret_cast<float4*>(crow + n) = make_float4(v[0], v[1], v[2], v[3]);
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const uint32_t ab = __float_as_uint(v[r]) & 0x7fffffffu;
                  amax_bits = amax_bits > ab ? amax_bits : ab;
                }
              } else {
    #pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (n + r < g.N) {
                    crow[n + r] = v[r];
                    const uint32_t ab = __float_as_uint(v[r]) & 0x7fffffffu;
                    amax_bits = amax_bits > ab ? amax_bits : ab;
                  }
              }
            } else {
              uint16_t h[4];
    #pragma unroll
              for (int r = 0; r < 4; ++r) h[r] = __builtin_bit_cast(uint16_t, (__bf16)v[r]);
              uint16_t* crow = reinterpret_cast<uint16_t*>(g.C) + m * g.ldc;
              if (g.vec_store && n + 3 < g.N) {
                *reinterpret_cast<uint2*>(crow + n) =
                    make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const uint32_t ab = ((uint32_t)h[r] & 0x7fffu) << 16;
                  amax_bits = amax_bits > ab ? amax_bits : ab;
                }
              } else {
    #pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (n + r < g.N) {
                    crow[n + r] = h[r];
                    const uint32_t ab = ((uint32_t)h[r] & 0x7fffu) << 16;
                    amax_bits = amax_bits > ab ? amax_bits : ab;
                  }
              }
            }
          }
        }
      }
    }
    // An edge epilogue issues a data-dependent number of stores: drain them,
    // so that the final wait below counts only the interior case's stores.
    if (!interior) wait_vm<0>();
    vb += P;
    if (!PERSIST || vb >= tiles) break;
    if constexpr (PERSIST) {
      cur = nxt;
      make_tile(vb + P, nxt);
    }
    pf_owner = owner_of(vb);
    gbase += ngroups;
  }
  // Every copy (the zero copies past the last tile, the last prefetch) has
  // landed in LDS before the workgroup ends; the C stores issued after them
  // may still be in flight (one tile per workgroup in the MX launch: the
  // next workgroup on this CU starts while they drain, +1.3% on the 70B-MLP
  // shape).
  wait_vm<kEpiStores>();
  if (g.out_amax) block_max_to_global(amax_bits, red, g.out_amax);
}

template <int FA, int FB, bool MX, bool TA, bool TB, bool TL = false>
static void launch_gemm(const GemmArgs& g, hipStream_t s) {
  const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  // the forward kernel copies MX scales 16 codes (4 stages) per row at a
  // time: row-major scale rows must be 4-byte aligned with K >= 512 (a
  // partial last group is copied from 16 codes before the row's end;
  // packed scales are padded to whole groups); one tile
  // per workgroup (or, with kFwdPersistent, per-tensor products walk tiles
  // with one workgroup per compute unit)
  // MN-major operands (TA / TB, per-tensor) take the forward kernel with
  // LDS transpose reads; K tails (K % 128 != 0) take it too
  const int64_t ncu = device_cu_count();
  if constexpr (!TL) {
    // the last K stage or group of 4 stages' row-major scale codes is
    // partial: the TL instantiation
    const bool tail = MX ? (g.K > 0 && g.scales_dma && (g.scales_packed ? (g.K % 128) != 0 : (g.K % 512) != 0))
                         : (g.K > 0 && (g.K % 128) != 0);
    if (tail) {
      launch_gemm<FA, FB, MX, TA, TB, true>(g, s);
      return;
    }
  }
  const bool fwd = g.K > 0 && (TL || (g.K % 128) == 0) && (!MX || g.scales_dma);
  if (fwd) {
    if (tiles < ncu) {
      // fewer 256 x 256 tiles than compute units: 128 x 256 tiles
      const int64_t t128 = ((g.M + 127) / 128) * ((g.N + BN - 1) / BN);
      // three LDS slots for long per-tensor products (see gemm_fwd_kernel)
      if constexpr (!MX) {
        if (g.K >= 4096) {
          hipLaunchKernelGGL((gemm_fwd_kernel<FA, FB, MX, 128, 3, TA, TB, TL>), dim3((unsigned)t128),
                             dim3(kGemmThreads), 0, s, g);
          return;
        }
      }
      hipLaunchKernelGGL((gemm_fwd_kernel<FA, FB, MX, 128, 2, TA, TB, TL>), dim3((unsigned)t128), dim3(kGemmThreads),
                         0, s, g);
      return;
    }
    const int64_t cus = (MX || !kFwdPersistent) ? tiles : ncu;
    const int64_t grid = tiles < cus ? tiles : cus;
    hipLaunchKernelGGL((gemm_fwd_kernel<FA, FB, MX, 256, 2, TA, TB, TL>), dim3((unsigned)grid), dim3(kGemmThreads), 0, s,
                       g);
  } else {
    hipLaunchKernelGGL((gemm_kernel<FA, FB, MX, TA, TB>), dim3((unsigned)tiles), dim3(kGemmThreads), 0, s, g);
  }
}

template <int FA, int FB>
static void dispatch_trans(const GemmArgs& g, bool ta, bool tb, hipStream_t s) {
  if (!ta && !tb) launch_gemm<FA, FB, false, false, false>(g, s);
  else if (!ta && tb) launch_gemm<FA, FB, false, false, true>(g, s);
  else if (ta && !tb) launch_gemm<FA, FB, false, true, false>(g, s);
  else launch_gemm<FA, FB, false, true, true>(g, s);
}

// Row-major E8M0 codes [rows x kb] -> the packed layout the forward MX GEMM
// copies whole lines of: chunk c (16 bytes) = codes [16 grp, 16 grp + 16) of
// row 256 t + r, with c = (t * sgroups + grp) * 256 + r; codes past the
// matrix (rows >= rows, blocks >= kb) are 127 (scale 1).  One lane per chunk:
// consecutive lanes write consecutive chunks.
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ src, int64_t rows, int64_t kb,
                                                          int64_t ld, uint8_t* __restrict__ dst, int64_t sgroups,
                                                          int64_t nchunks, int vec) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const int64_t r = c % kPackRows, tg = c / kPackRows;
  const int64_t grp = tg % sgroups, t = tg / sgroups;
  const int64_t row = t * kPackRows + r, j0 = grp * kPackBlocks;
  uint4 v;
  if (vec && row < rows && j0 + kPackBlocks <= kb) {
    v = *reinterpret_cast<const uint4*>(src + row * ld + j0);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t x = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t j = j0 + 4 * q + b;
        const uint32_t code = (row < rows && j < kb) ? src[row * ld + j] : 0x7fu;
        x |= code << (8 * b);
      }
      w[q] = x;
    }
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  *reinterpret_cast<uint4*>(dst + c * 16) = v;
}

// 16-byte loads need 16-byte aligned rows; buffer offsets are 32-bit, so a
// K-contiguous tile (256 rows) or a transposed operand (K rows) must span
// less than 2 GiB.
static int check_operand(const uint8_t* p, int64_t ld, bool trans, int64_t K) {
  if (!aligned(p, 16) || (ld % 16) != 0) return FP8_ERR_ALIGN;
  if (trans ? (K * ld >= (1LL << 31) - 4096) : (ld >= (1LL << 23))) return FP8_ERR_UNSUPPORTED;
  return FP8_OK;
}

}  // namespace sfp8

using namespace sfp8;

extern "C" {

int fp8_scaled_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* A, int fmt_a, int trans_a, int64_t lda,
                    const int32_t* bias_a, const uint8_t* B, int fmt_b, int trans_b, int64_t ldb,
                    const int32_t* bias_b, void* C, int out_dtype, int64_t ldc, float* out_amax,
                    hipStream_t stream) {
  if (!bias_a || !bias_b) return FP8_ERR_NULL;
  if (!valid_fmt(fmt_a) || !valid_fmt(fmt_b)) return FP8_ERR_FORMAT;
  if (!valid_dtype(out_dtype)) return FP8_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || (K % 16) != 0) return FP8_ERR_SHAPE;
  if (trans_a ? (lda < M || (M % 16) != 0) : (lda < K)) return FP8_ERR_SHAPE;
  if (trans_b ? (ldb < N || (N % 16) != 0) : (ldb < K)) return FP8_ERR_SHAPE;
  if (ldc < N) return FP8_ERR_SHAPE;
  if (check_matrix(M, N, ldc) || (trans_a ? check_matrix(K, M, lda) : check_matrix(M, K, lda)) ||
      (trans_b ? check_matrix(K, N, ldb) : check_matrix(N, K, ldb)))
    return FP8_ERR_SHAPE;
  if (M > 0 && N > 0 && !C) return FP8_ERR_NULL;
  if (M > 0 && N > 0 && K > 0 && (!A || !B)) return FP8_ERR_NULL;
  if (M > 0 && N > 0 && K > 0) {
    int st = check_operand(A, lda, trans_a != 0, K);
    if (st) return st;
    st = check_operand(B, ldb, trans_b != 0, K);
    if (st) return st;
  }
  if (out_amax) zero_float_async(out_amax, stream);
  if (M == 0 || N == 0) return launch_status();
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles > 0x7fffffffLL) return FP8_ERR_SHAPE;
  GemmArgs g;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb;
  g.bias_a = bias_a; g.bias_b = bias_b;
  g.sa = nullptr; g.lds_a = 0; g.sb = nullptr; g.lds_b = 0;
  g.sa_dword = 0; g.sb_dword = 0; g.scales_dma = 0;
  g.scales_packed = 0; g.sgroups = 0;
  g.C = C; g.ldc = ldc; g.out_amax = out_amax;
  g.out_f32 = out_dtype == FP8_DT_F32;
  g.vec_store = g.out_f32 ? (aligned(C, 16) && ldc % 4 == 0) : (aligned(C, 8) && ldc % 4 == 0);
  g.row16 = aligned(C, 16) && (ldc * (g.out_f32 ? 4 : 2)) % 16 == 0 && ldc * 2 * BM < (1LL << 32);
  const bool ta = trans_a != 0, tb = trans_b != 0;
  if (fmt_a == FP8_E4M3 && fmt_b == FP8_E4M3) dispatch_trans<FP8_E4M3, FP8_E4M3>(g, ta, tb, stream);
  else if (fmt_a == FP8_E5M2 && fmt_b == FP8_E4M3) dispatch_trans<FP8_E5M2, FP8_E4M3>(g, ta, tb, stream);
  else if (fmt_a == FP8_E4M3 && fmt_b == FP8_E5M2) dispatch_trans<FP8_E4M3, FP8_E5M2>(g, ta, tb, stream);
  else dispatch_trans<FP8_E5M2, FP8_E5M2>(g, ta, tb, stream);
  return launch_status();
}

int mx_scaled_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* A, int fmt_a, int64_t lda,
                   const uint8_t* A_scales, int64_t lds_a, const uint8_t* B, int fmt_b, int64_t ldb,
                   const uint8_t* B_scales, int64_t lds_b, void* C, int out_dtype, int64_t ldc, float* out_amax,
                   hipStream_t stream) {
  if (!valid_fmt(fmt_a) || !valid_fmt(fmt_b)) return FP8_ERR_FORMAT;
  if (!valid_dtype(out_dtype)) return FP8_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || (K % 32) != 0) return FP8_ERR_SHAPE;
  if (lda < K || ldb < K || ldc < N || lds_a < K / 32 || lds_b < K / 32) return FP8_ERR_SHAPE;
  if (check_matrix(M, N, ldc) || check_matrix(M, K, lda) || check_matrix(N, K, ldb) ||
      check_matrix(M, K / 32, lds_a) || check_matrix(N, K / 32, lds_b))
    return FP8_ERR_SHAPE;
  if (M > 0 && N > 0 && !C) return FP8_ERR_NULL;
  if (M > 0 && N > 0 && K > 0) {
    if (!A || !B || !A_scales || !B_scales) return FP8_ERR_NULL;
    int st = check_operand(A, lda, false, K);
    if (st) return st;
    st = check_operand(B, ldb, false, K);
    if (st) return st;
  }
  if (out_amax) zero_float_async(out_amax, stream);
  if (M == 0 || N == 0) return launch_status();
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles > 0x7fffffffLL) return FP8_ERR_SHAPE;
  GemmArgs g;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb;
  g.bias_a = nullptr; g.bias_b = nullptr;
  g.sa = A_scales; g.lds_a = lds_a; g.sb = B_scales; g.lds_b = lds_b;
  g.sa_dword = aligned(A_scales, 4) && (lds_a % 4) == 0;
  g.sb_dword = aligned(B_scales, 4) && (lds_b % 4) == 0;
  g.scales_dma = g.sa_dword && g.sb_dword && K >= 512 && lds_a < (1LL << 23) && lds_b < (1LL << 23);
  g.scales_packed = 0; g.sgroups = 0;
  g.C = C; g.ldc = ldc; g.out_amax = out_amax;
  g.out_f32 = out_dtype == FP8_DT_F32;
  g.vec_store = g.out_f32 ? (aligned(C, 16) && ldc % 4 == 0) : (aligned(C, 8) && ldc % 4 == 0);
  g.row16 = aligned(C, 16) && (ldc * (g.out_f32 ? 4 : 2)) % 16 == 0 && ldc * 2 * BM < (1LL << 32);
  if (fmt_a == FP8_E4M3 && fmt_b == FP8_E4M3) launch_gemm<FP8_E4M3, FP8_E4M3, true, false, false>(g, stream);
  else if (fmt_a == FP8_E5M2 && fmt_b == FP8_E4M3) launch_gemm<FP8_E5M2, FP8_E4M3, true, false, false>(g, stream);
  else if (fmt_a == FP8_E4M3 && fmt_b == FP8_E5M2) launch_gemm<FP8_E4M3, FP8_E5M2, true, false, false>(g, stream);
  else launch_gemm<FP8_E5M2, FP8_E5M2, true, false, false>(g, stream);
  return launch_status();
}

int64_t mx_packed_scales_bytes(int64_t rows, int64_t kblocks) {
  const int64_t b = packed_bytes_checked(rows, kblocks);
  return b < 0 ? FP8_ERR_SHAPE : b;
}

int mx_pack_scales(const uint8_t* scales, int64_t rows, int64_t kblocks, int64_t ld_scales, uint8_t* packed,
                   hipStream_t stream) {
  if (int st = check_matrix(rows, kblocks, ld_scales)) return st;
  const int64_t bytes = packed_bytes(rows, kblocks);
  if (bytes == 0) return FP8_OK;
  if (!packed || (kblocks > 0 && !scales)) return FP8_ERR_NULL;
  if (!aligned(packed, 16)) return FP8_ERR_ALIGN;
  const int64_t nchunks = bytes / 16;
  const int64_t blocks = (nchunks + 255) / 256;
  if (blocks > 0x7fffffffLL) return FP8_ERR_SHAPE;
  const int vec = aligned(scales, 16) && (ld_scales % 16) == 0;
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, scales, rows, kblocks,
                     ld_scales, packed, (kblocks + kPackBlocks - 1) / kPackBlocks, nchunks, vec);
  return launch_status();
}

int mx_scaled_gemm_packed(int64_t M, int64_t N, int64_t K, const uint8_t* A, int fmt_a, int64_t lda,
                          const uint8_t* A_packed, const uint8_t* B, int fmt_b, int64_t ldb, const uint8_t* B_packed,
                          void* C, int out_dtype, int64_t ldc, float* out_amax, hipStream_t stream) {
  if (!valid_fmt(fmt_a) || !valid_fmt(fmt_b)) return FP8_ERR_FORMAT;
  if (!valid_dtype(out_dtype)) return FP8_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || (K % 32) != 0) return FP8_ERR_SHAPE;
  if (lda < K || ldb < K || ldc < N) return FP8_ERR_SHAPE;
  if (check_matrix(M, N, ldc) || check_matrix(M, K, lda) || check_matrix(N, K, ldb)) return FP8_ERR_SHAPE;
  if (M > 0 && N > 0 && !C) return FP8_ERR_NULL;
  if (M > 0 && N > 0) {
    if (K == 0) return FP8_ERR_UNSUPPORTED;
    if (!A || !B || !A_packed || !B_packed) return FP8_ERR_NULL;
    if (!aligned(A_packed, 16) || !aligned(B_packed, 16)) return FP8_ERR_ALIGN;
    int st = check_operand(A, lda, false, K);
    if (st) return st;
    st = check_operand(B, ldb, false, K);
    if (st) return st;
  }
  if (out_amax) zero_float_async(out_amax, stream);
  if (M == 0 || N == 0) return launch_status();
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles > 0x7fffffffLL) return FP8_ERR_SHAPE;
  GemmArgs g;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb;
  g.bias_a = nullptr; g.bias_b = nullptr;
  g.sa = A_packed; g.lds_a = 0; g.sb = B_packed; g.lds_b = 0;
  g.sa_dword = 1; g.sb_dword = 1; g.scales_dma = 1;
  g.scales_packed = 1; g.sgroups = (K / 32 + kPackBlocks - 1) / kPackBlocks;
  g.C = C; g.ldc = ldc; g.out_amax = out_amax;
  g.out_f32 = out_dtype == FP8_DT_F32;
  g.vec_store = g.out_f32 ? (aligned(C, 16) && ldc % 4 == 0) : (aligned(C, 8) && ldc % 4 == 0);
  g.row16 = aligned(C, 16) && (ldc * (g.out_f32 ? 4 : 2)) % 16 == 0 && ldc * 2 * BM < (1LL << 32);
  if (fmt_a == FP8_E4M3 && fmt_b == FP8_E4M3) launch_gemm<FP8_E4M3, FP8_E4M3, true, false, false>(g, stream);
  else if (fmt_a == FP8_E5M2 && fmt_b == FP8_E4M3) launch_gemm<FP8_E5M2, FP8_E4M3, true, false, false>(g, stream);
  else if (fmt_a == FP8_E4M3 && fmt_b == FP8_E5M2) launch_gemm<FP8_E4M3, FP8_E5M2, true, false, false>(g, stream);
  else launch_gemm<FP8_E5M2, FP8_E5M2, true, false, false>(g, stream);
  return launch_status();
}

}  // extern "C"

// Host-side argument validation of every libscaled_fp8 entry point, built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py (CPU only).  Every call here must be
// rejected (or be a zero-sized call that returns FP8_OK) before any HIP
// call, so it runs on a machine without a GPU; the sanitizers check the
// checks themselves (out-of-bounds reads, signed overflow in the size
// arithmetic of extreme shapes, misaligned accesses).  Prints "ok" and
// exits 0 when every status equals the documented one.
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "scaled_fp8.h"

namespace {

int failures = 0;

void expect(const char* what, long long got, long long want) {
  if (got != want) {
    std::printf("FAIL %s: got %lld, want %lld\n", what, got, want);
    ++failures;
  }
}

// Device-looking pointers: 16-byte aligned (A16) or not (A1), never
// dereferenced on the host (validation fails before any use).
void* const A16 = reinterpret_cast<void*>(0x10000);
void* const A1 = reinterpret_cast<void*>(0x10001);
uint8_t* const U16 = static_cast<uint8_t*>(A16);
uint8_t* const U1 = static_cast<uint8_t*>(A1);
float* const F = static_cast<float*>(A16);
int32_t* const I = static_cast<int32_t*>(A16);
uint64_t* const Q = static_cast<uint64_t*>(A16);
const hipStream_t S = nullptr;
const int64_t BIG = int64_t(1) << 40;     // every product of two of these overflows int64 when squared twice
const int64_t HUGE_ = int64_t(1) << 62;

void status_strings() {
  const int codes[] = {FP8_OK, FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_ALIGN, FP8_ERR_DTYPE, FP8_ERR_FORMAT,
                       FP8_ERR_LAUNCH, FP8_ERR_UNSUPPORTED, -99, 12345};
  for (int c : codes) {
    const char* s = fp8_status_string(c);
    expect("status string not null", s != nullptr, 1);
    if (s) expect("status string terminated", std::strlen(s) > 0, 1);
  }
  expect("abi version", fp8_abi_version() >= 3, 1);
}

void amax_and_scale() {
  expect("amax null out", fp8_amax(A16, FP8_DT_BF16, 4, 4, 4, nullptr, S), FP8_ERR_NULL);
  expect("amax dtype", fp8_amax(A16, 7, 4, 4, 4, F, S), FP8_ERR_DTYPE);
  expect("amax ld < cols", fp8_amax(A16, FP8_DT_BF16, 4, 8, 4, F, S), FP8_ERR_SHAPE);
  expect("amax negative rows", fp8_amax(A16, FP8_DT_BF16, -1, 8, 8, F, S), FP8_ERR_SHAPE);
  expect("amax negative ld", fp8_amax(A16, FP8_DT_F32, 1, 8, -8, F, S), FP8_ERR_SHAPE);
  expect("amax null x", fp8_amax(nullptr, FP8_DT_BF16, 4, 4, 4, F, S), FP8_ERR_NULL);
  expect("amax huge", fp8_amax(A16, FP8_DT_BF16, BIG, BIG, BIG, F, S), FP8_ERR_SHAPE);
  expect("amax huge rows", fp8_amax(A16, FP8_DT_BF16, HUGE_, 2, 2, F, S), FP8_ERR_SHAPE);
  expect("amax_scale null workspace", fp8_amax_scale(A16, 0, 4, 4, 4, 0, 0, F, I, nullptr, nullptr, nullptr, S),
         FP8_ERR_NULL);
  expect("amax_scale null amax", fp8_amax_scale(A16, 0, 4, 4, 4, 0, 0, nullptr, I, nullptr, nullptr, A16, S),
         FP8_ERR_NULL);
  expect("amax_scale unaligned workspace", fp8_amax_scale(A16, 0, 4, 4, 4, 0, 0, F, I, nullptr, nullptr, A1, S),
         FP8_ERR_ALIGN);
  expect("amax_scale dtype", fp8_amax_scale(A16, 5, 4, 4, 4, 0, 0, F, I, nullptr, nullptr, A16, S), FP8_ERR_DTYPE);
  expect("amax_scale format", fp8_amax_scale(A16, 0, 4, 4, 4, 7, 0, F, I, nullptr, nullptr, A16, S), FP8_ERR_FORMAT);
  expect("amax_scale huge", fp8_amax_scale(A16, 0, BIG, BIG, BIG, 0, 0, F, I, nullptr, nullptr, A16, S),
         FP8_ERR_SHAPE);
  expect("amax_scale_noalloc null bias", fp8_amax_scale_noalloc(A16, 0, 4, 4, 4, 0, 0, F, nullptr, nullptr, nullptr, S),
         FP8_ERR_NULL);
  expect("amax_scale_noalloc dtype", fp8_amax_scale_noalloc(A16, 4, 4, 4, 4, 0, 0, F, I, nullptr, nullptr, S),
         FP8_ERR_DTYPE);
  expect("amax_scale_noalloc huge", fp8_amax_scale_noalloc(A16, 0, BIG, BIG, BIG, 0, 0, F, I, nullptr, nullptr, S),
         FP8_ERR_SHAPE);
  expect("scale null amax", fp8_compute_scale(nullptr, FP8_E4M3, 0, I, nullptr, nullptr, S), FP8_ERR_NULL);
  expect("scale null bias", fp8_compute_scale(F, FP8_E4M3, 0, nullptr, nullptr, nullptr, S), FP8_ERR_NULL);
  expect("scale format", fp8_compute_scale(F, 2, 0, I, nullptr, nullptr, S), FP8_ERR_FORMAT);
  expect("history init null", fp8_history_init(nullptr, I, 16, S), FP8_ERR_NULL);
  expect("history init window 0", fp8_history_init(F, I, 0, S), FP8_ERR_SHAPE);
  expect("history init window 4097", fp8_history_init(F, I, 4097, S), FP8_ERR_SHAPE);
  expect("history push null amax", fp8_history_push(F, I, 16, nullptr, S), FP8_ERR_NULL);
  expect("history push window", fp8_history_push(F, I, -3, F, S), FP8_ERR_SHAPE);
  expect("delayed format", fp8_compute_scale_delayed(F, I, 16, 9, 0, I, nullptr, nullptr, S), FP8_ERR_FORMAT);
  expect("delayed null state", fp8_compute_scale_delayed(F, nullptr, 16, 0, 0, I, nullptr, nullptr, S), FP8_ERR_NULL);
  expect("delayed window", fp8_compute_scale_delayed(F, I, 0, 0, 0, I, nullptr, nullptr, S), FP8_ERR_SHAPE);
}

void quantize() {
  for (int sat = 0; sat < 2; ++sat) {
    auto q = [&](const void* x, int dt, int64_t r, int64_t c, int64_t ld, int fmt, const int32_t* b, uint8_t* qq,
                 int64_t ldq, uint8_t* qt, int64_t ldqt) {
      return sat ? fp8_quantize_sat(x, dt, r, c, ld, fmt, b, qq, ldq, qt, ldqt, nullptr, Q, S)
                 : fp8_quantize(x, dt, r, c, ld, fmt, b, qq, ldq, qt, ldqt, nullptr, S);
    };
    expect("quantize null bias", q(A16, 0, 4, 4, 4, 0, nullptr, U16, 4, nullptr, 0), FP8_ERR_NULL);
    expect("quantize null q", q(A16, 0, 4, 4, 4, 0, I, nullptr, 4, nullptr, 0), FP8_ERR_NULL);
    expect("quantize dtype", q(A16, 3, 4, 4, 4, 0, I, U16, 4, nullptr, 0), FP8_ERR_DTYPE);
    expect("quantize format", q(A16, 0, 4, 4, 4, 5, I, U16, 4, nullptr, 0), FP8_ERR_FORMAT);
    expect("quantize ld", q(A16, 0, 4, 4, 2, 0, I, U16, 4, nullptr, 0), FP8_ERR_SHAPE);
    expect("quantize ldq", q(A16, 0, 4, 4, 4, 0, I, U16, 3, nullptr, 0), FP8_ERR_SHAPE);
    expect("quantize ldqT", q(A16, 0, 4, 8, 8, 0, I, U16, 8, U16, 2), FP8_ERR_SHAPE);
    expect("quantize null x", q(nullptr, 0, 4, 4, 4, 0, I, U16, 4, nullptr, 0), FP8_ERR_NULL);
    expect("quantize huge", q(A16, 0, BIG, BIG, BIG, 0, I, U16, BIG, nullptr, 0), FP8_ERR_SHAPE);
    expect("quantize huge qT", q(A16, 0, BIG, BIG, BIG, 0, I, U16, BIG, U16, BIG), FP8_ERR_SHAPE);
  }
  expect("quantize_sat null count",
         fp8_quantize_sat(A16, 0, 4, 4, 4, 0, I, U16, 4, nullptr, 0, nullptr, nullptr, S), FP8_ERR_NULL);
}

void quantize_delayed() {
  auto d = [](const void* x, int dt, int64_t r, int64_t c, int64_t ld, int fmt, int win, int64_t ldq, uint8_t* qt,
              int64_t ldqt, void* ws) {
    return fp8_quantize_delayed(x, dt, r, c, ld, fmt, 0, F, I, win, U16, ldq, qt, ldqt, I, F, Q, ws, S);
  };
  expect("delayed null workspace", d(A16, 0, 4, 4, 4, 0, 16, 4, nullptr, 0, nullptr), FP8_ERR_NULL);
  expect("delayed window 0", d(A16, 0, 4, 4, 4, 0, 0, 4, nullptr, 0, A16), FP8_ERR_SHAPE);
  expect("delayed window 4097", d(A16, 0, 4, 4, 4, 0, 4097, 4, nullptr, 0, A16), FP8_ERR_SHAPE);
  expect("delayed dtype", d(A16, 4, 4, 4, 4, 0, 16, 4, nullptr, 0, A16), FP8_ERR_DTYPE);
  expect("delayed format", d(A16, 0, 4, 4, 4, 2, 16, 4, nullptr, 0, A16), FP8_ERR_FORMAT);
  expect("delayed ld", d(A16, 0, 4, 4, 2, 0, 16, 4, nullptr, 0, A16), FP8_ERR_SHAPE);
  expect("delayed ldq", d(A16, 0, 4, 4, 4, 0, 16, 3, nullptr, 0, A16), FP8_ERR_SHAPE);
  expect("delayed ldqT", d(A16, 0, 4, 8, 8, 0, 16, 8, U16, 2, A16), FP8_ERR_SHAPE);
  expect("delayed null x", d(nullptr, 0, 4, 4, 4, 0, 16, 4, nullptr, 0, A16), FP8_ERR_NULL);
  expect("delayed workspace align", d(A16, 0, 4, 4, 4, 0, 16, 4, nullptr, 0, static_cast<char*>(A16) + 4),
         FP8_ERR_ALIGN);
  expect("delayed huge", d(A16, 0, BIG, BIG, BIG, 0, 16, BIG, nullptr, 0, A16), FP8_ERR_SHAPE);
  expect("delayed huge qT", d(A16, 0, BIG, BIG, BIG, 0, 16, BIG, U16, BIG, A16), FP8_ERR_SHAPE);
  expect("delayed null hist",
         fp8_quantize_delayed(A16, 0, 4, 4, 4, 0, 0, nullptr, I, 16, U16, 4, nullptr, 0, I, F, Q, A16, S),
         FP8_ERR_NULL);
}

void mx_casts() {
  for (int variant = 0; variant < 3; ++variant) {   // row-major, explicit rule, packed
    auto m = [&](const void* x, int dt, int64_t r, int64_t c, int64_t ld, int fmt, int rule, uint8_t* qq, int64_t ldq,
                 uint8_t* sc, int64_t lds) {
      if (variant == 0) return mx_quantize(x, dt, r, c, ld, fmt, qq, ldq, sc, lds, S);
      if (variant == 1) return mx_quantize_rule(x, dt, r, c, ld, fmt, rule, qq, ldq, sc, lds, S);
      return mx_quantize_packed(x, dt, r, c, ld, fmt, rule, qq, ldq, sc, S);
    };
    expect("mx cols % 32", m(A16, 0, 4, 48, 48, 0, 0, U16, 48, U16, 2), FP8_ERR_SHAPE);
    expect("mx null q", m(A16, 0, 4, 64, 64, 0, 0, nullptr, 64, U16, 2), FP8_ERR_NULL);
    expect("mx null scales", m(A16, 0, 4, 64, 64, 0, 0, U16, 64, nullptr, 2), FP8_ERR_NULL);
    expect("mx dtype", m(A16, 2, 4, 64, 64, 0, 0, U16, 64, U16, 2), FP8_ERR_DTYPE);
    expect("mx format", m(A16, 0, 4, 64, 64, 2, 0, U16, 64, U16, 2), FP8_ERR_FORMAT);
    expect("mx ld", m(A16, 0, 4, 64, 32, 0, 0, U16, 64, U16, 2), FP8_ERR_SHAPE);
    expect("mx null x", m(nullptr, 0, 4, 64, 64, 0, 0, U16, 64, U16, 2), FP8_ERR_NULL);
    expect("mx empty", m(nullptr, 0, 0, 64, 64, 0, 0, U16, 64, U16, 2), FP8_OK);
    expect("mx huge", m(A16, 0, BIG, BIG, BIG, 0, 0, U16, BIG, U16, BIG), FP8_ERR_SHAPE);
    if (variant == 0) expect("mx ld_scales", m(A16, 0, 4, 64, 64, 0, 0, U16, 64, U16, 1), FP8_ERR_SHAPE);
    if (variant == 1) expect("mx rule", m(A16, 0, 4, 64, 64, 0, 7, U16, 64, U16, 2), FP8_ERR_FORMAT);
    if (variant == 2) expect("mx packed unaligned", m(A16, 0, 4, 64, 64, 0, 0, U16, 64, U1, 2), FP8_ERR_ALIGN);
  }
  for (int variant = 0; variant < 3; ++variant) {
    auto t = [&](const void* x, int dt, int64_t r, int64_t c, int64_t ld, int fmt, int rule, uint8_t* qt, int64_t ldqt,
                 uint8_t* sc, int64_t lds) {
      if (variant == 0) return mx_quantize_t(x, dt, r, c, ld, fmt, qt, ldqt, sc, lds, S);
      if (variant == 1) return mx_quantize_t_rule(x, dt, r, c, ld, fmt, rule, qt, ldqt, sc, lds, S);
      return mx_quantize_t_packed(x, dt, r, c, ld, fmt, rule, qt, ldqt, sc, S);
    };
    expect("mx_t rows % 32", t(A16, 0, 48, 8, 8, 0, 0, U16, 48, U16, 2), FP8_ERR_SHAPE);
    expect("mx_t null qT", t(A16, 0, 64, 8, 8, 0, 0, nullptr, 64, U16, 2), FP8_ERR_NULL);
    expect("mx_t null scales", t(A16, 0, 64, 8, 8, 0, 0, U16, 64, nullptr, 2), FP8_ERR_NULL);
    expect("mx_t ldqT", t(A16, 0, 64, 8, 8, 0, 0, U16, 32, U16, 2), FP8_ERR_SHAPE);
    expect("mx_t ld", t(A16, 0, 64, 8, 4, 0, 0, U16, 64, U16, 2), FP8_ERR_SHAPE);
    expect("mx_t dtype", t(A16, 5, 64, 8, 8, 0, 0, U16, 64, U16, 2), FP8_ERR_DTYPE);
    expect("mx_t format", t(A16, 0, 64, 8, 8, 3, 0, U16, 64, U16, 2), FP8_ERR_FORMAT);
    expect("mx_t null x", t(nullptr, 0, 64, 8, 8, 0, 0, U16, 64, U16, 2), FP8_ERR_NULL);
    expect("mx_t empty", t(nullptr, 0, 64, 0, 0, 0, 0, U16, 64, U16, 2), FP8_OK);
    expect("mx_t huge", t(A16, 0, BIG, BIG, BIG, 0, 0, U16, BIG, U16, BIG), FP8_ERR_SHAPE);
    if (variant == 0) expect("mx_t ld_scales", t(A16, 0, 64, 8, 8, 0, 0, U16, 64, U16, 1), FP8_ERR_SHAPE);
    if (variant == 1) expect("mx_t rule", t(A16, 0, 64, 8, 8, 0, 9, U16, 64, U16, 2), FP8_ERR_FORMAT);
    if (variant == 2) expect("mx_t packed unaligned", t(A16, 0, 64, 8, 8, 0, 0, U16, 64, U1, 2), FP8_ERR_ALIGN);
  }
}

void packed_scales() {
  expect("packed bytes", mx_packed_scales_bytes(300, 20), 2LL * 2 * 4096);
  expect("packed bytes empty", mx_packed_scales_bytes(0, 5), 0);
  expect("packed bytes negative", mx_packed_scales_bytes(-1, 4), FP8_ERR_SHAPE);
  expect("packed bytes huge", mx_packed_scales_bytes(HUGE_, HUGE_), FP8_ERR_SHAPE);
  expect("packed bytes huge rows", mx_packed_scales_bytes(HUGE_, 16), FP8_ERR_SHAPE);
  expect("pack null", mx_pack_scales(U16, 4, 16, 16, nullptr, S), FP8_ERR_NULL);
  expect("pack null src", mx_pack_scales(nullptr, 4, 16, 16, U16, S), FP8_ERR_NULL);
  expect("pack unaligned", mx_pack_scales(U16, 4, 16, 16, U1, S), FP8_ERR_ALIGN);
  expect("pack ld", mx_pack_scales(U16, 4, 16, 8, U16, S), FP8_ERR_SHAPE);
  expect("pack empty", mx_pack_scales(nullptr, 0, 16, 16, nullptr, S), FP8_OK);
  expect("pack huge", mx_pack_scales(U16, HUGE_, HUGE_, HUGE_, U16, S), FP8_ERR_SHAPE);
}

void gemms() {
  auto g = [&](int64_t M, int64_t N, int64_t K, const uint8_t* A, int fa, int ta, int64_t lda, const int32_t* ba,
               const uint8_t* B, int fb, int tb, int64_t ldb, const int32_t* bb, void* C, int od, int64_t ldc) {
    return fp8_scaled_gemm(M, N, K, A, fa, ta, lda, ba, B, fb, tb, ldb, bb, C, od, ldc, nullptr, S);
  };
  expect("gemm null bias", g(64, 64, 64, U16, 0, 0, 64, nullptr, U16, 0, 0, 64, I, A16, 0, 64), FP8_ERR_NULL);
  expect("gemm format", g(64, 64, 64, U16, 4, 0, 64, I, U16, 0, 0, 64, I, A16, 0, 64), FP8_ERR_FORMAT);
  expect("gemm dtype", g(64, 64, 64, U16, 0, 0, 64, I, U16, 0, 0, 64, I, A16, 3, 64), FP8_ERR_DTYPE);
  expect("gemm K % 16", g(64, 64, 40, U16, 0, 0, 64, I, U16, 0, 0, 64, I, A16, 0, 64), FP8_ERR_SHAPE);
  expect("gemm lda", g(64, 64, 64, U16, 0, 0, 32, I, U16, 0, 0, 64, I, A16, 0, 64), FP8_ERR_SHAPE);
  expect("gemm trans_a M % 16", g(60, 64, 64, U16, 0, 1, 64, I, U16, 0, 0, 64, I, A16, 0, 64), FP8_ERR_SHAPE);
  expect("gemm ldc", g(64, 64, 64, U16, 0, 0, 64, I, U16, 0, 0, 64, I, A16, 0, 32), FP8_ERR_SHAPE);
  expect("gemm null C", g(64, 64, 64, U16, 0, 0, 64, I, U16, 0, 0, 64, I, nullptr, 0, 64), FP8_ERR_NULL);
  expect("gemm null A", g(64, 64, 64, nullptr, 0, 0, 64, I, U16, 0, 0, 64, I, A16, 0, 64), FP8_ERR_NULL);
  expect("gemm unaligned A", g(64, 64, 64, U1, 0, 0, 64, I, U16, 0, 0, 64, I, A16, 0, 64), FP8_ERR_ALIGN);
  expect("gemm lda % 16", g(64, 64, 64, U16, 0, 0, 72, I, U16, 0, 0, 64, I, A16, 0, 64), FP8_ERR_ALIGN);
  expect("gemm negative", g(-1, 64, 64, U16, 0, 0, 64, I, U16, 0, 0, 64, I, A16, 0, 64), FP8_ERR_SHAPE);
  expect("gemm huge", g(BIG, BIG, BIG, U16, 0, 0, BIG, I, U16, 0, 0, BIG, I, A16, 0, BIG), FP8_ERR_SHAPE);
  expect("gemm huge trans", g(BIG, BIG, BIG, U16, 0, 1, BIG, I, U16, 0, 1, BIG, I, A16, 0, BIG), FP8_ERR_SHAPE);
  expect("gemm huge ldc", g(64, 64, 64, U16, 0, 0, 64, I, U16, 0, 0, 64, I, A16, 0, HUGE_), FP8_ERR_SHAPE);

  auto m = [&](int64_t M, int64_t N, int64_t K, const uint8_t* A, int fa, int64_t lda, const uint8_t* sa,
               int64_t lsa, const uint8_t* B, int fb, int64_t ldb, const uint8_t* sb, int64_t lsb, void* C, int od,
               int64_t ldc) {
    return mx_scaled_gemm(M, N, K, A, fa, lda, sa, lsa, B, fb, ldb, sb, lsb, C, od, ldc, nullptr, S);
  };
  expect("mx gemm format", m(64, 64, 64, U16, 3, 64, U16, 2, U16, 0, 64, U16, 2, A16, 0, 64), FP8_ERR_FORMAT);
  expect("mx gemm dtype", m(64, 64, 64, U16, 0, 64, U16, 2, U16, 0, 64, U16, 2, A16, 9, 64), FP8_ERR_DTYPE);
  expect("mx gemm K % 32", m(64, 64, 48, U16, 0, 64, U16, 2, U16, 0, 64, U16, 2, A16, 0, 64), FP8_ERR_SHAPE);
  expect("mx gemm lds", m(64, 64, 64, U16, 0, 64, U16, 1, U16, 0, 64, U16, 2, A16, 0, 64), FP8_ERR_SHAPE);
  expect("mx gemm null scales", m(64, 64, 64, U16, 0, 64, nullptr, 2, U16, 0, 64, U16, 2, A16, 0, 64), FP8_ERR_NULL);
  expect("mx gemm null C", m(64, 64, 64, U16, 0, 64, U16, 2, U16, 0, 64, U16, 2, nullptr, 0, 64), FP8_ERR_NULL);
  expect("mx gemm unaligned B", m(64, 64, 64, U16, 0, 64, U16, 2, U1, 0, 64, U16, 2, A16, 0, 64), FP8_ERR_ALIGN);
  expect("mx gemm huge", m(BIG, BIG, BIG, U16, 0, BIG, U16, BIG, U16, 0, BIG, U16, BIG, A16, 0, BIG),
         FP8_ERR_SHAPE);

  auto p = [&](int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* pa, const uint8_t* B,
               int64_t ldb, const uint8_t* pb, void* C, int64_t ldc) {
    return mx_scaled_gemm_packed(M, N, K, A, 0, lda, pa, B, 0, ldb, pb, C, 0, ldc, nullptr, S);
  };
  expect("packed gemm K == 0", p(64, 64, 0, U16, 16, U16, U16, 16, U16, A16, 64), FP8_ERR_UNSUPPORTED);
  expect("packed gemm unaligned scales", p(64, 64, 512, U16, 512, U1, U16, 512, U16, A16, 64), FP8_ERR_ALIGN);
  expect("packed gemm null scales", p(64, 64, 512, U16, 512, nullptr, U16, 512, U16, A16, 64), FP8_ERR_NULL);
  expect("packed gemm null C", p(64, 64, 512, U16, 512, U16, U16, 512, U16, nullptr, 64), FP8_ERR_NULL);
  expect("packed gemm huge", p(BIG, BIG, BIG, U16, BIG, U16, U16, BIG, U16, A16, BIG), FP8_ERR_SHAPE);
}

}  // namespace

int main() {
  status_strings();
  amax_and_scale();
  quantize();
  quantize_delayed();
  mx_casts();
  packed_scales();
  gemms();
  std::printf(failures ? "FAILED (%d)\n" : "ok\n", failures);
  return failures ? 1 : 0;
}

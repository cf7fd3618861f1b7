// Random numbers beyond rounding on the library's position-keyed Philox
// stream: uniform and normal draws (for initialisation) and dropout.
//
// Sources (pages cited by title and section):
//   "Add stochastic rounding and philox RNG helpers" (FlyDSL pull request),
//     discussion: the counter-based generator as a general random-number
//     facility -- dropout, initialisation and the like -- rather than a
//     rounding detail.
//   "adamw-sr" (kernels hub page), Method: draws keyed by (seed, step) and
//     indexed by global element position, so any split of a tensor into
//     pieces that pass their own base_index reproduces the whole.
//
// The stream: position p = base_index + i takes 32-bit word p & 3 of the
// Philox4x32-10 call with counter (lo32(p >> 2), hi32(p >> 2), 0, 0), key
// (seed, step). From the word W of a position:
//   uniform  U = (W >> 8) * 2**-24 in [0, 1); y = low + (high - low) * U
//   normal   Box-Muller on the pair (2q, 2q+1), which shares a call:
//            u1 = ((W(2q) >> 8) + 1) * 2**-24, u2 = (W(2q+1) >> 8) * 2**-24,
//            r = sqrt(-2 ln u1), z(2q) = r cos(2 pi u2), z(2q+1) = r sin(2 pi u2);
//            y = mean + std * z (log, sin, cos on the hardware units)
//   dropout  dropped when W < floor(p * 2**32); y = x * (kept ? f32(1/(1-p)) : 0)
// Every kernel handles 4 consecutive positions per lane: one Philox call
// when they start on a group of four, two otherwise. All arithmetic is
// binary32 with no contraction; bf16 outputs are the round-to-nearest-even
// of the binary32 value.
#include "device.hpp"
#include "status.hpp"

#include <adamw_sr.h>

#include <algorithm>
#include <cmath>
#include <string>

#pragma clang fp contract(off)

namespace asr_rng {

constexpr int kBlock = 256;
constexpr int kVec = 4;                      // positions per lane
constexpr int64_t kSlot = kBlock * kVec;     // positions per workgroup
constexpr uint32_t kMaxGrid = 1u << 23;      // workgroups per launch
constexpr uint32_t kWindows = 8;             // one address window per XCD
constexpr float kTwoM24 = 1.0f / 16777216.0f;

enum Op { kUniform = 0, kNormal = 1, kDropout = 2 };

// Workgroup b works on slot w * q + min(w, r) + k of its launch (w = b % 8,
// k = b / 8): the workgroups that run on one XCD cover one contiguous range.
__device__ __forceinline__ uint32_t slot_of_block(uint32_t b, uint32_t grid) {
  const uint32_t w = b % kWindows, k = b / kWindows;
  const uint32_t q = grid / kWindows, r = grid % kWindows;
  return w * q + (w < r ? w : r) + k;
}

struct Params {
  const void* x;       // dropout input (f32 or bf16)
  void* y;             // output (f32 or bf16)
  uint8_t* mask;       // dropout keep mask, or null
  int64_t n;
  uint64_t slot0;      // first slot of this launch
  uint64_t base_index;
  float a, b;          // uniform: low, high - low; normal: mean, std; dropout: scale
  uint32_t threshold;  // dropout
  uint32_t seed, step;
  // Runs of 4 positions start `shift` elements before element 0 (the first
  // run's leading lanes touch nothing), so that whole runs are vector-
  // aligned in x and y; vec_ok says such a shift exists (else shift is 0
  // and every element moves on its own).
  uint32_t vec_ok;
  uint32_t shift;
};

// Words of positions (p0 & ~3) + k, k < 4 (PHASE == 0) or k < 8.
template <int PHASE>
__device__ __forceinline__ void run_words(uint64_t p0, uint32_t seed, uint32_t step,
                                          uint32_t (&w)[8]) {
  const uint64_t j0 = p0 >> 2;
  const asr::Words4 a = asr::stream_call(j0, seed, step);
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = a.w[k];
  if constexpr (PHASE > 0) {
    // a run that crosses position 2**64 continues at counter 0
    const asr::Words4 b = asr::stream_call((j0 + 1) & asr::kCounterMask, seed, step);
#pragma unroll
    for (int k = 0; k < 4; ++k) w[4 + k] = b.w[k];
  } else {
#pragma unroll
    for (int k = 4; k < 8; ++k) w[k] = 0;
  }
}

__device__ __forceinline__ float unit(uint32_t w) {
  return static_cast<float>(w >> 8) * kTwoM24;  // exact: 24-bit integer times 2**-24
}

// Standard normal pair of the words (W(2q), W(2q+1)), on the hardware
// transcendental units: v_log_f32 is log2, and v_sin_f32 / v_cos_f32 take
// their argument in revolutions, so sin(2 pi u2) is v_sin_f32(u2) with no
// argument reduction. Each of them only ever sees the 2**24 values
// (k + 1) * 2**-24 (u1) or k * 2**-24 (u2); the test suite measures their
// error over all of those inputs through asr_box_muller_given_words, which
// runs this function.
constexpr float kTwoLn2 = 1.38629436111989061883f;  // 2 ln 2, rounded to binary32

// Correctly rounded square root of an x that is +0 or a positive normal
// number (here x = 2 ln 2 |log2 u1| lies in [0, 34)). v_sqrt_f32 is within
// one ulp of the root, so the rounded root is y or one of its neighbours;
// Tuckerman's test picks it: with exact products (fma), the root lies below
// the midpoint of y- and y when x <= y- * y, and above the midpoint of y and
// y+ when x > y * y+. Without the range reduction and special cases of the
// general form, for inputs that need neither.
__device__ __forceinline__ float sqrt_rn_nonneg_normal(float x) {
  const float y = __builtin_amdgcn_sqrtf(x);
  const float below = __uint_as_float(__float_as_uint(y) - 1u);
  const float above = __uint_as_float(__float_as_uint(y) + 1u);
  float r = __builtin_fmaf(-below, y, x) <= 0.0f ? below : y;
  r = __builtin_fmaf(-y, above, x) > 0.0f ? above : r;
  return r;
}

__device__ __forceinline__ void box_muller(uint32_t w_even, uint32_t w_odd, float& zc,
                                           float& zs) {
  const float u1 = static_cast<float>((w_even >> 8) + 1u) * kTwoM24;  // (0, 1], exact
  const float u2 = unit(w_odd);
  // log2 u1 <= 0; its magnitude keeps r = +0 at u1 = 1
  const float r = sqrt_rn_nonneg_normal(kTwoLn2 * __builtin_fabsf(__builtin_amdgcn_logf(u1)));
  zc = r * __builtin_amdgcn_cosf(u2);
  zs = r * __builtin_amdgcn_sinf(u2);
}

__global__ void __launch_bounds__(kBlock)
box_muller_given_words(const uint32_t* __restrict__ w_even, const uint32_t* __restrict__ w_odd,
                       float* __restrict__ zc, float* __restrict__ zs, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride)
    box_muller(w_even[i], w_odd[i], zc[i], zs[i]);
}

// Elements i0 + e of a buffer, for the e in [lo, hi) that lie inside it.
template <typename T>
__device__ __forceinline__ void load4(const T* base, int64_t i0, bool full, int lo, int hi,
                                      float (&x)[4]) {
  if (full) asr::load_vec<false, 4>(base + i0, x);
  else asr::load_range(base, i0, lo, hi, x);
}

__device__ __forceinline__ void store4(float* base, int64_t i0, bool full, int lo, int hi,
                                       const float (&y)[4]) {
  if (full) asr::store_vec<false, 4>(base + i0, y);
  else asr::store_range(base, i0, lo, hi, y);
}

__device__ __forceinline__ void store4(uint16_t* base, int64_t i0, bool full, int lo, int hi,
                                       const float (&y)[4]) {
  uint32_t h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = asr::round_rn(__float_as_uint(y[e]));
  if (full) asr::store_vec_bf16<false, 4>(base + i0, h);
  else asr::store_range_bf16(base, i0, lo, hi, h);
}

// One lane: positions of elements i0 .. i0 + 3, of which lo <= e < hi lie
// inside the tensor.
template <int OP, typename T, int PHASE>
__device__ __forceinline__ void run(const Params& P, int64_t i0, int lo, int hi) {
  const bool full = P.vec_ok && lo == 0 && hi == kVec;
  const uint64_t p0 = P.base_index + static_cast<uint64_t>(i0);
  uint32_t w[8];
  run_words<PHASE>(p0, P.seed, P.step, w);
  float y[4];
  if constexpr (OP == kUniform) {
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = P.a + P.b * unit(w[PHASE + e]);
  } else if constexpr (OP == kNormal) {
    // pairs q = (PHASE >> 1) .. ((PHASE + 3) >> 1), each evaluated once
    constexpr int kFirst = PHASE >> 1, kLast = (PHASE + 3) >> 1;
    float z[8];
#pragma unroll
    for (int q = kFirst; q <= kLast; ++q) box_muller(w[2 * q], w[2 * q + 1], z[2 * q], z[2 * q + 1]);
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = P.a + P.b * z[PHASE + e];
  } else {
    float x[4];
    load4(static_cast<const T*>(P.x), i0, full, lo, hi, x);
    uint32_t keep = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool k = w[PHASE + e] >= P.threshold;
      keep |= static_cast<uint32_t>(k) << (8 * e);
      y[e] = x[e] * (k ? P.a : 0.0f);
    }
    if (P.mask) {
      if (lo == 0 && hi == kVec && ((reinterpret_cast<uintptr_t>(P.mask) + i0) & 3) == 0) {
        *reinterpret_cast<uint32_t*>(P.mask + i0) = keep;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e >= lo && e < hi) P.mask[i0 + e] = static_cast<uint8_t>((keep >> (8 * e)) & 1u);
      }
    }
  }
  store4(static_cast<T*>(P.y), i0, full, lo, hi, y);
}

template <int OP, typename T>
__global__ void __launch_bounds__(kBlock) rng_kernel(Params P) {
  const int64_t i0 = static_cast<int64_t>(P.slot0 + slot_of_block(blockIdx.x, gridDim.x)) * kSlot +
                     static_cast<int64_t>(threadIdx.x) * kVec - static_cast<int64_t>(P.shift);
  const int64_t left = P.n - i0;
  if (left <= 0) return;
  const int hi = left < kVec ? static_cast<int>(left) : kVec;
  const int lo = i0 < 0 ? static_cast<int>(-i0) : 0;
  // every run of the tensor starts at the same phase within its Philox call
  switch (static_cast<int>((P.base_index - P.shift) & 3u)) {
    case 0: run<OP, T, 0>(P, i0, lo, hi); break;
    case 1: run<OP, T, 1>(P, i0, lo, hi); break;
    case 2: run<OP, T, 2>(P, i0, lo, hi); break;
    default: run<OP, T, 3>(P, i0, lo, hi); break;
  }
}

}  // namespace asr_rng

// =========================================================== host side
namespace {

using asr_host::fail;
using asr_host::hip_fail;
using asr_host::ok;

bool aligned_to(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

template <int OP, typename T>
hipError_t launch_all(asr_rng::Params P, hipStream_t stream) {
  const uint64_t n_slots =
      (static_cast<uint64_t>(P.n) + P.shift + asr_rng::kSlot - 1) / asr_rng::kSlot;
  for (uint64_t slot0 = 0; slot0 < n_slots; slot0 += asr_rng::kMaxGrid) {
    P.slot0 = slot0;
    const uint32_t grid =
        static_cast<uint32_t>(std::min<uint64_t>(n_slots - slot0, asr_rng::kMaxGrid));
    void* argv[] = {&P};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&asr_rng::rng_kernel<OP, T>),
                                         dim3(grid), dim3(asr_rng::kBlock), argv, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int OP>
int dispatch(asr_rng::Params P, int32_t dtype, hipStream_t stream, const char* what) {
  const hipError_t e = dtype == ASR_F32 ? launch_all<OP, float>(P, stream)
                                        : launch_all<OP, uint16_t>(P, stream);
  if (e != hipSuccess) return hip_fail(e, what);
  return ok();
}

int check_common(const void* y, int32_t dtype, int64_t n) {
  if (dtype != ASR_F32 && dtype != ASR_BF16) return fail(ASR_EDTYPE, "dtype must be ASR_F32 or ASR_BF16");
  if (n < 0) return fail(ASR_EINVAL, "n < 0");
  if (n > (int64_t{1} << 62)) return fail(ASR_EINVAL, "n too large");
  if (n > 0 && !y) return fail(ASR_EINVAL, "NULL output");
  if (!aligned_to(y, dtype == ASR_F32 ? 4 : 2)) return fail(ASR_EALIGN, "output not aligned to its element size");
  return ASR_OK;
}

uint32_t vec_alignment(int32_t dtype) { return dtype == ASR_F32 ? 16 : 8; }

// Sets P.shift to the s in [0, 4) for which elements 4k - s of x (if
// given) and y sit on vector-aligned addresses, and P.vec_ok to whether
// there is one. A piece cut from aligned buffers at element offset o has
// s = o mod 4.
void choose_shift(asr_rng::Params& P, int32_t dtype) {
  const uintptr_t elem = dtype == ASR_F32 ? 4 : 2, vec = vec_alignment(dtype);
  P.vec_ok = 0;
  P.shift = 0;
  for (uint32_t s = 0; s < 4; ++s) {
    const bool y_ok = ((reinterpret_cast<uintptr_t>(P.y) + (4 - s) * elem) & (vec - 1)) == 0;
    const bool x_ok = !P.x || ((reinterpret_cast<uintptr_t>(P.x) + (4 - s) * elem) & (vec - 1)) == 0;
    if (y_ok && x_ok) {
      P.vec_ok = 1;
      P.shift = s;
      return;
    }
  }
}

// The draws are formed in binary32: a parameter must be a finite binary32 value.
bool fits_f32(double v) { return std::isfinite(v) && std::fabs(v) <= 3.4028234663852886e38; }

}  // namespace

extern "C" {

int asr_random_uniform(void* out, int32_t dtype, int64_t n, double low, double high,
                       uint32_t seed, uint32_t step, uint64_t base_index, void* stream) {
  if (int s = check_common(out, dtype, n)) return s;
  if (!fits_f32(low) || !fits_f32(high) || !fits_f32(high - low))
    return fail(ASR_EINVAL, "low, high and high - low must be finite in binary32");
  if (n == 0) return ok();
  asr_rng::Params P{};
  P.y = out;
  P.n = n;
  P.base_index = base_index;
  P.a = static_cast<float>(low);
  P.b = static_cast<float>(high - low);
  P.seed = seed;
  P.step = step;
  choose_shift(P, dtype);
  return dispatch<asr_rng::kUniform>(P, dtype, static_cast<hipStream_t>(stream), "uniform launch");
}

int asr_random_normal(void* out, int32_t dtype, int64_t n, double mean, double std,
                      uint32_t seed, uint32_t step, uint64_t base_index, void* stream) {
  if (int s = check_common(out, dtype, n)) return s;
  if (!fits_f32(mean) || !fits_f32(std) || std < 0.0)
    return fail(ASR_EINVAL, "mean and std must be finite in binary32, std >= 0");
  if (n == 0) return ok();
  asr_rng::Params P{};
  P.y = out;
  P.n = n;
  P.base_index = base_index;
  P.a = static_cast<float>(mean);
  P.b = static_cast<float>(std);
  P.seed = seed;
  P.step = step;
  choose_shift(P, dtype);
  return dispatch<asr_rng::kNormal>(P, dtype, static_cast<hipStream_t>(stream), "normal launch");
}

int asr_dropout(const void* x, void* y, uint8_t* mask, int32_t dtype, int64_t n, double p,
                uint32_t seed, uint32_t step, uint64_t base_index, void* stream) {
  if (int s = check_common(y, dtype, n)) return s;
  if (!(p >= 0.0 && p < 1.0)) return fail(ASR_EINVAL, "p must be in [0, 1)");
  if (n > 0 && !x) return fail(ASR_EINVAL, "NULL input");
  if (!aligned_to(x, dtype == ASR_F32 ? 4 : 2)) return fail(ASR_EALIGN, "input not aligned to its element size");
  if (n == 0) return ok();
  asr_rng::Params P{};
  P.x = x;
  P.y = y;
  P.mask = mask;
  P.n = n;
  P.base_index = base_index;
  P.a = static_cast<float>(1.0 / (1.0 - p));
  P.threshold = static_cast<uint32_t>(std::min(std::floor(p * 4294967296.0), 4294967295.0));
  P.seed = seed;
  P.step = step;
  choose_shift(P, dtype);
  return dispatch<asr_rng::kDropout>(P, dtype, static_cast<hipStream_t>(stream), "dropout launch");
}

int asr_box_muller_given_words(const uint32_t* w_even, const uint32_t* w_odd, float* zc,
                               float* zs, int64_t n, void* stream) {
  if (n < 0) return fail(ASR_EINVAL, "n < 0");
  if (n == 0) return ok();
  if (!w_even || !w_odd || !zc || !zs) return fail(ASR_EINVAL, "NULL buffer");
  if (!aligned_to(w_even, 4) || !aligned_to(w_odd, 4) || !aligned_to(zc, 4) || !aligned_to(zs, 4))
    return fail(ASR_EALIGN, "buffers must be 4-byte aligned");
  const int64_t blocks = (n + asr_rng::kBlock - 1) / asr_rng::kBlock;
  const uint32_t grid = static_cast<uint32_t>(std::min<int64_t>(blocks, 1 << 16));
  void* argv[] = {&w_even, &w_odd, &zc, &zs, &n};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&asr_rng::box_muller_given_words),
                                       dim3(grid), dim3(asr_rng::kBlock), argv, 0,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "box-muller launch");
  return ok();
}

}  // extern "C"

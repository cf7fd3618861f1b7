// Device building blocks of the AdamW-SR path for gfx950: Philox4x32-10,
// the f32 -> bf16 roundings, the per-element AdamW update and the 8-element
// vector loads/stores the streaming kernels use.
//
// Sources (pages cited by title and section):
//   "Add stochastic rounding and philox RNG helpers" (FlyDSL pull request),
//     Primitives: a counter-based generator returning four 32-bit words and
//     the add-and-truncate stochastic rounding.
//   "adamw-sr" (kernels hub page), intro/Usage/Method: the decoupled-weight-
//     decay Adam update, fp32 states, keying by (seed, step) and global
//     element position.
//   Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011):
//     the Philox4x32 round function and constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Every multiply and add below must round on its own: no contraction into
// fused multiply-adds, whatever the command line says.
#pragma clang fp contract(off)

namespace asr {

// ---------------------------------------------------------------- Philox
constexpr uint32_t kPhiloxMulA = 0xD2511F53u;   // multiplies counter word 0
constexpr uint32_t kPhiloxMulB = 0xCD9E8D57u;   // multiplies counter word 2
constexpr uint32_t kPhiloxBumpA = 0x9E3779B9u;  // added to key word 0 per round
constexpr uint32_t kPhiloxBumpB = 0xBB67AE85u;  // added to key word 1 per round

struct Words4 {
  uint32_t w[4];
};

// Philox4x32 with 10 rounds. One round replaces (c0, c1, c2, c3) by
// (hi(B*c2) ^ c1 ^ k0, lo(B*c2), hi(A*c0) ^ c3 ^ k1, lo(A*c0)); the key is
// bumped between rounds. The key words are wave-uniform in every caller, so
// the key schedule lives in scalar registers; each 32x32->64 product is one
// v_mad_u64_u32.
__device__ __forceinline__ Words4 philox4x32_10(uint32_t c0, uint32_t c1,
                                                uint32_t c2, uint32_t c3,
                                                uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t prod_a = static_cast<uint64_t>(c0) * kPhiloxMulA;
    const uint64_t prod_b = static_cast<uint64_t>(c2) * kPhiloxMulB;
    const uint32_t next0 = static_cast<uint32_t>(prod_b >> 32) ^ c1 ^ k0;
    const uint32_t next2 = static_cast<uint32_t>(prod_a >> 32) ^ c3 ^ k1;
    c1 = static_cast<uint32_t>(prod_b);
    c3 = static_cast<uint32_t>(prod_a);
    c0 = next0;
    c2 = next2;
    k0 += kPhiloxBumpA;
    k1 += kPhiloxBumpB;
  }
  return Words4{{c0, c1, c2, c3}};
}

// The call that serves global positions 4j .. 4j+3 of the random-bit stream:
// counter (lo32(j), hi32(j), 0, 0), key (seed, step).
__device__ __forceinline__ Words4 stream_call(uint64_t j, uint32_t seed,
                                              uint32_t step) {
  return philox4x32_10(static_cast<uint32_t>(j), static_cast<uint32_t>(j >> 32),
                       0u, 0u, seed, step);
}

// 16 random bits for the 8 consecutive positions pos0 .. pos0+7, where
// PHASE = pos0 & 3 is known at compile time. Position pos0+e takes word
// (PHASE+e) & 3 of call (pos0 >> 2) + ((PHASE+e) >> 2): two calls when the
// run starts on a group of four, three otherwise.
template <int PHASE>
__device__ __forceinline__ void stream_bits8(uint64_t pos0, uint32_t seed,
                                             uint32_t step, uint32_t (&r)[8]) {
  const uint64_t j0 = pos0 >> 2;
  const Words4 a = stream_call(j0, seed, step);
  const Words4 b = stream_call(j0 + 1, seed, step);
  uint32_t words[12];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    words[k] = a.w[k];
    words[4 + k] = b.w[k];
  }
  if constexpr (PHASE != 0) {
    const Words4 c = stream_call(j0 + 2, seed, step);
#pragma unroll
    for (int k = 0; k < 4; ++k) words[8 + k] = c.w[k];
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) words[8 + k] = 0u;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = words[PHASE + e] & 0xFFFFu;
}

// ------------------------------------------------------------- roundings
__device__ __forceinline__ bool f32_bits_is_nan(uint32_t u) {
  return (u & 0x7FFFFFFFu) > 0x7F800000u;
}

// Stochastic rounding: add the 16 random bits to the dropped half, keep the
// high half. A NaN keeps its high half with the quiet bit forced on, so no
// payload can carry into the exponent or the sign.
__device__ __forceinline__ uint32_t round_sr(uint32_t u, uint32_t r16) {
  return f32_bits_is_nan(u) ? ((u >> 16) | 0x0040u) : ((u + r16) >> 16);
}

// Round to nearest, ties to even; NaN as above.
__device__ __forceinline__ uint32_t round_rn(uint32_t u) {
  return f32_bits_is_nan(u) ? ((u >> 16) | 0x0040u)
                            : ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ----------------------------------------------------------- AdamW update
struct Coeffs {
  float decay;         // 1 - lr*wd
  float b1, omb1;      // beta1, 1 - beta1
  float b2, omb2;      // beta2, 1 - beta2
  float step_size;     // lr / (1 - beta1**t)
  float inv_bc2_sqrt;  // 1 / sqrt(1 - beta2**t)
  float eps;
};

// One element, binary32, fixed order. __builtin_sqrtf and '/' are the
// correctly rounded forms (HIP's default; the library is built without
// fast-math), and no multiply-add is fused (pragma above).
__device__ __forceinline__ void adamw_update(float& p, float g, float& m,
                                             float& v, const Coeffs& c) {
  m = c.b1 * m + c.omb1 * g;
  v = c.b2 * v + c.omb2 * (g * g);
  const float den = __builtin_sqrtf(v) * c.inv_bc2_sqrt + c.eps;
  const float upd = m / den;
  p = p * c.decay - c.step_size * upd;
}

// ------------------------------------------------------ element storage
struct F32 {
  using storage = float;
};
struct BF16 {
  using storage = uint16_t;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// 128-bit loads/stores of 8 elements starting at a 16-byte-aligned address.
__device__ __forceinline__ void load8(const float* src, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(src)[0];
  const float4 b = reinterpret_cast<const float4*>(src)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void load8(const uint16_t* src, float (&x)[8]) {
  const uint4 q = reinterpret_cast<const uint4*>(src)[0];
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void store8(float* dst, const float (&x)[8]) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(dst)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

__device__ __forceinline__ void store8_bf16(uint16_t* dst, const uint32_t (&h)[8]) {
  reinterpret_cast<uint4*>(dst)[0] =
      make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                 h[6] | (h[7] << 16));
}

// Element-wise forms for the ragged tail and for unaligned tensors: only
// elements e < count are touched.
__device__ __forceinline__ void load_n(const float* src, int count, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (e < count) ? src[e] : 0.0f;
}

__device__ __forceinline__ void load_n(const uint16_t* src, int count, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    x[e] = (e < count) ? bf16_bits_to_f32(src[e]) : 0.0f;
}

__device__ __forceinline__ void store_n(float* dst, int count, const float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e < count) dst[e] = x[e];
}

__device__ __forceinline__ void store_n_bf16(uint16_t* dst, int count,
                                             const uint32_t (&h)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e < count) dst[e] = static_cast<uint16_t>(h[e]);
}

}  // namespace asr

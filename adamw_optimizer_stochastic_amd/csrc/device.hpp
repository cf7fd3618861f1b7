// Device building blocks of the AdamW-SR path for gfx950: Philox4x32-10,
// the f32 -> bf16 roundings, the per-element AdamW update and the 4- or
// 8-element vector loads/stores the streaming kernels use.
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
    // three-input XOR in one gfx950 instruction (truth table 0x96 = a^b^c)
    const uint32_t next0 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(prod_b >> 32), c1, k0, 0x96);
    const uint32_t next2 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(prod_a >> 32), c3, k1, 0x96);
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

constexpr uint64_t kCounterMask = (uint64_t{1} << 62) - 1;

// 16 random bits for the V consecutive positions pos0 .. pos0+V-1, where
// PHASE = pos0 & 3 is known at compile time. Position pos0+e takes word
// (PHASE+e) & 3 of call (pos0 >> 2) + ((PHASE+e) >> 2): V/4 calls when the
// run starts on a group of four, one more otherwise.
template <int PHASE, int V>
__device__ __forceinline__ void stream_bits(uint64_t pos0, uint32_t seed, uint32_t step,
                                            uint32_t (&r)[V]) {
  constexpr int kCalls = (PHASE + V + 3) / 4;
  const uint64_t j0 = pos0 >> 2;
  uint32_t words[4 * kCalls];
#pragma unroll
  for (int k = 0; k < kCalls; ++k) {
    // Positions wrap modulo 2**64, so their counters p >> 2 wrap modulo
    // 2**62: a run that crosses 2**64 continues at counter 0.
    const uint64_t j = k == 0 ? j0 : ((j0 + k) & kCounterMask);
    const Words4 w = stream_call(j, seed, step);
#pragma unroll
    for (int q = 0; q < 4; ++q) words[4 * k + q] = w.w[q];
  }
#pragma unroll
  for (int e = 0; e < V; ++e) r[e] = words[PHASE + e] & 0xFFFFu;
}

// ------------------------------------------------------------- roundings
__device__ __forceinline__ bool f32_bits_is_nan(uint32_t u) {
  return (u & 0x7FFFFFFFu) > 0x7F800000u;
}

// Stochastic rounding: add the 16 random bits to the dropped half, keep the
// high half. A NaN keeps its high half with the quiet bit forced on, so no
// payload can carry into the exponent or the sign.
//
// gfx950 has this conversion in hardware (v_cvt_sr_bf16_f32). It takes its
// 16 random bits from the HIGH half of the 32-bit random operand and
// otherwise computes exactly the rule above, NaN, Inf, subnormals and
// overflow included; the test suite checks that against the reference
// implementation for every f32 input at several random values and for every
// random value at sampled inputs. ASR_HW_SR=0 selects the integer form.
#ifndef ASR_HW_SR
#define ASR_HW_SR 1
#endif
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t round_sr_int(uint32_t u, uint32_t r16) {
  return f32_bits_is_nan(u) ? ((u >> 16) | 0x0040u) : ((u + r16) >> 16);
}

__device__ __forceinline__ uint32_t round_sr(uint32_t u, uint32_t r16) {
  if constexpr (ASR_HW_SR) {
    const bf16x2 v = __builtin_amdgcn_cvt_sr_bf16_f32(bf16x2{}, __uint_as_float(u), r16 << 16, false);
    return __builtin_bit_cast(uint32_t, v) & 0xFFFFu;
  } else {
    return round_sr_int(u, r16);
  }
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

// Vector loads/stores of 4 or 8 consecutive elements from an aligned address.
// NT selects the non-temporal (streaming) form; the kernels measured faster
// without it and pass NT = false.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT, typename V>
__device__ __forceinline__ V vload(const V* src) {
  if constexpr (NT) return __builtin_nontemporal_load(src);
  else return *src;
}

template <bool NT, typename V>
__device__ __forceinline__ void vstore(V* dst, V x) {
  if constexpr (NT) __builtin_nontemporal_store(x, dst);
  else *dst = x;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// V consecutive elements (V = 4 or 8) from a 16-byte-aligned f32 address.
template <bool NT, int V>
__device__ __forceinline__ void load_vec(const float* src, float (&x)[V]) {
#pragma unroll
  for (int h = 0; h < V / 4; ++h) {
    const f32x4 a = vload<NT>(reinterpret_cast<const f32x4*>(src) + h);
    x[4 * h] = a.x; x[4 * h + 1] = a.y; x[4 * h + 2] = a.z; x[4 * h + 3] = a.w;
  }
}

// V consecutive bf16 elements (16 bytes for V = 8, 8 bytes for V = 4),
// upcast exactly: the bf16 pattern is the high half of the f32 pattern.
template <bool NT, int V>
__device__ __forceinline__ void load_vec(const uint16_t* src, float (&x)[V]) {
  uint32_t w[V / 2];
  if constexpr (V == 8) {
    const u32x4 q = vload<NT>(reinterpret_cast<const u32x4*>(src));
    w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
  } else {
    static_assert(V == 4, "4 or 8 elements per lane");
    const u32x2 q = vload<NT>(reinterpret_cast<const u32x2*>(src));
    w[0] = q.x; w[1] = q.y;
  }
#pragma unroll
  for (int k = 0; k < V / 2; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
  }
}

template <bool NT, int V>
__device__ __forceinline__ void store_vec(float* dst, const float (&x)[V]) {
#pragma unroll
  for (int h = 0; h < V / 4; ++h)
    vstore<NT>(reinterpret_cast<f32x4*>(dst) + h,
               f32x4{x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]});
}

template <bool NT, int V>
__device__ __forceinline__ void store_vec_bf16(uint16_t* dst, const uint32_t (&h)[V]) {
  if constexpr (V == 8) {
    vstore<NT>(reinterpret_cast<u32x4*>(dst),
               u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                     h[6] | (h[7] << 16)});
  } else {
    vstore<NT>(reinterpret_cast<u32x2*>(dst), u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
  }
}

// Element-wise forms for a run that is cut by either end of its tensor, or
// whose buffers are not vector-aligned: element e of the run is element
// i0 + e of the buffer, and only lo <= e < hi is touched (i0 is negative for
// the first run of a tensor whose runs start before it, see the kernels).
template <int V>
__device__ __forceinline__ void load_range(const float* base, int64_t i0, int lo, int hi,
                                           float (&x)[V]) {
#pragma unroll
  for (int e = 0; e < V; ++e) x[e] = (e >= lo && e < hi) ? base[i0 + e] : 0.0f;
}

template <int V>
__device__ __forceinline__ void load_range(const uint16_t* base, int64_t i0, int lo, int hi,
                                           float (&x)[V]) {
#pragma unroll
  for (int e = 0; e < V; ++e)
    x[e] = (e >= lo && e < hi) ? bf16_bits_to_f32(base[i0 + e]) : 0.0f;
}

template <int V>
__device__ __forceinline__ void store_range(float* base, int64_t i0, int lo, int hi,
                                            const float (&x)[V]) {
#pragma unroll
  for (int e = 0; e < V; ++e)
    if (e >= lo && e < hi) base[i0 + e] = x[e];
}

template <int V>
__device__ __forceinline__ void store_range_bf16(uint16_t* base, int64_t i0, int lo, int hi,
                                                 const uint32_t (&h)[V]) {
#pragma unroll
  for (int e = 0; e < V; ++e)
    if (e >= lo && e < hi) base[i0 + e] = static_cast<uint16_t>(h[e]);
}

}  // namespace asr

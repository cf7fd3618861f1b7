// Kernels and C ABI of the fused AdamW step with stochastic-rounding bf16
// write-back, for gfx950 (MI355X). The ABI is declared and documented in
// include/adamw_sr.h.
//
// Sources (pages cited by title and section):
//   "adamw-sr" (kernels hub page): intro (decoupled-weight-decay Adam step,
//     unbiased bf16 write-back, no fp32 master), Usage (drop-in for
//     torch.optim.AdamW; f32 states; f32|bf16 params and grads), Method
//     (Philox keyed by (seed, step), indexed by global element position),
//     Correctness (per-shard base_index equals the whole update bitwise).
//   "Add stochastic rounding and philox RNG helpers" (FlyDSL pull request):
//     Primitives (Philox words, add-and-truncate SR), discussion (SR as a
//     rounding mode of the f32 -> bf16 conversion).
//
// Design for the hardware: the step is a pure stream (22 bytes per bf16
// element, each byte read or written once), so the kernels are built around
// HBM bandwidth: 128-bit loads and stores of 8 elements per lane, Philox in
// registers with one call per 4 consecutive positions (no generator state in
// memory), no LDS and no matrix cores. A multi-tensor chunk table lets one
// launch cover thousands of tensors: every workgroup takes whole chunks of
// one tensor and finds its tensor by a wave-uniform binary search.
#include "device.hpp"

#include <adamw_sr.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <tuple>
#include <utility>
#include <type_traits>
#include <vector>

#pragma clang fp contract(off)

namespace asr {

constexpr int kBlock = 256;           // 4 waves of 64 lanes
constexpr int kVec = 8;               // elements per lane per iteration
constexpr int kMinChunkShift = 11;    // one block-iteration: 256 * 8 elements
#ifndef ASR_MAX_CHUNK_SHIFT
#define ASR_MAX_CHUNK_SHIFT 16
#endif
constexpr int kMaxChunkShift = ASR_MAX_CHUNK_SHIFT;
#ifndef ASR_TARGET_CHUNKS
#define ASR_TARGET_CHUNKS 32768
#endif
constexpr int64_t kTargetChunks = ASR_TARGET_CHUNKS;
constexpr uint32_t kMaxGrid = 1u << 20;  // blocks; larger work grid-strides
constexpr int kGroups = 4;               // (param dtype, grad dtype) pairs
constexpr int kUploadWords = 768;        // 3 KiB of metadata per upload launch

// Per-tensor metadata as the kernel reads it from the workspace.
struct DevTensor {
  void* param;
  const void* grad;
  float* m;
  float* v;
  int64_t numel;
  uint64_t base_index;
  uint32_t vec_ok;  // all four buffers 16-byte aligned: 128-bit path
  uint32_t reserved;
};
static_assert(sizeof(DevTensor) == 56, "metadata layout");

// ------------------------------------------------------- uniform loads
// Metadata is the same for the whole workgroup; keep it in scalar registers.
__device__ __forceinline__ uint32_t uniform_u32(const uint32_t* p) {
  return __builtin_amdgcn_readfirstlane(*p);
}
__device__ __forceinline__ uint64_t uniform_u64(const uint64_t* p) {
  const uint64_t x = *p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ DevTensor uniform_tensor(const DevTensor* t) {
  const uint64_t* w = reinterpret_cast<const uint64_t*>(t);
  DevTensor d;
  d.param = reinterpret_cast<void*>(uniform_u64(w + 0));
  d.grad = reinterpret_cast<const void*>(uniform_u64(w + 1));
  d.m = reinterpret_cast<float*>(uniform_u64(w + 2));
  d.v = reinterpret_cast<float*>(uniform_u64(w + 3));
  d.numel = static_cast<int64_t>(uniform_u64(w + 4));
  d.base_index = uniform_u64(w + 5);
  const uint64_t flags = uniform_u64(w + 6);
  d.vec_ok = static_cast<uint32_t>(flags);
  d.reserved = 0;
  return d;
}

enum : int { kRoundSR = ASR_ROUND_SR, kRoundRN = ASR_ROUND_RN };

// One span [start, stop) of one tensor; each lane takes 8 consecutive
// elements per iteration, the block strides by 2048 elements.
template <class PT, class GT, int ROUND, int PHASE, bool VEC>
__device__ __forceinline__ void adamw_span(const DevTensor& t, int64_t start,
                                           int64_t stop, const Coeffs& c,
                                           uint32_t seed, uint32_t step) {
  using PS = typename PT::storage;
  using GS = typename GT::storage;
  PS* __restrict__ param = static_cast<PS*>(t.param);
  const GS* __restrict__ grad = static_cast<const GS*>(t.grad);
  float* __restrict__ m = t.m;
  float* __restrict__ v = t.v;
  for (int64_t i0 = start + static_cast<int64_t>(threadIdx.x) * kVec; i0 < stop;
       i0 += static_cast<int64_t>(kBlock) * kVec) {
    const int64_t left = stop - i0;
    const int count = left < kVec ? static_cast<int>(left) : kVec;
    const bool full = VEC && count == kVec;
    float p[kVec], g[kVec], mm[kVec], vv[kVec];
    if (full) {
      load8(param + i0, p);
      load8(grad + i0, g);
      load8(m + i0, mm);
      load8(v + i0, vv);
    } else {
      load_n(param + i0, count, p);
      load_n(grad + i0, count, g);
      load_n(m + i0, count, mm);
      load_n(v + i0, count, vv);
    }
#pragma unroll
    for (int e = 0; e < kVec; ++e) adamw_update(p[e], g[e], mm[e], vv[e], c);

    if constexpr (std::is_same_v<PT, F32>) {
      if (full) store8(param + i0, p);
      else store_n(param + i0, count, p);
    } else {
      uint32_t h[kVec];
      if constexpr (ROUND == kRoundSR) {
        uint32_t r[kVec];
        stream_bits8<PHASE>(t.base_index + static_cast<uint64_t>(i0), seed, step, r);
#pragma unroll
        for (int e = 0; e < kVec; ++e) h[e] = round_sr(__float_as_uint(p[e]), r[e]);
      } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) h[e] = round_rn(__float_as_uint(p[e]));
      }
      if (full) store8_bf16(param + i0, h);
      else store_n_bf16(param + i0, count, h);
    }
    if (full) {
      store8(m + i0, mm);
      store8(v + i0, vv);
    } else {
      store_n(m + i0, count, mm);
      store_n(v + i0, count, vv);
    }
  }
}

template <class PT, class GT, int ROUND, bool VEC>
__device__ __forceinline__ void adamw_span_phase(const DevTensor& t, int64_t start,
                                                 int64_t stop, const Coeffs& c,
                                                 uint32_t seed, uint32_t step) {
  if constexpr (std::is_same_v<PT, BF16> && ROUND == kRoundSR) {
    switch (static_cast<int>(t.base_index & 3u)) {
      case 0: adamw_span<PT, GT, ROUND, 0, VEC>(t, start, stop, c, seed, step); break;
      case 1: adamw_span<PT, GT, ROUND, 1, VEC>(t, start, stop, c, seed, step); break;
      case 2: adamw_span<PT, GT, ROUND, 2, VEC>(t, start, stop, c, seed, step); break;
      default: adamw_span<PT, GT, ROUND, 3, VEC>(t, start, stop, c, seed, step); break;
    }
  } else {
    adamw_span<PT, GT, ROUND, 0, VEC>(t, start, stop, c, seed, step);
  }
}

// The multi-tensor step. chunk_begin[k] is the first chunk of tensor k
// (chunk_begin[0] = 0, chunk_begin[n_tensors] = n_chunks, every tensor has at
// least one chunk); a chunk is 2**chunk_shift consecutive elements of one
// tensor, the last one of a tensor possibly shorter.
template <class PT, class GT, int ROUND>
__global__ void __launch_bounds__(kBlock)
adamw_sr_multi_tensor(const DevTensor* __restrict__ tensors,
                      const uint32_t* __restrict__ chunk_begin, int32_t n_tensors,
                      uint32_t n_chunks, int32_t chunk_shift, Coeffs c,
                      uint32_t seed, uint32_t step) {
  for (uint32_t chunk = blockIdx.x; chunk < n_chunks; chunk += gridDim.x) {
    int32_t lo = 0, hi = n_tensors - 1;  // last tensor whose first chunk <= chunk
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (uniform_u32(chunk_begin + mid) <= chunk) lo = mid;
      else hi = mid - 1;
    }
    const DevTensor t = uniform_tensor(tensors + lo);
    const int64_t start =
        static_cast<int64_t>(chunk - uniform_u32(chunk_begin + lo)) << chunk_shift;
    const int64_t stop = std::min(start + (int64_t{1} << chunk_shift), t.numel);
    if (t.vec_ok) adamw_span_phase<PT, GT, ROUND, true>(t, start, stop, c, seed, step);
    else adamw_span_phase<PT, GT, ROUND, false>(t, start, stop, c, seed, step);
  }
}

// Copies up to kUploadWords words of metadata, passed by value in the kernel
// arguments, to device memory. Stream-ordered and allocation-free.
struct UploadBlock {
  uint32_t w[kUploadWords];
};

__global__ void __launch_bounds__(kBlock)
upload_words(UploadBlock src, uint32_t* __restrict__ dst, uint32_t n_words) {
  for (uint32_t i = threadIdx.x; i < n_words; i += kBlock) dst[i] = src.w[i];
}

// ---------------------------------------------------------- Philox fill
__global__ void __launch_bounds__(kBlock)
philox_fill(uint32_t* __restrict__ out, int64_t n_counters, uint64_t counter_base,
            uint32_t upper_lo, uint32_t upper_hi, uint32_t seed, uint32_t step,
            int vec_ok) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t k = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; k < n_counters;
       k += stride) {
    const uint64_t ctr = counter_base + static_cast<uint64_t>(k);
    const Words4 w = philox4x32_10(static_cast<uint32_t>(ctr),
                                   static_cast<uint32_t>(ctr >> 32), upper_lo,
                                   upper_hi, seed, step);
    uint32_t* dst = out + 4 * k;
    if (vec_ok) {
      reinterpret_cast<uint4*>(dst)[0] = make_uint4(w.w[0], w.w[1], w.w[2], w.w[3]);
    } else {
      dst[0] = w.w[0]; dst[1] = w.w[1]; dst[2] = w.w[2]; dst[3] = w.w[3];
    }
  }
}

// ------------------------------------------------------ f32 -> bf16 converts
template <int ROUND, int PHASE, bool VEC>
__device__ __forceinline__ void convert_all(const float* __restrict__ in,
                                            uint16_t* __restrict__ out, int64_t n,
                                            uint64_t base_index, uint32_t seed,
                                            uint32_t step) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock * kVec;
  for (int64_t i0 = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) * kVec; i0 < n;
       i0 += stride) {
    const int64_t left = n - i0;
    const int count = left < kVec ? static_cast<int>(left) : kVec;
    const bool full = VEC && count == kVec;
    float x[kVec];
    if (full) load8(in + i0, x);
    else load_n(in + i0, count, x);
    uint32_t h[kVec];
    if constexpr (ROUND == kRoundSR) {
      uint32_t r[kVec];
      stream_bits8<PHASE>(base_index + static_cast<uint64_t>(i0), seed, step, r);
#pragma unroll
      for (int e = 0; e < kVec; ++e) h[e] = round_sr(__float_as_uint(x[e]), r[e]);
    } else {
#pragma unroll
      for (int e = 0; e < kVec; ++e) h[e] = round_rn(__float_as_uint(x[e]));
    }
    if (full) store8_bf16(out + i0, h);
    else store_n_bf16(out + i0, count, h);
  }
}

template <int ROUND>
__global__ void __launch_bounds__(kBlock)
convert_f32_bf16(const float* __restrict__ in, uint16_t* __restrict__ out, int64_t n,
                 uint64_t base_index, uint32_t seed, uint32_t step, int vec_ok) {
  if constexpr (ROUND == kRoundSR) {
    const int phase = static_cast<int>(base_index & 3u);
    if (vec_ok) {
      switch (phase) {
        case 0: convert_all<ROUND, 0, true>(in, out, n, base_index, seed, step); break;
        case 1: convert_all<ROUND, 1, true>(in, out, n, base_index, seed, step); break;
        case 2: convert_all<ROUND, 2, true>(in, out, n, base_index, seed, step); break;
        default: convert_all<ROUND, 3, true>(in, out, n, base_index, seed, step); break;
      }
    } else {
      switch (phase) {
        case 0: convert_all<ROUND, 0, false>(in, out, n, base_index, seed, step); break;
        case 1: convert_all<ROUND, 1, false>(in, out, n, base_index, seed, step); break;
        case 2: convert_all<ROUND, 2, false>(in, out, n, base_index, seed, step); break;
        default: convert_all<ROUND, 3, false>(in, out, n, base_index, seed, step); break;
      }
    }
  } else {
    if (vec_ok) convert_all<ROUND, 0, true>(in, out, n, base_index, seed, step);
    else convert_all<ROUND, 0, false>(in, out, n, base_index, seed, step);
  }
}

// ------------------------------------------------ sqrt / division probe
__global__ void __launch_bounds__(kBlock)
sqrt_div(const float* __restrict__ a, const float* __restrict__ b,
         float* __restrict__ sqrt_out, float* __restrict__ div_out, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
    const float x = a[i];
    sqrt_out[i] = __builtin_sqrtf(x);
    div_out[i] = x / b[i];
  }
}

}  // namespace asr

// =========================================================== host side
namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int ok() {
  g_last_error.clear();
  return ASR_OK;
}

// Launches `kernel` with one block size for all kernels of the library;
// the arguments are converted to the kernel's parameter types first.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), uint32_t grid, hipStream_t stream,
                  Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> vals(std::forward<Args>(args)...);
  return std::apply(
      [&](auto&... v) {
        void* argv[] = {static_cast<void*>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid),
                               dim3(asr::kBlock), argv, 0, stream);
      },
      vals);
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ASR_EHIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                            hipGetErrorString(e) + ")");
}

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Binary64 power by binary powering from the low bit (same definition the
// bias corrections are specified with).
double powi(double b, int64_t t) {
  double r = 1.0;
  while (t) {
    if (t & 1) r *= b;
    b *= b;
    t >>= 1;
  }
  return r;
}

int check_hparams(double lr, double beta1, double beta2, double eps, double wd,
                  int64_t step) {
  if (!std::isfinite(lr) || lr < 0.0) return fail(ASR_EINVAL, "lr must be finite and >= 0");
  if (!(beta1 >= 0.0 && beta1 < 1.0)) return fail(ASR_EINVAL, "beta1 must be in [0, 1)");
  if (!(beta2 >= 0.0 && beta2 < 1.0)) return fail(ASR_EINVAL, "beta2 must be in [0, 1)");
  if (!std::isfinite(eps) || eps < 0.0) return fail(ASR_EINVAL, "eps must be finite and >= 0");
  if (!std::isfinite(wd) || wd < 0.0)
    return fail(ASR_EINVAL, "weight_decay must be finite and >= 0");
  if (step < 1 || step > int64_t{0xFFFFFFFF})
    return fail(ASR_EINVAL, "step must be in [1, 2**32 - 1]");
  return ASR_OK;
}

asr::Coeffs make_coeffs(double lr, double beta1, double beta2, double eps, double wd,
                        int64_t step) {
  const double bc1 = 1.0 - powi(beta1, step);
  const double bc2 = 1.0 - powi(beta2, step);
  asr::Coeffs c;
  c.decay = static_cast<float>(1.0 - lr * wd);
  c.b1 = static_cast<float>(beta1);
  c.omb1 = static_cast<float>(1.0 - beta1);
  c.b2 = static_cast<float>(beta2);
  c.omb2 = static_cast<float>(1.0 - beta2);
  c.step_size = static_cast<float>(lr / bc1);
  c.inv_bc2_sqrt = static_cast<float>(1.0 / std::sqrt(bc2));
  c.eps = static_cast<float>(eps);
  return c;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace layout: for each (param dtype, grad dtype) group in a fixed
// order, its DevTensor array then its chunk_begin array, each 16-byte
// aligned. The bound below covers any split of n tensors into the groups.
size_t workspace_bound(int32_t n) {
  if (n <= 0) return 0;
  const size_t per_group_pad = 2 * 16;
  return align_up(static_cast<size_t>(n) * sizeof(asr::DevTensor) +
                      (static_cast<size_t>(n) + asr::kGroups) * sizeof(uint32_t) +
                      asr::kGroups * per_group_pad,
                  256);
}

int chunk_shift_for(int64_t total) {
  int s = asr::kMinChunkShift;
  while (s < asr::kMaxChunkShift && ((total + (int64_t{1} << s) - 1) >> s) > asr::kTargetChunks)
    ++s;
  return s;
}

hipError_t launch_group(int group, int rounding, const asr::DevTensor* d_tensors,
                        const uint32_t* d_begin, int32_t n, uint32_t n_chunks,
                        int32_t shift, const asr::Coeffs& c, uint32_t seed,
                        uint32_t step, hipStream_t stream) {
  const uint32_t grid = std::min(n_chunks, asr::kMaxGrid);
  using asr::BF16;
  using asr::F32;
  using K = void (*)(const asr::DevTensor*, const uint32_t*, int32_t, uint32_t, int32_t,
                     asr::Coeffs, uint32_t, uint32_t);
  K k = nullptr;
  const bool sr = rounding == ASR_ROUND_SR;
  switch (group) {
    case ASR_F32 * 2 + ASR_F32: k = asr::adamw_sr_multi_tensor<F32, F32, asr::kRoundSR>; break;
    case ASR_F32 * 2 + ASR_BF16: k = asr::adamw_sr_multi_tensor<F32, BF16, asr::kRoundSR>; break;
    case ASR_BF16 * 2 + ASR_F32:
      k = sr ? asr::adamw_sr_multi_tensor<BF16, F32, asr::kRoundSR>
             : asr::adamw_sr_multi_tensor<BF16, F32, asr::kRoundRN>;
      break;
    default:
      k = sr ? asr::adamw_sr_multi_tensor<BF16, BF16, asr::kRoundSR>
             : asr::adamw_sr_multi_tensor<BF16, BF16, asr::kRoundRN>;
      break;
  }
  return launch(k, grid, stream, d_tensors, d_begin, n, n_chunks, shift, c, seed, step);
}

}  // namespace

extern "C" {

int asr_abi_version(void) { return ASR_ABI_VERSION; }

const char* asr_last_error(void) { return g_last_error.c_str(); }

size_t asr_adamw_workspace_bytes(int32_t n_tensors) { return workspace_bound(n_tensors); }

int asr_adamw_host_scalars(double lr, double beta1, double beta2, double eps,
                           double weight_decay, int64_t step, float* out) {
  if (int s = check_hparams(lr, beta1, beta2, eps, weight_decay, step)) return s;
  if (!out) return fail(ASR_EINVAL, "out is NULL");
  const asr::Coeffs c = make_coeffs(lr, beta1, beta2, eps, weight_decay, step);
  const float vals[8] = {c.decay, c.b1, c.omb1, c.b2, c.omb2, c.step_size, c.inv_bc2_sqrt, c.eps};
  std::memcpy(out, vals, sizeof(vals));
  return ok();
}

int asr_adamw_step(const asr_tensor* tensors, int32_t n_tensors, double lr, double beta1,
                   double beta2, double eps, double weight_decay, int64_t step,
                   uint32_t seed, int32_t rounding, void* workspace,
                   size_t workspace_bytes, void* stream_ptr) {
  if (n_tensors < 0) return fail(ASR_EINVAL, "n_tensors < 0");
  if (n_tensors > 0 && !tensors) return fail(ASR_EINVAL, "tensors is NULL");
  if (int s = check_hparams(lr, beta1, beta2, eps, weight_decay, step)) return s;
  if (rounding != ASR_ROUND_SR && rounding != ASR_ROUND_RN)
    return fail(ASR_EINVAL, "rounding must be ASR_ROUND_SR or ASR_ROUND_RN");

  // Validate and sort into dtype groups; drop empty tensors.
  std::vector<asr::DevTensor> group[asr::kGroups];
  int64_t group_elems[asr::kGroups] = {0, 0, 0, 0};
  for (int32_t i = 0; i < n_tensors; ++i) {
    const asr_tensor& t = tensors[i];
    const std::string at = "tensor " + std::to_string(i) + ": ";
    if (t.numel < 0) return fail(ASR_EINVAL, at + "numel < 0");
    if ((t.param_dtype != ASR_F32 && t.param_dtype != ASR_BF16) ||
        (t.grad_dtype != ASR_F32 && t.grad_dtype != ASR_BF16))
      return fail(ASR_EDTYPE, at + "dtype code must be ASR_F32 or ASR_BF16");
    if (t.numel == 0) continue;
    if (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq)
      return fail(ASR_EINVAL, at + "NULL buffer");
    const uintptr_t pa = t.param_dtype == ASR_F32 ? 4 : 2;
    const uintptr_t ga = t.grad_dtype == ASR_F32 ? 4 : 2;
    if (!aligned(t.param, pa) || !aligned(t.grad, ga) || !aligned(t.exp_avg, 4) ||
        !aligned(t.exp_avg_sq, 4))
      return fail(ASR_EALIGN, at + "buffer not aligned to its element size");
    const int g = t.param_dtype * 2 + t.grad_dtype;
    asr::DevTensor d;
    d.param = t.param;
    d.grad = t.grad;
    d.m = t.exp_avg;
    d.v = t.exp_avg_sq;
    d.numel = t.numel;
    d.base_index = t.base_index;
    d.vec_ok = aligned(t.param, 16) && aligned(t.grad, 16) && aligned(t.exp_avg, 16) &&
               aligned(t.exp_avg_sq, 16);
    d.reserved = 0;
    group[g].push_back(d);
    group_elems[g] += t.numel;
    if (group_elems[g] > (int64_t{1} << 47))
      return fail(ASR_EINVAL, "more than 2**47 elements of one dtype pair");
  }
  int64_t total = 0;
  for (int g = 0; g < asr::kGroups; ++g) total += group_elems[g];
  if (total == 0) return ok();

  const size_t need = workspace_bound(n_tensors);
  if (!workspace || workspace_bytes < need)
    return fail(ASR_EWORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (!aligned(workspace, 16)) return fail(ASR_EWORKSPACE, "workspace not 16-byte aligned");

  const int shift = chunk_shift_for(total);
  const asr::Coeffs c = make_coeffs(lr, beta1, beta2, eps, weight_decay, step);

  // Build the host image of the table.
  std::vector<uint8_t> image(need, 0);
  size_t off = 0;
  size_t tensors_off[asr::kGroups], begin_off[asr::kGroups];
  uint32_t n_chunks[asr::kGroups] = {0, 0, 0, 0};
  for (int g = 0; g < asr::kGroups; ++g) {
    if (group[g].empty()) continue;
    off = align_up(off, 16);
    tensors_off[g] = off;
    std::memcpy(image.data() + off, group[g].data(), group[g].size() * sizeof(asr::DevTensor));
    off += group[g].size() * sizeof(asr::DevTensor);
    off = align_up(off, 16);
    begin_off[g] = off;
    uint64_t chunks = 0;
    for (size_t k = 0; k <= group[g].size(); ++k) {
      const uint32_t b = static_cast<uint32_t>(chunks);
      std::memcpy(image.data() + off + k * sizeof(uint32_t), &b, sizeof(b));
      if (k < group[g].size())
        chunks += (static_cast<uint64_t>(group[g][k].numel) + (uint64_t{1} << shift) - 1) >> shift;
    }
    n_chunks[g] = static_cast<uint32_t>(chunks);
    off += (group[g].size() + 1) * sizeof(uint32_t);
  }

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t used = align_up(off, sizeof(uint32_t));
  for (size_t pos = 0; pos < used; pos += asr::kUploadWords * sizeof(uint32_t)) {
    asr::UploadBlock blk;
    const size_t bytes = std::min(used - pos, sizeof(blk.w));
    std::memset(blk.w, 0, sizeof(blk.w));
    std::memcpy(blk.w, image.data() + pos, bytes);
    hipError_t e = launch(asr::upload_words, 1, stream, blk,
                          reinterpret_cast<uint32_t*>(ws + pos),
                          static_cast<uint32_t>(bytes / sizeof(uint32_t)));
    if (e != hipSuccess) return hip_fail(e, "metadata upload launch");
  }
  for (int g = 0; g < asr::kGroups; ++g) {
    if (group[g].empty()) continue;
    hipError_t e = launch_group(
        g, rounding, reinterpret_cast<const asr::DevTensor*>(ws + tensors_off[g]),
        reinterpret_cast<const uint32_t*>(ws + begin_off[g]),
        static_cast<int32_t>(group[g].size()), n_chunks[g], shift, c, seed,
        static_cast<uint32_t>(step), stream);
    if (e != hipSuccess) return hip_fail(e, "adamw kernel launch");
  }
  return ok();
}

int asr_philox_4x32_fill(uint32_t* out, int64_t n_counters, uint64_t counter_base,
                         uint64_t counter_upper, uint32_t seed, uint32_t step,
                         void* stream_ptr) {
  if (n_counters < 0) return fail(ASR_EINVAL, "n_counters < 0");
  if (n_counters == 0) return ok();
  if (!out) return fail(ASR_EINVAL, "out is NULL");
  if (!aligned(out, 4)) return fail(ASR_EALIGN, "out not 4-byte aligned");
  if (n_counters > (int64_t{1} << 61)) return fail(ASR_EINVAL, "n_counters too large");
  const int64_t blocks = (n_counters + asr::kBlock - 1) / asr::kBlock;
  const uint32_t grid = static_cast<uint32_t>(std::min<int64_t>(blocks, 1 << 16));
  hipError_t e = launch(asr::philox_fill, grid, static_cast<hipStream_t>(stream_ptr), out,
                        n_counters, counter_base, static_cast<uint32_t>(counter_upper),
                        static_cast<uint32_t>(counter_upper >> 32), seed, step,
                        static_cast<int>(aligned(out, 16)));
  if (e != hipSuccess) return hip_fail(e, "philox fill launch");
  return ok();
}

static int convert(int rounding, const float* in, uint16_t* out, int64_t n, uint32_t seed,
                   uint32_t step, uint64_t base_index, void* stream_ptr) {
  if (n < 0) return fail(ASR_EINVAL, "n < 0");
  if (n == 0) return ok();
  if (!in || !out) return fail(ASR_EINVAL, "NULL buffer");
  if (!aligned(in, 4) || !aligned(out, 2))
    return fail(ASR_EALIGN, "buffer not aligned to its element size");
  if (n > (int64_t{1} << 62)) return fail(ASR_EINVAL, "n too large");
  const int64_t blocks = (n + asr::kBlock * asr::kVec - 1) / (asr::kBlock * asr::kVec);
  const uint32_t grid = static_cast<uint32_t>(std::min<int64_t>(blocks, 1 << 16));
  const int vec_ok = aligned(in, 16) && aligned(out, 16);
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  hipError_t e =
      rounding == ASR_ROUND_SR
          ? launch(asr::convert_f32_bf16<asr::kRoundSR>, grid, stream, in, out, n, base_index,
                   seed, step, vec_ok)
          : launch(asr::convert_f32_bf16<asr::kRoundRN>, grid, stream, in, out, n, base_index,
                   seed, step, vec_ok);
  if (e != hipSuccess) return hip_fail(e, "convert launch");
  return ok();
}

int asr_cvt_f32_bf16_sr(const float* in, uint16_t* out, int64_t n, uint32_t seed,
                        uint32_t step, uint64_t base_index, void* stream) {
  return convert(ASR_ROUND_SR, in, out, n, seed, step, base_index, stream);
}

int asr_cvt_f32_bf16_rn(const float* in, uint16_t* out, int64_t n, void* stream) {
  return convert(ASR_ROUND_RN, in, out, n, 0, 0, 0, stream);
}

int asr_f32_sqrt_div(const float* a, const float* b, float* sqrt_out, float* div_out,
                     int64_t n, void* stream_ptr) {
  if (n < 0) return fail(ASR_EINVAL, "n < 0");
  if (n == 0) return ok();
  if (!a || !b || !sqrt_out || !div_out) return fail(ASR_EINVAL, "NULL buffer");
  if (!aligned(a, 4) || !aligned(b, 4) || !aligned(sqrt_out, 4) || !aligned(div_out, 4))
    return fail(ASR_EALIGN, "buffer not 4-byte aligned");
  const int64_t blocks = (n + asr::kBlock - 1) / asr::kBlock;
  const uint32_t grid = static_cast<uint32_t>(std::min<int64_t>(blocks, 1 << 16));
  hipError_t e = launch(asr::sqrt_div, grid, static_cast<hipStream_t>(stream_ptr), a, b,
                        sqrt_out, div_out, n);
  if (e != hipSuccess) return hip_fail(e, "sqrt/div launch");
  return ok();
}

}  // extern "C"

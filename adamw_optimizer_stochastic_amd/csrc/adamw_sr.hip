// Kernels and C ABI of the fused AdamW step with stochastic-rounding bf16
// write-back, for gfx950 (MI355X). The ABI is declared and documented in
// include/adamw_sr.h.
//
// Sources (pages cited by title and section):
//   "adamw-sr" (kernels hub page): intro (decoupled-weight-decay Adam step,
//     unbiased bf16 write-back, no fp32 master), Usage (drop-in for
//     torch.optim.AdamW; f32 states; f32|bf16 params and grads), Method
//     (Philox keyed by (seed, step), indexed by global element position),
//     Correctness (shards that pass their own base_index reproduce the
//     one-piece update bit for bit).
//   "Add stochastic rounding and philox RNG helpers" (FlyDSL pull request):
//     Primitives (Philox words, add-and-truncate SR), discussion (SR as a
//     rounding mode of the f32 -> bf16 conversion).
//
// Design for the hardware: the step is a pure stream (22 bytes per bf16
// element, each byte read or written once), so the kernels are built around
// HBM bandwidth: vector loads and stores of 4 elements per lane (128-bit for
// f32, 64-bit for bf16), Philox in registers with one call per 4 consecutive
// positions (no generator state in memory), no LDS and no matrix cores.
// Every workgroup takes one slot of 1,024 elements and exits (no loop); the
// slots of a launch are spread over four address windows (XCDs x and x + 4
// share window x), and a residency cap (LDS reservation) keeps about 24 KiB
// in flight per CU. Tensors of equal size share a launch and find their
// tensor by a multiply-high division of the slot index; the rest use a
// slot-to-tensor table (built on the host when small, else filled on the
// device), so one call covers thousands of tensors. A list of at most 48
// tensors per launch passes its descriptors in the kernel arguments.
#include "device.hpp"
#include "status.hpp"

#include <adamw_sr.h>

#include <algorithm>
#include <map>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>
#include <type_traits>
#include <vector>

#pragma clang fp contract(off)

namespace asr {

constexpr int kBlock = 256;            // threads per workgroup of the helper kernels
// Threads per workgroup of the streaming kernels (the step, its traffic
// probe and the copy/read/write probes).
#ifndef ASR_STEP_BLOCK
#define ASR_STEP_BLOCK 256
#endif
constexpr int kStepBlock = ASR_STEP_BLOCK;
#ifndef ASR_VEC
#define ASR_VEC 4
#endif
constexpr int kVec = ASR_VEC;          // elements per lane of the step kernel
#ifndef ASR_CVT_VEC
#define ASR_CVT_VEC 8
#endif
constexpr int kCvtVec = ASR_CVT_VEC;   // elements per lane of the converts
constexpr int64_t kCvtSlot = kBlock * kCvtVec;
#ifndef ASR_CVT_BLOCKS_PER_CU
#define ASR_CVT_BLOCKS_PER_CU 6
#endif
constexpr int kCvtBlocksPerCU = ASR_CVT_BLOCKS_PER_CU;
constexpr int64_t kSlot = kStepBlock * kVec;  // elements per workgroup of the step kernel
// Blocks per launch; a larger list is covered by several launches.
constexpr uint32_t kMaxGrid = 1u << 23;
// Resident workgroups per CU for the step kernel. The path is bound by HBM
// with seven concurrent streams (four read, three written); measured on
// MI355X, the DRAM works best when the whole chip moves through one narrow
// window of addresses with about 24 KiB of loads in flight per CU, and four
// resident 4-element-per-lane workgroups keep that while hiding each slot's
// arithmetic (about 6.1 TB/s on a single large tensor, against 5.2 TB/s with
// the CU filled). The cap is applied by reserving LDS at launch (160 KiB per
// CU on gfx950); the kernel itself uses none.
#ifndef ASR_BLOCKS_PER_CU
#define ASR_BLOCKS_PER_CU 4
#endif
constexpr int kBlocksPerCU = ASR_BLOCKS_PER_CU;
constexpr uint32_t kLdsPerCU = 160u * 1024u;
constexpr bool kNonTemporal = false;   // streaming hints measured slower here
constexpr int kGroups = 4;             // (param dtype, grad dtype) pairs
constexpr int kUploadWords = 768;      // 3 KiB of metadata per upload launch

// Per-tensor metadata as the kernel reads it from the workspace.
struct DevTensor {
  void* param;
  const void* grad;
  float* m;
  float* v;
  int64_t numel;
  uint64_t base_index;
  // The tensor is walked in runs of kVec elements; run r covers elements
  // kVec*r - shift .. kVec*r - shift + kVec - 1, so the first run may start
  // before element 0 (its leading lanes then touch nothing). shift is chosen
  // so that every run starts on a vector-aligned address of all four
  // buffers (16 bytes for f32, 2*kVec bytes for bf16); vec_ok says such a
  // shift exists, else (buffers misaligned against each other) every
  // element moves on its own and shift is 0. Both sit in one 32-bit word
  // (bit 0: vec_ok, bits 8..15: shift) so that the descriptor is read with
  // scalar loads only (a sub-word field would be read with a vector load
  // that every lane then waits for).
  uint32_t runs;
  uint32_t first_slot;  // index of the tensor's first slot within its group
  __device__ __host__ bool vec_ok() const { return (runs & 1u) != 0; }
  __device__ __host__ uint32_t shift() const { return (runs >> 8) & 0xFFu; }
};
static_assert(sizeof(DevTensor) == 56, "metadata layout");

enum : int { kRoundSR = ASR_ROUND_SR, kRoundRN = ASR_ROUND_RN };

// How a lane's run moves: kRunsElem element by element (buffers misaligned
// against each other); kRunsEdge with vector accesses when the whole run is
// inside the tensor, else element by element; kRunsWhole with vector
// accesses and no per-lane checks (the caller knows every run of the slot
// is whole, so the branch is uniform and the code straight-line).
enum : int { kRunsElem = 0, kRunsEdge = 1, kRunsWhole = 2 };
#ifndef ASR_WHOLE_SLOTS
#define ASR_WHOLE_SLOTS 1
#endif

// One lane's run of kVec consecutive elements i0 .. i0+kVec-1 of tensor t,
// of which lo <= e < hi lie inside the tensor (i0 < 0 only for the first run
// of a shifted tensor). Whole runs of a tensor with vec_ok start on a
// vector-aligned address of all four buffers and move with vector accesses
// (128-bit for f32; 64- or 128-bit for bf16); cut runs, and every run of a
// tensor without vec_ok, move element by element (RUNS, above).
template <class PT, class GT, int ROUND, int PHASE, int RUNS>
__device__ __forceinline__ void adamw_run(const DevTensor& t, int64_t i0, int lo, int hi,
                                           const Coeffs& c, uint32_t seed, uint32_t step) {
  using PS = typename PT::storage;
  using GS = typename GT::storage;
  PS* __restrict__ param = static_cast<PS*>(t.param);
  const GS* __restrict__ grad = static_cast<const GS*>(t.grad);
  float* __restrict__ m = t.m;
  float* __restrict__ v = t.v;
  const bool full = RUNS == kRunsWhole || (RUNS == kRunsEdge && lo == 0 && hi == kVec);
  float p[kVec], g[kVec], mm[kVec], vv[kVec];
  if (full) {
    load_vec<kNonTemporal, kVec>(param + i0, p);
    load_vec<kNonTemporal, kVec>(grad + i0, g);
    load_vec<kNonTemporal, kVec>(m + i0, mm);
    load_vec<kNonTemporal, kVec>(v + i0, vv);
  } else {
    load_range(param, i0, lo, hi, p);
    load_range(grad, i0, lo, hi, g);
    load_range(m, i0, lo, hi, mm);
    load_range(v, i0, lo, hi, vv);
  }
#pragma unroll
  for (int e = 0; e < kVec; ++e) adamw_update(p[e], g[e], mm[e], vv[e], c);

  if constexpr (std::is_same_v<PT, F32>) {
    if (full) store_vec<kNonTemporal, kVec>(param + i0, p);
    else store_range(param, i0, lo, hi, p);
  } else {
    uint32_t h[kVec];
    if constexpr (ROUND == kRoundSR) {
      uint32_t r[kVec];
      stream_bits<PHASE, kVec>(t.base_index + static_cast<uint64_t>(i0), seed, step, r);
#pragma unroll
      for (int e = 0; e < kVec; ++e) h[e] = round_sr(__float_as_uint(p[e]), r[e]);
    } else {
#pragma unroll
      for (int e = 0; e < kVec; ++e) h[e] = round_rn(__float_as_uint(p[e]));
    }
    if (full) store_vec_bf16<kNonTemporal, kVec>(param + i0, h);
    else store_range_bf16(param, i0, lo, hi, h);
  }
  if (full) {
    store_vec<kNonTemporal, kVec>(m + i0, mm);
    store_vec<kNonTemporal, kVec>(v + i0, vv);
  } else {
    store_range(m, i0, lo, hi, mm);
    store_range(v, i0, lo, hi, vv);
  }
}

// The phase of a run's first position within its Philox call, (base_index
// + i0) & 3, is the same for every run of a tensor: (base_index - shift) & 3.
template <class PT, class GT, int ROUND, int RUNS>
__device__ __forceinline__ void adamw_run_phase(const DevTensor& t, int64_t i0, int lo, int hi,
                                                 const Coeffs& c, uint32_t seed, uint32_t step) {
  if constexpr (std::is_same_v<PT, BF16> && ROUND == kRoundSR) {
    switch (static_cast<int>((t.base_index - t.shift()) & 3u)) {
      case 0: adamw_run<PT, GT, ROUND, 0, RUNS>(t, i0, lo, hi, c, seed, step); break;
      case 1: adamw_run<PT, GT, ROUND, 1, RUNS>(t, i0, lo, hi, c, seed, step); break;
      case 2: adamw_run<PT, GT, ROUND, 2, RUNS>(t, i0, lo, hi, c, seed, step); break;
      default: adamw_run<PT, GT, ROUND, 3, RUNS>(t, i0, lo, hi, c, seed, step); break;
    }
  } else {
    adamw_run<PT, GT, ROUND, 0, RUNS>(t, i0, lo, hi, c, seed, step);
  }
}

// Slot `local` (kSlot elements) of tensor t: one kVec-element run per lane.
// A slot whose runs all lie inside a vector-aligned tensor (every slot but
// the first and last of a tensor) takes the straight-line vector path; at
// the ends, lanes past either end get an empty range and touch nothing (no
// early exit, so the whole descriptor is fetched in one round).
template <class PT, class GT, int ROUND>
__device__ __forceinline__ void adamw_slot(const DevTensor& t, uint32_t local, const Coeffs& c,
                                           uint32_t seed, uint32_t step) {
  const int64_t s0 = static_cast<int64_t>(local) * kSlot - static_cast<int64_t>(t.shift());
  const int64_t i0 = s0 + static_cast<int64_t>(threadIdx.x) * kVec;
  if (ASR_WHOLE_SLOTS && t.vec_ok() && s0 >= 0 && s0 + kSlot <= t.numel) {
    adamw_run_phase<PT, GT, ROUND, kRunsWhole>(t, i0, 0, kVec, c, seed, step);
    return;
  }
  const int64_t left = t.numel - i0;
  const int hi = left <= 0 ? 0 : (left < kVec ? static_cast<int>(left) : kVec);
  const int lo = i0 < 0 ? static_cast<int>(-i0) : 0;
  if (t.vec_ok()) adamw_run_phase<PT, GT, ROUND, kRunsEdge>(t, i0, lo, hi, c, seed, step);
  else adamw_run_phase<PT, GT, ROUND, kRunsElem>(t, i0, lo, hi, c, seed, step);
}

// The multi-tensor step, one slot per workgroup, no loop: the workgroups in
// flight (dispatched in order) sweep the memory as one narrow window. All
// descriptor reads come before any store and have uniform addresses, so they
// are scalar loads.
//
// Size-class form: every tensor of the launch has the same numel, so slot s
// belongs to tensor s / slots_per_tensor. The quotient is taken as the high
// half of s * magic, magic = floor((2**32 - 1) / slots_per_tensor), which
// falls short of the true quotient by at most one (s < 2**32), then
// corrected; the descriptor table is small and stays in the scalar cache.
#ifndef ASR_WINDOWS
#define ASR_WINDOWS 4
#endif
// Workgroup -> slot. MI355X hands workgroups to its 8 XCDs round-robin in
// dispatch order. With kWindows windows, workgroup b takes the next slot of
// window b % kWindows, a contiguous 1/kWindows of the launch; with 4, XCDs x
// and x + 4 share window x. Several windows instead of one average the DRAM
// bank/channel conflicts between the seven streams over unrelated sets of
// physical pages (5.33 to 6.28 TB/s across buffer placements with one
// window); measured on the Llama-3-8B list in three processes, alternating
// builds: 1, 2, 4, 8 and 16 windows gave 5.61-5.76, 5.83-5.98, 5.85-6.12,
// 5.67-5.97 and 5.38-5.63 TB/s. Any bijection is correct; this only changes
// the order of work.
constexpr uint32_t kWindows = ASR_WINDOWS;
// The plain copy, read and write streams measured best with one window per
// XCD (8); they keep that.
constexpr uint32_t kCopyWindows = 8;
template <uint32_t W = kWindows>
__device__ __forceinline__ uint32_t slot_of_block(uint32_t b, uint32_t grid) {
  if constexpr (W > 1) {
    const uint32_t w = b % W, k = b / W;
    const uint32_t q = grid / W, r = grid % W;
    return w * q + (w < r ? w : r) + k;
  } else {
    (void)grid;
    return b;
  }
}

template <class PT, class GT, int ROUND>
__global__ void __launch_bounds__(kStepBlock)
adamw_sr_class(const DevTensor* __restrict__ tensors, uint32_t slots_per_tensor, uint32_t magic,
               uint32_t slot0, Coeffs c, uint32_t seed, uint32_t step) {
  const uint32_t slot = slot0 + slot_of_block(blockIdx.x, gridDim.x);
  uint32_t ti = __umulhi(slot, magic);
  if (static_cast<uint64_t>(ti + 1) * slots_per_tensor <= slot) ++ti;
  const DevTensor t = tensors[ti];
  adamw_slot<PT, GT, ROUND>(t, slot - ti * slots_per_tensor, c, seed, step);
}

// Inline form, for lists of at most kInlineTensors tensors per launch: the
// descriptors travel in the kernel arguments, so a small step needs neither
// an upload launch nor a slot table. A workgroup finds its tensor as the
// class form does (equal sizes: a multiply-high division), or else by a
// binary search of the first slots (at most 6 probes); both are
// wave-uniform, on scalar loads from the kernel-argument segment.
#ifndef ASR_INLINE_TENSORS
#define ASR_INLINE_TENSORS 48
#endif
constexpr int kInlineTensors = ASR_INLINE_TENSORS;
struct InlineTensors {
  DevTensor t[kInlineTensors > 0 ? kInlineTensors : 1];  // first_slot ascending from 0
  uint32_t n;
  uint32_t per, magic;  // size class: slots per tensor and its magic; per = 0: any sizes
};

__device__ __forceinline__ uint32_t inline_tensor(const InlineTensors& L, uint32_t slot) {
  if (L.per != 0) {
    uint32_t ti = __umulhi(slot, L.magic);
    if (static_cast<uint64_t>(ti + 1) * L.per <= slot) ++ti;
    return ti;
  }
  uint32_t lo = 0, hi = L.n - 1;  // the last k with t[k].first_slot <= slot
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) >> 1;
    if (L.t[mid].first_slot <= slot) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <class PT, class GT, int ROUND>
__global__ void __launch_bounds__(kStepBlock)
adamw_sr_inline(const InlineTensors L, uint32_t slot0, Coeffs c, uint32_t seed, uint32_t step) {
  const uint32_t slot = slot0 + slot_of_block(blockIdx.x, gridDim.x);
  const DevTensor t = L.t[inline_tensor(L, slot)];
  adamw_slot<PT, GT, ROUND>(t, slot - t.first_slot, c, seed, step);
}

// Table form, for tensors of any sizes: slot_tensor[s] names the tensor of
// slot s (filled on the device from the tensors' first slots).
template <class PT, class GT, int ROUND>
__global__ void __launch_bounds__(kStepBlock)
adamw_sr_slots(const DevTensor* __restrict__ tensors, const uint32_t* __restrict__ slot_tensor,
               uint32_t slot0, Coeffs c, uint32_t seed, uint32_t step) {
  const uint32_t slot = slot0 + slot_of_block(blockIdx.x, gridDim.x);
  const DevTensor t = tensors[slot_tensor[slot]];
  adamw_slot<PT, GT, ROUND>(t, slot - t.first_slot, c, seed, step);
}

// slot_tensor[s] = the last k with first_slot[k] <= s (first_slot ascending,
// first_slot[0] = 0, every tensor at least one slot).
__global__ void __launch_bounds__(kBlock)
fill_slot_table(const uint32_t* __restrict__ first_slot, int32_t n_tensors,
                uint32_t* __restrict__ slot_tensor, uint32_t n_slots) {
  const uint32_t stride = gridDim.x * kBlock;
  for (uint32_t s = blockIdx.x * kBlock + threadIdx.x; s < n_slots; s += stride) {
    int32_t lo = 0, hi = n_tensors - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (first_slot[mid] <= s) lo = mid;
      else hi = mid - 1;
    }
    slot_tensor[s] = static_cast<uint32_t>(lo);
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

// Device workspace of the allocation-free step (see asr_adamw_step_noalloc):
// 4 MiB, one copy per GPU.
constexpr size_t kScratchBytes = size_t{4} << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

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
// One lane's run of kCvtVec elements i0 .. of the conversion, of which
// lo <= e < hi lie inside the array (i0 < 0 only for the first run when the
// runs are shifted, as for the step).
template <int ROUND, int PHASE, bool VEC>
__device__ __forceinline__ void convert_run(const float* __restrict__ in,
                                            uint16_t* __restrict__ out, int64_t i0, int lo, int hi,
                                            uint64_t base_index, uint32_t seed, uint32_t step) {
  constexpr int V = kCvtVec;
  const bool full = VEC && lo == 0 && hi == V;
  float x[V];
  if (full) load_vec<kNonTemporal, V>(in + i0, x);
  else load_range(in, i0, lo, hi, x);
  uint32_t h[V];
  if constexpr (ROUND == kRoundSR) {
    uint32_t r[V];
    stream_bits<PHASE, V>(base_index + static_cast<uint64_t>(i0), seed, step, r);
#pragma unroll
    for (int e = 0; e < V; ++e) h[e] = round_sr(__float_as_uint(x[e]), r[e]);
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) h[e] = round_rn(__float_as_uint(x[e]));
  }
  if (full) store_vec_bf16<kNonTemporal, V>(out + i0, h);
  else store_range_bf16(out, i0, lo, hi, h);
}

#ifndef ASR_CVT_WINDOWS
#define ASR_CVT_WINDOWS 8
#endif
// One window per XCD and six resident workgroups per CU measured best for
// the conversion (6.13-6.15 TB/s on 2**30 elements against 5.74-6.06 for
// one window at four to eight workgroups).
constexpr uint32_t kCvtWindows = ASR_CVT_WINDOWS;
__device__ __forceinline__ uint32_t cvt_slot_of_block(uint32_t b, uint32_t grid) {
  if constexpr (kCvtWindows > 1) {
    const uint32_t w = b % kCvtWindows, k = b / kCvtWindows;
    const uint32_t q = grid / kCvtWindows, r = grid % kCvtWindows;
    return w * q + (w < r ? w : r) + k;
  } else {
    (void)grid;
    return b;
  }
}

// One slot of kCvtSlot elements per workgroup, no loop (as for the step).
// shift: elements the runs start before in[0] (the first run's leading
// lanes touch nothing), chosen so that whole runs are vector-aligned in both
// buffers; vec_ok says such a shift exists (else shift is 0 and every
// element moves on its own).
template <int ROUND>
__global__ void __launch_bounds__(kBlock)
convert_f32_bf16(const float* __restrict__ in, uint16_t* __restrict__ out, int64_t n,
                 uint64_t slot0, uint64_t base_index, uint32_t seed, uint32_t step, int vec_ok,
                 int shift) {
  const int64_t i0 = static_cast<int64_t>(slot0 + cvt_slot_of_block(blockIdx.x, gridDim.x)) * kCvtSlot +
                     static_cast<int64_t>(threadIdx.x) * kCvtVec - shift;
  const int64_t left = n - i0;
  const int hi = left <= 0 ? 0 : (left < kCvtVec ? static_cast<int>(left) : kCvtVec);
  const int lo = i0 < 0 ? static_cast<int>(-i0) : 0;
  if constexpr (ROUND == kRoundSR) {
    const int phase = static_cast<int>((base_index - static_cast<uint64_t>(shift)) & 3u);
    if (vec_ok) {
      switch (phase) {
        case 0: convert_run<ROUND, 0, true>(in, out, i0, lo, hi, base_index, seed, step); break;
        case 1: convert_run<ROUND, 1, true>(in, out, i0, lo, hi, base_index, seed, step); break;
        case 2: convert_run<ROUND, 2, true>(in, out, i0, lo, hi, base_index, seed, step); break;
        default: convert_run<ROUND, 3, true>(in, out, i0, lo, hi, base_index, seed, step); break;
      }
    } else {
      switch (phase) {
        case 0: convert_run<ROUND, 0, false>(in, out, i0, lo, hi, base_index, seed, step); break;
        case 1: convert_run<ROUND, 1, false>(in, out, i0, lo, hi, base_index, seed, step); break;
        case 2: convert_run<ROUND, 2, false>(in, out, i0, lo, hi, base_index, seed, step); break;
        default: convert_run<ROUND, 3, false>(in, out, i0, lo, hi, base_index, seed, step); break;
      }
    }
  } else {
    if (vec_ok) convert_run<ROUND, 0, true>(in, out, i0, lo, hi, base_index, seed, step);
    else convert_run<ROUND, 0, false>(in, out, i0, lo, hi, base_index, seed, step);
  }
}

// ------------------------------------------------- measurement: a copy
// A plain copy built like the step: one slot of kStepBlock lanes x 4 x 16
// bytes per workgroup, no loop, 128-bit loads and stores, the step's
// residency cap, and one address window per XCD (the copy's best; the step
// itself runs best on 4). It measures what this launch structure gets from
// HBM for a 1:1 read/write stream, the reference the step's bandwidth is
// also quoted against.
constexpr int kCopyVec = 4;  // 16-byte units per lane, one wave-wide 1 KiB access each
__global__ void __launch_bounds__(kStepBlock)
stream_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, uint64_t n16,
            uint64_t slot0) {
  const uint64_t base = (slot0 + slot_of_block<kCopyWindows>(blockIdx.x, gridDim.x)) * (kStepBlock * kCopyVec) +
                        threadIdx.x;
  u32x4 x[kCopyVec];
#pragma unroll
  for (int k = 0; k < kCopyVec; ++k)
    if (base + k * kStepBlock < n16) x[k] = src[base + k * kStepBlock];
#pragma unroll
  for (int k = 0; k < kCopyVec; ++k)
    if (base + k * kStepBlock < n16) dst[base + k * kStepBlock] = x[k];
}

// A read-only and a write-only stream in the copy's form (one 16 KiB slot
// per workgroup, windows, residency cap). The read keeps its loads alive by
// XOR-ing them and storing the result to sink[0] only if it equals a value
// that a buffer of equal 16-byte words (the benchmark fills it so) cannot
// give, so it moves no bytes to memory.
__global__ void __launch_bounds__(kStepBlock)
stream_read(const u32x4* __restrict__ src, u32x4* __restrict__ sink, uint64_t n16,
            uint64_t slot0) {
  const uint64_t base = (slot0 + slot_of_block<kCopyWindows>(blockIdx.x, gridDim.x)) * (kStepBlock * kCopyVec) +
                        threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < kCopyVec; ++k)
    if (base + k * kStepBlock < n16) acc ^= src[base + k * kStepBlock];
  if (acc.x == 0x9E3779B9u && acc.y == 0xBB67AE85u && acc.z == 0xD2511F53u &&
      acc.w == 0xCD9E8D57u)
    sink[0] = acc;
}

__global__ void __launch_bounds__(kStepBlock)
stream_write(u32x4* __restrict__ dst, uint64_t n16, uint64_t slot0, uint32_t value) {
  const uint64_t base = (slot0 + slot_of_block<kCopyWindows>(blockIdx.x, gridDim.x)) * (kStepBlock * kCopyVec) +
                        threadIdx.x;
  const u32x4 x = {value, value, value, value};
#pragma unroll
  for (int k = 0; k < kCopyVec; ++k)
    if (base + k * kStepBlock < n16) dst[base + k * kStepBlock] = x;
}

// The step's memory traffic with its arithmetic taken out: the same runs,
// vector and element accesses, slots, windows and residency cap as
// adamw_run, but the new parameter is the old one XOR the gradient (the
// high halves, for a bf16 parameter) and m and v are written back as read.
// It measures what HBM gives this access pattern (four streams read, three
// written) under the step's launch structure; the benchmark reports it
// beside the step.
template <class PT, class GT, int RUNS>
__device__ __forceinline__ void probe_run(const DevTensor& t, int64_t i0, int lo, int hi) {
  using PS = typename PT::storage;
  using GS = typename GT::storage;
  PS* __restrict__ param = static_cast<PS*>(t.param);
  const GS* __restrict__ grad = static_cast<const GS*>(t.grad);
  float* __restrict__ m = t.m;
  float* __restrict__ v = t.v;
  const bool full = RUNS == kRunsWhole || (RUNS == kRunsEdge && lo == 0 && hi == kVec);
  float p[kVec], g[kVec], mm[kVec], vv[kVec];
  if (full) {
    load_vec<kNonTemporal, kVec>(param + i0, p);
    load_vec<kNonTemporal, kVec>(grad + i0, g);
    load_vec<kNonTemporal, kVec>(m + i0, mm);
    load_vec<kNonTemporal, kVec>(v + i0, vv);
  } else {
    load_range(param, i0, lo, hi, p);
    load_range(grad, i0, lo, hi, g);
    load_range(m, i0, lo, hi, mm);
    load_range(v, i0, lo, hi, vv);
  }
#pragma unroll
  for (int e = 0; e < kVec; ++e) p[e] = __uint_as_float(__float_as_uint(p[e]) ^ __float_as_uint(g[e]));
  if constexpr (std::is_same_v<PT, F32>) {
    if (full) store_vec<kNonTemporal, kVec>(param + i0, p);
    else store_range(param, i0, lo, hi, p);
  } else {
    uint32_t h[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) h[e] = __float_as_uint(p[e]) >> 16;
    if (full) store_vec_bf16<kNonTemporal, kVec>(param + i0, h);
    else store_range_bf16(param, i0, lo, hi, h);
  }
  if (full) {
    store_vec<kNonTemporal, kVec>(m + i0, mm);
    store_vec<kNonTemporal, kVec>(v + i0, vv);
  } else {
    store_range(m, i0, lo, hi, mm);
    store_range(v, i0, lo, hi, vv);
  }
}

template <class PT, class GT>
__device__ __forceinline__ void probe_slot(const DevTensor& t, uint32_t local) {
  const int64_t s0 = static_cast<int64_t>(local) * kSlot - static_cast<int64_t>(t.shift());
  const int64_t i0 = s0 + static_cast<int64_t>(threadIdx.x) * kVec;
  if (ASR_WHOLE_SLOTS && t.vec_ok() && s0 >= 0 && s0 + kSlot <= t.numel) {
    probe_run<PT, GT, kRunsWhole>(t, i0, 0, kVec);
    return;
  }
  const int64_t left = t.numel - i0;
  const int hi = left <= 0 ? 0 : (left < kVec ? static_cast<int>(left) : kVec);
  const int lo = i0 < 0 ? static_cast<int>(-i0) : 0;
  if (t.vec_ok()) probe_run<PT, GT, kRunsEdge>(t, i0, lo, hi);
  else probe_run<PT, GT, kRunsElem>(t, i0, lo, hi);
}

// Launched exactly like adamw_sr_class / adamw_sr_slots (same arguments;
// the coefficients, seed and step are unused).
template <class PT, class GT>
__global__ void __launch_bounds__(kStepBlock)
stream_probe_class(const DevTensor* __restrict__ tensors, uint32_t slots_per_tensor,
                   uint32_t magic, uint32_t slot0, Coeffs, uint32_t, uint32_t) {
  const uint32_t slot = slot0 + slot_of_block(blockIdx.x, gridDim.x);
  uint32_t ti = __umulhi(slot, magic);
  if (static_cast<uint64_t>(ti + 1) * slots_per_tensor <= slot) ++ti;
  const DevTensor t = tensors[ti];
  probe_slot<PT, GT>(t, slot - ti * slots_per_tensor);
}

template <class PT, class GT>
__global__ void __launch_bounds__(kStepBlock)
stream_probe_slots(const DevTensor* __restrict__ tensors, const uint32_t* __restrict__ slot_tensor,
                   uint32_t slot0, Coeffs, uint32_t, uint32_t) {
  const uint32_t slot = slot0 + slot_of_block(blockIdx.x, gridDim.x);
  const DevTensor t = tensors[slot_tensor[slot]];
  probe_slot<PT, GT>(t, slot - t.first_slot);
}

template <class PT, class GT>
__global__ void __launch_bounds__(kStepBlock)
stream_probe_inline(const InlineTensors L, uint32_t slot0, Coeffs, uint32_t, uint32_t) {
  const uint32_t slot = slot0 + slot_of_block(blockIdx.x, gridDim.x);
  const DevTensor t = L.t[inline_tensor(L, slot)];
  probe_slot<PT, GT>(t, slot - t.first_slot);
}

// ---------------------------------------------- SR with caller's bits
// out[i] = SR(x[i], r16[i]): the rounding with its random bits supplied.
__global__ void __launch_bounds__(kBlock)
sr_given_bits(const float* __restrict__ x, const uint16_t* __restrict__ r16,
              uint16_t* __restrict__ out, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride)
    out[i] = static_cast<uint16_t>(round_sr(__float_as_uint(x[i]), r16[i]));
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
namespace asr_host {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int ok() {
  g_last_error.clear();
  return ASR_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ASR_EHIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                            hipGetErrorString(e) + ")");
}

}  // namespace asr_host

namespace {

using asr_host::fail;
using asr_host::hip_fail;
using asr_host::ok;

// Launches `kernel` with one block size for all kernels of the library;
// the arguments are converted to the kernel's parameter types first.
template <typename... KArgs, typename... Args>
hipError_t launch_lds(void (*kernel)(KArgs...), uint32_t grid, uint32_t block, uint32_t lds_bytes,
                      hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> vals(std::forward<Args>(args)...);
  return std::apply(
      [&](auto&... v) {
        void* argv[] = {static_cast<void*>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block),
                               argv, lds_bytes, stream);
      },
      vals);
}

template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), uint32_t grid, hipStream_t stream,
                  Args&&... args) {
  return launch_lds(kernel, grid, asr::kBlock, 0, stream, std::forward<Args>(args)...);
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

uint64_t slots_of(int64_t numel) {
  return (static_cast<uint64_t>(numel) + asr::kSlot - 1) / asr::kSlot;
}

// Slots of a tensor: its runs start `shift` elements before element 0.
uint64_t tensor_slots(const asr::DevTensor& d) { return slots_of(d.numel + d.shift()); }

// The most slots a tensor of this size can take, whatever its shift (the
// workspace size must not depend on where the buffers are).
uint64_t max_slots(int64_t numel) { return slots_of(numel + asr::kVec - 1); }

// Whether element s of a buffer of this dtype (and so every kVec-th element
// from there) starts a vector access: 16 bytes for f32 (one or two 128-bit
// accesses), 2*kVec bytes for bf16.
bool run_aligned(const void* p, int32_t dtype, int s) {
  const uintptr_t elem = dtype == ASR_F32 ? 4 : 2;
  const uintptr_t vec = dtype == ASR_F32 ? 16 : 2 * asr::kVec;
  return ((reinterpret_cast<uintptr_t>(p) + (asr::kVec - s) * elem) & (vec - 1)) == 0;
}

// The shift 0 <= s < kVec for which runs starting at elements k*kVec - s
// are vector-aligned in all four buffers of the tensor, or -1 (buffers
// misaligned against each other: the tensor goes element by element). A
// piece cut from aligned buffers at any element offset o has one: s =
// o mod kVec.
int vector_shift(const asr_tensor& t) {
  for (int s = 0; s < asr::kVec; ++s)
    if (run_aligned(t.param, t.param_dtype, s) && run_aligned(t.grad, t.grad_dtype, s) &&
        run_aligned(t.exp_avg, ASR_F32, s) && run_aligned(t.exp_avg_sq, ASR_F32, s))
      return s;
  return -1;
}

// A (param dtype, grad dtype) pair's tensors are launched as size classes
// (equal slot counts, at least kClassMinSlots slots in total; up to
// kMaxClassLaunches per pair) plus one table-driven launch for the rest.
constexpr uint64_t kClassMinSlots = 2048;
constexpr int kMaxClassLaunches = 64;
constexpr int kMaxLaunches = asr::kGroups * (kMaxClassLaunches + 1);

// Workspace layout: first every launch's DevTensor array and, for a table
// launch, its slot table when the host builds it (at most kHostTableSlots
// entries) or else its first_slot array, each 16-byte aligned (this prefix
// is uploaded from the host); then the slot tables filled on the device.
// A plan whose launches all take their descriptors in the kernel arguments
// uses none of it. The bound covers any split of the tensors into launches.
size_t workspace_bound(int32_t n, uint64_t total_slots) {
  if (n <= 0) return 0;
  const size_t pad = 3 * 16 * static_cast<size_t>(kMaxLaunches);
  return align_up(static_cast<size_t>(n) * sizeof(asr::DevTensor) +
                      static_cast<size_t>(n) * sizeof(uint32_t) +
                      static_cast<size_t>(total_slots) * sizeof(uint32_t) + pad,
                  256);
}

// Table launches of at most this many slots get their slot table from the
// host, inside the uploaded metadata: that never takes more launches than
// the device fill (a table of this size adds at most one upload launch and
// saves the fill launch), and a small step takes two launches instead of
// three.
constexpr uint64_t kHostTableSlots = asr::kUploadWords;

struct Launch {
  int group = 0;
  bool by_class = false;
  bool host_table = false;        // table launches: slot table uploaded with the metadata
  bool inline_desc = false;       // descriptors in the kernel arguments (adamw_sr_inline)
  std::vector<asr::DevTensor> tensors;
  uint32_t slots_per_tensor = 0;  // size-class launches
  uint64_t n_slots = 0;
  size_t tensors_off = 0, first_off = 0, table_off = 0;
};

// Splits each dtype pair into size-class launches and one table launch.
// Returns an empty string or an error message.
std::string plan_launches(const std::vector<asr::DevTensor> (&group)[asr::kGroups],
                          std::vector<Launch>* out) {
  for (int g = 0; g < asr::kGroups; ++g) {
    if (group[g].empty()) continue;
    std::map<uint64_t, std::vector<size_t>> by_slots;
    for (size_t i = 0; i < group[g].size(); ++i)
      by_slots[tensor_slots(group[g][i])].push_back(i);
    Launch rest;
    rest.group = g;
    int classes = 0;
    for (const auto& [per, idx] : by_slots) {
      const uint64_t total = per * idx.size();
      if (total >= kClassMinSlots && classes < kMaxClassLaunches) {
        if (total > 0xFFFFFFFFull) return "more than 2**32 slots of one size";
        Launch l;
        l.group = g;
        l.by_class = true;
        l.slots_per_tensor = static_cast<uint32_t>(per);
        l.n_slots = total;
        for (size_t i : idx) {
          asr::DevTensor d = group[g][i];
          d.first_slot = static_cast<uint32_t>(l.tensors.size() * per);
          l.tensors.push_back(d);
        }
        out->push_back(std::move(l));
        ++classes;
      } else {
        for (size_t i : idx) {
          asr::DevTensor d = group[g][i];
          d.first_slot = static_cast<uint32_t>(rest.n_slots);
          rest.tensors.push_back(d);
          rest.n_slots += per;  // = tensor_slots(d)
          if (rest.n_slots > 0xFFFFFFFFull) return "more than 2**32 slots of mixed sizes";
        }
      }
    }
    rest.host_table = rest.n_slots <= kHostTableSlots;
    if (!rest.tensors.empty()) out->push_back(std::move(rest));
  }
  return "";
}

using TableKernel = void (*)(const asr::DevTensor*, const uint32_t*, uint32_t, asr::Coeffs,
                             uint32_t, uint32_t);
using InlineKernel = void (*)(const asr::InlineTensors, uint32_t, asr::Coeffs, uint32_t, uint32_t);
using ClassKernel = void (*)(const asr::DevTensor*, uint32_t, uint32_t, uint32_t, asr::Coeffs,
                             uint32_t, uint32_t);

template <template <class, class, int> class Pick>
auto pick_kernel(int group, int rounding) {
  using asr::BF16;
  using asr::F32;
  const bool sr = rounding == ASR_ROUND_SR;
  switch (group) {
    case ASR_F32 * 2 + ASR_F32: return Pick<F32, F32, asr::kRoundSR>::get();
    case ASR_F32 * 2 + ASR_BF16: return Pick<F32, BF16, asr::kRoundSR>::get();
    case ASR_BF16 * 2 + ASR_F32:
      return sr ? Pick<BF16, F32, asr::kRoundSR>::get() : Pick<BF16, F32, asr::kRoundRN>::get();
    default:
      return sr ? Pick<BF16, BF16, asr::kRoundSR>::get() : Pick<BF16, BF16, asr::kRoundRN>::get();
  }
}
template <class PT, class GT, int R>
struct PickTable {
  static TableKernel get() { return asr::adamw_sr_slots<PT, GT, R>; }
};
template <class PT, class GT, int R>
struct PickClass {
  static ClassKernel get() { return asr::adamw_sr_class<PT, GT, R>; }
};
template <class PT, class GT, int R>
struct PickInline {
  static InlineKernel get() { return asr::adamw_sr_inline<PT, GT, R>; }
};
// the traffic probe of the same launch (the rounding does not apply)
template <class PT, class GT, int>
struct PickProbeTable {
  static TableKernel get() { return asr::stream_probe_slots<PT, GT>; }
};
template <class PT, class GT, int>
struct PickProbeClass {
  static ClassKernel get() { return asr::stream_probe_class<PT, GT>; }
};
template <class PT, class GT, int>
struct PickProbeInline {
  static InlineKernel get() { return asr::stream_probe_inline<PT, GT>; }
};

// LDS reserved per workgroup to hold the step kernel at kBlocksPerCU
// resident workgroups per CU (0 = no cap).
hipError_t occupancy_lds(const void* kernel, uint32_t* lds) {
  *lds = 0;
  if (asr::kBlocksPerCU <= 0) return hipSuccess;
  *lds = (asr::kLdsPerCU / asr::kBlocksPerCU) & ~1023u;
  if (*lds > 64u * 1024u)
    return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(*lds));
  return hipSuccess;
}

// One launch of the plan: (table launches) the slot table, then the step (or
// the traffic probe) in launches of at most kMaxGrid slots.
hipError_t run_launch(const Launch& l, uint8_t* ws, bool probe, int rounding,
                      const asr::Coeffs& c, uint32_t seed, uint32_t step, hipStream_t stream) {
  const auto* d_tensors = reinterpret_cast<const asr::DevTensor*>(ws + l.tensors_off);
  const uint32_t n_slots = static_cast<uint32_t>(l.n_slots);
  hipError_t e;
  uint32_t lds = 0;
  if (l.inline_desc) {
    asr::InlineTensors L{};
    std::copy(l.tensors.begin(), l.tensors.end(), L.t);
    L.n = static_cast<uint32_t>(l.tensors.size());
    L.per = l.by_class ? l.slots_per_tensor : 0;
    L.magic = l.by_class ? 0xFFFFFFFFu / l.slots_per_tensor : 0;
    const InlineKernel k = probe ? pick_kernel<PickProbeInline>(l.group, rounding)
                                 : pick_kernel<PickInline>(l.group, rounding);
    if ((e = occupancy_lds(reinterpret_cast<const void*>(k), &lds)) != hipSuccess) return e;
    for (uint32_t slot0 = 0; slot0 < n_slots; slot0 += std::min(n_slots - slot0, asr::kMaxGrid)) {
      const uint32_t grid = std::min(n_slots - slot0, asr::kMaxGrid);
      e = launch_lds(k, grid, asr::kStepBlock, lds, stream, L, slot0, c, seed, step);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (l.by_class) {
    const ClassKernel k = probe ? pick_kernel<PickProbeClass>(l.group, rounding)
                                : pick_kernel<PickClass>(l.group, rounding);
    if ((e = occupancy_lds(reinterpret_cast<const void*>(k), &lds)) != hipSuccess) return e;
    const uint32_t magic = 0xFFFFFFFFu / l.slots_per_tensor;
    for (uint32_t slot0 = 0; slot0 < n_slots; slot0 += std::min(n_slots - slot0, asr::kMaxGrid)) {
      const uint32_t grid = std::min(n_slots - slot0, asr::kMaxGrid);
      e = launch_lds(k, grid, asr::kStepBlock, lds, stream, d_tensors, l.slots_per_tensor, magic,
                     slot0, c, seed,
                     step);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  auto* d_table = reinterpret_cast<uint32_t*>(ws + l.table_off);
  if (!l.host_table) {
    const uint32_t fill_grid = std::min<uint32_t>((n_slots + asr::kBlock - 1) / asr::kBlock, 4096u);
    e = launch(asr::fill_slot_table, fill_grid, stream,
               reinterpret_cast<const uint32_t*>(ws + l.first_off),
               static_cast<int32_t>(l.tensors.size()), d_table, n_slots);
    if (e != hipSuccess) return e;
  }
  const TableKernel k = probe ? pick_kernel<PickProbeTable>(l.group, rounding)
                              : pick_kernel<PickTable>(l.group, rounding);
  if ((e = occupancy_lds(reinterpret_cast<const void*>(k), &lds)) != hipSuccess) return e;
  for (uint32_t slot0 = 0; slot0 < n_slots; slot0 += std::min(n_slots - slot0, asr::kMaxGrid)) {
    const uint32_t grid = std::min(n_slots - slot0, asr::kMaxGrid);
    e = launch_lds(k, grid, asr::kStepBlock, lds, stream, d_tensors,
                   static_cast<const uint32_t*>(d_table), slot0,
                   c, seed, step);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ------------------------------------------------------------- the plan
// What one step call enqueues: the launches and the metadata image that is
// uploaded to the front of the workspace (device-filled slot tables follow).
struct StepPlan {
  std::vector<Launch> launches;
  std::vector<uint8_t> image;  // metadata, uploaded to workspace[0, meta_bytes)
  size_t used_bytes = 0;       // workspace bytes this plan writes (metadata + tables)
  size_t bound_bytes = 0;      // asr_adamw_workspace_bytes of the list
};

// Validates the list (statuses and messages as documented for
// asr_adamw_step), groups it by dtype pair, plans the launches and lays out
// the workspace. An all-empty list gives a plan without launches.
int make_plan(const asr_tensor* tensors, int32_t n_tensors, StepPlan* plan) {
  if (n_tensors < 0) return fail(ASR_EINVAL, "n_tensors < 0");
  if (n_tensors > 0 && !tensors) return fail(ASR_EINVAL, "tensors is NULL");
  // Validate and sort into dtype groups; drop empty tensors.
  std::vector<asr::DevTensor> group[asr::kGroups];
  uint64_t group_slots[asr::kGroups] = {0, 0, 0, 0};
  uint64_t bound_slots = 0;
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
    const int shift = vector_shift(t);
    d.runs = shift >= 0 ? 1u | (static_cast<uint32_t>(shift) << 8) : 0u;
    d.first_slot = 0;  // set by the launch plan
    group[g].push_back(d);
    group_slots[g] += tensor_slots(d);
    bound_slots += max_slots(t.numel);
    if (group_slots[g] > 0xFFFFFFFFull)
      return fail(ASR_EINVAL, "more than 2**32 slots of one dtype pair");
  }
  plan->bound_bytes = workspace_bound(n_tensors, bound_slots);
  const std::string err = plan_launches(group, &plan->launches);
  if (!err.empty()) return fail(ASR_EINVAL, err);
  // A plan whose every launch fits the kernel arguments uploads nothing.
  bool all_inline = true;
  for (const Launch& l : plan->launches)
    all_inline = all_inline && l.tensors.size() <= static_cast<size_t>(asr::kInlineTensors);
  for (Launch& l : plan->launches) l.inline_desc = all_inline;

  // Workspace offsets: uploaded metadata first (descriptors; first slots for
  // a device-filled table, or the host-filled table itself), device-filled
  // tables after.
  size_t off = 0;
  for (Launch& l : plan->launches) {
    if (l.inline_desc) continue;
    off = align_up(off, 16);
    l.tensors_off = off;
    off += l.tensors.size() * sizeof(asr::DevTensor);
    if (l.by_class) continue;
    off = align_up(off, 16);
    if (l.host_table) {
      l.table_off = off;
      off += l.n_slots * sizeof(uint32_t);
    } else {
      l.first_off = off;
      off += l.tensors.size() * sizeof(uint32_t);
    }
  }
  const size_t meta_bytes = align_up(off, 16);
  off = meta_bytes;
  for (Launch& l : plan->launches) {
    if (l.inline_desc || l.by_class || l.host_table) continue;
    off = align_up(off, 16);
    l.table_off = off;
    off += l.n_slots * sizeof(uint32_t);
  }
  plan->used_bytes = off;
  if (!plan->launches.empty() && off > plan->bound_bytes)
    return fail(ASR_EWORKSPACE, "internal: workspace plan exceeds its bound");
  plan->image.assign(meta_bytes, 0);
  for (const Launch& l : plan->launches) {
    if (l.inline_desc) continue;
    std::memcpy(plan->image.data() + l.tensors_off, l.tensors.data(),
                l.tensors.size() * sizeof(asr::DevTensor));
    if (l.by_class) continue;
    for (size_t k = 0; k < l.tensors.size(); ++k) {
      if (!l.host_table) {
        std::memcpy(plan->image.data() + l.first_off + k * sizeof(uint32_t),
                    &l.tensors[k].first_slot, sizeof(uint32_t));
        continue;
      }
      // slots first_slot .. first_slot + tensor_slots - 1 belong to tensor k
      const uint32_t idx = static_cast<uint32_t>(k);
      const uint64_t end = l.tensors[k].first_slot + tensor_slots(l.tensors[k]);
      for (uint64_t sl = l.tensors[k].first_slot; sl < end; ++sl)
        std::memcpy(plan->image.data() + l.table_off + sl * sizeof(uint32_t), &idx,
                    sizeof(uint32_t));
    }
  }
  return ASR_OK;
}

int check_workspace(const StepPlan& plan, const void* workspace, size_t workspace_bytes) {
  if (!workspace || workspace_bytes < plan.bound_bytes)
    return fail(ASR_EWORKSPACE, "workspace needs " + std::to_string(plan.bound_bytes) + " bytes");
  if (!aligned(workspace, 16)) return fail(ASR_EWORKSPACE, "workspace not 16-byte aligned");
  return ASR_OK;
}

// Uploads the metadata to ws (kernel-argument copies: stream-ordered,
// allocation-free) and enqueues every launch of the plan on the stream.
int enqueue_plan(const StepPlan& plan, uint8_t* ws, bool probe, int rounding,
                 const asr::Coeffs& c, uint32_t seed, uint32_t step, hipStream_t stream) {
  const size_t meta_bytes = plan.image.size();
  for (size_t pos = 0; pos < meta_bytes; pos += asr::kUploadWords * sizeof(uint32_t)) {
    asr::UploadBlock blk;
    const size_t bytes = std::min(meta_bytes - pos, sizeof(blk.w));
    std::memset(blk.w, 0, sizeof(blk.w));
    std::memcpy(blk.w, plan.image.data() + pos, bytes);
    hipError_t e = launch(asr::upload_words, 1, stream, blk,
                          reinterpret_cast<uint32_t*>(ws + pos),
                          static_cast<uint32_t>(bytes / sizeof(uint32_t)));
    if (e != hipSuccess) return hip_fail(e, "metadata upload launch");
  }
  for (const Launch& l : plan.launches) {
    hipError_t e = run_launch(l, ws, probe, rounding, c, seed, step, stream);
    if (e != hipSuccess) return hip_fail(e, probe ? "probe kernel launch" : "adamw kernel launch");
  }
  return ok();
}

// ----------------------------------------------- allocation-free variant
// The workspace of asr_adamw_step_noalloc: a fixed device array, one copy
// per GPU, held until the process ends. Host code never passes `scratch`
// itself to a kernel (on the host that name is a stand-in, not a device
// address): it uses the address hipGetSymbolAddress returns for the
// current device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device, looked up on the first call
// on that device (with it current) and kept.
int current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ASR_EINVAL, "device index beyond the " + std::to_string(kMaxDevices) +
                                " devices the scratch table holds");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(asr::scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(ASR_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ASR_OK;
}

}  // namespace

extern "C" {

int asr_abi_version(void) { return ASR_ABI_VERSION; }

const char* asr_last_error(void) { return asr_host::g_last_error.c_str(); }

size_t asr_adamw_workspace_bytes(const asr_tensor* tensors, int32_t n_tensors) {
  if (n_tensors <= 0 || !tensors) return 0;
  uint64_t slots = 0;
  for (int32_t i = 0; i < n_tensors; ++i)
    if (tensors[i].numel > 0) slots += max_slots(tensors[i].numel);
  return workspace_bound(n_tensors, slots);
}

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
  if (int s = check_hparams(lr, beta1, beta2, eps, weight_decay, step)) return s;
  if (rounding != ASR_ROUND_SR && rounding != ASR_ROUND_RN)
    return fail(ASR_EINVAL, "rounding must be ASR_ROUND_SR or ASR_ROUND_RN");
  StepPlan plan;
  if (int s = make_plan(tensors, n_tensors, &plan)) return s;
  if (plan.launches.empty()) return ok();
  if (int s = check_workspace(plan, workspace, workspace_bytes)) return s;
  const asr::Coeffs c = make_coeffs(lr, beta1, beta2, eps, weight_decay, step);
  return enqueue_plan(plan, static_cast<uint8_t*>(workspace), false, rounding, c, seed,
                      static_cast<uint32_t>(step), static_cast<hipStream_t>(stream_ptr));
}

int asr_adamw_step_noalloc(const asr_tensor* tensors, int32_t n_tensors, double lr,
                           double beta1, double beta2, double eps, double weight_decay,
                           int64_t step, uint32_t seed, int32_t rounding, void* stream_ptr) {
  if (int s = check_hparams(lr, beta1, beta2, eps, weight_decay, step)) return s;
  if (rounding != ASR_ROUND_SR && rounding != ASR_ROUND_RN)
    return fail(ASR_EINVAL, "rounding must be ASR_ROUND_SR or ASR_ROUND_RN");
  StepPlan plan;
  if (int s = make_plan(tensors, n_tensors, &plan)) return s;
  if (plan.launches.empty()) return ok();
  if (plan.used_bytes > asr::kScratchBytes)
    return fail(ASR_EWORKSPACE, "this list needs " + std::to_string(plan.used_bytes) +
                                    " bytes of scratch; the static scratch holds " +
                                    std::to_string(asr::kScratchBytes) +
                                    " (use asr_adamw_step with a workspace)");
  void* ws = nullptr;
  if (int s = current_scratch(&ws)) return s;
  const asr::Coeffs c = make_coeffs(lr, beta1, beta2, eps, weight_decay, step);
  return enqueue_plan(plan, static_cast<uint8_t*>(ws), false, rounding, c, seed,
                      static_cast<uint32_t>(step), static_cast<hipStream_t>(stream_ptr));
}

int asr_adamw_stream_probe(const asr_tensor* tensors, int32_t n_tensors, void* workspace,
                           size_t workspace_bytes, void* stream_ptr) {
  StepPlan plan;
  if (int s = make_plan(tensors, n_tensors, &plan)) return s;
  if (plan.launches.empty()) return ok();
  if (int s = check_workspace(plan, workspace, workspace_bytes)) return s;
  return enqueue_plan(plan, static_cast<uint8_t*>(workspace), true, ASR_ROUND_SR, asr::Coeffs{},
                      0, 0, static_cast<hipStream_t>(stream_ptr));
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
  // runs of kCvtVec elements start `shift` elements before in[0], on
  // 16-byte addresses of both buffers if some shift allows it
  int shift = -1;
  for (int s = 0; s < asr::kCvtVec && shift < 0; ++s) {
    const uintptr_t ia = reinterpret_cast<uintptr_t>(in) + (asr::kCvtVec - s) * 4;
    const uintptr_t oa = reinterpret_cast<uintptr_t>(out) + (asr::kCvtVec - s) * 2;
    if ((ia & 15) == 0 && (oa & (2 * asr::kCvtVec - 1)) == 0) shift = s;
  }
  const int vec_ok = shift >= 0;
  if (shift < 0) shift = 0;
  const uint64_t n_slots =
      (static_cast<uint64_t>(n) + static_cast<uint64_t>(shift) + asr::kCvtSlot - 1) / asr::kCvtSlot;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  using K = void (*)(const float*, uint16_t*, int64_t, uint64_t, uint64_t, uint32_t, uint32_t, int,
                     int);
  const K k = rounding == ASR_ROUND_SR ? asr::convert_f32_bf16<asr::kRoundSR>
                                       : asr::convert_f32_bf16<asr::kRoundRN>;
  uint32_t lds = 0;
  if (asr::kCvtBlocksPerCU > 0) {
    lds = (asr::kLdsPerCU / asr::kCvtBlocksPerCU) & ~1023u;
    if (lds > 64u * 1024u) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds));
      if (e != hipSuccess) return hip_fail(e, "convert attribute");
    }
  }
  for (uint64_t slot0 = 0; slot0 < n_slots; slot0 += asr::kMaxGrid) {
    const uint32_t grid = static_cast<uint32_t>(std::min<uint64_t>(n_slots - slot0, asr::kMaxGrid));
    hipError_t e = launch_lds(k, grid, asr::kBlock, lds, stream, in, out, n, slot0, base_index,
                              seed, step,
                              vec_ok, shift);
    if (e != hipSuccess) return hip_fail(e, "convert launch");
  }
  return ok();
}

int asr_cvt_f32_bf16_sr(const float* in, uint16_t* out, int64_t n, uint32_t seed,
                        uint32_t step, uint64_t base_index, void* stream) {
  return convert(ASR_ROUND_SR, in, out, n, seed, step, base_index, stream);
}

int asr_cvt_f32_bf16_rn(const float* in, uint16_t* out, int64_t n, void* stream) {
  return convert(ASR_ROUND_RN, in, out, n, 0, 0, 0, stream);
}

int asr_stream_copy(void* dst, const void* src, int64_t bytes, void* stream_ptr) {
  if (bytes < 0) return fail(ASR_EINVAL, "bytes < 0");
  if (bytes == 0) return ok();
  if (!dst || !src) return fail(ASR_EINVAL, "NULL buffer");
  if (bytes % 16 != 0 || !aligned(dst, 16) || !aligned(src, 16))
    return fail(ASR_EALIGN, "buffers and size must be multiples of 16 bytes");
  const uint64_t n16 = static_cast<uint64_t>(bytes) / 16;
  const uint64_t per_slot = static_cast<uint64_t>(asr::kStepBlock) * asr::kCopyVec;
  const uint64_t n_slots = (n16 + per_slot - 1) / per_slot;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  uint32_t lds = 0;
  hipError_t e = occupancy_lds(reinterpret_cast<const void*>(asr::stream_copy), &lds);
  if (e != hipSuccess) return hip_fail(e, "copy attribute");
  for (uint64_t slot0 = 0; slot0 < n_slots; slot0 += asr::kMaxGrid) {
    const uint32_t grid = static_cast<uint32_t>(std::min<uint64_t>(n_slots - slot0, asr::kMaxGrid));
    e = launch_lds(asr::stream_copy, grid, asr::kStepBlock, lds, stream,
                   static_cast<const asr::u32x4*>(src),
                   static_cast<asr::u32x4*>(dst), n16, slot0);
    if (e != hipSuccess) return hip_fail(e, "copy launch");
  }
  return ok();
}

int asr_hbm_probe(int32_t kind, void* dst, const void* src, int64_t bytes, void* stream_ptr) {
  if (kind == ASR_PROBE_COPY) return asr_stream_copy(dst, src, bytes, stream_ptr);
  if (kind != ASR_PROBE_READ && kind != ASR_PROBE_WRITE)
    return fail(ASR_EINVAL, "kind must be ASR_PROBE_READ, ASR_PROBE_WRITE or ASR_PROBE_COPY");
  if (bytes < 0) return fail(ASR_EINVAL, "bytes < 0");
  if (bytes == 0) return ok();
  const void* buf = kind == ASR_PROBE_READ ? src : dst;
  if (!buf || (kind == ASR_PROBE_READ && !dst)) return fail(ASR_EINVAL, "NULL buffer");
  if (bytes % 16 != 0 || !aligned(buf, 16) || !aligned(dst, 16))
    return fail(ASR_EALIGN, "buffers and size must be multiples of 16 bytes");
  const uint64_t n16 = static_cast<uint64_t>(bytes) / 16;
  const uint64_t per_slot = static_cast<uint64_t>(asr::kStepBlock) * asr::kCopyVec;
  const uint64_t n_slots = (n16 + per_slot - 1) / per_slot;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const void* k = kind == ASR_PROBE_READ ? reinterpret_cast<const void*>(asr::stream_read)
                                         : reinterpret_cast<const void*>(asr::stream_write);
  uint32_t lds = 0;
  hipError_t e = occupancy_lds(k, &lds);
  if (e != hipSuccess) return hip_fail(e, "probe attribute");
  for (uint64_t slot0 = 0; slot0 < n_slots; slot0 += asr::kMaxGrid) {
    const uint32_t grid = static_cast<uint32_t>(std::min<uint64_t>(n_slots - slot0, asr::kMaxGrid));
    if (kind == ASR_PROBE_READ)
      e = launch_lds(asr::stream_read, grid, asr::kStepBlock, lds, stream,
                     static_cast<const asr::u32x4*>(src),
                     static_cast<asr::u32x4*>(dst), n16, slot0);
    else
      e = launch_lds(asr::stream_write, grid, asr::kStepBlock, lds, stream,
                     static_cast<asr::u32x4*>(dst), n16,
                     slot0, 0x3F803F80u);
    if (e != hipSuccess) return hip_fail(e, "probe launch");
  }
  return ok();
}

int asr_sr_bf16_given_bits(const float* x, const uint16_t* r16, uint16_t* out, int64_t n,
                           void* stream_ptr) {
  if (n < 0) return fail(ASR_EINVAL, "n < 0");
  if (n == 0) return ok();
  if (!x || !r16 || !out) return fail(ASR_EINVAL, "NULL buffer");
  if (!aligned(x, 4) || !aligned(r16, 2) || !aligned(out, 2))
    return fail(ASR_EALIGN, "buffer not aligned to its element size");
  const int64_t blocks = (n + asr::kBlock - 1) / asr::kBlock;
  const uint32_t grid = static_cast<uint32_t>(std::min<int64_t>(blocks, 1 << 16));
  hipError_t e = launch(asr::sr_given_bits, grid, static_cast<hipStream_t>(stream_ptr), x, r16,
                        out, n);
  if (e != hipSuccess) return hip_fail(e, "sr launch");
  return ok();
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

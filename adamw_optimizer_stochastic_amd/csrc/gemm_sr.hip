// bf16 GEMM on gfx950 matrix cores whose f32 result is rounded to bf16 by
// stochastic rounding (or round-to-nearest) in the epilogue.
//
// Sources (pages cited by title and section):
//   "Add stochastic rounding and philox RNG helpers" (FlyDSL pull request):
//     GEMM section (a bf16 GEMM whose f32 accumulator goes to bf16 by SR
//     instead of RN, the random bits keyed per output element from a seed;
//     RN stays the default) and Tests (SR stays within tolerance of RN,
//     changes with the seed, reproducible for a fixed seed).
//   "adamw-sr" (kernels hub page), Method: the keying used throughout this
//     library -- Philox4x32-10 keyed by (seed, step), indexed by the global
//     position of the element.
//
// What is computed: C[m][n] = sum_k A[m][k] * B[n][k] (A is M x K, B is N x K,
// both row-major with K contiguous, i.e. C = A * B^T as in a linear layer
// y = x W^T), accumulated in f32 on the matrix cores, then rounded to bf16.
// Output element (m, n) takes its 16 random bits from stream position
// base_index + m*N + n: the same stream, and the same rounding, as the
// standalone conversion, so the SR output equals the conversion of the f32
// result bit for bit.
//
// Kernel design (CDNA4):
//   * v_mfma_f32_32x32x16_bf16 with the operands swapped (B rows feed the
//     instruction's row side, A rows its column side): each lane then ends
//     up holding runs of 4 consecutive output columns of one row, which is
//     exactly one Philox call's 4 words and one 8-byte bf16 store.
//   * Workgroup tile BM x BN, K in stages of 64 (128 bytes per row), two
//     stages in LDS. Global -> LDS by the gfx950 16-byte LDS-direct load
//     (global_load_lds_dwordx4): no VGPR staging. Each wave-wide load fills
//     1 KiB = 8 rows; the 16-byte chunks of a row are XOR-swizzled so that
//     the fragment reads (ds_read_b128, 32 rows per instruction) are free of
//     bank conflicts.
//   * Rows past M or N and chunks past K load from a 16-byte zero block, so
//     ragged edges need no masking in the main loop.
//   * Tiles are handed to XCDs in contiguous ranges (workgroup b runs on XCD
//     b % 8) and grouped along M inside each range, so the workgroups that
//     share an L2 also share A and B panels.
#include "device.hpp"
#include "status.hpp"

#include <adamw_sr.h>

#include <algorithm>
#include <string>
#include <type_traits>

#pragma clang fp contract(off)

namespace asr_gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kBK = 64;            // K elements per LDS stage
constexpr int kRowBytes = kBK * 2;  // 128 bytes: 8 chunks of 16 bytes
constexpr int kSlabRows = 8;       // rows one wave-wide 16-byte DMA fills
constexpr int kXcds = 8;
constexpr int kGroupM = 4;         // tile rows per group in the tile order

// Byte offset of 16-byte chunk c of tile row r within a stage region. The
// XOR spreads the rows a ds_read_b128 touches over all banks: rows r and
// r+1 share a 256-byte bank period, and (r >> 1) & 7 takes eight values over
// 16 consecutive rows.
__device__ __forceinline__ uint32_t chunk_offset(uint32_t r, uint32_t c) {
  return r * kRowBytes + ((c ^ ((r >> 1) & 7u)) << 4);
}

// Source of chunks outside the matrices (rows past M or N, columns past K).
__device__ __align__(16) uint4 g_zero_chunk;

template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
  static constexpr int kWaves = kWavesM * kWavesN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kFragM = WM / 32, kFragN = WN / 32;
  static constexpr int kSlabs = (BM + BN) / kSlabRows;
  static constexpr int kSlabsPerWave = kSlabs / kWaves;
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kLdsBytes = 2 * kStageBytes;
  static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
  static_assert(kSlabs % kWaves == 0, "every wave fills the same number of slabs");
  static_assert(BM % kSlabRows == 0, "a slab lies in A or in B");
};

struct GemmArgs {
  const uint16_t* a;
  const uint16_t* b;
  uint16_t* c;
  float* c32;          // optional f32 copy of the accumulator (may be null)
  int64_t lda, ldb, ldc;
  uint64_t base_index;
  int32_t m, n, k;
  uint32_t tiles_m, tiles_n;
  uint32_t seed, step;
  uint32_t vec_store;  // ldc % 4 == 0 and C (and c32) aligned for 8 (16) bytes
  uint32_t pos4;       // base_index % 4 == 0 and N % 4 == 0
};

// Tile index of workgroup b: XCD x = b % 8 owns a contiguous range of
// tiles, then tiles are taken in groups of kGroupM tile rows.
__device__ __forceinline__ void tile_of_block(uint32_t b, uint32_t tiles_m, uint32_t tiles_n,
                                              uint32_t& tm, uint32_t& tn) {
  const uint32_t total = tiles_m * tiles_n;
  const uint32_t q = total / kXcds, r = total % kXcds;
  const uint32_t x = b % kXcds, k = b / kXcds;
  const uint32_t t = x * q + min(x, r) + k;
  const uint32_t group = kGroupM * tiles_n;
  const uint32_t first_m = (t / group) * kGroupM;
  const uint32_t rows = min(tiles_m - first_m, static_cast<uint32_t>(kGroupM));
  const uint32_t in_group = t % group;
  tm = first_m + in_group % rows;
  tn = in_group / rows;
}

template <int ROUND>
__device__ __forceinline__ void round4(const float (&x)[4], const uint32_t (&r16)[4],
                                       uint32_t (&h)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t u = __float_as_uint(x[e]);
    h[e] = ROUND == ASR_ROUND_SR ? asr::round_sr(u, r16[e]) : asr::round_rn(u);
  }
}

// 16 random bits for positions p .. p+3 (any alignment).
__device__ __forceinline__ void bits4(uint64_t p, bool pos4, uint32_t seed, uint32_t step,
                                      uint32_t (&r16)[4]) {
  if (pos4) {
    asr::stream_bits<0, 4>(p, seed, step, r16);
  } else {
    const uint32_t phase = static_cast<uint32_t>(p) & 3u;
    const asr::Words4 w0 = asr::stream_call(p >> 2, seed, step);
    const asr::Words4 w1 = asr::stream_call((p >> 2) + 1, seed, step);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t s = phase + e;
      uint32_t w = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (s == static_cast<uint32_t>(q)) w = q < 4 ? w0.w[q] : w1.w[q - 4];
      r16[e] = w & 0xFFFFu;
    }
  }
}

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// Writes output elements (m, n .. n+3) that lie inside C: the f32 values
// when requested, and their bf16 roundings.
template <int ROUND, bool F32OUT>
__device__ __forceinline__ void store_out(const GemmArgs& args, int64_t m, int64_t n,
                                          const float (&x)[4]) {
  const bool full = n + 4 <= args.n && args.vec_store;
  if constexpr (F32OUT) {
    float* d = args.c32 + m * args.ldc + n;
    if (full) {
      *reinterpret_cast<asr::f32x4*>(d) = asr::f32x4{x[0], x[1], x[2], x[3]};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < args.n) d[e] = x[e];
    }
  }
  uint32_t r16[4] = {0, 0, 0, 0};
  if constexpr (ROUND == ASR_ROUND_SR)
    bits4(args.base_index + static_cast<uint64_t>(m) * static_cast<uint64_t>(args.n) +
              static_cast<uint64_t>(n),
          args.pos4 != 0, args.seed, args.step, r16);
  uint32_t h[4];
  round4<ROUND>(x, r16, h);
  uint16_t* d = args.c + m * args.ldc + n;
  if (full) {
    *reinterpret_cast<asr::u32x2*>(d) = asr::u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < args.n) d[e] = static_cast<uint16_t>(h[e]);
  }
}

template <typename Cfg, int ROUND, bool F32OUT>
__global__ __launch_bounds__(Cfg::kThreads) void gemm_bf16(GemmArgs args) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN;
  __shared__ __align__(1024) unsigned char smem[Cfg::kLdsBytes];

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = threadIdx.x >> 6;
  uint32_t tm, tn;
  tile_of_block(blockIdx.x, args.tiles_m, args.tiles_n, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int64_t n0 = static_cast<int64_t>(tn) * BN;

  // ---- this lane's share of the global -> LDS copies: one 16-byte chunk
  // of row R = slab*8 + lane/8, at position lane%8 of that row.
  const uint16_t* src[Cfg::kSlabsPerWave];
  uint32_t kchunk[Cfg::kSlabsPerWave];  // element offset of the chunk in the stage
#pragma unroll
  for (int j = 0; j < Cfg::kSlabsPerWave; ++j) {
    const uint32_t slab = wave + j * Cfg::kWaves;
    const uint32_t row = slab * kSlabRows + (lane >> 3);
    const uint32_t c = (lane & 7u) ^ ((row >> 1) & 7u);  // inverse of chunk_offset's XOR
    kchunk[j] = c * 8;
    if (row < static_cast<uint32_t>(BM)) {
      const int64_t gm = m0 + row;
      src[j] = gm < args.m ? args.a + gm * args.lda + c * 8 : nullptr;
    } else {
      const int64_t gn = n0 + (row - BM);
      src[j] = gn < args.n ? args.b + gn * args.ldb + c * 8 : nullptr;
    }
  }
  const uint16_t* zero = reinterpret_cast<const uint16_t*>(&g_zero_chunk);

  auto load_stage = [&](int stage, int k0) {
    unsigned char* base = smem + stage * Cfg::kStageBytes;
#pragma unroll
    for (int j = 0; j < Cfg::kSlabsPerWave; ++j) {
      const uint32_t slab = wave + j * Cfg::kWaves;
      const bool in = src[j] != nullptr && static_cast<int>(k0 + kchunk[j]) < args.k;
      const uint16_t* g = in ? src[j] + k0 : zero;
      __builtin_amdgcn_global_load_lds(g, (lds_void_ptr)(base + slab * 1024u),
                                       16, 0, 0);
    }
  };

  f32x16 acc[Cfg::kFragM][Cfg::kFragN];
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j) acc[i][j] = f32x16{};

  const uint32_t wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const uint32_t frag_row = lane & 31u, frag_half = lane >> 5;
  const int ktiles = (args.k + kBK - 1) / kBK;

  if (ktiles > 0) load_stage(0, 0);
  for (int kt = 0; kt < ktiles; ++kt) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this stage's copies have landed
    __syncthreads();                     // ... for every wave; the other stage is free
    if (kt + 1 < ktiles) load_stage((kt + 1) & 1, (kt + 1) * kBK);
    const unsigned char* sa = smem + (kt & 1) * Cfg::kStageBytes;
    const unsigned char* sb = sa + BM * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const uint32_t c = 2 * kk + frag_half;
      bf16x8 fa[Cfg::kFragM], fb[Cfg::kFragN];
#pragma unroll
      for (int i = 0; i < Cfg::kFragM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(
            sa + chunk_offset(wm * Cfg::WM + i * 32 + frag_row, c));
#pragma unroll
      for (int j = 0; j < Cfg::kFragN; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(
            sb + chunk_offset(wn * Cfg::WN + j * 32 + frag_row, c));
#pragma unroll
      for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::kFragN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue. acc[i][j] register r of lane l holds C[m][n] with
  // m = row base + l%32 and n = column base + 8*(r/4) + 4*(l/32) + r%4.
  // Compile-time loops keep every accumulator index constant (a runtime
  // index would move the accumulators to scratch memory).
  static_for<Cfg::kFragM>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int64_t m = m0 + wm * Cfg::WM + i * 32 + frag_row;
    if (m >= args.m) return;
    static_for<Cfg::kFragN>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      static_for<4>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        const int64_t n = n0 + wn * Cfg::WN + j * 32 + 8 * q + 4 * frag_half;
        if (n >= args.n) return;
        const float x[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                            acc[i][j][4 * q + 3]};
        store_out<ROUND, F32OUT>(args, m, n, x);
      });
    });
  });
}

using Big = TileCfg<256, 256, 128, 64>;   // 8 waves, 2 per SIMD
using Small = TileCfg<128, 128, 64, 64>;  // 4 waves, for grids too small for Big

}  // namespace asr_gemm

// =========================================================== host side
namespace {

using asr_host::fail;
using asr_host::hip_fail;
using asr_host::ok;

bool aligned_to(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

template <typename Cfg, int ROUND, bool F32OUT>
hipError_t launch_gemm(asr_gemm::GemmArgs args, hipStream_t stream) {
  args.tiles_m = static_cast<uint32_t>((args.m + Cfg::BM - 1) / Cfg::BM);
  args.tiles_n = static_cast<uint32_t>((args.n + Cfg::BN - 1) / Cfg::BN);
  const uint64_t tiles = static_cast<uint64_t>(args.tiles_m) * args.tiles_n;
  void* argv[] = {&args};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&asr_gemm::gemm_bf16<Cfg, ROUND, F32OUT>),
      dim3(static_cast<uint32_t>(tiles)), dim3(Cfg::kThreads), argv, 0, stream);
}

template <typename Cfg>
hipError_t dispatch(const asr_gemm::GemmArgs& args, int32_t rounding, hipStream_t stream) {
  const bool f32 = args.c32 != nullptr;
  if (rounding == ASR_ROUND_SR)
    return f32 ? launch_gemm<Cfg, ASR_ROUND_SR, true>(args, stream)
               : launch_gemm<Cfg, ASR_ROUND_SR, false>(args, stream);
  return f32 ? launch_gemm<Cfg, ASR_ROUND_RN, true>(args, stream)
             : launch_gemm<Cfg, ASR_ROUND_RN, false>(args, stream);
}

}  // namespace

extern "C" {

int asr_gemm_bf16(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, uint16_t* c,
                  int64_t ldc, float* c_f32, int64_t m, int64_t n, int64_t k, int32_t rounding,
                  uint32_t seed, uint32_t step, uint64_t base_index, void* stream) {
  constexpr int64_t kMaxDim = int64_t{1} << 31;
  if (m < 0 || n < 0 || k < 0 || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim)
    return fail(ASR_EINVAL, "gemm: m, n, k must be in [0, 2**31)");
  if (rounding != ASR_ROUND_SR && rounding != ASR_ROUND_RN)
    return fail(ASR_EINVAL, "gemm: rounding must be ASR_ROUND_SR or ASR_ROUND_RN");
  if (m == 0 || n == 0) return ok();
  if (!c || (k > 0 && (!a || !b))) return fail(ASR_EINVAL, "gemm: null matrix pointer");
  if (lda < k || ldb < k || ldc < n) return fail(ASR_EINVAL, "gemm: lda, ldb >= k and ldc >= n");
  if (k % 8 != 0 || lda % 8 != 0 || ldb % 8 != 0)
    return fail(ASR_EALIGN, "gemm: k, lda and ldb must be multiples of 8");
  if (!aligned_to(a, 16) || !aligned_to(b, 16))
    return fail(ASR_EALIGN, "gemm: A and B must be 16-byte aligned");
  if (!aligned_to(c, 2) || (c_f32 && !aligned_to(c_f32, 4)))
    return fail(ASR_EALIGN, "gemm: C must be aligned to its element size");
  if (static_cast<uint64_t>(m) * static_cast<uint64_t>(n) - 1 > ~base_index)
    return fail(ASR_EINVAL, "gemm: base_index + m*n exceeds 2**64");

  asr_gemm::GemmArgs args{};
  args.a = a;
  args.b = b;
  args.c = c;
  args.c32 = c_f32;
  args.lda = lda;
  args.ldb = ldb;
  args.ldc = ldc;
  args.base_index = base_index;
  args.m = static_cast<int32_t>(m);
  args.n = static_cast<int32_t>(n);
  args.k = static_cast<int32_t>(k);
  args.seed = seed;
  args.step = step;
  args.vec_store = ldc % 4 == 0 && aligned_to(c, 8) && (!c_f32 || aligned_to(c_f32, 16));
  args.pos4 = (base_index % 4 == 0) && (n % 4 == 0);

  const uint64_t big_tiles = static_cast<uint64_t>((m + 255) / 256) * ((n + 255) / 256);
  const uint64_t small_tiles = static_cast<uint64_t>((m + 127) / 128) * ((n + 127) / 128);
  if (small_tiles > 0x7FFFFFFFull) return fail(ASR_EINVAL, "gemm: too many tiles");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The big tile halves the LDS and L2 traffic per flop; it needs enough
  // tiles to give every CU at least one.
  const hipError_t e = big_tiles >= 256 ? dispatch<asr_gemm::Big>(args, rounding, s)
                                        : dispatch<asr_gemm::Small>(args, rounding, s);
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return ok();
}

}  // extern "C"

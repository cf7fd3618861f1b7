// bf16 GEMM on gfx950 matrix cores whose f32 result is rounded to bf16 by
// stochastic rounding (or round-to-nearest) in the epilogue.
//
// Sources (pages cited by title and section):
//   "Add stochastic rounding and philox RNG helpers" (FlyDSL pull request):
//     Consumer section (a bf16 GEMM whose f32 accumulator goes to bf16 by SR
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
//   * Workgroup tile BM x BN (256 x 256, 8 waves of 128 x 64, two per SIMD),
//     K in tiles of BK = 64 (one 128-byte cache line per row) through a ring
//     of STAGES = 2 LDS buffers (128 KiB). Global -> LDS by gfx950's 16-byte
//     buffer loads to LDS (buffer_load_dwordx4 ... lds): no VGPR staging.
//     Each wave-wide load fills 1 KiB; the 16-byte chunks of a row are
//     XOR-swizzled so that the fragment reads (ds_read_b128, 32 rows per
//     instruction) are free of bank conflicts. A K tile's copies are issued
//     into the buffer of the tile two before it as soon as every wave has
//     passed that tile's barrier, the ring waits with vmcnt for exactly the
//     tile it needs, and its barrier carries no release fence.
//   * Copy sources are a buffer resource at the tile origin and K offset
//     (scalar) plus 32-bit lane offsets. Rows past M or N are clamped to the
//     last row (their products only reach outputs that are not stored);
//     chunks past K take an out-of-range offset, for which the buffer load
//     returns zeros, so ragged edges need no masking in the MFMA loop.
//   * Each MFMA step runs in a fixed order, fenced with sched_barrier so
//     the compiler keeps it: after every MFMA one fragment read for the
//     next step. The tile's barrier sits inside its last MFMA step, so the
//     next tile's first fragments and the copies of the tile two ahead
//     issue under the MFMAs that follow it.
//   * Tiles are handed to XCDs in contiguous ranges (workgroup b runs on XCD
//     b % 8) and grouped along M inside each range, so the workgroups that
//     share an L2 also share A and B panels.
//   * Epilogue: lanes l and l + 32 hold alternate runs of 4 columns of one
//     row; v_permlane32_swap pairs them into runs of 8, each written with
//     one 16-byte store (RN swaps the f32 values; SR rounds each lane's own
//     runs first, one Philox call per run, and swaps the packed bf16 words).
//   * With more big tiles than CUs the launch is persistent: one workgroup
//     per CU runs output tiles b, b + #CUs, ... (the same order), and the
//     ring carries on across them: the next tile's first two K tiles are
//     copied during the current tile's last two, so a tile starts with its
//     operands in LDS, and its waits leave the previous tile's output stores
//     in flight (vector-memory operations complete in issue order).
//   * Grids of fewer than 256 big tiles use a 128 x 128 tile: 8 waves of
//     64 x 32 when there are no more such tiles than CUs, else 4 waves of
//     64 x 64 (two workgroups to a CU). With at most half as many
//     128 x 128 tiles as CUs, a 64 x 64 tile in 4 waves of 32 x 32 gives
//     four times as many workgroups. Where a CU runs a single workgroup
//     (the 8-wave 128 x 128 tile, the 64 x 64 tile) the ring is 3 and 4
//     K tiles deep: such grids are latency-bound, and the LDS is free.
#include "device.hpp"
#include "status.hpp"

#include <adamw_sr.h>

#include <algorithm>
#include <atomic>
#include <string>
#include <type_traits>

#pragma clang fp contract(off)

namespace asr_gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kXcds = 8;
#ifndef ASR_GEMM_GROUP_M
#define ASR_GEMM_GROUP_M 4
#endif
constexpr int kGroupM = ASR_GEMM_GROUP_M;  // tile rows per group in the tile order
// SR epilogue: 1 = lanes pair up their rounded runs into 16-byte stores,
// 0 = each lane stores its runs of 4 (8 bytes); the results are identical.
#ifndef ASR_GEMM_SR_SWAP
#define ASR_GEMM_SR_SWAP 1
#endif
constexpr int kDmaBytes = 1024;    // LDS bytes one wave-wide 16-byte-per-lane DMA fills

// Copies go through buffer resources: a resource spans kBufferRecords bytes
// from a tile's first row at one K tile, and a lane offset at or past that
// reads zeros (a buffer load's out-of-range result) without touching memory.
// Valid offsets stay below it: a tile's rows are at most 255 leading
// dimensions (< 2**22 elements, so < 2**23 bytes) past its first row.
constexpr uint32_t kBufferRecords = 0x80000000u;
constexpr uint32_t kOutOfRange = kBufferRecords;
constexpr int32_t kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const char* base) {
  // (the builtin takes a non-const pointer; the resource is only read)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), static_cast<short>(0),
                                           static_cast<int32_t>(kBufferRecords), kBufferWord3);
}

// Workgroup tile BM x BN, wave tile WM x WN, K in stages of BK (32 or 64),
// STAGES stages in LDS.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int STAGES_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, STAGES = STAGES_;
  static constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
  static constexpr int kWaves = kWavesM * kWavesN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kFragM = WM / 32, kFragN = WN / 32;
  static constexpr int kRowBytes = BK * 2;                 // one row of a stage
  static constexpr int kChunks = BK / 8;                   // 16-byte chunks per row
  static constexpr int kSlabRows = kDmaBytes / kRowBytes;  // rows per wave-wide DMA
  static constexpr int kSlabs = (BM + BN) / kSlabRows;
  // Waves that issue the copies: one per SIMD (waves 0 .. 3; wave w runs on
  // SIMD w % 4). With two waves per SIMD the other one keeps issuing MFMAs
  // while its partner's copies wait to issue, instead of both stalling at
  // once.
  static constexpr int kCopyWaves = kWaves > 4 ? 4 : kWaves;
  static constexpr int kSlabsPerWave = kSlabs / kCopyWaves;  // DMAs per copying lane per stage
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kLdsBytes = STAGES * kStageBytes;
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
  static_assert(kSlabs % kCopyWaves == 0, "every copying wave fills the same number of slabs");
  static_assert(BM % kSlabRows == 0, "a slab lies in A or in B");
  static_assert(STAGES >= 2 && kLdsBytes <= 160 * 1024, "LDS budget");

  // Position of 16-byte chunk c in tile row r. A ds_read_b128 is served 16
  // lanes at a time over 64 four-byte banks (256 bytes); its 16 lanes read
  // one chunk index from 16 consecutive rows, and the XOR gives those rows
  // 16 distinct bank ranges: 128-byte rows pair up in a 256-byte period and
  // (r >> 1) & 7 separates the 8 pairs; 64-byte rows come four to a period
  // and (r >> 2) & 3 separates the 4 periods.
  __device__ static __forceinline__ uint32_t chunk_pos(uint32_t r, uint32_t c) {
    return BK == 64 ? (c ^ ((r >> 1) & 7u)) : (c ^ ((r >> 2) & 3u));
  }
  __device__ static __forceinline__ uint32_t chunk_offset(uint32_t r, uint32_t c) {
    return r * kRowBytes + (chunk_pos(r, c) << 4);
  }
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
  uint32_t vec16;      // ldc % 8 == 0 and C and c32 aligned for 16 bytes
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

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ int32_t row_clamp(int32_t row, int32_t last) {
  return row < last ? row : last;
}

// Workgroup barrier for the LDS ring: this wave's LDS reads are complete
// (lgkmcnt(0)) and every wave has arrived. Unlike __syncthreads() it does
// not wait for this wave's outstanding global->LDS copies (a release fence
// would), which is the point of the ring; the caller waits for exactly the
// copies it needs with wait_vmcnt. The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

// Writes output elements (m, n .. n+7), n a multiple of 8, that lie inside
// C: with 16-byte stores when the whole run is inside and aligned, else as
// two runs of 4.
template <int ROUND, bool F32OUT>
__device__ __forceinline__ void store_out8(const GemmArgs& args, int64_t m, int64_t n,
                                           const float (&x)[8]) {
  if (args.vec16 && n + 8 <= args.n) {
    if constexpr (F32OUT) {
      float* d = args.c32 + m * args.ldc + n;
      reinterpret_cast<asr::f32x4*>(d)[0] = asr::f32x4{x[0], x[1], x[2], x[3]};
      reinterpret_cast<asr::f32x4*>(d)[1] = asr::f32x4{x[4], x[5], x[6], x[7]};
    }
    const uint64_t p = args.base_index + static_cast<uint64_t>(m) * static_cast<uint64_t>(args.n) +
                       static_cast<uint64_t>(n);
    uint32_t r16[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (ROUND == ASR_ROUND_SR) {
      uint32_t lo[4], hi[4];
      bits4(p, args.pos4 != 0, args.seed, args.step, lo);
      bits4(p + 4, args.pos4 != 0, args.seed, args.step, hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r16[e] = lo[e];
        r16[4 + e] = hi[e];
      }
    }
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      h[e] = ROUND == ASR_ROUND_SR ? asr::round_sr(__float_as_uint(x[e]), r16[e])
                                   : asr::round_rn(__float_as_uint(x[e]));
    *reinterpret_cast<asr::u32x4*>(args.c + m * args.ldc + n) =
        asr::u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                   h[6] | (h[7] << 16)};
  } else {
    const float a[4] = {x[0], x[1], x[2], x[3]};
    const float b[4] = {x[4], x[5], x[6], x[7]};
    store_out<ROUND, F32OUT>(args, m, n, a);
    if (n + 4 < args.n) store_out<ROUND, F32OUT>(args, m, n + 4, b);
  }
}

template <typename Cfg, int ROUND, bool F32OUT, bool PERSIST>
__global__ __launch_bounds__(Cfg::kThreads) void gemm_bf16(GemmArgs args) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN;
  __shared__ __align__(1024) unsigned char smem[Cfg::kLdsBytes];

  const uint32_t lane = threadIdx.x & 63u;
  // The wave index as a scalar: every LDS destination and global base below
  // is then uniform and lives in scalar registers.
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---- this lane's share of the global -> LDS copies. Slab j of this wave
  // is rows slab * kSlabRows .. + kSlabRows - 1 of the stage (slab = wave +
  // j * kWaves; the first kSlabsA slabs of every wave lie in A, the rest in
  // B); the lane copies the 16-byte chunk at position lane % kChunks of row
  // lane / kChunks. Its source is a buffer resource at the tile origin and
  // K offset (scalar) plus a 32-bit per-lane byte offset. Rows past the edge
  // of A or B are clamped to the last row: they only feed outputs that are
  // not stored.
  constexpr int kChunks = Cfg::kChunks;
  constexpr int kCopiers = Cfg::kCopyWaves;
  constexpr int kSlabsA = BM / Cfg::kSlabRows / kCopiers;
  static_assert((BM / Cfg::kSlabRows) % kCopiers == 0, "A slabs split evenly over waves");
  const bool copier = kCopiers == Cfg::kWaves || wave < static_cast<uint32_t>(kCopiers);
  // The tile the copies fetch (origin m0, n0): the workgroup's current tile,
  // and in the persistent form, during the current tile's last STAGES K
  // tiles, the next one.
  int64_t m0 = 0, n0 = 0;
  uint32_t voff[Cfg::kSlabsPerWave];
  const char* a_tile = nullptr;
  const char* b_tile = nullptr;
  auto aim_copies = [&](uint32_t tile) {
    uint32_t tm, tn;
    tile_of_block(tile, args.tiles_m, args.tiles_n, tm, tn);
    m0 = static_cast<int64_t>(tm) * BM;
    n0 = static_cast<int64_t>(tn) * BN;
    const int32_t last_a = args.m - 1 - static_cast<int32_t>(m0);
    const int32_t last_b = args.n - 1 - static_cast<int32_t>(n0);
#pragma unroll
    for (int j = 0; j < Cfg::kSlabsPerWave; ++j) {
      const uint32_t row = (wave + j * kCopiers) * Cfg::kSlabRows + lane / kChunks;
      const uint32_t c = Cfg::chunk_pos(row, lane % kChunks);  // the XOR is its own inverse
      if (j < kSlabsA)
        voff[j] = (static_cast<uint32_t>(row_clamp(static_cast<int32_t>(row), last_a)) *
                       static_cast<uint32_t>(args.lda) + c * 8) * 2;
      else
        voff[j] = (static_cast<uint32_t>(row_clamp(static_cast<int32_t>(row) - BM, last_b)) *
                       static_cast<uint32_t>(args.ldb) + c * 8) * 2;
    }
    a_tile = reinterpret_cast<const char*>(args.a + m0 * args.lda);
    b_tile = reinterpret_cast<const char*>(args.b + n0 * args.ldb);
  };
  uint32_t tile = blockIdx.x;
  aim_copies(tile);
  bool has_next = false;  // persistent form: this workgroup has another output tile
  // persistent form: the previous output tile's kStoresPerWave stores were
  // issued after this tile's first STAGES K tiles of copies
  bool stores_behind = false;

  // Copy of slab j of K tile kt into LDS buffer `stage`: a buffer load to
  // LDS (buffer_load_dwordx4 ... lds) from a resource at the tile's first
  // row and K tile, with the lane's 32-bit offset. Lanes whose offset is
  // kOutOfRange write zeros.
  auto dma_off = [&](int stage, int j, int kt, uint32_t off) {
    const char* base = (j < kSlabsA ? a_tile : b_tile) + static_cast<int64_t>(kt) * Cfg::kRowBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        buffer_of(base),
        (lds_void_ptr)(smem + stage * Cfg::kStageBytes + (wave + j * kCopiers) * kDmaBytes),
        16, off, 0, 0, 0);
  };
  auto dma = [&](int stage, int j, int kt) { dma_off(stage, j, kt, voff[j]); };
  // The last K tile when K is not a multiple of BK: chunks at or past K read
  // zeros (K is a multiple of 8, so a chunk is wholly inside or outside).
  auto dma_tail = [&](int stage, int j, int kt) {
    const uint32_t row = (wave + j * kCopiers) * Cfg::kSlabRows + lane / kChunks;
    const uint32_t c = Cfg::chunk_pos(row, lane % kChunks);
    const int k = kt * Cfg::BK + static_cast<int>(c) * 8;
    dma_off(stage, j, kt, k < args.k ? voff[j] : kOutOfRange);
  };

  f32x16 acc[Cfg::kFragM][Cfg::kFragN];
  // Vector-memory instructions one wave's epilogue issues for a tile that
  // lies wholly inside C: one 16-byte store per 8 outputs (one 8-byte store
  // per 4 for SR without the swap), more with the f32 copy or unaligned C
  // (never fewer).
  constexpr int kStoresPerWave =
      Cfg::kFragM * Cfg::kFragN * (ROUND == ASR_ROUND_RN || ASR_GEMM_SR_SWAP ? 2 : 4);
  static_assert((Cfg::STAGES - 1) * Cfg::kSlabsPerWave + kStoresPerWave < 64, "vmcnt range");

  const uint32_t wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const uint32_t frag_row = lane & 31u, frag_half = lane >> 5;
  const int ktiles = (args.k + Cfg::BK - 1) / Cfg::BK;
  const int kfull = args.k / Cfg::BK;  // K tiles with no chunk past K
  constexpr int kSteps = Cfg::BK / 16;  // MFMA steps per K tile

  // Ring of STAGES buffers: tile kt lives in buffer kt % STAGES. The copies
  // of tile kt + STAGES go into tile kt's own buffer as soon as every wave
  // has passed the barrier inside tile kt's last MFMA step (by then all of
  // tile kt's fragments are in registers), so they have STAGES - 1 tiles
  // and the rest of that step to land. Fragments are read one step ahead,
  // the first step's across the tile boundary (see tile_body).
  int cur = 0;                     // buffer of tile kt
  bf16x8 fa[2][Cfg::kFragM], fb[2][Cfg::kFragN];

  // LOAD (the copies a tile body issues, of tile kt + STAGES): 0 = none,
  // 1 = a whole tile, 2 = the partial last tile, 3 = a whole K tile of the
  // next output tile (K tile kt + STAGES - ktiles; persistent form).
  // The barrier sits inside the last MFMA step of each tile.
  // Half of that step's MFMAs are issued, then the wave waits for tile
  // kt + 1, passes the barrier, and issues tile kt + 1's first fragment
  // reads and the copies of tile kt + STAGES between the other half of the
  // MFMAs. The next tile then starts with its fragments in registers
  // instead of behind a barrier and a round trip to the LDS.
  auto read_frags_from = [&](const unsigned char* sa, int kk, int buf) {
    const unsigned char* sb = sa + BM * Cfg::kRowBytes;
    const uint32_t c = 2 * kk + frag_half;
#pragma unroll
    for (int i = 0; i < Cfg::kFragM; ++i)
      fa[buf][i] = *reinterpret_cast<const bf16x8*>(
          sa + Cfg::chunk_offset(wm * Cfg::WM + i * 32 + frag_row, c));
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j)
      fb[buf][j] = *reinterpret_cast<const bf16x8*>(
          sb + Cfg::chunk_offset(wn * Cfg::WN + j * 32 + frag_row, c));
  };
  // Fragment read r of step kk into set buf: A fragment r for r < kFragM,
  // else B fragment r - kFragM.
  auto read_frag = [&](const unsigned char* sa, int kk, int buf, auto rc) {
    constexpr int r = decltype(rc)::value;
    const uint32_t c = 2 * kk + frag_half;
    if constexpr (r < Cfg::kFragM)
      fa[buf][r] = *reinterpret_cast<const bf16x8*>(
          sa + Cfg::chunk_offset(wm * Cfg::WM + r * 32 + frag_row, c));
    else
      fb[buf][r - Cfg::kFragM] = *reinterpret_cast<const bf16x8*>(
          sa + BM * Cfg::kRowBytes +
          Cfg::chunk_offset(wn * Cfg::WN + (r - Cfg::kFragM) * 32 + frag_row, c));
  };
  auto mfma = [&](int kk, auto ic, auto jc) {
    constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk & 1][j], fa[kk & 1][i], acc[i][j],
                                                         0, 0, 0);
  };
  auto wait_for = [&](int tile) {  // this lane's copies of tile `tile` have landed
    if (tile + Cfg::STAGES - 2 < ktiles) wait_vmcnt<(Cfg::STAGES - 2) * Cfg::kSlabsPerWave>();
    else wait_vmcnt<0>();
  };
  auto tile_body = [&](int kt, auto load_c) {
    constexpr int LOAD = decltype(load_c)::value;
    static_assert(kSteps % 2 == 0, "fragment sets alternate per step");
    const int next = kt + Cfg::STAGES - (LOAD == 3 ? ktiles : 0);
    const unsigned char* sa = smem + cur * Cfg::kStageBytes;
    const unsigned char* na = smem + (cur + 1 == Cfg::STAGES ? 0 : cur + 1) * Cfg::kStageBytes;
    // Explicit order, fenced so the compiler keeps it: in every step, group
    // g is MFMA g, then fragment read g for the next step. No MFMA moves
    // into another step, so each accumulator is updated once per step and
    // the reads have a step's worth of MFMAs to land in.
    static_for<kSteps>([&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      constexpr bool kLast = kk + 1 == kSteps;
      constexpr int kReads = kLast ? 0 : Cfg::kFragM + Cfg::kFragN;
      constexpr int kRows = kLast ? Cfg::kFragM / 2 : Cfg::kFragM;
      constexpr int kMf = kRows * Cfg::kFragN;
      static_for<kMf>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        mfma(kk, std::integral_constant<int, g / Cfg::kFragN>{},
             std::integral_constant<int, g % Cfg::kFragN>{});
        if constexpr (g < kReads) read_frag(sa, kk + 1, (kk + 1) & 1, gc);
        __builtin_amdgcn_sched_barrier(0);
      });
      static_for<(kReads > kMf ? kReads - kMf : 0)>([&](auto rc) {
        read_frag(sa, kk + 1, (kk + 1) & 1,
                  std::integral_constant<int, kMf + decltype(rc)::value>{});
      });
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kLast) {
        // the barrier, then the other half of the MFMAs, each followed by
        // a read of the next tile's first step (harmless after the last
        // tile: the LDS is only read, and the values are not used)
        if (kt + 1 < ktiles) {
          // (K tile 1 of a tile whose predecessor's stores follow its copies:
          // those stores may stay outstanding)
          if (PERSIST && kt == 0 && stores_behind)
            wait_vmcnt<(Cfg::STAGES - 2) * Cfg::kSlabsPerWave + kStoresPerWave>();
          else
            wait_for(kt + 1);
          barrier_lds();  // tile kt + 1 visible; every wave is done with tile kt - 1's buffer
        } else if constexpr (LOAD == 3) {
          barrier_lds();  // every wave is done with this buffer before the next tile's copies
        }
        __builtin_amdgcn_sched_barrier(0);
        constexpr int kRest = (Cfg::kFragM - kRows) * Cfg::kFragN;
        constexpr int kNext = Cfg::kFragM + Cfg::kFragN;
        // the copies of K tile kt + STAGES, into this tile's buffer (every
        // wave has read it once past the barrier), two or so after each MFMA
        constexpr int kEarlyDmas = LOAD != 0 ? Cfg::kSlabsPerWave : 0;
        constexpr int kPer = (kEarlyDmas + kRest - 1) / kRest;
        static_for<kRest>([&](auto gc) {
          constexpr int g = decltype(gc)::value;
          if constexpr (g < kNext) read_frag(na, 0, 0, gc);
          mfma(kk, std::integral_constant<int, kRows + g / Cfg::kFragN>{},
               std::integral_constant<int, g % Cfg::kFragN>{});
          static_for<kPer>([&](auto dc) {
            constexpr int j = g * kPer + decltype(dc)::value;
            if constexpr (j < kEarlyDmas) {
              if (copier && (LOAD != 3 || has_next)) {
                if constexpr (LOAD == 2) dma_tail(cur, j, next);
                else dma(cur, j, next);
              }
            }
          });
          __builtin_amdgcn_sched_barrier(0);
        });
        static_for<(kNext > kRest ? kNext - kRest : 0)>([&](auto rc) {
          read_frag(na, 0, 0, std::integral_constant<int, kRest + decltype(rc)::value>{});
        });
        __builtin_amdgcn_sched_barrier(0);
      }
    });
    cur = cur + 1 == Cfg::STAGES ? 0 : cur + 1;
  };

  static_assert(!PERSIST || Cfg::STAGES == 2, "the persistent form assumes a 2-deep ring");
  // The prologue copies K tiles 0 .. STAGES - 1. Then, per output tile,
  // three phases, each a loop over one instance of the body (an if/else of
  // two instances inside one loop costs registers): bodies that copy a
  // whole K tile; the one that copies the partial last K tile, if K has one
  // the prologue did not cover; bodies that copy the next output tile's
  // first K tiles (persistent form) or nothing.
  //
  // Persistent form (one workgroup per CU, output tiles blockIdx.x,
  // blockIdx.x + gridDim.x, ...; needs kfull >= STAGES): the ring carries on
  // across output tiles, so the next tile's first K tiles are in flight
  // during this tile's last K tiles and its epilogue. Vector-memory
  // operations complete in issue order, so the next tile's waits for its K
  // tiles 0 and 1 may leave this tile's stores outstanding: exactly
  // kStoresPerWave of them when the tile is interior; otherwise they also
  // wait for the stores.
#pragma unroll
  for (int s = 0; s < Cfg::STAGES; ++s) {
    if (!copier) {
    } else if (s < kfull) {
#pragma unroll
      for (int j = 0; j < Cfg::kSlabsPerWave; ++j) dma(s, j, s);
    } else if (s < ktiles) {
#pragma unroll
      for (int j = 0; j < Cfg::kSlabsPerWave; ++j) dma_tail(s, j, s);
    }
  }
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::kFragN; ++j) acc[i][j] = f32x16{};
  };
  // K tile 0 has landed (up to STAGES K tiles were issued, then maybe the
  // previous output tile's stores): make it visible, read its first step.
  auto start_tile = [&]() {
    if (stores_behind) wait_vmcnt<(Cfg::STAGES - 1) * Cfg::kSlabsPerWave + kStoresPerWave>();
    else if (Cfg::STAGES - 1 < ktiles) wait_vmcnt<(Cfg::STAGES - 1) * Cfg::kSlabsPerWave>();
    else wait_vmcnt<0>();
    barrier_lds();
    read_frags_from(smem + cur * Cfg::kStageBytes, 0, 0);
  };
  // Phases 1 and 2; returns the first K tile of the last phase.
  auto own_copies = [&]() {
    int kt = 0;
    for (; kt + Cfg::STAGES < kfull; ++kt) tile_body(kt, std::integral_constant<int, 1>{});
    if (kfull < ktiles && kt + Cfg::STAGES == kfull) {
      tile_body(kt, std::integral_constant<int, 2>{});
      ++kt;
    }
    return kt;
  };
  // acc[i][j] register r of lane l holds C[m][n] with m = row base + l%32
  // and n = column base + 8*(r/4) + 4*(l/32) + r%4: lanes l and l + 32 hold
  // alternate runs of 4 columns of the same row. v_permlane32_swap on the
  // pair of groups 2p and 2p + 1 gives lane l < 32 columns 16p .. +7 and
  // lane l + 32 columns 16p + 8 .. +15, written with one 16-byte store (half
  // the store instructions of 8-byte runs). RN swaps the f32 values (4 swaps
  // per 8 outputs); SR first rounds each lane's own runs of 4 (one Philox
  // call each, as the keying lays them out) and swaps the packed bf16 words
  // (2 swaps per 8 outputs; swapping the f32 values before SR measured
  // slower). The swaps run with every lane active, before the bounds
  // checks; runs that are ragged or unaligned fall back to 4-wide stores.
  // Compile-time loops keep every accumulator index constant (a runtime
  // index would move the accumulators to scratch memory).
  auto epilogue = [&](int64_t em0, int64_t en0, uint32_t e_row, uint32_t e_half) {
    if constexpr (ROUND != ASR_ROUND_RN && ASR_GEMM_SR_SWAP) {
      static_for<Cfg::kFragM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int64_t m = em0 + wm * Cfg::WM + i * 32 + e_row;
        static_for<Cfg::kFragN>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          static_for<2>([&](auto pc) {
            constexpr int qp = decltype(pc)::value;
            // this lane's own runs of 4 (groups 2qp and 2qp + 1), rounded
            const int64_t n0q = en0 + wn * Cfg::WN + j * 32 + 16 * qp + 4 * e_half;
            uint32_t w[2][2];
            float xs[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
              for (int e = 0; e < 4; ++e) xs[h][e] = acc[i][j][8 * qp + 4 * h + e];
              uint32_t r16[4];
              bits4(args.base_index + static_cast<uint64_t>(m) * static_cast<uint64_t>(args.n) +
                        static_cast<uint64_t>(n0q + 8 * h),
                    args.pos4 != 0, args.seed, args.step, r16);
              uint32_t hb[4];
              round4<ROUND>(xs[h], r16, hb);
              w[h][0] = hb[0] | (hb[1] << 16);
              w[h][1] = hb[2] | (hb[3] << 16);
            }
            // lane l < 32 then holds columns 16qp .. +7, lane l + 32 16qp + 8 .. +15
            const auto s0 = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
            // Both lanes of the pair must take the same branch: the 16-byte
            // stores write the partner's run too, so they are taken only when
            // all 16 columns of the pair are inside the row; otherwise each
            // lane writes its own two runs.
            const int64_t n16 = en0 + wn * Cfg::WN + j * 32 + 16 * qp;
            const int64_t n8 = n16 + 8 * e_half;
            if (m < args.m) {
              if (args.vec16 && !F32OUT && n16 + 16 <= args.n) {
                *reinterpret_cast<asr::u32x4*>(args.c + m * args.ldc + n8) =
                    asr::u32x4{s0[0], s1[0], s0[1], s1[1]};
              } else {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                  if (n0q + 8 * h < args.n) store_out<ROUND, F32OUT>(args, m, n0q + 8 * h, xs[h]);
              }
            }
          });
        });
      });
      return;
    }
    if constexpr (ROUND != ASR_ROUND_RN) {
      static_for<Cfg::kFragM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int64_t m = em0 + wm * Cfg::WM + i * 32 + e_row;
        if (m >= args.m) return;
        static_for<Cfg::kFragN>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          static_for<4>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            const int64_t n = en0 + wn * Cfg::WN + j * 32 + 8 * q + 4 * e_half;
            if (n >= args.n) return;
            const float x[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                acc[i][j][4 * q + 3]};
            store_out<ROUND, F32OUT>(args, m, n, x);
          });
        });
      });
      return;
    }
    static_for<Cfg::kFragM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int64_t m = em0 + wm * Cfg::WM + i * 32 + e_row;
      static_for<Cfg::kFragN>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        static_for<2>([&](auto pc) {
          constexpr int qp = decltype(pc)::value;
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const auto r = __builtin_amdgcn_permlane32_swap(
                __float_as_uint(acc[i][j][8 * qp + e]), __float_as_uint(acc[i][j][8 * qp + 4 + e]),
                false, false);
            x[e] = __uint_as_float(r[0]);
            x[4 + e] = __uint_as_float(r[1]);
          }
          const int64_t n = en0 + wn * Cfg::WN + j * 32 + 16 * qp + 8 * e_half;
          if (m < args.m && n < args.n) store_out8<ROUND, F32OUT>(args, m, n, x);
        });
      });
    });
  };

  if constexpr (!PERSIST) {
    zero_acc();
    if (ktiles > 0) start_tile();
    int kt = own_copies();
    for (; kt < ktiles; ++kt) tile_body(kt, std::integral_constant<int, 0>{});
    epilogue(m0, n0, frag_row, frag_half);
  } else {
    for (;;) {
      const int64_t em0 = m0, en0 = n0;  // this output tile
      const uint32_t next_tile = tile + gridDim.x;
      has_next = next_tile < args.tiles_m * args.tiles_n;
      zero_acc();
      start_tile();  // (ktiles >= STAGES here)
      int kt = own_copies();
      aim_copies(has_next ? next_tile : tile);  // (no copies are issued without a next tile)
      for (; kt < ktiles; ++kt) tile_body(kt, std::integral_constant<int, 3>{});
      // The lane index goes through an empty asm so that no part of the
      // store addresses is hoisted out of the tile loop (it would stay live
      // through the K loop).
      uint32_t el = lane;
      asm volatile("" : "+v"(el));
      epilogue(em0, en0, el & 31u, el >> 5);
      if (!has_next) break;
      stores_behind = em0 + BM <= args.m && en0 + BN <= args.n;
      tile = next_tile;
    }
  }
}

#ifndef ASR_GEMM_BIG
#define ASR_GEMM_BIG 256, 256, 128, 64, 64, 2
#endif
#ifndef ASR_GEMM_SMALL
#define ASR_GEMM_SMALL 128, 128, 64, 64, 64, 2
#endif
#ifndef ASR_GEMM_SMALL8
#define ASR_GEMM_SMALL8 128, 128, 64, 32, 64, 3
#endif
#ifndef ASR_GEMM_TINY
#define ASR_GEMM_TINY 64, 64, 32, 32, 64, 4
#endif
#ifndef ASR_GEMM_PERSIST
#define ASR_GEMM_PERSIST 1
#endif
#ifndef ASR_GEMM_SMALL_WAVES8
#define ASR_GEMM_SMALL_WAVES8 1
#endif
#ifndef ASR_GEMM_USE_TINY
#define ASR_GEMM_USE_TINY 1
#endif
#ifndef ASR_GEMM_TINY_DIV
#define ASR_GEMM_TINY_DIV 2
#endif
using Big = TileCfg<ASR_GEMM_BIG>;        // 8 waves, 2 per SIMD
using Small = TileCfg<ASR_GEMM_SMALL>;    // 4 waves, for grids too small for Big
using Small8 = TileCfg<ASR_GEMM_SMALL8>;  // the same tile in 8 waves, for at most one tile per CU
using Tiny = TileCfg<ASR_GEMM_TINY>;      // 4 waves of 32 x 32, for grids of up to half as many tiles as CUs

}  // namespace asr_gemm

// =========================================================== host side
namespace {

using asr_host::fail;
using asr_host::hip_fail;
using asr_host::ok;

bool aligned_to(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Compute units of the current device (cached per device, safe to call from
// several threads; 0 if unknown).
int cu_count() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Launches one workgroup per output tile, or with `persist_grid` > 0 that
// many workgroups, each looping over output tiles.
template <typename Cfg, int ROUND, bool F32OUT, bool PERSIST>
hipError_t launch_gemm(asr_gemm::GemmArgs args, uint32_t persist_grid, hipStream_t stream) {
  args.tiles_m = static_cast<uint32_t>((args.m + Cfg::BM - 1) / Cfg::BM);
  args.tiles_n = static_cast<uint32_t>((args.n + Cfg::BN - 1) / Cfg::BN);
  const uint64_t tiles = static_cast<uint64_t>(args.tiles_m) * args.tiles_n;
  const uint32_t grid = PERSIST ? persist_grid : static_cast<uint32_t>(tiles);
  void* argv[] = {&args};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&asr_gemm::gemm_bf16<Cfg, ROUND, F32OUT, PERSIST>),
      dim3(grid), dim3(Cfg::kThreads), argv, 0, stream);
}

template <typename Cfg, bool PERSIST>
hipError_t dispatch(const asr_gemm::GemmArgs& args, int32_t rounding, uint32_t persist_grid,
                    hipStream_t stream) {
  const bool f32 = args.c32 != nullptr;
  if (rounding == ASR_ROUND_SR)
    return f32 ? launch_gemm<Cfg, ASR_ROUND_SR, true, PERSIST>(args, persist_grid, stream)
               : launch_gemm<Cfg, ASR_ROUND_SR, false, PERSIST>(args, persist_grid, stream);
  return f32 ? launch_gemm<Cfg, ASR_ROUND_RN, true, PERSIST>(args, persist_grid, stream)
             : launch_gemm<Cfg, ASR_ROUND_RN, false, PERSIST>(args, persist_grid, stream);
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
  // the copies address a tile's rows by byte offsets below 2**31 from its first row
  if (lda >= (int64_t{1} << 22) || ldb >= (int64_t{1} << 22))
    return fail(ASR_EINVAL, "gemm: lda and ldb must be below 2**22");
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
  args.vec16 = ldc % 8 == 0 && aligned_to(c, 16) && (!c_f32 || aligned_to(c_f32, 16));
  args.pos4 = (base_index % 4 == 0) && (n % 4 == 0);

  const uint64_t big_tiles = static_cast<uint64_t>((m + 255) / 256) * ((n + 255) / 256);
  const uint64_t small_tiles = static_cast<uint64_t>((m + 127) / 128) * ((n + 127) / 128);
  if (small_tiles > 0x7FFFFFFFull) return fail(ASR_EINVAL, "gemm: too many tiles");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The big tile halves the LDS and L2 traffic per flop; it needs enough
  // tiles to give every CU at least one. With more tiles than CUs (one big
  // tile fills a CU's LDS) the persistent form runs one workgroup per CU;
  // it needs STAGES whole K tiles.
  const int cus = cu_count();
  const bool persist = ASR_GEMM_PERSIST && cus > 0 && big_tiles > static_cast<uint64_t>(cus) &&
                       k / asr_gemm::Big::BK >= asr_gemm::Big::STAGES;
  // With no more 128 x 128 tiles than CUs, each CU runs about one small
  // workgroup, so the tile runs as 8 waves (two per SIMD, one hiding the
  // other's latency); with more tiles, 4-wave workgroups share the CUs.
  const bool small8 = ASR_GEMM_SMALL_WAVES8 && cus > 0 && small_tiles <= static_cast<uint64_t>(cus);
  const bool tiny = ASR_GEMM_USE_TINY && cus > 0 && small_tiles * ASR_GEMM_TINY_DIV <= static_cast<uint64_t>(cus);
  hipError_t e;
  if (big_tiles < 256 && tiny) e = dispatch<asr_gemm::Tiny, false>(args, rounding, 0, s);
  else if (big_tiles < 256 && small8) e = dispatch<asr_gemm::Small8, false>(args, rounding, 0, s);
  else if (big_tiles < 256) e = dispatch<asr_gemm::Small, false>(args, rounding, 0, s);
  else if (persist) e = dispatch<asr_gemm::Big, true>(args, rounding, static_cast<uint32_t>(cus), s);
  else e = dispatch<asr_gemm::Big, false>(args, rounding, 0, s);
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return ok();
}

}  // extern "C"

/*
 * adamw_sr.h -- C ABI of the fused AdamW step with stochastic-rounding bf16
 * write-back, for AMD Instinct MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *   - "adamw-sr" (kernels hub page), intro, Usage, Method, Correctness:
 *     a decoupled-weight-decay Adam step with float32 moment states, f32 or
 *     bf16 parameters and gradients, bf16 parameters written back by
 *     unbiased stochastic rounding with no fp32 master copy; the random bits
 *     come from a counter-based Philox whose key is the pair (seed, step)
 *     and whose counter is derived from the element's position in the whole
 *     parameter set, so a tensor updated in one piece or in shards (each
 *     shard passing the position of its first element) gets the same bits;
 *   - "Add stochastic rounding and philox RNG helpers" (FlyDSL pull request),
 *     Primitives: philox_4x32(counter, key) -> four 32-bit words, and
 *     stochastic rounding f32 -> bf16 by adding 16 random bits to the 16
 *     dropped mantissa bits and truncating; discussion: stochastic rounding
 *     as a rounding mode of the narrowing conversion.
 *
 * Conventions shared by every entry point:
 *   - All device pointers are HIP device (or managed) memory owned by the
 *     caller; the library allocates no device memory and keeps no generator
 *     state (the generator is counter-based).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream of
 *     the current device). The current device must be the stream's device.
 *     Work is enqueued asynchronously; no call synchronizes the host. A
 *     device-side fault surfaces at the caller's next synchronization.
 *   - Every call returns an asr_status. On a non-zero status nothing was
 *     enqueued (argument errors are found before any launch) unless the
 *     status is ASR_EHIP, and asr_last_error() describes the problem.
 *   - Element counts are int64_t; global positions are uint64_t and wrap
 *     modulo 2**64.
 *
 * Random-bit contract (the "stream"), used by asr_adamw_step and
 * asr_cvt_f32_bf16_sr: element i of a tensor whose first element sits at
 * global position base_index has position p = base_index + i (64-bit).
 * Its 16 random bits are the low 16 bits of word (p & 3) of
 * Philox4x32-10(counter = (lo32(p >> 2), hi32(p >> 2), 0, 0),
 *              key     = (seed, step)).
 * Philox4x32-10 is the published generator of Salmon et al. (SC 2011):
 * multipliers 0xD2511F53 (word 0) and 0xCD9E8D57 (word 2), key bumps
 * 0x9E3779B9 and 0xBB67AE85, 10 rounds.
 *
 * Rounding rules (bit patterns u of f32, results are bf16 patterns):
 *   SR: NaN -> (u >> 16) | 0x0040 (stays NaN, sign and top payload kept);
 *       otherwise (u + r16) >> 16 in 32-bit arithmetic.
 *   RN: NaN as above; otherwise round to nearest, ties to even.
 */
#ifndef ADAMW_SR_H
#define ADAMW_SR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum asr_status {
  ASR_OK = 0,
  ASR_EINVAL = 1,     /* an argument value is out of its documented range      */
  ASR_EDTYPE = 2,     /* a dtype code is neither ASR_F32 nor ASR_BF16          */
  ASR_EALIGN = 3,     /* a pointer is not aligned to its element size          */
  ASR_EWORKSPACE = 4, /* workspace NULL, smaller than required, or misaligned  */
  ASR_EHIP = 5        /* the HIP runtime reported an error (see last_error)    */
} asr_status;

enum { ASR_F32 = 0, ASR_BF16 = 1 };
enum { ASR_ROUND_SR = 0, ASR_ROUND_RN = 1 };

/* One tensor of the optimizer's list, flattened and contiguous. */
typedef struct asr_tensor {
  void* param;          /* numel elements of param_dtype, updated in place   */
  const void* grad;     /* numel elements of grad_dtype, read only           */
  float* exp_avg;       /* numel f32: first moment m, updated in place       */
  float* exp_avg_sq;    /* numel f32: second moment v, updated in place      */
  int64_t numel;        /* >= 0; a tensor with numel 0 is skipped            */
  uint64_t base_index;  /* global position of element 0 (random-bit stream)  */
  int32_t param_dtype;  /* ASR_F32 | ASR_BF16                                */
  int32_t grad_dtype;   /* ASR_F32 | ASR_BF16                                */
} asr_tensor;

/* Bytes of device workspace asr_adamw_step needs for this list (0 when
 * n_tensors <= 0 or tensors is NULL). Only the count of tensors and their
 * numel matter, so the size stays valid across steps of a fixed list. The
 * workspace holds the list's metadata and a table of one 32-bit entry per
 * 1,024-element slot (under 0.4% of the bf16 parameter bytes). A step whose
 * launches each cover at most 48 tensors (any list of at most 48 tensors)
 * passes the metadata in its kernel arguments and leaves the workspace
 * untouched; the workspace is still required. */
size_t asr_adamw_workspace_bytes(const asr_tensor* tensors, int32_t n_tensors);

/*
 * One AdamW step over a list of tensors, in one pass over memory.
 * ("adamw-sr" page: intro, Usage, Method, Correctness.)
 *
 * For every element, in binary32, each operation rounded to nearest even
 * and never fused into a multiply-add:
 *     m   = b1*m + omb1*g
 *     v   = b2*v + omb2*(g*g)
 *     p   = p*decay - step_size * (m / (sqrt(v)*inv_bc2_sqrt + eps32))
 * where g and p are the gradient and parameter upcast exactly to f32, and the
 * constants are formed once per call in binary64 (bc1 = 1 - beta1**step,
 * bc2 = 1 - beta2**step by binary powering) and rounded to binary32:
 *     decay = 1 - lr*weight_decay, b1 = beta1, omb1 = 1 - beta1, b2 = beta2,
 *     omb2 = 1 - beta2, step_size = lr/bc1, inv_bc2_sqrt = 1/sqrt(bc2),
 *     eps32 = eps    (asr_adamw_host_scalars returns them).
 * m and v are stored as f32. An f32 parameter is stored as computed; a bf16
 * parameter is rounded by SR (rounding = ASR_ROUND_SR; key (seed, step),
 * position base_index + i) or by RN (ASR_ROUND_RN).
 *
 * tensors      host array of n_tensors descriptors (read during the call only);
 *              the param, grad, exp_avg and exp_avg_sq buffers of all tensors
 *              must be pairwise disjoint (not checked here; the Python
 *              binding checks).
 * lr           >= 0, finite.       beta1, beta2   in [0, 1).
 * eps          >= 0, finite.       weight_decay   >= 0, finite.
 * step         1-based step count t, in [1, 2**32 - 1]; used for the bias
 *              corrections and as key word 1.
 * seed         key word 0.
 * workspace    device buffer of at least asr_adamw_workspace_bytes(tensors,
 *              n_tensors) bytes, 16-byte aligned, owned by the caller. Its
 *              contents are overwritten (stream-ordered); it must not be used
 *              by other work that runs concurrently with this step.
 * Errors: ASR_EINVAL (n_tensors < 0, NULL tensors with n_tensors > 0,
 * numel < 0, a NULL buffer in a non-empty tensor, hyperparameter or step out
 * of range, rounding code unknown, more than 2**32 slots of 1,024 elements
 * of one dtype pair), ASR_EDTYPE, ASR_EALIGN (param/grad not aligned to 2 or 4 bytes as
 * their dtype needs, m/v not 4-byte aligned), ASR_EWORKSPACE, ASR_EHIP.
 * Layout of the work: each tensor is walked in runs of 4 consecutive
 * elements, one run per GPU lane, shifted by s elements (0 <= s < 4) so
 * that every whole run starts on a vector-aligned address of all four
 * buffers (16 bytes for f32, 8 for bf16) -- a tensor cut out of aligned
 * buffers at any element offset has such a shift. Whole runs move with
 * vector accesses; the cut runs at either end, and every run of a tensor
 * whose buffers are misaligned against each other (no such shift), move
 * element by element. The results are the same either way.
 */
int asr_adamw_step(const asr_tensor* tensors, int32_t n_tensors,
                   double lr, double beta1, double beta2, double eps,
                   double weight_decay, int64_t step, uint32_t seed,
                   int32_t rounding, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * asr_adamw_step without a workspace argument, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc. The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine): its
 * kernels use a static device array of 4 MiB ("scratch", one copy per GPU,
 * held until the process ends) in place of the workspace, found on the
 * first call on each device with that device current. Results are those
 * of asr_adamw_step bit for bit (the same kernels).
 * Limit: the list's metadata (60 bytes per tensor plus a few hundred) plus
 * a 4-byte slot-table entry per 1,024 elements of the tensors that are not
 * in a size class must fit in 4 MiB (a Llama-3-8B list needs about 18 KiB);
 * a larger list is rejected with ASR_EWORKSPACE before anything is
 * enqueued. Nothing in the scratch needs to start at zero: each call
 * writes all it reads. All calls on one GPU share its scratch, so calls
 * that may overlap on one GPU (other streams, other threads, several
 * replays of graphs in flight at once) race: order them on one stream.
 * Other arguments and errors as for asr_adamw_step.
 */
int asr_adamw_step_noalloc(const asr_tensor* tensors, int32_t n_tensors,
                           double lr, double beta1, double beta2, double eps,
                           double weight_decay, int64_t step, uint32_t seed,
                           int32_t rounding, void* stream);

/*
 * The eight binary32 constants asr_adamw_step uses for these
 * hyperparameters, in this order: decay, b1, omb1, b2, omb2, step_size,
 * inv_bc2_sqrt, eps32 (see asr_adamw_step). Host only; touches no device.
 * out: host array of 8 floats. Errors: ASR_EINVAL as for asr_adamw_step.
 */
int asr_adamw_host_scalars(double lr, double beta1, double beta2, double eps,
                           double weight_decay, int64_t step, float* out);

/*
 * Philox4x32-10 words of n_counters consecutive counters.
 * ("Add stochastic rounding and philox RNG helpers", Primitives.)
 * Call k (0 <= k < n_counters) uses counter
 *   (lo32(c), hi32(c), lo32(counter_upper), hi32(counter_upper)),
 *   c = counter_base + k (mod 2**64),
 * and key (seed, step); its words 0..3 go to out[4k .. 4k+3].
 * With counter_upper = 0 these are the calls of the random-bit stream.
 * out: device buffer of 4*n_counters uint32, 4-byte aligned.
 * Errors: ASR_EINVAL (n_counters < 0, out NULL with n_counters > 0),
 * ASR_EALIGN, ASR_EHIP.
 */
int asr_philox_4x32_fill(uint32_t* out, int64_t n_counters,
                         uint64_t counter_base, uint64_t counter_upper,
                         uint32_t seed, uint32_t step, void* stream);

/*
 * Stochastic-rounding conversion f32 -> bf16 of n elements.
 * ("Add stochastic rounding and philox RNG helpers", Primitives and
 * discussion: SR as a rounding mode of the conversion.)
 * out[i] = SR(in[i], r16(base_index + i)) with key (seed, step).
 * in: device, n f32, 4-byte aligned; out: device, n bf16 patterns, 2-byte
 * aligned; in and out must not overlap.
 * Errors: ASR_EINVAL (n < 0, NULL buffer with n > 0), ASR_EALIGN, ASR_EHIP.
 */
int asr_cvt_f32_bf16_sr(const float* in, uint16_t* out, int64_t n,
                        uint32_t seed, uint32_t step, uint64_t base_index,
                        void* stream);

/*
 * Round-to-nearest-even conversion f32 -> bf16 (the comparison mode; the
 * FlyDSL page's Consumer section keeps "rn" as the default rounding).
 * Same buffers and errors as asr_cvt_f32_bf16_sr.
 */
int asr_cvt_f32_bf16_rn(const float* in, uint16_t* out, int64_t n,
                        void* stream);

/*
 * Stochastic rounding f32 -> bf16 with the random bits supplied by the
 * caller: out[i] = SR(x[i], r16[i]) under the rule at the top of this file.
 * ("Add stochastic rounding and philox RNG helpers", Primitives: the
 * rounding primitive takes its random bits as an input.) The same device
 * rounding as asr_adamw_step and asr_cvt_f32_bf16_sr, so it is the hook
 * that checks the rounding apart from the generator.
 * x: device, n f32; r16: device, n uint16 random values; out: device, n bf16
 * patterns. Natural alignment. Errors: ASR_EINVAL, ASR_EALIGN, ASR_EHIP.
 */
int asr_sr_bf16_given_bits(const float* x, const uint16_t* r16, uint16_t* out,
                           int64_t n, void* stream);

/*
 * bf16 GEMM with a stochastic-rounding (or round-to-nearest) epilogue.
 * ("Add stochastic rounding and philox RNG helpers", Consumer section: the f32
 * accumulator of a bf16 GEMM is converted to bf16 by SR keyed per output
 * element from a seed, RN being the other rounding; Tests: SR within
 * tolerance of RN, seed-dependent, reproducible.)
 *
 *   C[m][n] = round( sum_k A[m][k] * B[n][k] )     0 <= m < M, 0 <= n < N
 *
 * i.e. C = A * B^T with A (M x K) and B (N x K) both row-major, K
 * contiguous (the layout of x and W in a linear layer y = x W^T). The sum
 * is accumulated in f32 on the matrix cores in an order of the library's
 * choosing (fixed for given M, N, K, so results are reproducible).
 * rounding ASR_ROUND_SR: element (m, n) is rounded with the 16 random bits
 * of stream position base_index + m*N + n under key (seed, step) -- the
 * stream and rule of asr_cvt_f32_bf16_sr, so C equals that conversion of
 * the f32 result bit for bit, and a block of rows [r0, r1) computed alone
 * with base_index + r0*N reproduces those rows of the whole product.
 * rounding ASR_ROUND_RN: round to nearest even (seed, step, base_index
 * unused).
 *
 * a: device bf16 patterns, row m at a + m*lda; b: device, row n at
 * b + n*ldb; c: device bf16 patterns, row m at c + m*ldc; c_f32: NULL, or
 * a device f32 buffer with the same row stride ldc that receives the
 * unrounded f32 result. No output may overlap an input.
 * Requirements: 0 <= M, N, K < 2**31; K, lda, ldb multiples of 8;
 * K <= lda < 2**22, K <= ldb < 2**22, ldc >= N; a and b 16-byte aligned; c and c_f32 aligned to
 * their element size; base_index + M*N <= 2**64. M or N = 0 writes
 * nothing; K = 0 writes zeros.
 * Errors: ASR_EINVAL (sizes, strides, rounding, NULL), ASR_EALIGN,
 * ASR_EHIP (launch failure). Runs on `stream`; does not synchronize.
 */
int asr_gemm_bf16(const uint16_t* a, int64_t lda, const uint16_t* b,
                  int64_t ldb, uint16_t* c, int64_t ldc, float* c_f32,
                  int64_t m, int64_t n, int64_t k, int32_t rounding,
                  uint32_t seed, uint32_t step, uint64_t base_index,
                  void* stream);

/*
 * Random numbers on the library's stream, beyond rounding.
 * ("Add stochastic rounding and philox RNG helpers", discussion: the
 * counter-based generator as a general facility for dropout and
 * initialisation; "adamw-sr", Method: keyed by (seed, step), indexed by the
 * global position of the element.)
 * Position p = base_index + i takes 32-bit word W = word p & 3 of the
 * Philox4x32-10 call with counter (lo32(p >> 2), hi32(p >> 2), 0, 0) and key
 * (seed, step) -- the stream asr_philox_4x32_fill writes. All arithmetic is
 * binary32 without contraction; an ASR_BF16 output is the round-to-nearest-
 * even of the binary32 value. A tensor split into pieces that each pass
 * their own base_index reproduces the whole bit for bit.
 *
 * asr_random_uniform: out[i] = f32(low) + f32(high - low) * U,
 *   U = (W >> 8) * 2**-24 in [0, 1). low, high and high - low finite in
 *   binary32.
 * asr_random_normal: Box-Muller on position pairs (2q, 2q + 1):
 *   u1 = ((W(2q) >> 8) + 1) * 2**-24, u2 = (W(2q + 1) >> 8) * 2**-24,
 *   r = sqrt(-2 ln u1); z(2q) = r cos(2 pi u2), z(2q + 1) = r sin(2 pi u2);
 *   out[i] = f32(mean) + f32(std) * z. ln is 2 ln 2 * |log2|, and log2,
 *   sin and cos are gfx950's transcendental instructions (v_log_f32,
 *   v_sin_f32, v_cos_f32), whose error over every input they can receive
 *   here is measured by asr_box_muller_given_words; values are reproducible
 *   on this library but not bit-identical to other implementations.
 *   mean and std finite in binary32, std >= 0.
 * asr_dropout: drop probability p in [0, 1). Element i is dropped when
 *   W < floor(p * 2**32); y[i] = x[i] * (dropped ? 0 : f32(1 / (1 - p))), one
 *   binary32 multiply (a dropped Inf or NaN gives NaN, a dropped negative
 *   value -0). mask: NULL, or n bytes receiving 1 for kept, 0 for dropped.
 *   x and y may be the same buffer (in place).
 *
 * out, x, y: device, n elements of dtype (ASR_F32 or ASR_BF16), aligned to
 * the element size (16-byte f32 / 8-byte bf16 alignment takes the vector
 * path). Errors: ASR_EDTYPE, ASR_EINVAL (sizes, parameters, NULL),
 * ASR_EALIGN, ASR_EHIP. Run on `stream`; do not synchronize.
 */
int asr_random_uniform(void* out, int32_t dtype, int64_t n, double low,
                       double high, uint32_t seed, uint32_t step,
                       uint64_t base_index, void* stream);
int asr_random_normal(void* out, int32_t dtype, int64_t n, double mean,
                      double std, uint32_t seed, uint32_t step,
                      uint64_t base_index, void* stream);
int asr_dropout(const void* x, void* y, uint8_t* mask, int32_t dtype,
                int64_t n, double p, uint32_t seed, uint32_t step,
                uint64_t base_index, void* stream);

/*
 * Measurement support: copies `bytes` bytes from src to dst with a kernel
 * built like the AdamW step (one slot of 16 KiB per workgroup, 128-bit loads
 * and stores, the step's residency cap; one address window per XCD). The benchmark
 * quotes the step's bandwidth against this copy's as well as against the
 * HBM peak. src, dst: device, 16-byte aligned, not overlapping; bytes a
 * multiple of 16. Errors: ASR_EINVAL, ASR_EALIGN, ASR_EHIP.
 */
int asr_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);

/*
 * Measurement support: what HBM gives a plain stream under the launch
 * structure of asr_stream_copy (16 KiB slot per workgroup, 128-bit
 * accesses, XCD windows, residency cap). The benchmark reports these
 * beside the AdamW step as the memory ceiling it is measured against.
 *   ASR_PROBE_READ   reads `bytes` bytes of src. Fill src with equal 16-byte
 *                    words (e.g. all bytes alike): the kernel then writes
 *                    nothing; dst is a 16-byte sink that it could write
 *                    otherwise.
 *   ASR_PROBE_WRITE  writes `bytes` bytes of dst (src unused, may be NULL).
 *   ASR_PROBE_COPY   asr_stream_copy(dst, src, bytes).
 * Buffers device, 16-byte aligned; bytes a multiple of 16.
 * Errors: ASR_EINVAL (kind, bytes < 0, NULL), ASR_EALIGN, ASR_EHIP.
 */
enum { ASR_PROBE_READ = 0, ASR_PROBE_WRITE = 1, ASR_PROBE_COPY = 2 };
int asr_hbm_probe(int32_t kind, void* dst, const void* src, int64_t bytes,
                  void* stream);

/*
 * Measurement support: the memory traffic of asr_adamw_step over this list
 * without its arithmetic -- the same launch plan, slots, runs, vector and
 * element accesses, windows and residency cap, reading param, grad,
 * exp_avg and exp_avg_sq and writing param, exp_avg and exp_avg_sq of
 * every element, with param := param XOR grad (for a bf16 param, the high
 * halves of the upcast values) and the moments written back as read. It
 * DESTROYS the parameters; it is a bandwidth probe of the step's access
 * pattern (four streams read, three written), not an optimizer.
 * Arguments, workspace and errors as for asr_adamw_step.
 */
int asr_adamw_stream_probe(const asr_tensor* tensors, int32_t n_tensors,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Test support: the Box-Muller pair of asr_random_normal from given words:
 * zc[i], zs[i] = r cos(2 pi u2), r sin(2 pi u2) with u1, u2 from
 * w_even[i], w_odd[i] as above -- the same device function, so its error
 * can be measured over every possible input. All buffers: device, n
 * 4-byte elements. Errors: ASR_EINVAL, ASR_EALIGN, ASR_EHIP.
 */
int asr_box_muller_given_words(const uint32_t* w_even, const uint32_t* w_odd,
                               float* zc, float* zs, int64_t n, void* stream);

/*
 * Test support: the binary32 square root and division exactly as the AdamW
 * kernel evaluates them: sqrt_out[i] = sqrt(a[i]), div_out[i] = a[i] / b[i],
 * both correctly rounded (to nearest even, subnormals kept).
 * All buffers: device, n floats, 4-byte aligned.
 * Errors: ASR_EINVAL, ASR_EALIGN, ASR_EHIP.
 */
int asr_f32_sqrt_div(const float* a, const float* b, float* sqrt_out,
                     float* div_out, int64_t n, void* stream);

/* Text for the last non-OK status returned on this thread ("" if none). The
 * pointer stays valid until the next library call on this thread. */
const char* asr_last_error(void);

/* ABI version of this header and library (major * 100 + minor). */
int asr_abi_version(void);

#define ASR_ABI_VERSION 107

#ifdef __cplusplus
}
#endif

#endif /* ADAMW_SR_H */

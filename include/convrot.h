/*
 * convrot.h -- C ABI of the MI355X (gfx950) int8_tensorwise "convrot" linear layer.
 *
 * The layer (as the pages describe it):
 *   - weights are stored int8 after a rotation of their input axis in g-wide
 *     groups, with one fp32 scale per tensor (convert_to_quant guide, "What is
 *     INT8 ConvRot?" and "How INT8 ConvRot Quantization Works");
 *   - the default path dequantizes and derotates the weight on every forward
 *     as an [out, in/g, g] @ [g, g] block matmul, then runs a bf16 linear
 *     (PR "share the int8_convrot scheme ... Krea-2 and Z-Image", "What it is
 *     worth");
 *   - int8_compute rotates the input, quantizes it to int8 per token and
 *     multiplies int8 by int8, slicing the tokens so that its working memory
 *     stays within the default path's (Invoke docs "int8 Compute",
 *     introduction and "Memory").
 *
 * The rotation R is not printed on the pages. This library fixes
 *   R = H_g . diag(d) / sqrt(g),  g in {4, 16, 64, 256},
 * with H_g Sylvester's Hadamard matrix (H[i][j] = (-1)^popcount(i & j)) and
 * d[i] = -1 where bit 63 of SplitMix64 output i (counter form:
 * mix(rot_seed + (i + 1) * 0x9E3779B97F4A7C15)) is set, else +1. The same R
 * serves every group of every layer and both paths. `g` and `rot_seed` must
 * be the same at quantize time and at use time; a mismatch is not detectable
 * here, and decoding with the wrong rotation raises no error but gives noise
 * (PR "share the int8_convrot scheme ... Krea-2 and Z-Image", QA Instructions).
 *
 * Numerics (bit-exact contract):
 *   x_r  = each rotated element is the exact sum rounded once to fp32
 *          (nearest-even);
 *   s    = RN(amax / 127), inv = RN(127 / amax) (amax and the values scaled by
 *          2^64 first when amax < 2^-64), q = rint_even(RN(x_r * inv)), so
 *          |q| <= 127; amax == 0 gives s = 0 and q = 0;
 *   W_hat = bf16(RN(float(S) * RN(s_w * 2^-log2(sqrt g)))), S = (Wq . D) . H;
 *   y    = bf16(RN(RN(float(acc) * s_w) * s_x[m]) [+ bias[n] in fp32]).
 *
 * Per-output-channel weight scales (the *_per_channel entry points): s_w is a
 * vector of n fp32, one per row of W (= per output column of y). Row r of the
 * rotated weight is quantized with its own amax exactly as a token row is;
 * the dequant uses RN(s_w[r] * 2^-log2(sqrt g)) for row r and the epilogue
 * s_w[n] for column n. Published int8 convrot checkpoints carry one scale per
 * output channel, and a weight scale always multiplies output rows, never the
 * input axis (PR "share the int8_convrot scheme ... Krea-2 and Z-Image",
 * "Z-Image: the fused QKV", and the scale-layout fix in its commits: a scale
 * broadcast along the input axis decodes square weights wrongly).
 * These vectors must be 16-byte aligned.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers to row-major, contiguous memory whose
 *     last axis is K (input features). bf16 tensors are passed as uint16_t*.
 *     Scales (s_w, s_x) live in device memory too.
 *   - The caller owns every buffer. The library allocates and frees nothing
 *     and keeps no state between calls (apart from a per-thread error string),
 *     except for the convrot_streamer object below, which owns its staging
 *     memory, copy stream and events from create to destroy.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; the library never synchronizes. The
 *     return value covers argument checks and launch errors; a fault inside a
 *     kernel surfaces at the caller's next synchronization.
 *   - Arguments are checked before anything is launched. On any error nothing
 *     is enqueued and no output is touched.
 *   - Shapes: K % 64 == 0, K % g == 0, K <= 16384 for the rotating entry points;
 *     N % 16 == 0 and K <= 133144 (int32 accumulator bound) for the GEMM;
 *     all dimensions < 2^31, and ceil(M/128) * ceil(N/128) < 2^31 for the
 *     GEMM. M == 0 is a no-op (the M-sized buffers may then be null).
 *   - Alignment: tensor base pointers 16-byte aligned, per-tensor scales and
 *     s_x 4-byte aligned, per-channel scale vectors 16-byte aligned.
 *   - Results are bit-identical from run to run and independent of slicing.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CONVROT_ABI_VERSION 7

typedef enum convrot_status {
  CONVROT_OK = 0,
  CONVROT_E_INVALID_ARG = 1,       /* null pointer, negative or zero dim, overlapping in/out  */
  CONVROT_E_UNSUPPORTED_GROUP = 2, /* g not in {4,16,64,256}, or K % g != 0                   */
  CONVROT_E_UNSUPPORTED_SHAPE = 3, /* a shape limit above is not met                          */
  CONVROT_E_MISALIGNED = 4,        /* a pointer is not aligned as required                    */
  CONVROT_E_WORKSPACE = 5,         /* workspace too small for one token row                   */
  CONVROT_E_HIP = 6,               /* a HIP call failed; see convrot_last_error_string()      */
  CONVROT_E_SELFCHECK = 7          /* a session's first-call check failed (latched)           */
} convrot_status;

/* 16-bit float format of activations, bias, outputs and W_hat (the *_ex
 * entry points). The pages' kernels run in BF16 and FP16 (Invoke docs "int8
 * Compute", the table of layers that keep unpacking). With FP16 every step is
 * the same; only the input decoding and the final rounding (to nearest even,
 * overflow to inf) change. IEEE half inputs never need the exact row pass:
 * each value is a multiple of 2^-24 below 2^16, so the float64 transform of a
 * group is exact. Non-finite inputs are out of contract for both formats. */
typedef enum convrot_dtype { CONVROT_DTYPE_BF16 = 0, CONVROT_DTYPE_F16 = 1 } convrot_dtype;

/* Weight scale granularity (the *_ex entry points): one fp32 for the tensor,
 * or one per output channel (n fp32, 16-byte aligned; see above). */
typedef enum convrot_scale_mode {
  CONVROT_SCALE_PER_TENSOR = 0,
  CONVROT_SCALE_PER_CHANNEL = 1
} convrot_scale_mode;

/* Rotate, absmax and quantize a weight to int8 with one scale per tensor.
 *   w   [n, k] bf16 (in)     the unquantized weight (out features x in features)
 *   wq  [n, k] int8 (out)    Wq = q(W . blockdiag(R)) under the numerics above
 *   s_w [1]    fp32 (out)    s_w = RN(amax / 127) over the whole rotated tensor
 * Offline step of the format (convert_to_quant guide, "How INT8 ConvRot
 * Quantization Works": --int8 --scaling_mode tensor --convrot
 * --convrot-group-size). s_w's slot is also used as scratch while the call
 * runs, so no other work may read it meanwhile. */
convrot_status convrot_quantize_weights(const uint16_t* w, int64_t n, int64_t k, int g,
                                        uint64_t rot_seed, int8_t* wq, float* s_w,
                                        void* stream);

/* Dequantize and derotate an int8 weight to bf16 (the default path's per-forward
 * decode: PR "share the int8_convrot scheme ... Krea-2 and Z-Image", "What it is
 * worth": an [out, in/g, g] @ [g, g] block matmul after the scale).
 *   wq    [n, k] int8 (in), s_w [1] fp32 (in)
 *   w_out [n, k] bf16 (out)  W_hat = s_w . Wq . blockdiag(R)^T, rounded as above */
convrot_status convrot_dequant_derotate(const int8_t* wq, const float* s_w, int64_t n, int64_t k,
                                        int g, uint64_t rot_seed, uint16_t* w_out, void* stream);

/* Per-channel variant of convrot_quantize_weights: s_w [n] fp32 (out, 16-byte
 * aligned), s_w[r] = RN(amax_r / 127) over row r of the rotated weight; row r of
 * wq is quantized with s_w[r]. Same kernels as convrot_quantize_activations. */
convrot_status convrot_quantize_weights_per_channel(const uint16_t* w, int64_t n, int64_t k,
                                                    int g, uint64_t rot_seed, int8_t* wq,
                                                    float* s_w, void* stream);

/* Per-channel variant of convrot_dequant_derotate: s_w [n] fp32 (in, 16-byte
 * aligned); row r of w_out is bf16(RN(float(S) * RN(s_w[r] * 2^-log2(sqrt g)))). */
convrot_status convrot_dequant_derotate_per_channel(const int8_t* wq, const float* s_w, int64_t n,
                                                    int64_t k, int g, uint64_t rot_seed,
                                                    uint16_t* w_out, void* stream);

/* Dequantize + derotate several weights in one launch (the default path
 * decodes every weight of a model on each forward: PR "share the
 * int8_convrot scheme ... Krea-2 and Z-Image", "What it is worth"; one launch
 * for many layers spares each small layer the fixed cost of its own launch).
 * Each job is convrot_dequant_derotate_ex on its own weight; all jobs share
 * g, rot_seed, scale_mode and out_dtype:
 *   wq    [n, k] int8 (in, device, 16-byte aligned)
 *   s_w   [1] or, per channel, [n] fp32 (in, device; 16-byte aligned per channel)
 *   w_out [n, k] in out_dtype (out, device, 16-byte aligned)
 * `jobs` is an array of njobs descriptors in HOST memory, read during the
 * call only: the library copies them into the kernel arguments (up to 48
 * weights per launch; longer lists take several launches, in order). The
 * call allocates nothing and reads no device memory on the host, so it can be
 * captured in a graph. Errors as for the single call, per job; an output that
 * overlaps another job's output or any job's inputs is CONVROT_E_INVALID_ARG
 * (inputs may be shared). njobs == 0 is a no-op. Each W_hat is bit-identical
 * to the single call's. */
typedef struct convrot_dequant_job {
  const int8_t* wq;
  const float* s_w;
  void* w_out;
  int64_t n, k;
} convrot_dequant_job;
convrot_status convrot_dequant_derotate_batched(const convrot_dequant_job* jobs, int njobs,
                                                convrot_scale_mode scale_mode, int g,
                                                uint64_t rot_seed, convrot_dtype out_dtype,
                                                void* stream);

/* Rotate each token row of x by blockdiag(R), take its absmax and quantize it to
 * int8 with one fp32 scale per row (Invoke docs "int8 Compute", introduction).
 *   x   [m, k] bf16 (in)
 *   xq  [m, k] int8 (out), s_x [m] fp32 (out) */
convrot_status convrot_quantize_activations(const uint16_t* x, int64_t m, int64_t k, int g,
                                            uint64_t rot_seed, int8_t* xq, float* s_x,
                                            void* stream);

/* Test hook: the same result as convrot_quantize_activations, computed for every
 * row by the exact (banded) kernel, whose row pass otherwise only finishes,
 * inside the fast kernel's launch, the rows that kernel cannot decide. */
convrot_status convrot_quantize_activations_exact(const uint16_t* x, int64_t m, int64_t k, int g,
                                                  uint64_t rot_seed, int8_t* xq, float* s_x,
                                                  void* stream);

/* int8 GEMM with the scaling epilogue (the int8 x int8 multiply of int8_compute:
 * Invoke docs "int8 Compute", introduction).
 *   xq [m, k] int8, s_x [m] fp32, wq [n, k] int8, s_w [1] fp32 (in)
 *   bias [n] bf16 (in, nullable)
 *   y   [m, n] bf16 (out, nullable)   y = bf16(RN(RN(float(acc) s_w) s_x[m]) [+ bias])
 *   acc [m, n] int32 (out, nullable)  acc = xq . wq^T, exact
 * At least one of y and acc must be non-null. */
convrot_status convrot_gemm_int8(const int8_t* xq, const float* s_x, const int8_t* wq,
                                 const float* s_w, const uint16_t* bias, int64_t m, int64_t n,
                                 int64_t k, uint16_t* y, int32_t* acc, void* stream);

/* Test / tuning hook: convrot_gemm_int8 with a forced block tile: 128, 192 or
 * 256 (tile x tile outputs), 384 (384 x 192 outputs; only for k % 128 == 0),
 * or 0 = the automatic choice. Same results. Any other tile value, or 384 with
 * k % 128 != 0, is CONVROT_E_INVALID_ARG before anything is launched. */
convrot_status convrot_gemm_int8_tile(const int8_t* xq, const float* s_x, const int8_t* wq,
                                      const float* s_w, const uint16_t* bias, int64_t m,
                                      int64_t n, int64_t k, uint16_t* y, int32_t* acc, int tile,
                                      void* stream);

/* Per-channel variants of the two GEMM calls above: s_w [n] fp32 (in, 16-byte
 * aligned) and y = bf16(RN(RN(float(acc) s_w[n]) s_x[m]) [+ bias[n]]). */
convrot_status convrot_gemm_int8_per_channel(const int8_t* xq, const float* s_x,
                                             const int8_t* wq, const float* s_w,
                                             const uint16_t* bias, int64_t m, int64_t n,
                                             int64_t k, uint16_t* y, int32_t* acc, void* stream);
convrot_status convrot_gemm_int8_per_channel_tile(const int8_t* xq, const float* s_x,
                                                  const int8_t* wq, const float* s_w,
                                                  const uint16_t* bias, int64_t m, int64_t n,
                                                  int64_t k, uint16_t* y, int32_t* acc, int tile,
                                                  void* stream);

/* The int8_compute forward: for each slice of token rows, rotate + quantize the
 * slice into the workspace, then run the int8 GEMM with the scaling epilogue.
 * Slices hold as many rows as the workspace fits (Invoke docs "int8 Compute",
 * "Memory": slices of at most twice the output width keep the working memory
 * within the default path's bf16 unpack).
 *   x [m, k] bf16, wq [n, k] int8, s_w [1] fp32, bias [n] bf16 nullable (in)
 *   y [m, n] bf16 (out)
 *   workspace: device memory, 256-byte aligned, workspace_bytes long; holds
 *     slice_rows * k bytes of int8 activations (rounded up to 256) followed by
 *     slice_rows fp32 scales. The output does not depend on the slice size. */
convrot_status convrot_linear_int8(const uint16_t* x, const int8_t* wq, const float* s_w,
                                   const uint16_t* bias, int64_t m, int64_t n, int64_t k, int g,
                                   uint64_t rot_seed, uint16_t* y, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Per-channel variant of convrot_linear_int8: s_w [n] fp32 (in, 16-byte
 * aligned); same slicing and workspace. */
convrot_status convrot_linear_int8_per_channel(const uint16_t* x, const int8_t* wq,
                                               const float* s_w, const uint16_t* bias, int64_t m,
                                               int64_t n, int64_t k, int g, uint64_t rot_seed,
                                               uint16_t* y, void* workspace,
                                               size_t workspace_bytes, void* stream);

/* General forms: every combination of activation format (dtype) and weight
 * scale granularity (scale_mode). x, bias, y and w_out are 16-bit tensors of
 * the given format; everything else is as in the entry points above, and an
 * unknown dtype or scale_mode value is CONVROT_E_INVALID_ARG.
 *   convrot_quantize_activations_ex: x [m, k] -> xq [m, k] int8, s_x [m]
 *   convrot_dequant_derotate_ex:     wq [n, k], s_w -> w_out [n, k] in out_dtype
 *   convrot_gemm_int8_ex:            y (nullable) in dtype, acc (nullable);
 *                                    tile as for convrot_gemm_int8_tile
 *   convrot_linear_int8_ex:          x, bias, y in dtype; same workspace rules */
convrot_status convrot_quantize_activations_ex(const void* x, convrot_dtype dtype, int64_t m,
                                               int64_t k, int g, uint64_t rot_seed, int8_t* xq,
                                               float* s_x, void* stream);
convrot_status convrot_dequant_derotate_ex(const int8_t* wq, const float* s_w,
                                           convrot_scale_mode scale_mode, int64_t n, int64_t k,
                                           int g, uint64_t rot_seed, void* w_out,
                                           convrot_dtype out_dtype, void* stream);
convrot_status convrot_gemm_int8_ex(const int8_t* xq, const float* s_x, const int8_t* wq,
                                    const float* s_w, convrot_scale_mode scale_mode,
                                    const void* bias, int64_t m, int64_t n, int64_t k, void* y,
                                    int32_t* acc, convrot_dtype dtype, int tile, void* stream);
convrot_status convrot_linear_int8_ex(const void* x, const int8_t* wq, const float* s_w,
                                      convrot_scale_mode scale_mode, const void* bias, int64_t m,
                                      int64_t n, int64_t k, int g, uint64_t rot_seed, void* y,
                                      convrot_dtype dtype, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* The int8 forward of convrot_linear_int8_ex without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). The token slices go
 * through a scratch array of CONVROT_NOALLOC_SCRATCH_BYTES (64 MiB) that the
 * library holds per device from its load to the end of the process: slices of
 * up to floor(64 MiB / (k + 4)) token rows (rounded down to whole 256-row
 * GEMM tiles; e.g. 13096 rows at k = 5120, 4608 at k = 13824). The call
 * allocates and frees nothing, and synchronizes nothing.
 *   x, bias, y, wq, s_w, scale_mode, dtype, m, n, k, g, rot_seed, stream: as
 *     for convrot_linear_int8_ex; y is bit-identical to its output for every
 *     workspace size.
 * Errors as for convrot_linear_int8_ex; CONVROT_E_WORKSPACE if one token row
 * (k + 4 bytes) would not fit the scratch (never for k <= 16384). The scratch
 * is shared by every call on a device and keeps the last call's contents
 * (nothing in it needs to start at zero): calls that overlap in time on one
 * device race, so callers serialize them (one stream, or stream order). */
#define CONVROT_NOALLOC_SCRATCH_BYTES (64u << 20)
convrot_status convrot_linear_int8_noalloc(const void* x, const int8_t* wq, const float* s_w,
                                           convrot_scale_mode scale_mode, const void* bias,
                                           int64_t m, int64_t n, int64_t k, int g,
                                           uint64_t rot_seed, void* y, convrot_dtype dtype,
                                           void* stream);

/* Host-streamed int8 layers (Invoke docs "int8 Compute", the table of a
 * transformer kept in host memory: a non-resident layer's int8 weight is
 * moved to the device on every call, at half the bytes of its bf16 form, and
 * then runs the same forward as a resident layer; "Memory": the staging stays
 * within the default path's working memory).
 *
 * A convrot_streamer owns `slots` device staging buffers of slot_bytes each, a
 * copy stream of its own (default priority) and two events per slot; it is
 * the one object of this library that allocates (at create; destroy frees).
 * convrot_streamer_linear_int8 is convrot_linear_int8_ex with the weight wq_host
 * in host memory (pinned, from hipHostMalloc, for the copy to run
 * asynchronously; device memory also works): it copies the weight into the
 * next slot on the copy stream (after that slot's previous forward has
 * finished), makes `stream` wait for the copy, and enqueues the forward
 * reading the slot. Calls return at once, so the copies of later layers
 * overlap the forwards of earlier ones; the output is bit-identical to
 * convrot_linear_int8_ex on a resident copy of the weight. wq_host must stay
 * unchanged until the forward that reads it has finished. A streamer is used
 * by one host thread at a time, on the device current at create. Errors as
 * for convrot_linear_int8_ex, plus CONVROT_E_WORKSPACE when n*k exceeds
 * slot_bytes; a HIP error after the copy was enqueued may leave it enqueued. */
#define CONVROT_STREAMER_MAX_SLOTS 8
typedef struct convrot_streamer convrot_streamer;
convrot_status convrot_streamer_create(size_t slot_bytes, int slots, convrot_streamer** out);
convrot_status convrot_streamer_destroy(convrot_streamer* streamer);
convrot_status convrot_streamer_linear_int8(convrot_streamer* streamer, const void* x,
                                            convrot_dtype dtype, const int8_t* wq_host,
                                            const float* s_w, convrot_scale_mode scale_mode,
                                            const void* bias, int64_t m, int64_t n, int64_t k,
                                            int g, uint64_t rot_seed, void* y, void* workspace,
                                            size_t workspace_bytes, void* stream);

/* First-call tuning and self-check (Invoke docs "int8 Compute", "Memory" and
 * "When something goes wrong": per layer shape and range of token counts, the
 * kernels are tuned once with a buffer the size of the last-level cache, and
 * that first output is compared on 256 rows with the dequant path; a
 * mismatch or a kernel fault sends that GPU back to the dequant path until
 * the application restarts).
 *
 * A convrot_session (one per device, made on the current device) runs
 * convrot_linear_int8_ex through a table keyed by (n, k, token bucket, g,
 * dtype, scale_mode), the token bucket being ceil(log2 m). On the first call
 * for a key, synchronously on `stream`:
 *   1. the first token slice is quantized and every GEMM tile that exists
 *      for k is timed on it (two runs each, after 256 MB - the MI355X MALL -
 *      have been written to the session's buffer); the fastest is kept (a
 *      key given a tile by convrot_session_import skips this step);
 *   2. the forward runs with that tile and writes y;
 *   3. W_hat (convrot_dequant_derotate_ex in dtype) is formed in the
 *      session's buffer, a chunk of weight rows at a time, the first
 *      min(m, 256) rows of x . W_hat^T (+ bias) are computed in fp32 over the
 *      chunk's columns, and their relative Frobenius distance e from the same
 *      rows of y (summed over all chunks) is kept. e <= check_tolerance passes.
 * Later calls for the key run the forward with the kept tile and enqueue
 * asynchronously, like convrot_linear_int8_ex (same results: every tile gives
 * the same bits). If the check fails, or a HIP call of a first call fails,
 * the session latches: that call (which has written y) and every later call
 * return CONVROT_E_SELFCHECK (later calls enqueue nothing), and the caller takes the
 * default path (convrot_dequant_derotate_ex and its own bf16 / fp16 matmul).
 * The library never switches paths silently. The quantization noise of the
 * int8 path is a few percent at most (per-token int8 after the rotation);
 * check_tolerance <= 0 selects 0.1. convrot_session_create allocates the
 * session's buffer (256 MB of device memory) and two events on the current
 * device; convrot_session_destroy frees them. The calls allocate no device
 * memory. A session is safe to share between threads (calls are serialized). */
typedef struct convrot_session convrot_session;
convrot_status convrot_session_create(double check_tolerance, convrot_session** out);
convrot_status convrot_session_destroy(convrot_session* session);
convrot_status convrot_session_linear_int8(convrot_session* session, const void* x,
                                           convrot_dtype dtype, const int8_t* wq,
                                           const float* s_w, convrot_scale_mode scale_mode,
                                           const void* bias, int64_t m, int64_t n, int64_t k,
                                           int g, uint64_t rot_seed, void* y, void* workspace,
                                           size_t workspace_bytes, void* stream);
/* The tile kept for a key and the check's relative error e; CONVROT_E_INVALID_ARG
 * if the key has had no first call. *latched (nullable) reports the latch. */
convrot_status convrot_session_lookup(convrot_session* session, int64_t m, int64_t n, int64_t k,
                                      int g, convrot_dtype dtype, convrot_scale_mode scale_mode,
                                      int* tile, double* check_error, int* latched);

/* The tuned tiles across processes (the tuning of a key's first call costs a
 * dozen GEMM runs and cache flushes; a serving process can start from the
 * last run's choices). For callers that keep a small table between runs.
 *
 * convrot_session_export: the session's table as text, host memory: the line
 * "convrot-session-tiles 1", then one line per key, "n k bucket g dtype
 * scale_mode tile" (decimal integers; bucket = ceil(log2 m); dtype and
 * scale_mode the enum values), for every key with a first call and every
 * imported key without one, in a fixed order. Writes at most buf_bytes
 * bytes, NUL-terminated when buf_bytes > 0 (buf nullable when buf_bytes is
 * 0) and returns the bytes the whole text needs, NUL included; 0 for a null
 * session. Check errors are not exported.
 *
 * convrot_session_import: reads such text (host memory, NUL-terminated).
 * Each line gives its key a tile: that key's first call then skips the
 * timing and runs with the tile, and still runs the check against the
 * default path (the same results: every tile gives the same bits). Keys that
 * already had a first call keep their entry. The text must be well formed:
 * the header line, seven integers per line with k % 64 == 0, k <= 16384,
 * k % g == 0, g in {4, 16, 64, 256}, n % 16 == 0, a tile in {128, 192, 256,
 * 384} that exists for k (384: k % 128 == 0); otherwise CONVROT_E_INVALID_ARG
 * naming the line, and nothing is imported. Touches no GPU. */
size_t convrot_session_export(convrot_session* session, char* buf, size_t buf_bytes);
convrot_status convrot_session_import(convrot_session* session, const char* text);

/* Workspace bytes that convrot_linear_int8 uses for slices of `rows` token rows. */
size_t convrot_linear_int8_workspace_for_rows(int64_t rows, int64_t k);

/* Default workspace: slices of min(m, 2n) rows (Invoke docs "int8 Compute",
 * "Memory"). Returns 0 for invalid dimensions. */
size_t convrot_linear_int8_workspace_size(int64_t m, int64_t n, int64_t k);

/* Host-only: the rotation signs d[0..g) for (g, rot_seed) as +1/-1 bytes into
 * host memory `d` (g bytes). Touches no GPU. */
convrot_status convrot_rotation_signs(uint64_t rot_seed, int g, int8_t* d);

/* Machine shape. Persistent grids, the GEMM's tile choice and its XCD-aware
 * tile order are sized from the device's compute-unit count, queried once
 * per device (hipDeviceAttributeMultiprocessorCount: 256 on an MI355X, fewer
 * on a compute partition); the XCD count is CUs / 32, the CUs of one gfx950
 * XCD (1 below 64 CUs). Sizing changes speed only, never results.
 *
 * convrot_compute_units: the count that launches on the current device use.
 * convrot_set_compute_units: a process-wide override of that count for
 *   tests and tuning (0 restores the device's count); e.g. a small count
 *   makes every persistent grid walk many passes. It affects launches
 *   enqueued after the call, from any thread.
 * convrot_plan_launch: host only (touches no GPU when compute_units > 0):
 *   the launch geometry of `kernel` for the given shape (m rows for the
 *   activation kernels, n x k for the dequant, m x n x k for the GEMM; g for
 *   the rotating kernels) on `compute_units` CUs (0 = the current device's).
 *   Shape errors as for the corresponding entry point. */
typedef enum convrot_kernel {
  CONVROT_KERNEL_ACT_QUANT = 0,          /* activation rotate + quantize, fast kernel   */
  CONVROT_KERNEL_ACT_QUANT_DEFERRED = 1, /* its blocks' pass over the rows they defer   */
  CONVROT_KERNEL_EXACT = 2,              /* exact kernel (weights, the _exact hook)     */
  CONVROT_KERNEL_DEQUANT = 3,            /* dequant + derotate                          */
  CONVROT_KERNEL_GEMM = 4                /* int8 GEMM, automatic tile                   */
} convrot_kernel;
typedef struct convrot_launch_plan {
  int64_t grid;           /* workgroups                                                  */
  int64_t passes;         /* persistent kernels: batches per workgroup (rounded up)      */
  int32_t block;          /* threads per workgroup                                       */
  int32_t rows_per_block; /* act-quant: token rows per batch (its deferred rows: rows of
                             K/32 lanes per step); dequant: 32-row tiles per step        */
  int32_t tile_m, tile_n; /* GEMM block tile (0 otherwise)                               */
  int32_t xcds;           /* XCDs of the GEMM's tile order                                */
  int32_t compute_units;  /* the CU count the plan was made for                          */
} convrot_launch_plan;
int convrot_compute_units(void);
convrot_status convrot_set_compute_units(int compute_units_override);
convrot_status convrot_plan_launch(convrot_kernel kernel, int64_t m, int64_t n, int64_t k, int g,
                                   int compute_units, convrot_launch_plan* out);

const char* convrot_status_string(convrot_status s);
/* Details of the last error on the calling thread ("" if none). */
const char* convrot_last_error_string(void);
int convrot_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */

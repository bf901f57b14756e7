// Internal launcher declarations of the convrot library.
#pragma once

#include "common.h"

namespace convrot {

// 16-bit float format of activations, bias and outputs.
enum class DType { kBF16 = 0, kF16 = 1 };

// Compute units that launches size their grids for: the current device's
// count (queried once per device), or the process-wide override of
// convrot_set_compute_units.
int compute_units();

// Launch geometry of a kernel (host-side sizing, testable without a GPU).
struct LaunchPlan {
  int64_t grid = 0;        // workgroups
  int block = 0;           // threads per workgroup
  int rows_per_block = 0;  // rows of a batch (act-quant) / 32-row tiles per step (dequant)
  int tile_m = 0, tile_n = 0;  // GEMM block tile
  int xcds = 1;            // XCDs the GEMM's tile order spreads over
  int64_t passes = 0;      // batches per workgroup of a persistent grid (ceil)
};
// Act-quant fast kernel (deferred = false) or its deferred-row pass.
LaunchPlan plan_act_quant(int64_t rows, int K, bool deferred, int cus);
// Exact kernel over every row (weight quantization and the exact entry point).
LaunchPlan plan_exact(int64_t rows, int K, int cus);
LaunchPlan plan_dequant(int64_t n, int64_t k, int g, int cus);
// tile 0 = automatic choice
LaunchPlan plan_gemm(int64_t m, int64_t n, int64_t k, int tile, int cus);

// Rotate + quantize rows (per-row scales): fast kernel, then the exact kernel
// over the rows it deferred (bf16 only: half rows are never deferred).
hipError_t launch_quantize_rows(const uint16_t* x, int8_t* xq, float* s, int64_t rows, int K,
                                int g, const SignMask& sm, DType dt, hipStream_t st);
// Same result through the exact kernel only (used by tests of the fast path).
hipError_t launch_quantize_rows_exact(const uint16_t* x, int8_t* xq, float* s, int64_t rows,
                                      int K, int g, const SignMask& sm, hipStream_t st);
// Rotate + quantize a tensor with one scale (the scale slot doubles as the
// absmax accumulator until the last launch).
hipError_t launch_quantize_tensor(const uint16_t* w, int8_t* wq, float* s_w, int64_t rows, int K,
                                  int g, const SignMask& sm, hipStream_t st);
// One weight of a batched dequant.
struct DequantJob {
  const int8_t* wq;
  const float* s_w;
  uint16_t* w_out;
  int64_t n, k;
};
// The weights of one dequant launch, passed by value as kernel arguments
// (a single weight gets a table of one: the argument block stays small, and
// with it the launch).
constexpr int kMaxDequantJobs = 48;
template <int N>
struct DequantJobs {
  struct Desc {
    const int8_t* wq;
    const float* s_w;
    uint16_t* w_out;
    int64_t nrows;            // view rows of max(g, 32) bytes
    double inv_vrows_per_ch;  // per-channel: 1 / view rows per weight row
    int vrows_per_ch;
  };
  int njobs;
  int64_t chunk_begin[N + 1];
  Desc job[N];
};
// W_hat of several weights that share g, the signs, the scale mode and the
// output format, in launches of up to kMaxDequantJobs weights each.
hipError_t launch_dequant_jobs(const DequantJob* job, int njobs, bool sw_per_channel, int g,
                               const SignMask& sm, DType dt, hipStream_t st);
// W_hat = RN16(float(S) * RN(s_w * 2^-log2(sqrt g))), S = (Wq . D) . H per
// group, RN16 to bf16 or half (dt); with sw_per_channel, row r uses s_w[r].
hipError_t launch_dequant(const int8_t* wq, const float* s_w, bool sw_per_channel, int64_t n,
                          int64_t k, int g, const SignMask& sm, uint16_t* w_out, DType dt,
                          hipStream_t st);
// acc = xq . wq^T (int32); y = RN16(RN(RN(float(acc) * s_w) * s_x[m]) [+ bias[n]]),
// bias and y in dt; with sw_per_channel, column n uses s_w[n] (s_w then
// 16-byte aligned).
hipError_t launch_gemm(const int8_t* xq, const float* s_x, const int8_t* wq, const float* s_w,
                       bool sw_per_channel, const uint16_t* bias, int64_t m, int64_t n, int64_t k,
                       uint16_t* y, int32_t* acc, DType dt, hipStream_t st);
// The same GEMM with a forced block tile (128, 192 or 256; 0 = automatic).
hipError_t launch_gemm_tile(const int8_t* xq, const float* s_x, const int8_t* wq,
                            const float* s_w, bool sw_per_channel, const uint16_t* bias,
                            int64_t m, int64_t n, int64_t k, uint16_t* y, int32_t* acc, int tile,
                            DType dt, hipStream_t st);

// First-call check: write `bytes` of buf (evicts the operands from the caches).
hipError_t launch_flush(void* buf, size_t bytes, hipStream_t st);
// y_ref[rows, n] = x[:rows] . w_hat^T (+ bias) in fp32 (x, w_hat, bias, y in dt;
// y rows ldy apart), then for each row r < rows: partial[2r] = sum_c (y - y_ref)^2
// and partial[2r + 1] = sum_c y_ref^2 in float64, added to partial's values when
// `accumulate` is set (a check over column chunks: w_hat, bias and y offset to
// the chunk's first column, n its width).
hipError_t launch_check_rows(const uint16_t* x, const uint16_t* w_hat, const uint16_t* bias,
                             const uint16_t* y, int64_t ldy, int rows, int n, int k, DType dt,
                             bool accumulate, float* y_ref, double* partial, hipStream_t st);

}  // namespace convrot

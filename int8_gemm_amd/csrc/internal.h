// Internal launcher declarations of the convrot library.
#pragma once

#include "common.h"

namespace convrot {

// 16-bit float format of activations, bias and outputs.
enum class DType { kBF16 = 0, kF16 = 1 };

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
// y_ref[rows, n] = x[:rows] . w_hat^T (+ bias) in fp32 (x, w_hat, bias, y in dt),
// then partial[2r] = sum_c (y - y_ref)^2 and partial[2r + 1] = sum_c y_ref^2
// (float64) for each row r < rows.
hipError_t launch_check_rows(const uint16_t* x, const uint16_t* w_hat, const uint16_t* bias,
                             const uint16_t* y, int rows, int n, int k, DType dt, float* y_ref,
                             double* partial, hipStream_t st);

}  // namespace convrot

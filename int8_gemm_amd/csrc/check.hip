// Kernels of the first-call check (Invoke docs "int8 Compute", "Memory" and
// "When something goes wrong"): once per layer shape and range of token
// counts, up to 256 output rows of the int8 forward are compared with the
// dequant path, and the GEMM tile is tuned after a buffer the size of the
// last-level cache has been written (on MI355X the 256 MB MALL).
//
//   ref_rows_kernel:  y_ref[r, c] = sum_k x[r, k] * W_hat[c, k] (+ bias[c]) in
//                     fp32, W_hat the dequantized (default-path) weight;
//   diff_rows_kernel: per row, sum (y[r, c] - y_ref[r, c])^2 and
//                     sum y_ref[r, c]^2 in float64 (added up over the
//                     column chunks the check is taken in);
//   flush_kernel:     writes a buffer, evicting the operands from the caches.
//
// None of this is on the forward's hot path: it runs once per key.

#include "common.h"
#include "internal.h"

namespace convrot {

namespace {

template <bool F16>
__device__ __forceinline__ float to_f32(uint16_t v) {
  return F16 ? (float)__builtin_bit_cast(_Float16, (unsigned short)v)
             : __uint_as_float((uint32_t)v << 16);
}

// 64 x 64 output tile per block, 4 x 4 outputs per thread, K in chunks of 32
template <bool F16>
__global__ __launch_bounds__(256) void ref_rows_kernel(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ w,
                                                       const uint16_t* __restrict__ bias,
                                                       int rows, int n, int k,
                                                       float* __restrict__ out) {
  __shared__ float xs[64][33];
  __shared__ float wsm[64][33];
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = 0; k0 < k; k0 += 32) {
    for (int i = tid; i < 64 * 32; i += 256) {
      const int rr = i / 32, kk = i % 32;
      const int gk = k0 + kk;
      const int gr = r0 + rr, gc = c0 + rr;
      xs[rr][kk] = (gr < rows && gk < k) ? to_f32<F16>(x[(int64_t)gr * k + gk]) : 0.0f;
      wsm[rr][kk] = (gc < n && gk < k) ? to_f32<F16>(w[(int64_t)gc * k + gk]) : 0.0f;
    }
    __syncthreads();
    for (int kk = 0; kk < 32; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_fmaf(xs[tr * 4 + i][kk], wsm[tc * 4 + j][kk], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + tr * 4 + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + tc * 4 + j;
      if (r < rows && c < n) out[(int64_t)r * n + c] = acc[i][j] + (bias ? to_f32<F16>(bias[c]) : 0.0f);
    }
  }
}

// one block per row; the sums are added to partial when `accumulate` is set
// (a check taken over column chunks)
template <bool F16>
__global__ __launch_bounds__(256) void diff_rows_kernel(const uint16_t* __restrict__ y, int64_t ldy,
                                                        const float* __restrict__ y_ref, int n,
                                                        int accumulate,
                                                        double* __restrict__ partial) {
  __shared__ double s0[256], s1[256];
  const int row = blockIdx.x, tid = threadIdx.x;
  double d2 = 0.0, r2 = 0.0;
  for (int c = tid; c < n; c += 256) {
    const double a = to_f32<F16>(y[(int64_t)row * ldy + c]);
    const double b = y_ref[(int64_t)row * n + c];
    d2 += (a - b) * (a - b);
    r2 += b * b;
  }
  s0[tid] = d2;
  s1[tid] = r2;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) {
      s0[tid] += s0[tid + h];
      s1[tid] += s1[tid + h];
    }
    __syncthreads();
  }
  if (tid == 0) {
    partial[2 * row] = (accumulate ? partial[2 * row] : 0.0) + s0[0];
    partial[2 * row + 1] = (accumulate ? partial[2 * row + 1] : 0.0) + s1[0];
  }
}

__global__ __launch_bounds__(256) void flush_kernel(u4* __restrict__ buf, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * 256)
    buf[i] = (u4){(uint32_t)i, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_flush(void* buf, size_t bytes, hipStream_t st) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(flush_kernel, dim3(compute_units() * 8), dim3(256), 0, st, static_cast<u4*>(buf),
                     n16);
  return hipGetLastError();
}

hipError_t launch_check_rows(const uint16_t* x, const uint16_t* w_hat, const uint16_t* bias,
                             const uint16_t* y, int64_t ldy, int rows, int n, int k, DType dt,
                             bool accumulate, float* y_ref, double* partial, hipStream_t st) {
  if (rows <= 0 || n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((rows + 63) / 64));
  const int acc = accumulate ? 1 : 0;
  if (dt == DType::kF16) {
    hipLaunchKernelGGL(ref_rows_kernel<true>, grid, dim3(256), 0, st, x, w_hat, bias, rows, n, k,
                       y_ref);
    hipLaunchKernelGGL(diff_rows_kernel<true>, dim3((unsigned)rows), dim3(256), 0, st, y, ldy,
                       y_ref, n, acc, partial);
  } else {
    hipLaunchKernelGGL(ref_rows_kernel<false>, grid, dim3(256), 0, st, x, w_hat, bias, rows, n,
                       k, y_ref);
    hipLaunchKernelGGL(diff_rows_kernel<false>, dim3((unsigned)rows), dim3(256), 0, st, y, ldy,
                       y_ref, n, acc, partial);
  }
  return hipGetLastError();
}

}  // namespace convrot

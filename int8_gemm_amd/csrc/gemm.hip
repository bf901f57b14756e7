// int8 x int8 -> int32 GEMM with the convrot scaling epilogue (gfx950).
//
// acc[m, n] = sum_k xq[m, k] * wq[n, k] (exact int32: |acc| <= 127^2 K < 2^31)
// y[m, n]   = bf16(RN32(RN32(float(acc) * s_w) * s_x[m]) [+ bias[n] in fp32])
//
// This is the int8 tensor-core multiply of int8_compute (Invoke docs
// "int8 Compute", introduction: the input is quantized per token and int8 is
// multiplied by int8); the pages run it through Triton on NVIDIA, this is a
// gfx950 design of its own:
//   * block tile 256 x 256, 4 waves (2 x 2), wave tile 128 x 128;
//   * v_mfma_i32_16x16x64_i8 with the weight rows in the A operand, so each
//     lane's accumulators are 4 consecutive output columns of one row;
//   * K-step 128 bytes, double-buffered in LDS (2 x 64 KB), global loads for
//     the next step issued before the current step's MFMAs;
//   * LDS rows of 128 B with the 16-byte chunk index XOR-swizzled by the row,
//     so the 16-byte fragment reads of consecutive rows hit distinct banks;
//   * tiles are walked in groups of rows, with the block index remapped so
//     that the 8 XCDs each get a contiguous range of tiles (L2 reuse).
// Both operands are K-contiguous ("TN"). K % 64 == 0, N % 16 == 0.

#include "common.h"
#include "internal.h"

namespace convrot {

namespace {

constexpr int BM = 256;         // rows of xq per block
constexpr int BN = 256;         // rows of wq per block
constexpr int BK = 128;         // K bytes per stage
constexpr int NTHR = 256;
constexpr int CHUNKS = BK / 16; // 16-byte chunks per tile row

__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7); }

__global__ __launch_bounds__(NTHR, 1) void gemm_i8_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ s_x, const int8_t* __restrict__ wq,
    const float* __restrict__ s_w, const uint16_t* __restrict__ bias, int M, int N, int K,
    int tiles_m, int tiles_n, uint16_t* __restrict__ y, int32_t* __restrict__ acc_out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  // stage s: A(wq) tile at s*64K, B(xq) tile at s*64K + 32K
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1;   // wave column block in N
  const int wm = wave >> 1;  // wave row block in M

  // ---- tile index: XCD-contiguous, grouped rows ----
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  {
    const int nx = 8;
    const int per = (ntiles + nx - 1) / nx;
    const int xcd = bid % nx;
    const int loc = bid / nx;
    const int full = ntiles - (per - 1) * nx;  // XCDs that get `per` tiles
    bid = (xcd < full) ? xcd * per + loc : full * per + (xcd - full) * (per - 1) + loc;
  }
  constexpr int GROUP = 8;
  const int group_sz = GROUP * tiles_n;
  const int grp = bid / group_sz;
  const int first_m = grp * GROUP;
  const int gm = min(tiles_m - first_m, GROUP);
  const int in_grp = bid - grp * group_sz;
  const int tile_m = first_m + in_grp % gm;
  const int tile_n = in_grp / gm;
  const int m0 = tile_m * BM;
  const int n0 = tile_n * BN;

  // ---- global -> register staging (8 chunks of each operand per thread) ----
  uint4 ra[8], rb[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int id = u * NTHR + tid;
      const int row = id >> 3;
      const int c = id & 7;
      const int k = k0 + 16 * c;
      const int n = min(n0 + row, N - 1);
      const int m = min(m0 + row, M - 1);
      if (k < K) {
        ra[u] = *reinterpret_cast<const uint4*>(wq + (int64_t)n * K + k);
        rb[u] = *reinterpret_cast<const uint4*>(xq + (int64_t)m * K + k);
      } else {
        ra[u] = make_uint4(0, 0, 0, 0);
        rb[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int stage) {
    uint8_t* a = lds + stage * 65536;
    uint8_t* b = a + 32768;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int id = u * NTHR + tid;
      const int row = id >> 3;
      const int c = id & 7;
      const int off = row * BK + 16 * swz(row, c);
      *reinterpret_cast<uint4*>(a + off) = ra[u];
      *reinterpret_cast<uint4*>(b + off) = rb[u];
    }
  };

  v4i acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

  const int nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();

  const int fr = lane & 15;  // fragment row within a 16-row block
  const int fq = lane >> 4;  // k-slice (16 B) within a 64-byte sub-step
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < nk) gload((ks + 1) * BK);
    const uint8_t* a = lds + cur * 65536;
    const uint8_t* b = a + 32768;
    const int subs = min(2, (K - ks * BK) / 64);
    for (int sub = 0; sub < subs; ++sub) {
      const int c = 4 * sub + fq;
      v4i af[8], bf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = wn * 128 + i * 16 + fr;
        af[i] = *reinterpret_cast<const v4i*>(a + row * BK + 16 * swz(row, c));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = wm * 128 + j * 16 + fr;
        bf[j] = *reinterpret_cast<const v4i*>(b + row * BK + 16 * swz(row, c));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nk) {
      __syncthreads();
      lstore(cur ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds n = 4*(lane/16) + e (e < 4), m = lane % 16 ----
  const float sw = *s_w;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = m0 + wm * 128 + j * 16 + fr;
    if (m >= M) continue;
    const float sx = s_x[m];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + wn * 128 + i * 16 + 4 * fq;
      if (n >= N) continue;
      const v4i v = acc[i][j];
      if (acc_out) {
        *reinterpret_cast<int4*>(acc_out + (int64_t)m * N + n) = make_int4(v[0], v[1], v[2], v[3]);
      }
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = (float)v[e] * sw;
        f[e] = f[e] * sx;
      }
      if (bias) {
        const uint2 bb = *reinterpret_cast<const uint2*>(bias + n);
        f[0] = f[0] + bf16lo(bb.x);
        f[1] = f[1] + bf16hi(bb.x);
        f[2] = f[2] + bf16lo(bb.y);
        f[3] = f[3] + bf16hi(bb.y);
      }
      if (y) {
        uint2 o;
        o.x = pack_bf16x2(f[0], f[1]);
        o.y = pack_bf16x2(f[2], f[3]);
        *reinterpret_cast<uint2*>(y + (int64_t)m * N + n) = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const int8_t* xq, const float* s_x, const int8_t* wq, const float* s_w,
                       const uint16_t* bias, int64_t m, int64_t n, int64_t k, uint16_t* y,
                       int32_t* acc, hipStream_t st) {
  if (m == 0 || n == 0) return hipSuccess;
  const int tiles_m = (int)((m + BM - 1) / BM);
  const int tiles_n = (int)((n + BN - 1) / BN);
  const int ntiles = tiles_m * tiles_n;
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_i8_kernel),
                        hipFuncAttributeMaxDynamicSharedMemorySize, 131072);
    attr_set = true;
  }
  hipLaunchKernelGGL(gemm_i8_kernel, dim3(ntiles), dim3(NTHR), 131072, st, xq, s_x, wq, s_w, bias,
                     (int)m, (int)n, (int)k, tiles_m, tiles_n, y, acc);
  return hipGetLastError();
}

}  // namespace convrot

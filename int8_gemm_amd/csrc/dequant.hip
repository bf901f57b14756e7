// Dequantize + derotate (the default path's per-forward weight decode).
//
// For each g-group of the input axis: S[j] = sum_i Wq[i] d[i] H[i, j] (exact
// int32, |S| <= 127 g) and W_hat[j] = bf16(RN32(float(S) * c)),
// c = RN32(s_w * 2^-log2(sqrt g)). This is s_w . Wq . blockdiag(R)^T with
// R = H . diag(d) / sqrt(g), done as the [out, in/g, g] @ [g, g] block matmul
// of PR "share the int8_convrot scheme ... Krea-2 and Z-Image", section
// "What it is worth" (there with g = 256 and bf16 math).
//
// gfx950 mapping: the flat weight is viewed as rows of R = max(g, 32) bytes.
// One wave computes a 32-row tile with v_mfma_i32_32x32x32_i8, the +-1 matrix
// in the A operand (rows = output j) and the weight rows in the B operand
// (columns = groups). H_g = H_{g/32} (x) H_32 for g >= 64, so the A operand
// needs only the g/32 blocks d-scaled H_32 and their negatives, built once
// per lane from the sign mask. For g < 32 the A operand is block-diagonal.
// The kernel is bound by HBM: 1 byte read and 2 bytes written per element.

#include "common.h"
#include "internal.h"

namespace convrot {

namespace {

// parity of popcount
__device__ __forceinline__ uint32_t par(uint32_t v) { return __builtin_popcount(v) & 1u; }

// 16-bit mask: bit b = parity(b & x) for b < 16 (a row of H_16 as sign bits)
__device__ __forceinline__ uint32_t hrow16(uint32_t x) {
  uint32_t m = 0u;
  if (x & 1u) m ^= 0xAAAAu;
  if (x & 2u) m ^= 0xCCCCu;
  if (x & 4u) m ^= 0xF0F0u;
  if (x & 8u) m ^= 0xFF00u;
  return m;
}

__device__ __forceinline__ uint32_t nib_bytes(uint32_t nib) {
  return ((nib * 0x00204081u) & 0x01010101u) * 0xFFu;
}

// 16 int8 entries (one A-operand slice) from 16-bit masks: negative where
// neg bit is set, zero where nz bit is clear, +1 otherwise.
__device__ __forceinline__ v4i frag_from_masks(uint32_t neg, uint32_t nz) {
  v4i f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t nb = nib_bytes((neg >> (4 * q)) & 0xFu);
    const uint32_t zb = nib_bytes((nz >> (4 * q)) & 0xFu);
    f[q] = (int)((0x01010101u ^ (nb & 0xFEFEFEFEu)) & zb);
  }
  return f;
}

template <int G>
__global__ __launch_bounds__(256) void dequant_kernel(const int8_t* __restrict__ wq,
                                                      const float* __restrict__ s_w,
                                                      int64_t nrows, SignMask sm,
                                                      uint16_t* __restrict__ out) {
  constexpr int R = G > 32 ? G : 32;  // bytes per view row
  constexpr int NB = R / 32;          // 32-blocks per view row
  constexpr int KS = ilog2(G) / 2;
  const int lane = threadIdx.x & 63;
  const uint32_t jl = lane & 31;      // A row (output j within a 32-block)
  const uint32_t kh = lane >> 5;      // k-slice: il = 16*kh + b

  // ---- A fragments ----
  v4i fragP[NB], fragN[NB];
  if constexpr (G >= 32) {
    const uint32_t h = hrow16(jl & 15u) ^ (par(kh & (jl >> 4)) ? 0xFFFFu : 0u);
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
      const uint32_t dm = (sm.w[ib] >> (16 * kh)) & 0xFFFFu;
      fragP[ib] = frag_from_masks(h ^ dm, 0xFFFFu);
      fragN[ib] = frag_from_masks(h ^ dm ^ 0xFFFFu, 0xFFFFu);
    }
  } else {
    // block-diagonal: entry (jl, il) nonzero iff il/G == jl/G
    uint32_t nz = 0u, neg = 0u;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const uint32_t il = 16u * kh + (uint32_t)b;
      if (il / G == jl / G) {
        nz |= 1u << b;
        const uint32_t hpar = par(il & jl & (uint32_t)(G - 1));
        const uint32_t dneg = (sm.w[0] >> (il % G)) & 1u;
        neg |= (hpar ^ dneg) << b;
      }
    }
    fragP[0] = frag_from_masks(neg, nz);
    fragN[0] = fragP[0];
  }

  const float c = *s_w * (1.0f / (float)(1 << KS));
  // work item = (32-row tile, JW consecutive output 32-blocks): the NB*NB
  // MFMAs of a tile are spread over NB/JW waves (the tile's input bytes are
  // re-read from L2 by each), which shortens each wave's serial MFMA chain.
  constexpr int JW = NB < 2 ? NB : 2;
  constexpr int NQ = NB / JW;
  const int64_t nitems = (nrows + 31) / 32 * NQ;
  const int64_t wave0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t wstride = (int64_t)gridDim.x * 4;

  for (int64_t item = wave0; item < nitems; item += wstride) {
    const int64_t tile = item / NQ;
    const int jq = (int)(item % NQ);
    const int64_t r = tile * 32 + jl;                   // B column = this lane's view row
    const int64_t rr = r < nrows ? r : nrows - 1;
    v4i bfr[NB];
#pragma unroll
    for (int ib = 0; ib < NB; ++ib)
      bfr[ib] = *reinterpret_cast<const v4i*>(wq + rr * R + 32 * ib + 16 * kh);
    const bool ok = r < nrows;
#pragma unroll
    for (int jw = 0; jw < JW; ++jw) {
      const int jb = jq * JW + jw;
      v16i acc = {};
#pragma unroll
      for (int ib = 0; ib < NB; ++ib) {
        const bool negb = (__builtin_popcount(ib & jb) & 1) != 0;
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(negb ? fragN[ib] : fragP[ib], bfr[ib], acc,
                                                     0, 0, 0);
      }
      // lane (jl, kh) holds outputs j = 8a + 4kh + e of view row r; pack to
      // bf16 pairs, then swap halves with lane jl + 32 (v_permlane32_swap) so
      // that lane kh = 0 holds j = 16h .. 16h+7 and lane kh = 1 holds
      // j = 16h+8 .. 16h+15 for h = 0, 1: two 16-byte stores per lane.
      uint32_t pk[4][2];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        pk[a][0] = pack_bf16x2((float)acc[4 * a + 0] * c, (float)acc[4 * a + 1] * c);
        pk[a][1] = pack_bf16x2((float)acc[4 * a + 2] * c, (float)acc[4 * a + 3] * c);
      }
      uint16_t* o = out + r * R + 32 * jb + 8 * kh;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u4 v;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          // swap lanes 32..63 of pk[2h] with lanes 0..31 of pk[2h+1]
          const auto sw = __builtin_amdgcn_permlane32_swap(pk[2 * h][e], pk[2 * h + 1][e],
                                                           false, false);
          v[e] = sw[0];      // kh = 0: own a = 2h; kh = 1: partner's a = 2h+1
          v[2 + e] = sw[1];  // kh = 0: partner's a = 2h; kh = 1: own a = 2h+1
        }
        if (ok) *reinterpret_cast<u4*>(o + 16 * h) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_dequant(const int8_t* wq, const float* s_w, int64_t n, int64_t k, int g,
                          const SignMask& sm, uint16_t* w_out, hipStream_t st) {
  const int64_t ne = n * k;
  if (ne == 0) return hipSuccess;
  const int R = g > 32 ? g : 32;
  const int64_t nrows = ne / R;
  const int64_t items = (nrows + 31) / 32 * (R >= 64 ? R / 64 : 1);
  int64_t blocks = (items + 3) / 4;
  const int64_t cap = 256 * 8;
  if (blocks > cap) blocks = cap;
  switch (g) {
    case 4:
      hipLaunchKernelGGL(dequant_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st, wq, s_w,
                         nrows, sm, w_out);
      break;
    case 16:
      hipLaunchKernelGGL(dequant_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, st, wq, s_w,
                         nrows, sm, w_out);
      break;
    case 64:
      hipLaunchKernelGGL(dequant_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, st, wq, s_w,
                         nrows, sm, w_out);
      break;
    default:
      hipLaunchKernelGGL(dequant_kernel<256>, dim3((unsigned)blocks), dim3(256), 0, st, wq, s_w,
                         nrows, sm, w_out);
      break;
  }
  return hipGetLastError();
}

}  // namespace convrot

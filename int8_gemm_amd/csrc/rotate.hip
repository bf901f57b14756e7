// Rotation + absmax + int8 quantization kernels (gfx950).
//
// Rotation: x_r[j] = sum_i x[i] R[i, j] over each g-group of a row, with
// R = H_g . diag(d) / sqrt(g) (Sylvester H, d = +-1). The value kept is the
// exact sum rounded once to fp32 (nearest-even). Every product bf16 * (+-2^-k)
// is exact, so this is order independent; the kernels compute it with a
// Walsh-Hadamard transform (butterflies) in float64:
//
//   * Fast kernel: if a group's nonzero elements span at most 45 - log2(g)
//     binades, every butterfly partial sum is a multiple of the smallest
//     element's quantum and below g times the largest element, so it fits
//     53 bits and float64 is exact. Rows holding a group outside that bound
//     (or rows too small for the folded scaling below) are left to the exact
//     kernel: their scale slot receives the kDeferredRow NaN.
//   * Deferred rows (the exact kernel's deferred mode) first get one rounded
//     float64 transform: each output is within log2(g) * 2^-53 * sum|x| of
//     the exact sum (a depth-log2(g) tree of rounded additions), so with
//     that bound (and margin) an element either provably rounds to
//     RN32(y), or to one of RN32(y) and its neighbour. The row is finished
//     there unless such an undecided element could be the row's absmax or
//     quantizes differently for its two candidates (ties decided only by
//     elements the float64 sum lost: GELU-tailed activations).
//   * Exact kernel: splits each group's elements into bands of kBand
//     binades (each band's transform is exact in float64), turns each band's
//     sums into integers of the band's quantum and adds the bands bottom-up
//     with exact floor division, carrying a sticky bit for the dropped
//     fraction. The rounding is then exact whenever the top band's integer
//     has at least 27 bits; otherwise the element is at least 2^16 times
//     below the row's absmax and quantizes to 0 whatever its fp32 value.
//
// IEEE half inputs (the fast kernel's F16 form): every half value is a
// multiple of 2^-24 below 2^16, so a group's signed sums are multiples of
// 2^-24 below 2^24 and every float64 partial sum is exact. No half row is
// ever deferred (its absmax also lies far inside the scaling range).
//
// Quantization (per row or per tensor): s = RN(amax/127), inv = RN(127/amax)
// (both operands scaled by 2^64 first when amax < 2^-64),
// q = rint_even(RN(x_r * inv)); |q| <= 127 always; amax == 0 gives s = q = 0.
//
// Pages: the per-token rotate + quantize of int8_compute is the Invoke docs
// "int8 Compute" introduction; the weight quantization (one scale per tensor,
// rotation in groups of g) is the convert_to_quant guide, "How INT8 ConvRot
// Quantization Works" and "Determining the Right ConvRot Group Size".

#include "common.h"
#include "internal.h"

namespace convrot {

namespace {

constexpr float kQuantBias = 12583040.0f;   // 1.5 * 2^23 + 128: low byte = q + 128
constexpr float kQuantPlain = 12582912.0f;  // 1.5 * 2^23: low byte = q (two's complement)

// --- cross-lane helpers ------------------------------------------------------

// quad permutations write every lane, so no "old" operand is needed
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kQuadRev = 0x1B;   // quad_perm [3,2,1,0]: lane i <- i ^ 3
constexpr int kHalfMirror = 0x141;  // row_half_mirror: lane i <- 7 - i within 8 lanes

// lane i <- lane i ^ M (M = 1, 2, 4) with DPP moves; xor 4 is the half-row
// mirror (i ^ 7) followed by the quad reversal (i ^ 3)
template <int M>
__device__ __forceinline__ uint32_t xor_lanes_u32(uint32_t v) {
  static_assert(M == 1 || M == 2 || M == 4, "lane xor");
  if constexpr (M == 1) return dpp_u32<kQuadXor1>(v);
  if constexpr (M == 2) return dpp_u32<kQuadXor2>(v);
  return dpp_u32<kQuadRev>(dpp_u32<kHalfMirror>(v));
}
template <int M>
__device__ __forceinline__ double xor_lanes_f64(double v) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = xor_lanes_u32<M>((uint32_t)b);
  const uint32_t hi = xor_lanes_u32<M>((uint32_t)(b >> 32));
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

// In-lane radix-2 Walsh-Hadamard stages over the low log2(min(G, N)) index
// bits of v[N]; stage h combines (j, j+h) into (a+b, a-b).
template <int G, int N>
__device__ __forceinline__ void fwht_inlane(double (&v)[N]) {
  constexpr int L = G < N ? G : N;
#pragma unroll
  for (int h = 1; h < L; h <<= 1) {
#pragma unroll
    for (int i = 0; i < N; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const double a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

// Spread the 4 bits of a nibble to bytes: bit i -> byte i = 0xFF.
__device__ __forceinline__ uint32_t nibble_to_bytemask(uint32_t nib) {
  return ((nib * 0x00204081u) & 0x01010101u) * 0xFFu;
}

// Exponent fields of a packed bf16 pair (sign cleared): the max, and the min
// over nonzero elements taken as (field of bits-1), so zeros drop out (they
// wrap to 0xFFFF) and a mantissa-zero power of two reads one binade low,
// which only widens the measured span.
__device__ __forceinline__ void span_acc(uint32_t w, us2& mx, us2& mn) {
  const us2 m = __builtin_bit_cast(us2, w & 0x7FFF7FFFu);
  mx = __builtin_elementwise_max(mx, m);
  mn = __builtin_elementwise_min(mn, m - (us2)(1));
}

__device__ __forceinline__ uint32_t lane_pack(us2 v, bool is_max) {
  const uint32_t a = v.x, b = v.y;
  return is_max ? (a > b ? a : b) : (a < b ? a : b);
}

// span of a group in binades, from the reduced max bits and min (bits-1).
// Returns -1 for an all-zero group.
__device__ __forceinline__ int group_span(uint32_t mxbits, uint32_t mnbits) {
  if (mnbits == 0xFFFFu) return -1;
  const int emax = (int)(mxbits >> 7);
  int emin = (int)((mnbits + 1u) >> 7);
  if (mnbits >= 0x7F80u) emin = (int)(mnbits >> 7);  // cannot happen for finite input
  emin = emin < 1 ? 1 : emin;
  return emax - emin;
}

}  // namespace

// ============================================================================
// Fast kernel: 64 contiguous elements per lane; a row is spread over a team
// of T = K/64 lanes; a block holds rows_per_block rows (one "batch") at a
// time and walks batches blockIdx.x, blockIdx.x + gridDim.x, ... (persistent
// grid). The next batch's bf16 words are loaded into registers while the
// current batch is transformed (16-bit words: bf16, or half when F16). The per-row max and flag go through LDS
// slots used round-robin over 3 batches, so one barrier per batch suffices:
// the slot reset after batch b's barrier is that of batch b-1 (whose readers
// all passed the barrier) and it is next written after batch b+1's barrier.
// ============================================================================

template <int G, bool F16>
__global__ __launch_bounds__(512) void rotate_quant_fast_kernel(
    const uint16_t* __restrict__ x, int8_t* __restrict__ xq, float* __restrict__ scale,
    int64_t rows, int K, int T, int rows_per_block, int64_t nbatches, SignMask sm) {
  constexpr int CH = 64;
  constexpr int LOGG = ilog2(G);
  constexpr int kMaxSpan = 45 - LOGG;
  constexpr int NGL = G >= CH ? 1 : CH / G;  // groups held by one lane
  constexpr int KS = LOGG / 2;               // 1/sqrt(g) = 2^-KS
  __shared__ uint32_t s_rowmax[3][256];
  __shared__ uint32_t s_rowflag[3][256];

  const int tid = threadIdx.x;
  const int r_in = tid / T;
  const int c = tid - r_in * T;
  const bool in_team = r_in < rows_per_block;
  if (tid < rows_per_block) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      s_rowmax[q][tid] = 0u;
      s_rowflag[q][tid] = 0u;
    }
  }

  // sign bits of this lane's 64 outputs
  uint32_t sg0, sg1;
  if constexpr (G == 256) {
    const int q = c & 3;
    sg0 = sm.w[2 * q];
    sg1 = sm.w[2 * q + 1];
  } else if constexpr (G == 64) {
    sg0 = sm.w[0];
    sg1 = sm.w[1];
  } else if constexpr (G == 16) {
    sg0 = (sm.w[0] & 0xFFFFu) * 0x00010001u;
    sg1 = sg0;
  } else {
    sg0 = (sm.w[0] & 0xFu) * 0x11111111u;
    sg1 = sg0;
  }

  auto load = [&](int64_t batch, uint32_t (&w)[32]) {
    const int64_t row = batch * rows_per_block + r_in;
    if (in_team && batch < nbatches && row < rows) {
      const u4* p = reinterpret_cast<const u4*>(x + row * (int64_t)K + (int64_t)CH * c);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u4 q = p[i];
        w[4 * i + 0] = q.x;
        w[4 * i + 1] = q.y;
        w[4 * i + 2] = q.z;
        w[4 * i + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) w[i] = 0u;
    }
  };

  uint32_t w[32];
  int64_t batch = blockIdx.x;
  load(batch, w);
  __syncthreads();  // slot initialisation visible

  for (int it = 0; batch < nbatches; ++it, batch += gridDim.x) {
    const int64_t row = batch * rows_per_block + r_in;
    const bool active = in_team && row < rows;
    uint32_t wn[32];
    load(batch + gridDim.x, wn);

    // ---- exponent span per group (half groups are always exact) ----
    bool flagged = false;
    if constexpr (!F16) {
      constexpr int DW = (G >= CH ? CH : G) / 2;  // dwords per (lane part of a) group
#pragma unroll
      for (int gidx = 0; gidx < NGL; ++gidx) {
        us2 mx = (us2)(0), mn = (us2)(0xFFFF);
#pragma unroll
        for (int i = 0; i < DW; ++i) span_acc(w[gidx * DW + i], mx, mn);
        uint32_t a = lane_pack(mx, true), b = lane_pack(mn, false);
        if constexpr (G == 256) {
          uint32_t t = dpp_u32<kQuadXor1>(a); a = a > t ? a : t;
          t = dpp_u32<kQuadXor2>(a); a = a > t ? a : t;
          t = dpp_u32<kQuadXor1>(b); b = b < t ? b : t;
          t = dpp_u32<kQuadXor2>(b); b = b < t ? b : t;
        }
        flagged |= group_span(a, b) > kMaxSpan;
      }
    }

    // ---- widen, transform ----
    double v[CH];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[2 * i] = (double)(F16 ? half_lo(w[i]) : bf16lo(w[i]));
      v[2 * i + 1] = (double)(F16 ? half_hi(w[i]) : bf16hi(w[i]));
    }
    fwht_inlane<G, CH>(v);
    if constexpr (G == 256) {
      const int q = c & 3;  // position of this lane's 64-element part in its group
      const double s1 = (q & 1) ? -1.0 : 1.0;
      const double s2 = (q & 2) ? -1.0 : 1.0;
#pragma unroll
      for (int i = 0; i < CH; ++i) v[i] = __builtin_fma(v[i], s1, dpp_f64<kQuadXor1>(v[i]));
#pragma unroll
      for (int i = 0; i < CH; ++i) v[i] = __builtin_fma(v[i], s2, dpp_f64<kQuadXor2>(v[i]));
    }

    // u = RN32(y) (y = unscaled, unsigned sum); x_r = d_j * u * 2^-k for normal x_r
    float u[CH];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      u[i] = (float)v[i];
      amax = fmaxf(amax, fabsf(u[i]));
    }

    const int slot = it % 3;
    if (active) {
      atomicMax(&s_rowmax[slot][r_in], __float_as_uint(amax));
      if (flagged) atomicOr(&s_rowflag[slot][r_in], 1u);
    }
    __syncthreads();
    if (tid < rows_per_block) {
      const int nslot = (it + 2) % 3;
      s_rowmax[nslot][tid] = 0u;
      s_rowflag[nslot][tid] = 0u;
    }

    if (active) {
      const float amax_u = __uint_as_float(s_rowmax[slot][r_in]);
      const float amax_x = amax_u * (1.0f / (float)(1 << KS));  // exact unless deferred
      const bool deferred = s_rowflag[slot][r_in] != 0u || !(amax_u <= 3.0e38f) ||
                            (amax_u > 0.0f && amax_x < 0x1p-100f);
      if (deferred) {
        if (c == 0) scale[row] = __uint_as_float(kDeferredRow);
      } else {
        float sc, inv_u;
        if (amax_u > 0.0f) {
          sc = amax_x / 127.0f;
          const float inv = 127.0f / amax_x;
          inv_u = inv * (1.0f / (float)(1 << KS));
        } else {
          sc = 0.0f;
          inv_u = 0.0f;
        }
        if (c == 0) scale[row] = sc;

        uint32_t outw[16];
#pragma unroll
        for (int d = 0; d < 16; ++d) {
          uint32_t b[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = u[4 * d + e] * inv_u;
            b[e] = __float_as_uint(p + kQuantBias);  // q + 128 in the low byte
          }
          const uint32_t t0 = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);
          const uint32_t t1 = __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
          const uint32_t packed = t0 | t1;
          const uint32_t nib = ((d < 8 ? sg0 : sg1) >> ((4 * d) & 31)) & 0xFu;
          const uint32_t m = nibble_to_bytemask(nib);
          // negate the bytes with d = -1 (biased: 256 - v never carries), unbias
          outw[d] = ((packed ^ m) + (m & 0x01010101u)) ^ 0x80808080u;
        }
        u4* o = reinterpret_cast<u4*>(xq + row * (int64_t)K + (int64_t)CH * c);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = (u4){outw[4 * i], outw[4 * i + 1], outw[4 * i + 2], outw[4 * i + 3]};
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = wn[i];
  }
}

// ============================================================================
// Exact kernel: 32 contiguous elements per lane, team of T = K/32 lanes per
// row. Modes: per-row quantize (optionally only rows carrying kDeferredRow),
// per-tensor absmax (pass 1) and per-tensor quantize (pass 2).
// ============================================================================

enum ExactMode : int { kRowAll = 0, kRowDeferred = 1, kTensorMax = 2, kTensorQuant = 3 };

template <int G, bool WIDE>
__global__ __launch_bounds__(512) void rotate_quant_exact_kernel(
    const uint16_t* __restrict__ x, int8_t* __restrict__ xq, float* __restrict__ scale,
    uint32_t* __restrict__ tensor_amax, int64_t rows, int K, int T, int rows_per_block,
    int64_t nbatches, SignMask sm, int mode) {
  constexpr int CH = 32;
  constexpr int LOGG = ilog2(G);
  constexpr int KS = LOGG / 2;
  constexpr int NGL = G >= CH ? 1 : CH / G;  // groups held by one lane
  constexpr int GE = G >= CH ? CH : G;       // elements of a group in one lane
  constexpr int LPG = G >= CH ? G / CH : 1;  // lanes per group
  __shared__ uint32_t s_rowmax[256];
  __shared__ uint32_t s_rowflag[256];
  __shared__ uint32_t s_rowunc[256];   // 1 + bits of an undecided element's larger candidate
  __shared__ uint32_t s_rowconf[256];  // an undecided element quantizes both ways

  const int tid = threadIdx.x;
  const int r_in = tid / T;
  const int c = tid - r_in * T;
  if (mode == kRowDeferred) {
    // one parallel look at the scale slots of all rows this block would
    // visit; usually none is deferred and the block is done
    bool any = false;
    const int64_t per_pass = (int64_t)gridDim.x * rows_per_block;
    for (int64_t i = tid; ; i += blockDim.x) {
      const int64_t pass = i / rows_per_block;
      const int64_t r = (int64_t)blockIdx.x * rows_per_block + pass * per_pass +
                        (i - pass * rows_per_block);
      if (r >= rows) break;
      any |= __float_as_uint(scale[r]) == kDeferredRow;
    }
    if (__syncthreads_or(any) == 0) return;
  }
  // persistent grid: batches of rows_per_block rows, strided by gridDim.x
  for (int64_t batch = blockIdx.x; batch < nbatches; batch += gridDim.x) {
  __syncthreads();  // the previous batch's readers of the LDS slots are done
  const int64_t row = batch * rows_per_block + r_in;
  bool active = (r_in < rows_per_block) && (row < rows);
  if (tid < rows_per_block) {
    s_rowmax[tid] = 0u;
    s_rowflag[tid] = 0u;
    s_rowunc[tid] = 0u;
    s_rowconf[tid] = 0u;
  }
  if (mode == kRowDeferred) {
    // rows that the fast kernel finished are skipped as a whole
    if (active) active = __float_as_uint(scale[row]) == kDeferredRow;
    if (__syncthreads_or(active) == 0) continue;
  }

  uint32_t w[16];
  if (active) {
    const uint4* p = reinterpret_cast<const uint4*>(x + row * (int64_t)K + (int64_t)CH * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = p[i];
      w[4 * i + 0] = q.x;
      w[4 * i + 1] = q.y;
      w[4 * i + 2] = q.z;
      w[4 * i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = 0u;
  }

  // per group: largest exponent field E and band count
  int egrp[NGL];
  int nb_lane = 0;
  uint32_t gmask = 0u;  // bit gidx: group gidx spans more than float64 adds exactly
#pragma unroll
  for (int gidx = 0; gidx < NGL; ++gidx) {
    us2 mx = (us2)(0), mn = (us2)(0xFFFF);
#pragma unroll
    for (int i = 0; i < GE / 2; ++i) span_acc(w[gidx * (GE / 2) + i], mx, mn);
    uint32_t a = lane_pack(mx, true), b = lane_pack(mn, false);
    // over the LPG lanes of the group (consecutive lanes within 8: DPP)
    auto xred = [&](auto mt) {
      constexpr int m = decltype(mt)::value;
      const uint32_t ta = xor_lanes_u32<m>(a);
      const uint32_t tb = xor_lanes_u32<m>(b);
      a = a > ta ? a : ta;
      b = b < tb ? b : tb;
    };
    if constexpr (LPG > 1) xred(std::integral_constant<int, 1>{});
    if constexpr (LPG > 2) xred(std::integral_constant<int, 2>{});
    if constexpr (LPG > 4) xred(std::integral_constant<int, 4>{});
    const int span = group_span(a, b);
    if (span > 45 - LOGG) gmask |= 1u << gidx;
    int e = (int)(a >> 7);
    egrp[gidx] = e < 1 ? 1 : e;
    const int nb = span < 0 ? 0 : span / kBand + 1;
    nb_lane = nb_lane > nb ? nb_lane : nb;
  }
  if constexpr (WIDE) {
    // ---- one rounded float64 transform first (rows the fast kernel left:
    // mostly wide-span groups). Each output is a depth-LOGG tree of correctly
    // rounded additions, so it is within LOGG * 2^-53 * S of the exact sum
    // (S = sum |x| over the group); delta = 2^-46 * S' bounds that with a wide
    // margin (S' = fp32 sum of |x| over the group for g >= 32, over the lane
    // otherwise). With u = RN32(y) and d = y - u (exact), the exact sum rounds
    // to u when |d| + delta is below the half-gap h from u to its next
    // rounding boundary (ulp/2, ulp/4 at a power of two, 2^-151 at zero);
    // h is a power of two, so the float64 test is exact. Otherwise, with
    // delta < h, it rounds to u or to u's neighbour on the side of y
    // (undecided). The row is finished here unless an undecided element
    // could be its absmax or quantizes differently for its two candidates.
    float u[CH];
    uint64_t umask = 0ull, dmask = 0ull;
    uint32_t unc_hi = 0u;
    bool unsafe = false;
    float wamax = 0.0f;
    {
      double y[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i)
        y[i] = (double)__uint_as_float((i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16));
      float sabs = 0.0f;
#pragma unroll
      for (int i = 0; i < CH; ++i) sabs += fabsf((float)y[i]);
      fwht_inlane<G, CH>(y);
      // cross-lane stages over the LPG lanes of a group (DPP, in-row)
      auto xstage = [&](auto mt) {
        constexpr int m = decltype(mt)::value;
        const double sg = ((c & m) != 0) ? -1.0 : 1.0;
#pragma unroll
        for (int i = 0; i < CH; ++i) y[i] = __builtin_fma(y[i], sg, xor_lanes_f64<m>(y[i]));
        sabs += __uint_as_float(xor_lanes_u32<m>(__float_as_uint(sabs)));
      };
      if constexpr (LPG > 1) xstage(std::integral_constant<int, 1>{});
      if constexpr (LPG > 2) xstage(std::integral_constant<int, 2>{});
      if constexpr (LPG > 4) xstage(std::integral_constant<int, 4>{});
      static_assert(LPG <= 8, "group spans at most 8 lanes");
      const double delta = (double)sabs * 0x1p-46;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        u[i] = (float)y[i];
        wamax = fmaxf(wamax, fabsf(u[i]));
        const uint32_t rb = __float_as_uint(u[i]);
        uint32_t ef = (rb >> 23) & 0xFFu;
        ef = ef < 1u ? 1u : ef;
        const uint32_t pow2 = (rb & 0x7FFFFFu) == 0u ? 1u : 0u;
        const double h =
            __longlong_as_double((int64_t)(uint64_t)(ef + (1023u - 151u) - pow2) << 52);
        const double d = y[i] - (double)u[i];
        const bool wide = (gmask >> (i / GE)) & 1u;
        const bool und = wide && !(fabs(d) + delta < h);
        unsafe |= und && !(delta < h);
        const uint32_t mb = rb & 0x7FFFFFFFu;
        const bool away = (d > 0.0) == !(rb >> 31) || mb == 0u;
        umask |= (uint64_t)und << i;
        dmask |= (uint64_t)(und && away) << i;
        const uint32_t hb = und ? mb + (away ? 1u : 0u) : 0u;
        unc_hi = hb > unc_hi ? hb : unc_hi;
      }
    }
    if (active) {
      atomicMax(&s_rowmax[r_in], __float_as_uint(wamax));
      if (unsafe) atomicOr(&s_rowflag[r_in], 1u);
      if (umask != 0ull) atomicMax(&s_rowunc[r_in], unc_hi + 1u);
    }
    __syncthreads();
    const float amax_u = __uint_as_float(s_rowmax[r_in]);
    const float amax_x = amax_u * (1.0f / (float)(1 << KS));  // exact when not deferred
    const uint32_t rowunc = s_rowunc[r_in];
    bool wide_ok = active && s_rowflag[r_in] == 0u && amax_u <= 3.0e38f &&
                   !(amax_u > 0.0f && amax_x < 0x1p-100f) &&
                   !(rowunc != 0u && rowunc - 1u >= __float_as_uint(amax_u));
    float wsc = 0.0f;
    uint32_t wout[CH / 4];
    if (wide_ok) {
      float inv_u = 0.0f;
      if (amax_u > 0.0f) {
        wsc = amax_x / 127.0f;
        inv_u = (127.0f / amax_x) * (1.0f / (float)(1 << KS));
      }
      const int base_j = (G >= CH) ? CH * (c % LPG) : 0;
      bool conflict = false;
#pragma unroll
      for (int d4 = 0; d4 < CH / 4; ++d4) {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * d4 + e;
          const int j = (G >= CH) ? base_j + i : (i % G);
          const float sgn = sign_bit(sm, j) ? -1.0f : 1.0f;
          b[e] = __float_as_uint((sgn * u[i]) * inv_u + kQuantPlain);
          // the other candidate of an undecided element (u's sign; a zero's
          // sign does not reach q)
          const uint32_t rb = __float_as_uint(u[i]);
          const uint32_t mb = rb & 0x7FFFFFFFu;
          const uint32_t nb = ((dmask >> i) & 1ull) ? mb + 1u : mb - 1u;
          const float un = __uint_as_float((rb & 0x80000000u) | nb);
          const uint32_t b2 = __float_as_uint((sgn * un) * inv_u + kQuantPlain);
          conflict |= ((umask >> i) & 1ull) && ((b[e] ^ b2) & 0xFFu) != 0u;
        }
        const uint32_t t0 = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);
        const uint32_t t1 = __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
        wout[d4] = t0 | t1;
      }
      if (conflict) atomicOr(&s_rowconf[r_in], 1u);
    }
    __syncthreads();  // conflicts published; s_rowmax readers done
    wide_ok = wide_ok && s_rowconf[r_in] == 0u;
    if (wide_ok) {
      uint4* o = reinterpret_cast<uint4*>(xq + row * (int64_t)K + (int64_t)CH * c);
#pragma unroll
      for (int i = 0; i < CH / 16; ++i)
        o[i] = make_uint4(wout[4 * i], wout[4 * i + 1], wout[4 * i + 2], wout[4 * i + 3]);
      if (c == 0) scale[row] = wsc;
    }
    // the banded algorithm below for the rows still open
    active = active && !wide_ok;
    if (tid < rows_per_block) s_rowmax[tid] = 0u;  // published by the barrier below
    if (__syncthreads_or(active) == 0) continue;
  }

  // all lanes run the same number of bands (empty bands add nothing)
  int nb_all = nb_lane;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int t = __shfl_xor(nb_all, m);
    nb_all = nb_all > t ? nb_all : t;
  }

  double V[CH];
  uint32_t sticky = 0u;
#pragma unroll
  for (int i = 0; i < CH; ++i) V[i] = 0.0;

  for (int band = nb_all - 1; band >= 0; --band) {
    // keep the widened inputs out of registers across bands: recompute them
    // from the packed bf16 words each band (an empty asm marks the words as
    // changed, so the conversions are not hoisted out of the loop)
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(w[i]));
    double F[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
      const int f = (int)((bits >> 7) & 0xFFu);
      const int fe = f < 1 ? 1 : f;
      const int eg = egrp[i / GE];
      const bool in_band = ((bits & 0x7FFFu) != 0u) && ((eg - fe) / kBand == band);
      const float xv = __uint_as_float(bits << 16);
      F[i] = in_band ? (double)xv : 0.0;
    }
    fwht_inlane<G, CH>(F);
    // cross-lane stages over the LPG lanes of a group (DPP, in-row)
    auto bstage = [&](auto mt) {
      constexpr int m = decltype(mt)::value;
      const double sg = ((c & m) != 0) ? -1.0 : 1.0;
#pragma unroll
      for (int i = 0; i < CH; ++i) F[i] = __builtin_fma(F[i], sg, xor_lanes_f64<m>(F[i]));
    };
    if constexpr (LPG > 1) bstage(std::integral_constant<int, 1>{});
    if constexpr (LPG > 2) bstage(std::integral_constant<int, 2>{});
    if constexpr (LPG > 4) bstage(std::integral_constant<int, 4>{});
    // integers of the band quantum 2^q_b, q_b = E - (band+1)*kBand - 133
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int eg = egrp[i / GE];
      const double I = __builtin_ldexp(F[i], (band + 1) * kBand + 133 - eg);
      const double fl = __builtin_floor(V[i] * 0x1p-36);
      sticky |= (V[i] != fl * 0x1p36) ? (1u << i) : 0u;
      V[i] = I + fl;
    }
  }

  // x_r = d_j * (2V + sticky) * 2^(q_0 - 1 - KS), rounded once to fp32
  float xr[CH];
  float amax = 0.0f;
  const int base_j = (G >= CH) ? CH * (c % LPG) : 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int eg = egrp[i / GE];
    const double W = 2.0 * V[i] + (double)((sticky >> i) & 1u);
    const int j = (G >= CH) ? base_j + i : (i % G);
    const double sgn = sign_bit(sm, j) ? -1.0 : 1.0;
    xr[i] = (float)(sgn * __builtin_ldexp(W, eg - kBand - 133 - 1 - KS));
    amax = fmaxf(amax, fabsf(xr[i]));
  }

  if (mode == kTensorMax) {
    // wave max, then one atomic per wave
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    if ((tid & 63) == 0 && amax > 0.0f) atomicMax(tensor_amax, __float_as_uint(amax));
    continue;
  }

  float rmax;
  if (mode == kTensorQuant) {
    rmax = __uint_as_float(*tensor_amax);
  } else {
    __syncthreads();
    if (active) atomicMax(&s_rowmax[r_in], __float_as_uint(amax));
    __syncthreads();
    rmax = __uint_as_float(s_rowmax[r_in]);
  }
  if (!active) continue;

  float s = 0.0f, inv = 0.0f, pre = 1.0f;
  if (rmax > 0.0f) {
    s = rmax / 127.0f;
    float a = rmax;
    if (a < 0x1p-64f) {
      a *= 0x1p64f;
      pre = 0x1p64f;
    }
    inv = 127.0f / a;
  }
  if (mode != kTensorQuant && c == 0) scale[row] = s;

  uint32_t outw[CH / 4];
#pragma unroll
  for (int d = 0; d < CH / 4; ++d) {
    uint32_t b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = (xr[4 * d + e] * pre) * inv;
      b[e] = __float_as_uint(p + kQuantPlain);
    }
    const uint32_t t0 = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);
    const uint32_t t1 = __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
    outw[d] = t0 | t1;
  }
  uint4* o = reinterpret_cast<uint4*>(xq + row * (int64_t)K + (int64_t)CH * c);
#pragma unroll
  for (int i = 0; i < CH / 16; ++i)
    o[i] = make_uint4(outw[4 * i], outw[4 * i + 1], outw[4 * i + 2], outw[4 * i + 3]);
  }  // batch loop
}

__global__ void tensor_scale_init_kernel(uint32_t* amax_bits) { *amax_bits = 0u; }

__global__ void tensor_scale_final_kernel(float* s_w) {
  const float amax = __uint_as_float(*reinterpret_cast<uint32_t*>(s_w));
  *s_w = amax > 0.0f ? amax / 127.0f : 0.0f;
}

// ============================================================================
// Launchers
// ============================================================================

namespace {

struct TeamShape {
  int T;      // lanes per row
  int block;  // threads per block
  int rpb;    // rows per block
};

// Choose a block of whole waves holding whole rows of T lanes (at most 512
// threads, at most 256 rows) for a persistent kernel with `wpc` resident
// waves per CU: the most row lanes at work per CU (resident blocks x rows per
// block x T), ties to the smaller block.
TeamShape team_shape(int T, int wpc) {
  TeamShape best{T, 0, 0};
  int best_lanes = 0;
  for (int waves = 1; waves <= 8; ++waves) {
    const int threads = 64 * waves;
    int rpb = threads / T;
    if (rpb < 1) continue;
    if (rpb > 256) rpb = 256;
    const int blocks = wpc / waves > 0 ? wpc / waves : 1;
    const int lanes = blocks * rpb * T;
    if (lanes > best_lanes) {
      best_lanes = lanes;
      best.block = threads;
      best.rpb = rpb;
    }
  }
  return best;
}

// Resident waves per CU that the persistent fast kernel aims for
// (compile-time tunable).
#ifndef CONVROT_FAST_WAVES_PER_CU
#define CONVROT_FAST_WAVES_PER_CU 8
#endif
constexpr int kFastWavesPerCU = CONVROT_FAST_WAVES_PER_CU;

template <int G>
hipError_t launch_fast(const uint16_t* x, int8_t* xq, float* s, int64_t rows, int K,
                       const SignMask& sm, bool f16, hipStream_t st) {
  const TeamShape ts = team_shape(K / 64, kFastWavesPerCU);
  const int64_t nbatches = (rows + ts.rpb - 1) / ts.rpb;
  // whole blocks per CU that stay resident together: a grid beyond that would
  // run a second, partial round of blocks
  const int per_cu = kFastWavesPerCU / (ts.block / 64);
  const int64_t cap = (int64_t)kNumCUs * (per_cu > 0 ? per_cu : 1);
  const int64_t blocks = nbatches < cap ? nbatches : cap;
  auto kern = f16 ? rotate_quant_fast_kernel<G, true> : rotate_quant_fast_kernel<G, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(ts.block), 0, st, x, xq, s, rows, K,
                     ts.T, ts.rpb, nbatches, sm);
  return hipGetLastError();
}

// Resident waves per CU of the persistent exact kernel. Over the rows the
// fast kernel deferred, each block first scans its rows' scale slots in one
// parallel pass and returns at once when none is deferred, so a full grid
// costs little on ordinary inputs and keeps the chip busy on inputs (GELU
// tails) that defer most rows.
constexpr int kExactWavesPerCU = 8;
#ifndef CONVROT_DEFERRED_WAVES_PER_CU
#define CONVROT_DEFERRED_WAVES_PER_CU 8
#endif
constexpr int kDeferredWavesPerCU = CONVROT_DEFERRED_WAVES_PER_CU;

template <int G>
hipError_t launch_exact(const uint16_t* x, int8_t* xq, float* s, uint32_t* tensor_amax,
                        int64_t rows, int K, const SignMask& sm, int mode, hipStream_t st) {
  const int wpc = mode == kRowDeferred ? kDeferredWavesPerCU : kExactWavesPerCU;
  const TeamShape ts = team_shape(K / 32, wpc);
  const int64_t nbatches = (rows + ts.rpb - 1) / ts.rpb;
  const int per_cu = wpc / (ts.block / 64);  // whole resident blocks per CU
  const int64_t cap = (int64_t)kNumCUs * (per_cu > 0 ? per_cu : 1);
  const int64_t blocks = nbatches < cap ? nbatches : cap;
  // rows the fast kernel left get a rounded float64 transform first
  auto kern = mode == kRowDeferred ? rotate_quant_exact_kernel<G, true>
                                   : rotate_quant_exact_kernel<G, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(ts.block), 0, st, x, xq, s, tensor_amax,
                     rows, K, ts.T, ts.rpb, nbatches, sm, mode);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(const uint16_t* x, int8_t* xq, float* s, int64_t rows, int K,
                                int g, const SignMask& sm, DType dt, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const bool f16 = dt == DType::kF16;
  hipError_t e;
  switch (g) {
    case 4: e = launch_fast<4>(x, xq, s, rows, K, sm, f16, st); break;
    case 16: e = launch_fast<16>(x, xq, s, rows, K, sm, f16, st); break;
    case 64: e = launch_fast<64>(x, xq, s, rows, K, sm, f16, st); break;
    default: e = launch_fast<256>(x, xq, s, rows, K, sm, f16, st); break;
  }
  if (e != hipSuccess || f16) return e;  // half rows are never deferred
  switch (g) {
    case 4: return launch_exact<4>(x, xq, s, nullptr, rows, K, sm, kRowDeferred, st);
    case 16: return launch_exact<16>(x, xq, s, nullptr, rows, K, sm, kRowDeferred, st);
    case 64: return launch_exact<64>(x, xq, s, nullptr, rows, K, sm, kRowDeferred, st);
    default: return launch_exact<256>(x, xq, s, nullptr, rows, K, sm, kRowDeferred, st);
  }
}

hipError_t launch_quantize_rows_exact(const uint16_t* x, int8_t* xq, float* s, int64_t rows,
                                      int K, int g, const SignMask& sm, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  switch (g) {
    case 4: return launch_exact<4>(x, xq, s, nullptr, rows, K, sm, kRowAll, st);
    case 16: return launch_exact<16>(x, xq, s, nullptr, rows, K, sm, kRowAll, st);
    case 64: return launch_exact<64>(x, xq, s, nullptr, rows, K, sm, kRowAll, st);
    default: return launch_exact<256>(x, xq, s, nullptr, rows, K, sm, kRowAll, st);
  }
}

hipError_t launch_quantize_tensor(const uint16_t* w, int8_t* wq, float* s_w, int64_t rows, int K,
                                  int g, const SignMask& sm, hipStream_t st) {
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(s_w);
  hipLaunchKernelGGL(tensor_scale_init_kernel, dim3(1), dim3(1), 0, st, amax_bits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows == 0) {
    if (e == hipSuccess) {
      hipLaunchKernelGGL(tensor_scale_final_kernel, dim3(1), dim3(1), 0, st, s_w);
      e = hipGetLastError();
    }
    return e;
  }
  for (int mode : {(int)kTensorMax, (int)kTensorQuant}) {
    switch (g) {
      case 4: e = launch_exact<4>(w, wq, nullptr, amax_bits, rows, K, sm, mode, st); break;
      case 16: e = launch_exact<16>(w, wq, nullptr, amax_bits, rows, K, sm, mode, st); break;
      case 64: e = launch_exact<64>(w, wq, nullptr, amax_bits, rows, K, sm, mode, st); break;
      default: e = launch_exact<256>(w, wq, nullptr, amax_bits, rows, K, sm, mode, st); break;
    }
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(tensor_scale_final_kernel, dim3(1), dim3(1), 0, st, s_w);
  return hipGetLastError();
}

}  // namespace convrot

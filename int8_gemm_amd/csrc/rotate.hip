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
//     53 bits and float64 is exact. A group outside that bound ("wide") gets
//     an error bound instead (from its largest exponent and its sum of |x|):
//     an output whose bound interval rounds to one fp32 is decided, the
//     others are "open" between two neighbouring floats. The row is finished
//     unless an open element could be its absmax, has more than two
//     candidates, or quantizes differently for its two candidates; such rows
//     (and rows too small for the folded scaling below) are deferred: their
//     scale slot receives the kDeferredRow NaN, and the block that deferred
//     them runs the exact row pass on them after its last batch.
//   * Deferred rows (the exact row pass's deferred mode) first get one
//     rounded float64 transform: each output is within log2(g) * 2^-53 * sum|x| of
//     the exact sum (a depth-log2(g) tree of rounded additions), so with
//     that bound (and margin) an element either provably rounds to
//     RN32(y), or to one of RN32(y) and its neighbour. The undecided
//     elements that could be the row's absmax are then summed again with
//     error-free additions, which decides nearly all of them. The row is
//     finished there unless an undecided element is still a candidate for
//     the absmax or quantizes differently for its two candidates (ties
//     decided only by elements the float64 sum lost).
//   * Exact row pass (the exact kernel, and the rest of a deferred row):
//     splits each group's elements into bands of kBand
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
// Exact row pass: 32 contiguous elements per lane, a team of T = K/32 lanes
// per row, rows row0 .. row0 + nrows - 1 in one call (nrows <= blockDim / T).
// Modes: per-row quantize of every row, or of the rows carrying kDeferredRow
// (the fast kernel's blocks call it for the rows they defer), per-tensor
// absmax (pass 1) and per-tensor quantize (pass 2). Every thread of the block
// calls it with the same arguments (it holds block barriers).
// ============================================================================

enum ExactMode : int { kRowAll = 0, kRowDeferred = 1, kTensorMax = 2, kTensorQuant = 3 };

// per-row LDS slots of one call
template <bool WIDE>
struct ExactLds {
  uint32_t rowmax[256];
  uint32_t rowflag[256];
  uint32_t rowunc[256];   // 1 + bits of an undecided element's larger candidate
  uint32_t rowconf[256];  // an undecided element quantizes both ways
  // after the resolution of a row's absmax-risk elements: the row's absmax,
  // its largest undecided candidate (+1), and a flag for an element too close
  uint32_t rowmax2[WIDE ? 256 : 1];
  uint32_t rowunc2[WIDE ? 256 : 1];
  uint32_t rowflag2[WIDE ? 256 : 1];
};

// The 32 sign bits of a lane's 32 outputs (bit i: output i has d = -1): word
// c % LPG of the mask for groups across lanes, else word 0 at i % G. Chosen
// with selects (no indexed access, which would put the mask in scratch).
template <int G, int CH>
__device__ __forceinline__ uint32_t lane_sign_word(const SignMask& sm, int c) {
  constexpr int LPG = G >= CH ? G / CH : 1;
  uint32_t w = sm.w[0];
#pragma unroll
  for (int q = 1; q < LPG; ++q) w = (c % LPG) == q ? sm.w[q] : w;
  return w;
}

// WIDE: the rows first get one rounded float64 transform with an error bound
// (the rows the fast kernel deferred: mostly wide-span groups); rows it does
// not finish, and every row when !WIDE, take the banded algorithm.
template <int G, bool WIDE>
__device__ __forceinline__ void exact_rows(ExactLds<WIDE>& L, const uint16_t* __restrict__ x,
                                           int8_t* __restrict__ xq, float* __restrict__ scale,
                                           uint32_t* __restrict__ tensor_amax, int64_t rows, int K,
                                           int T, int64_t row0, int nrows, const SignMask& sm,
                                           int mode) {
  constexpr int CH = 32;
  constexpr int LOGG = ilog2(G);
  constexpr int KS = LOGG / 2;
  constexpr int NGL = G >= CH ? 1 : CH / G;  // groups held by one lane
  constexpr int GE = G >= CH ? CH : G;       // elements of a group in one lane
  constexpr int LPG = G >= CH ? G / CH : 1;  // lanes per group

  const int tid = threadIdx.x;
  const int r_in = tid / T;
  const int c = tid - r_in * T;
  __syncthreads();  // the previous call's readers of the LDS slots are done
  const int64_t row = row0 + r_in;
  bool active = (r_in < nrows) && (row < rows);
  if (tid < nrows) {
    L.rowmax[tid] = 0u;
    L.rowflag[tid] = 0u;
    L.rowunc[tid] = 0u;
    L.rowconf[tid] = 0u;
    if constexpr (WIDE) {
      L.rowmax2[tid] = 0u;
      L.rowunc2[tid] = 0u;
      L.rowflag2[tid] = 0u;
    }
  }
  if (mode == kRowDeferred) {
    // rows that the fast kernel finished are skipped as a whole
    if (active) active = __float_as_uint(scale[row]) == kDeferredRow;
    if (__syncthreads_or(active) == 0) return;
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
    // (S = sum |x| over the group); delta = 2^-49 * S' is at least twice that
    // (LOGG <= 8; S' = fp32 sum of |x| over the group for g >= 32, over the
    // lane otherwise, S' >= S (1 - 2^-16)). With u = RN32(y) and d = y - u
    // (exact), the exact sum rounds to u when |d| + delta is below the
    // half-gap h from u to its next rounding boundary (ulp/2, ulp/4 at a
    // power of two, 2^-151 at zero);
    // h is a power of two, so the float64 test is exact. Otherwise, with
    // delta < h, it rounds to u or to u's neighbour on the side of y
    // (undecided). The row is finished here unless an undecided element
    // could be its absmax or quantizes differently for its two candidates.
    float u[CH];
    uint64_t umask = 0ull, dmask = 0ull;
    uint32_t unc_hi = 0u;
    bool unsafe = false;
    float wamax = 0.0f;
    float sabs_g = 0.0f;  // fp32 sum of |x| over the group (over the lane for g < 32)
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
      sabs_g = sabs;
      // twice the bound log2 g * 2^-53 * S <= 2^-50 S (sabs >= S (1 - 2^-16))
      const double delta = (double)sabs * 0x1p-49;
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
        if (und) {  // rare: the bookkeeping of an undecided element
          unsafe |= !(delta < h);
          const uint32_t mb = rb & 0x7FFFFFFFu;
          const bool away = (d > 0.0) == !(rb >> 31) || mb == 0u;
          umask |= 1ull << i;
          dmask |= (uint64_t)away << i;
          const uint32_t hb = mb + (away ? 1u : 0u);
          unc_hi = hb > unc_hi ? hb : unc_hi;
        }
      }
    }
    if (active) {
      atomicMax(&L.rowmax[r_in], __float_as_uint(wamax));
      if (unsafe) atomicOr(&L.rowflag[r_in], 1u);
      if (umask != 0ull) atomicMax(&L.rowunc[r_in], unc_hi + 1u);
    }
    __syncthreads();
    // ---- rows whose absmax an undecided element could be: those elements
    // (larger candidate reaching the row's absmax) get their exact rounding,
    // then the row takes its absmax again; the rest of the row is unchanged.
    bool risky = false;
    {
      const uint32_t au0 = L.rowmax[r_in], ru0 = L.rowunc[r_in];
      risky = active && L.rowflag[r_in] == 0u && ru0 != 0u && ru0 - 1u >= au0 &&
              __uint_as_float(au0) <= 3.0e38f;
      if (__syncthreads_or(risky)) {
        uint64_t pend = 0ull;
        if (risky) {
#pragma unroll
          for (int i = 0; i < CH; ++i) {
            const uint32_t mb = __float_as_uint(u[i]) & 0x7FFFFFFFu;
            const uint32_t hb = mb + (uint32_t)((dmask >> i) & 1ull);
            pend |= (uint64_t)(((umask >> i) & 1ull) && hb >= au0) << i;
          }
        }
        bool left = false;
        // ---- the exact rounding of the undecided elements: per position i a
        // group's lanes sum their part's inputs again with error-free
        // additions (value s, rounding errors summed apart in e), then run the
        // cross-lane stages on (s, e) the same way, so that every lane holds
        // its own output at position i as s + e, within 2^-93 sum |x| of the
        // exact sum. From r = RN32(s): if s + e lies farther than that margin
        // from r's rounding boundaries it rounds to r; else, from the midpoint
        // of r and its neighbour on the side of s + e, to one of the two.
        // What is too close to decide leaves the row to the banded algorithm.
        // The float64 differences used are exact (Sterbenz: the operands lie
        // within a factor two of each other). ----
        const double bnd = (double)sabs_g * 0x1p-88;  // margin for |s + e - exact| (sabs: fp32 group sum)
        for (;;) {
          uint32_t code = pend != 0ull ? (uint32_t)__builtin_ctzll(pend) : 0xFFFFu;
          auto gmin = [&](auto mt) {
            constexpr int m = decltype(mt)::value;
            const uint32_t t = xor_lanes_u32<m>(code);
            code = t < code ? t : code;
          };
          if constexpr (LPG > 1) gmin(std::integral_constant<int, 1>{});
          if constexpr (LPG > 2) gmin(std::integral_constant<int, 2>{});
          if constexpr (LPG > 4) gmin(std::integral_constant<int, 4>{});
          if (__ballot(code != 0xFFFFu) == 0ull) break;  // wave-uniform exit
          if (code == 0xFFFFu) continue;                  // uniform over the group's lanes
          const int i = (int)code;
          const int gb = G >= CH ? 0 : (i / G) * G;  // first element of the element's group
          const int jj = i - gb;                      // position within this lane's part
          double ps = 0.0, pe = 0.0;
          // the part's inputs again from memory (the packed words' registers
          // stay free through the transform): for groups across lanes all four
          // loads in flight at once (the loop's latency decides the pass on
          // GELU-tailed rows), for in-lane groups 8 at a time (registers)
          constexpr int NQ8 = G >= 64 ? CH / 8 : 1;
          const uint4* xp = reinterpret_cast<const uint4*>(x + row * (int64_t)K + (int64_t)CH * c);
          uint4 q4[NQ8];
#pragma unroll
          for (int b = 0; b < NQ8; ++b) q4[b] = xp[b];
#pragma unroll(NQ8)
          for (int k0 = 0; k0 < CH; k0 += 8) {
            const uint4 q8 = G >= 64 ? q4[(k0 >> 3) % NQ8] : xp[k0 >> 3];
            const uint32_t w4[4] = {q8.x, q8.y, q8.z, q8.w};
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const int k = k0 + t;
              const double xk = (double)__uint_as_float((t & 1) ? (w4[t >> 1] & 0xFFFF0000u)
                                                                : (w4[t >> 1] << 16));
              const bool in_grp = G >= CH || (k >= gb && k < gb + G);
              const double tk0 = (__builtin_popcount((uint32_t)(jj & (k - gb))) & 1) ? -xk : xk;
              const double tk = in_grp ? tk0 : 0.0;
              const double sn = ps + tk;
              const double bb = sn - ps;
              pe += (ps - (sn - bb)) + (tk - bb);
              ps = sn;
            }
          }
          auto tstage = [&](auto mt) {
            constexpr int m = decltype(mt)::value;
            const double os = xor_lanes_f64<m>(ps), oe = xor_lanes_f64<m>(pe);
            const bool hi_lane = (c & m) != 0;  // the difference: partner - own
            const double a = hi_lane ? os : ps, b = hi_lane ? -ps : os;
            const double sn = a + b;
            const double bb = sn - a;
            pe = (hi_lane ? oe - pe : pe + oe) + ((a - (sn - bb)) + (b - bb));
            ps = sn;
          };
          if constexpr (LPG > 1) tstage(std::integral_constant<int, 1>{});
          if constexpr (LPG > 2) tstage(std::integral_constant<int, 2>{});
          if constexpr (LPG > 4) tstage(std::integral_constant<int, 4>{});
          if ((pend >> i) & 1ull) {
            const float r = (float)ps;
            const uint32_t rb = __float_as_uint(r);
            uint32_t ef = (rb >> 23) & 0xFFu;
            ef = ef < 1u ? 1u : ef;
            const uint32_t pow2 = (rb & 0x7FFFFFu) == 0u ? 1u : 0u;
            const double h =
                __longlong_as_double((int64_t)(uint64_t)(ef + (1023u - 151u) - pow2) << 52);
            const double d = (ps - (double)r) + pe;
            float un = r;
            bool ok = fabs(ps) <= 3.0e38;
            if (ok && !(fabs(d) + (bnd + h * 0x1p-50) < h)) {
              // between r and its neighbour on the side of d
              const uint32_t up = rb == 0x80000000u ? 1u : ((rb >> 31) ? rb - 1u : rb + 1u);
              const uint32_t dn = rb == 0u ? 0x80000001u : ((rb >> 31) ? rb + 1u : rb - 1u);
              const float nb = __uint_as_float(d > 0.0 ? up : dn);
              const double mid = 0.5 * ((double)r + (double)nb);
              const double dd = (ps - mid) + pe;
              ok = r != 0.0f && nb != 0.0f && (r > 0.0f) == (nb > 0.0f) && fabs(dd) > 2.0 * bnd;
              un = (dd > 0.0) == (nb > r) ? nb : r;
            }
            if (ok) {
#pragma unroll
              for (int e2 = 0; e2 < CH; ++e2) u[e2] = e2 == i ? un : u[e2];
              umask &= ~(1ull << i);
              dmask &= ~(1ull << i);
            } else {
              left = true;
            }
            pend &= ~(1ull << i);
          }
        }
        if (risky) {
          float am2 = 0.0f;
          uint32_t un2 = 0u;
#pragma unroll
          for (int i = 0; i < CH; ++i) {
            am2 = fmaxf(am2, fabsf(u[i]));
            const uint32_t mb = __float_as_uint(u[i]) & 0x7FFFFFFFu;
            const uint32_t hb = ((umask >> i) & 1ull) ? mb + (uint32_t)((dmask >> i) & 1ull) : 0u;
            un2 = hb > un2 ? hb : un2;
          }
          atomicMax(&L.rowmax2[r_in], __float_as_uint(am2));
          if (left) atomicOr(&L.rowflag2[r_in], 1u);
          if (umask != 0ull) atomicMax(&L.rowunc2[r_in], un2 + 1u);
        }
        __syncthreads();
      }
    }
    const float amax_u = __uint_as_float(risky ? L.rowmax2[r_in] : L.rowmax[r_in]);
    const float amax_x = amax_u * (1.0f / (float)(1 << KS));  // exact when not deferred
    const uint32_t rowunc = risky ? L.rowunc2[r_in] : L.rowunc[r_in];
    bool wide_ok = active && (risky ? L.rowflag2[r_in] : L.rowflag[r_in]) == 0u && amax_u <= 3.0e38f &&
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
      const uint32_t sgw = lane_sign_word<G, CH>(sm, c);
      bool conflict = false;
#pragma unroll
      for (int d4 = 0; d4 < CH / 4; ++d4) {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * d4 + e;
          const float sgn = ((sgw >> (G >= CH ? i : i % G)) & 1u) ? -1.0f : 1.0f;
          b[e] = __float_as_uint((sgn * u[i]) * inv_u + kQuantPlain);
          if ((umask >> i) & 1ull) {
            // the other candidate of an undecided element (u's sign; a zero's
            // sign does not reach q)
            const uint32_t rb = __float_as_uint(u[i]);
            const uint32_t mb = rb & 0x7FFFFFFFu;
            const uint32_t nb = ((dmask >> i) & 1ull) ? mb + 1u : mb - 1u;
            const float un = __uint_as_float((rb & 0x80000000u) | nb);
            const uint32_t b2 = __float_as_uint((sgn * un) * inv_u + kQuantPlain);
            conflict |= ((b[e] ^ b2) & 0xFFu) != 0u;
          }
        }
        const uint32_t t0 = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);
        const uint32_t t1 = __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
        wout[d4] = t0 | t1;
      }
      if (conflict) atomicOr(&L.rowconf[r_in], 1u);
    }
    __syncthreads();  // conflicts published; L.rowmax readers done
    wide_ok = wide_ok && L.rowconf[r_in] == 0u;
    if (wide_ok) {
      uint4* o = reinterpret_cast<uint4*>(xq + row * (int64_t)K + (int64_t)CH * c);
#pragma unroll
      for (int i = 0; i < CH / 16; ++i)
        o[i] = make_uint4(wout[4 * i], wout[4 * i + 1], wout[4 * i + 2], wout[4 * i + 3]);
      if (c == 0) scale[row] = wsc;
    }
    // the banded algorithm below for the rows still open
    active = active && !wide_ok;
    if (tid < nrows) L.rowmax[tid] = 0u;  // published by the barrier below
    if (__syncthreads_or(active) == 0) return;
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
  const uint32_t sgw = lane_sign_word<G, CH>(sm, c);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int eg = egrp[i / GE];
    const double W = 2.0 * V[i] + (double)((sticky >> i) & 1u);
    const double sgn = ((sgw >> (G >= CH ? i : i % G)) & 1u) ? -1.0 : 1.0;
    xr[i] = (float)(sgn * __builtin_ldexp(W, eg - kBand - 133 - 1 - KS));
    amax = fmaxf(amax, fabsf(xr[i]));
  }

  if (mode == kTensorMax) {
    // wave max, then one atomic per wave
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    if ((tid & 63) == 0 && amax > 0.0f) atomicMax(tensor_amax, __float_as_uint(amax));
    return;
  }

  float rmax;
  if (mode == kTensorQuant) {
    rmax = __uint_as_float(*tensor_amax);
  } else {
    __syncthreads();
    if (active) atomicMax(&L.rowmax[r_in], __float_as_uint(amax));
    __syncthreads();
    rmax = __uint_as_float(L.rowmax[r_in]);
  }
  if (!active) return;

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
}

template <int G>
__global__ __launch_bounds__(512) void rotate_quant_exact_kernel(
    const uint16_t* __restrict__ x, int8_t* __restrict__ xq, float* __restrict__ scale,
    uint32_t* __restrict__ tensor_amax, int64_t rows, int K, int T, int rows_per_block,
    int64_t nbatches, SignMask sm, int mode) {
  __shared__ ExactLds<false> L;
  // persistent grid: batches of rows_per_block rows, strided by gridDim.x
  for (int64_t batch = blockIdx.x; batch < nbatches; batch += gridDim.x)
    exact_rows<G, false>(L, x, xq, scale, tensor_amax, rows, K, T, batch * rows_per_block,
                         rows_per_block, sm, mode);
}

// The exact row pass over rows a fast-kernel block deferred, as a call of its
// own: inlined into the fast kernel, its register needs reshaped the
// allocation of the kernel's batch loop (2-3% slower on ordinary rows,
// measured on MI355X). Its LDS slots arrive as a generic pointer.
template <int G>
__device__ __noinline__ void exact_rows_deferred(ExactLds<true>* L, const uint16_t* x,
                                                 int8_t* xq, float* scale, int64_t rows, int K,
                                                 int T, int64_t row0, int nrows, SignMask sm) {
  exact_rows<G, true>(*L, x, xq, scale, nullptr, rows, K, T, row0, nrows, sm, kRowDeferred);
}

// Per-thread masks of the fast kernel's open elements (bf16 only) during its
// batches; the slots of the exact row pass for its deferred rows after them.
template <bool F16>
struct OpenMasks {
  union {
    uint32_t open[4][512];
    ExactLds<true> ex;
  };
};
template <>
struct OpenMasks<true> {
  uint32_t open[1][1];
};

// ============================================================================
// Fast kernel: 64 contiguous elements per lane; a row is spread over a team
// of T = K/64 lanes; a block holds rows_per_block rows (one "batch") at a
// time and walks batches blockIdx.x, blockIdx.x + gridDim.x, ... (persistent
// grid). The next batch's bf16 words are loaded into registers while the
// current batch is transformed (16-bit words: bf16, or half when F16). The per-row max and flag go through LDS
// slots used round-robin over 3 batches, so one barrier per batch suffices:
// the slot reset after batch b's barrier is that of batch b-1 (whose readers
// all passed the barrier) and it is next written after batch b+1's barrier.
// A bf16 row the kernel cannot finish gets the kDeferredRow NaN in its scale
// slot and a mark for its batch in an LDS bitmap; after its last batch the
// block runs the exact row pass (deferred mode) over the marked batches, so
// on ordinary inputs nothing runs after the batch loop (the launch makes the
// block hold at least two fast rows, i.e. one row of the exact pass's team of
// K/32 lanes).
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
  // open elements of wide groups (bf16 only): per row, 1 + the bits of the
  // largest candidate magnitude, and a flag set when an open element's two
  // candidates quantize differently (read one batch later); per thread, the
  // masks of its open elements and of those whose other candidate is the
  // next float up
  __shared__ uint32_t s_rowunc[3][F16 ? 1 : 256];
  __shared__ uint32_t s_rowconf[3][F16 ? 1 : 256];
  // (the masks' LDS holds the exact row pass's slots after the last batch)
  __shared__ OpenMasks<F16> s_u;
  auto& s_open = s_u.open;
  // g = 256: the byte masks of the sign step (0xFF where d = -1), per part q
  // of a group and output word: the four parts differ, so in registers they
  // would cost a lane 32 VGPRs, and rebuilt per word ~5 VALU instructions
  __shared__ __attribute__((aligned(16))) uint32_t s_sgn[G == 256 ? 4 : 1][16];
  __shared__ __attribute__((aligned(16))) uint32_t s_sgn1[G == 256 ? 4 : 1][16];  // & 0x01010101
  // batches (by pass number it) holding a deferred row: bit it of the
  // bitmap for the first kMarked passes, one flag for any later pass
  constexpr int kMarked = F16 ? 32 : 2048;
  __shared__ uint32_t s_dpass[kMarked / 32];
  __shared__ uint32_t s_dover;
  // the sign mask again for that pass (from LDS: kept in SGPRs through the
  // batch loop it would crowd the loop's scalar registers)
  __shared__ uint32_t s_smask[F16 ? 1 : 8];

  const int tid = threadIdx.x;
  const int r_in = tid / T;
  const int c = tid - r_in * T;
  const bool in_team = r_in < rows_per_block;
  if constexpr (!F16) {
    for (int i = tid; i < kMarked / 32; i += blockDim.x) s_dpass[i] = 0u;
    if (tid == 0) s_dover = 0u;
    if (tid == 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) s_smask[q] = sm.w[q];
    }
  }
  auto mark = [&](int pass) {
    if constexpr (!F16) {
      if (pass < kMarked)
        atomicOr(&s_dpass[pass >> 5], 1u << (pass & 31));
      else
        atomicOr(&s_dover, 1u);
    }
  };
  if (tid < rows_per_block) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      s_rowmax[q][tid] = 0u;
      if constexpr (!F16) {
        s_rowunc[q][tid] = 0u;
        s_rowconf[q][tid] = 0u;
      }
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
  if constexpr (G == 256) {
    if (tid < 64) {
      const int q = tid >> 4, d = tid & 15;
      const uint32_t word = sm.w[2 * q + (d >> 3)];
      const uint32_t m = nibble_to_bytemask((word >> ((4 * d) & 31)) & 0xFu);
      s_sgn[q][d] = m;
      s_sgn1[q][d] = m & 0x01010101u;
    }
  }
  __syncthreads();  // slot and table initialisation visible

  int it = 0;
  for (; batch < nbatches; ++it, batch += gridDim.x) {
    const int64_t row = batch * rows_per_block + r_in;
    const bool active = in_team && row < rows;

    // ---- exponent span per group (half groups are always exact) ----
    // wide_mask bit gidx: group gidx of this lane spans more binades than the
    // float64 transform adds exactly; emax_f: the largest exponent field of
    // those groups
    uint32_t wide_mask = 0u, emax_f = 0u;
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
        if (group_span(a, b) > kMaxSpan) {
          wide_mask |= 1u << gidx;
          emax_f = (a >> 7) > emax_f ? (a >> 7) : emax_f;
        }
      }
    }

    // ---- widen, transform ----
    double v[CH];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[2 * i] = (double)(F16 ? half_lo(w[i]) : bf16lo(w[i]));
      v[2 * i + 1] = (double)(F16 ? half_hi(w[i]) : bf16hi(w[i]));
    }
    // The next batch's words, in flight during the rest of this batch. For
    // g = 256 they are loaded here, while the transform runs (the current
    // words are dead once widened): 3-4% faster on 5120- and 13824-wide rows
    // than after the transform. For smaller groups after the transform (here
    // they would cost spills: up to 19% slower at g = 4).
    // sum |x| over the lane (over its quad's group at g = 256), for the error
    // bound of wide groups below
    double sabs = 0.0;
    if constexpr (!F16) {
      if (wide_mask != 0u) {
#pragma unroll
        for (int i = 0; i < CH; ++i) sabs += fabs(v[i]);
        if constexpr (G == 256) {
          sabs += dpp_f64<kQuadXor1>(sabs);
          sabs += dpp_f64<kQuadXor2>(sabs);
        }
      }
    }
    uint32_t wn[32];
    if constexpr (G == 256) load(batch + gridDim.x, wn);
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
    bool unsafe = false;    // an open element with more than two candidates
    bool has_open = false;  // this lane holds an open element
    uint32_t open_hi = 0u;  // bits of the largest candidate magnitude of those
    if (wide_mask != 0u) {
      // A wide group's float64 transform is rounded: each output is within
      // LOGG * 2^-53 * S of the exact sum (a depth-LOGG tree of correctly
      // rounded additions whose nodes at one level partition the inputs),
      // S = sum |x| < G * 2^(E+1), E the group's largest exponent. With twice
      // that bound, delta = 2^(E + ceil(log2 LOGG) + LOGG - 51), the exact
      // sum lies in [y - delta, y + delta], and since rounding is monotonic
      // it rounds to RN32(y) when both ends do (the two float64 end points err
      // by less than the margin). Otherwise the element is open: when the two
      // ends round to neighbouring floats lo and hi, the exact sum rounds to
      // one of them and u = RN32(y) is one of them; the row is finished from
      // u unless an open element's larger candidate could be the row's
      // absmax, or its two candidates quantize to different bytes (checked
      // once the scale is known). Wider intervals defer the row.
      // The same bound from the computed sum of |x| (the lane's, which covers
      // each of its groups; the whole group's at g = 256): S < 2^(e_S + 1)
      // (1 + 2^-46) with e_S the exponent of the float64 sum, so
      // 2^(e_S + ceil(log2 LOGG) - 51) is again twice the bound; the smaller
      // of the two is used (tighter for groups with few large elements).
      constexpr int LL = LOGG <= 2 ? 1 : (LOGG <= 4 ? 2 : 3);
      const uint32_t fe = emax_f + (uint32_t)(1023 - 127 + LL + LOGG - 51);
      const uint32_t fs = (uint32_t)((uint64_t)__double_as_longlong(sabs) >> 52) + (uint32_t)(LL - 51);
      const double delta = __longlong_as_double((int64_t)(uint64_t)(fs < fe ? fs : fe) << 52);
      uint32_t om[2] = {0u, 0u}, um[2] = {0u, 0u};  // open elements; other candidate above u
      // One group per lane (g >= 64, so the whole lane is wide here): eight
      // elements at a time, which are open without a branch, the details
      // only under one branch per eight (open elements are rare; -2 to -7%
      // on GELU-tailed rows). Smaller groups test each element under its
      // group's wide bit.
      if constexpr (NGL > 1) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          u[i] = (float)v[i];
          amax = fmaxf(amax, fabsf(u[i]));
          if ((wide_mask >> (i / G)) & 1u) {
            const float lo = (float)(v[i] - delta), hi = (float)(v[i] + delta);
            if (lo != hi) {
              const uint32_t lb = __float_as_uint(lo);
              const uint32_t nb = lb == 0x80000000u ? 1u : ((lb >> 31) ? lb - 1u : lb + 1u);
              unsafe |= __uint_as_float(nb) != hi;
              om[i >> 5] |= 1u << (i & 31);
              um[i >> 5] |= (u[i] == lo ? 1u : 0u) << (i & 31);
              const uint32_t mb = __float_as_uint(fmaxf(fabsf(lo), fabsf(hi)));
              open_hi = mb > open_hi ? mb : open_hi;
            }
          }
        }
      } else {
#pragma unroll
        for (int i0 = 0; i0 < CH; i0 += 8) {
          float lo8[8], hi8[8];
          uint32_t op8 = 0u;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int i = i0 + t;
            u[i] = (float)v[i];
            amax = fmaxf(amax, fabsf(u[i]));
            lo8[t] = (float)(v[i] - delta);
            hi8[t] = (float)(v[i] + delta);
            op8 |= (lo8[t] != hi8[t] ? 1u : 0u) << t;
          }
          if (op8 != 0u) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const int i = i0 + t;
              if ((op8 >> t) & 1u) {
                const float lo = lo8[t], hi = hi8[t];
                // the float right above lo (bit patterns: -0 -> +2^-149)
                const uint32_t lb = __float_as_uint(lo);
                const uint32_t nb = lb == 0x80000000u ? 1u : ((lb >> 31) ? lb - 1u : lb + 1u);
                unsafe |= __uint_as_float(nb) != hi;
                om[i >> 5] |= 1u << (i & 31);
                um[i >> 5] |= (u[i] == lo ? 1u : 0u) << (i & 31);
                const uint32_t mb = __float_as_uint(fmaxf(fabsf(lo), fabsf(hi)));
                open_hi = mb > open_hi ? mb : open_hi;
              }
            }
          }
        }
      }
      if (om[0] | om[1]) {
        has_open = true;
        s_open[0][tid] = om[0];
        s_open[1][tid] = om[1];
        s_open[2][tid] = um[0];
        s_open[3][tid] = um[1];
      }
    } else {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        u[i] = (float)v[i];
        amax = fmaxf(amax, fabsf(u[i]));
      }
    }

    if constexpr (G != 256) load(batch + gridDim.x, wn);
    const int slot = it % 3;
    if (active) {
      atomicMax(&s_rowmax[slot][r_in], __float_as_uint(amax));
      if constexpr (!F16) {
        // an unsafe element defers the row: all ones fails every comparison below
        if (has_open || unsafe) atomicMax(&s_rowunc[slot][r_in], unsafe ? ~0u : open_hi + 1u);
      }
    }
    __syncthreads();
    if (tid < rows_per_block) {
      const int nslot = (it + 2) % 3;
      s_rowmax[nslot][tid] = 0u;
      if constexpr (!F16) {
        s_rowunc[nslot][tid] = 0u;
        s_rowconf[(it + 1) % 3][tid] = 0u;  // read one batch ago, written next batch
      }
    }
    if constexpr (!F16) {
      // the previous batch's row had an open element whose candidates quantize
      // differently: defer it (this thread wrote its scale, so the marker
      // lands after it)
      const int64_t prev = row - (int64_t)gridDim.x * rows_per_block;
      if (it > 0 && in_team && c == 0 && prev < rows && s_rowconf[(it + 2) % 3][r_in] != 0u) {
        scale[prev] = __uint_as_float(kDeferredRow);
        mark(it - 1);
      }
    }

    if (active) {
      const float amax_u = __uint_as_float(s_rowmax[slot][r_in]);
      const float amax_x = amax_u * (1.0f / (float)(1 << KS));  // exact unless deferred
      bool deferred = !(amax_u <= 3.0e38f) || (amax_u > 0.0f && amax_x < 0x1p-100f);
      if constexpr (!F16) {
        // an open element's larger candidate reaches the decided absmax
        const uint32_t ru = s_rowunc[slot][r_in];
        deferred |= ru != 0u && ru - 1u >= __float_as_uint(amax_u);
      }
      if (deferred) {
        if (c == 0) {
          scale[row] = __uint_as_float(kDeferredRow);
          mark(it);
        }
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

        // sign masks of this lane's output words (g = 256: from the table)
        uint32_t mk[16], mk1[16];
        if constexpr (G == 256) {
          const u4* tm = reinterpret_cast<const u4*>(s_sgn[c & 3]);
          const u4* t1 = reinterpret_cast<const u4*>(s_sgn1[c & 3]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u4 a = tm[i], b = t1[i];
            mk[4 * i] = a.x; mk[4 * i + 1] = a.y; mk[4 * i + 2] = a.z; mk[4 * i + 3] = a.w;
            mk1[4 * i] = b.x; mk1[4 * i + 1] = b.y; mk1[4 * i + 2] = b.z; mk1[4 * i + 3] = b.w;
          }
        } else {
#pragma unroll
          for (int d = 0; d < 16; ++d) {
            mk[d] = nibble_to_bytemask(((d < 8 ? sg0 : sg1) >> ((4 * d) & 31)) & 0xFu);
            mk1[d] = mk[d] & 0x01010101u;
          }
        }
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
          // negate the bytes with d = -1 (biased: 256 - v never carries), unbias
          outw[d] = ((packed ^ mk[d]) + mk1[d]) ^ 0x80808080u;
        }
        u4* o = reinterpret_cast<u4*>(xq + row * (int64_t)K + (int64_t)CH * c);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = (u4){outw[4 * i], outw[4 * i + 1], outw[4 * i + 2], outw[4 * i + 3]};
        if constexpr (!F16) {
          if (has_open) {
            // both candidates of each open element must give the same byte
            const uint32_t om0 = s_open[0][tid], om1 = s_open[1][tid];
            const uint32_t um0 = s_open[2][tid], um1 = s_open[3][tid];
            bool conflict = false;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
              const uint32_t om = i < 32 ? om0 : om1, um = i < 32 ? um0 : um1;
              if ((om >> (i & 31)) & 1u) {
                // the other candidate: the float right above u (um bit set) or
                // right below it
                const uint32_t b = __float_as_uint(u[i]);
                const bool up = (um >> (i & 31)) & 1u;
                const uint32_t bu = b == 0x80000000u ? 1u : ((b >> 31) ? b - 1u : b + 1u);
                const uint32_t bd = b == 0u ? 0x80000001u : ((b >> 31) ? b + 1u : b - 1u);
                const float other = __uint_as_float(up ? bu : bd);
                const uint32_t q1 = __float_as_uint(u[i] * inv_u + kQuantBias);
                const uint32_t q2 = __float_as_uint(other * inv_u + kQuantBias);
                conflict |= ((q1 ^ q2) & 0xFFu) != 0u;
              }
            }
            if (conflict) atomicOr(&s_rowconf[slot][r_in], 1u);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = wn[i];
  }
  if constexpr (!F16) {
    // conflicts of the last batch
    __syncthreads();
    const int64_t last = (batch - gridDim.x) * rows_per_block + r_in;
    if (it > 0 && in_team && c == 0 && last < rows && s_rowconf[(it - 1) % 3][r_in] != 0u) {
      scale[last] = __uint_as_float(kDeferredRow);
      mark(it - 1);
    }

    // ---- the rows this block deferred: the exact row pass with its team of
    // 2T lanes per row (at most blockDim), over the marked batches in order.
    // The scale slots and the bitmap are read after the barrier, so every
    // thread sees the marks and takes the same steps. ----
    auto& s_ex = s_u.ex;
    __syncthreads();
    const int T2 = 2 * T;
    const int rpb2 = (int)blockDim.x / T2;
    SignMask sm2;
#pragma unroll
    for (int i = 0; i < 8; ++i) sm2.w[i] = s_smask[i];
    // lane l of every wave holds bitmap word l: one ballot finds the marked
    // words (none on ordinary inputs), the same in every wave
    static_assert(kMarked / 32 == 64, "one bitmap word per lane");
    const uint32_t word = s_dpass[tid & 63];
    const bool over = s_dover != 0u;
    // the marked passes in order, then (flag) every pass from kMarked on;
    // one call site of the exact row pass
    int pass = -1;
    for (;;) {
      const int from = pass + 1;
      if (from < kMarked) {
        // bits of words >= from / 32 at positions >= from
        const int lane = tid & 63;
        uint32_t wl = lane < (from >> 5) ? 0u : word;
        if (lane == (from >> 5)) wl &= ~0u << (from & 31);
        const uint64_t nz = __ballot(wl != 0u);
        if (nz != 0ull) {
          const int wd = __builtin_ctzll(nz);
          pass = wd * 32 + __builtin_ctz((uint32_t)__shfl((int)wl, wd));
        } else {
          pass = over ? kMarked : it;
        }
      } else {
        pass = from;
      }
      if (pass >= it) break;
      const int64_t row0 = ((int64_t)blockIdx.x + (int64_t)pass * gridDim.x) * rows_per_block;
      const int64_t left = rows - row0;
      const int nr = (int)(left < rows_per_block ? left : rows_per_block);
      for (int r0 = 0; r0 < nr; r0 += rpb2)
        exact_rows_deferred<G>(&s_ex, x, xq, scale, rows, K, T2, row0 + r0,
                               nr - r0 < rpb2 ? nr - r0 : rpb2, sm2);
    }
  }
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

// Choose a block of whole waves holding whole rows of T lanes (at least
// min_rows of them, at most 256; at most 512 threads) for a persistent kernel
// with `wpc` resident waves per CU: the most row lanes at work per CU
// (resident blocks x rows per block x T), ties to the smaller block.
TeamShape team_shape(int T, int wpc, int min_rows) {
  TeamShape best{T, 0, 0};
  int best_lanes = 0;
  for (int waves = 1; waves <= 8; ++waves) {
    const int threads = 64 * waves;
    int rpb = threads / T;
    if (rpb < min_rows) continue;
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

// Grid of a persistent rotate kernel: blocks of whole rows of T lanes, as
// many as stay resident together at `wpc` waves per CU (a grid beyond that
// would run a second, partial round of blocks), no more than there are
// batches.
LaunchPlan plan_rotate(int64_t rows, int T, int wpc, int cus, int min_rows) {
  const TeamShape ts = team_shape(T, wpc, min_rows);
  LaunchPlan p;
  p.block = ts.block;
  p.rows_per_block = ts.rpb;
  const int64_t nbatches = (rows + ts.rpb - 1) / ts.rpb;
  const int per_cu = wpc / (ts.block / 64);
  const int64_t cap = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  p.grid = nbatches < cap ? nbatches : cap;
  p.passes = p.grid > 0 ? (nbatches + p.grid - 1) / p.grid : 0;
  return p;
}

template <int G>
hipError_t launch_fast(const uint16_t* x, int8_t* xq, float* s, int64_t rows, int K,
                       const SignMask& sm, bool f16, hipStream_t st) {
  // half rows are never deferred, so their blocks need not fit a K/32-lane row
  const LaunchPlan p = f16 ? plan_rotate(rows, K / 64, kFastWavesPerCU, compute_units(), 1)
                           : plan_act_quant(rows, K, false, compute_units());
  // a bf16 block resolves its deferred rows with teams of K/32 lanes
  if ((!f16 && p.block < K / 32) || p.block > 512) return hipErrorInvalidConfiguration;
  const int64_t nbatches = (rows + p.rows_per_block - 1) / p.rows_per_block;
  auto kern = f16 ? rotate_quant_fast_kernel<G, true> : rotate_quant_fast_kernel<G, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.grid), dim3(p.block), 0, st, x, xq, s, rows, K,
                     K / 64, p.rows_per_block, nbatches, sm);
  return hipGetLastError();
}

// Resident waves per CU of the persistent exact kernel.
constexpr int kExactWavesPerCU = 8;

template <int G>
hipError_t launch_exact(const uint16_t* x, int8_t* xq, float* s, uint32_t* tensor_amax,
                        int64_t rows, int K, const SignMask& sm, int mode, hipStream_t st) {
  const LaunchPlan p = plan_exact(rows, K, compute_units());
  const int64_t nbatches = (rows + p.rows_per_block - 1) / p.rows_per_block;
  hipLaunchKernelGGL(rotate_quant_exact_kernel<G>, dim3((unsigned)p.grid), dim3(p.block), 0, st, x,
                     xq, s, tensor_amax, rows, K, K / 32, p.rows_per_block, nbatches, sm, mode);
  return hipGetLastError();
}

}  // namespace

// The fast kernel's blocks hold at least two rows of K/64 lanes (K <= 16384),
// so that one row of the exact pass's K/32 lanes fits a block (bf16 rows;
// half rows, never deferred, take the shape without that floor). deferred:
// the blocks' pass over the rows they defer, in the fast kernel's grid, with
// rows_per_block rows of K/32 lanes per step.
LaunchPlan plan_act_quant(int64_t rows, int K, bool deferred, int cus) {
  LaunchPlan p = plan_rotate(rows, K / 64, kFastWavesPerCU, cus, 2);
  if (deferred && p.block > 0) p.rows_per_block = p.block / (K / 32);
  return p;
}

LaunchPlan plan_exact(int64_t rows, int K, int cus) {
  return plan_rotate(rows, K / 32, kExactWavesPerCU, cus, 1);
}

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
  return e;
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

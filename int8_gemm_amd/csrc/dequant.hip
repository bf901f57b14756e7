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
//
// Per-channel scales (one s_w per weight row): a weight row holds K/R whole
// view rows, so the scale is a per-lane value: lane jl of a tile decodes view
// row jl, whose weight row is (tile*32 + jl) / (K/R).

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

template <int G, bool PC, bool F16, int NJ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PC ? 4 : 1))) void dequant_kernel(
    const DequantJobs<NJ> jobs, SignMask sm) {
  constexpr int R = G > 32 ? G : 32;   // bytes per view row
  constexpr int NB = R / 32;           // 32-blocks per view row
  constexpr int KS = ilog2(G) / 2;
  // A block takes 4 tiles of 32 view rows, or one tile whose 8 output
  // 32-blocks are spread over its 4 waves (g = 256): a contiguous chunk of
  // CHUNK input bytes of one weight, loaded coalesced into LDS and
  // prefetched one chunk ahead through registers.
  constexpr int NQ = NB >= 4 ? 4 : 1;      // waves per tile
  constexpr int JW = NB / NQ;              // output 32-blocks per wave
  constexpr int TPB = 4 / NQ;              // tiles per block
  constexpr int CHUNK = TPB * 32 * R;      // input bytes per block step (<= 8 KB)
  constexpr int NLD = CHUNK / (256 * 16);  // 16-byte loads per thread per chunk
  static_assert(CHUNK % (256 * 16) == 0 || CHUNK < 256 * 16, "chunk");
  constexpr int LR = R + 16;               // LDS bytes per staged input row (padded)
  constexpr int OW = JW * 32;              // outputs per row per wave
  constexpr int OSTR = OW * 2 + 16;        // LDS bytes per staged output row (padded)
  __shared__ __attribute__((aligned(16))) uint8_t s_in[TPB * 32 * LR];
  __shared__ __attribute__((aligned(16))) uint8_t s_out[4][32 * OSTR];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const uint32_t jl = lane & 31;  // A row (output j within a 32-block) / B column (view row)
  const uint32_t kh = lane >> 5;  // k-slice: il = 16*kh + b
  const int tl = wave / NQ;       // tile of this wave within the chunk
  const int jq = wave % NQ;       // its share of the output 32-blocks

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

  // The chunks of all weights form one sequence (weight j owns chunks
  // [chunk_begin[j], chunk_begin[j + 1])); a block walks chunks blockIdx.x,
  // blockIdx.x + gridDim.x, ... The fields of the weight of the current and
  // of the next chunk stay in registers and are read again only when the
  // weight changes (chunks only grow).
  const int64_t nchunks = jobs.chunk_begin[NJ == 1 ? 1 : jobs.njobs];
  struct Cur {
    int j;
    int64_t begin, end;  // its chunks
    const int8_t* wq;
    uint16_t* out;
    int64_t nrows;
    float ct;  // per tensor: RN(s_w * 2^-KS)
  };
  auto fetch = [&](int64_t ch, int j) {
    while (NJ > 1 && j + 1 < jobs.njobs && ch >= jobs.chunk_begin[j + 1]) ++j;
    Cur c;
    c.j = j;
    c.begin = NJ == 1 ? 0 : jobs.chunk_begin[j];  // a table of one starts at chunk 0
    c.end = jobs.chunk_begin[j + 1];
    c.wq = jobs.job[j].wq;
    c.out = jobs.job[j].w_out;
    c.nrows = jobs.job[j].nrows;
    c.ct = PC ? 0.0f : *jobs.job[j].s_w * (1.0f / (float)(1 << KS));
    return c;
  };

  // coalesced chunk load: thread tid takes 16-byte pieces tid, tid + 256, ...
  // (bytes past the weight's end read as zero)
  auto load_chunk = [&](int64_t ch, const Cur& w, u4 (&r)[NLD > 0 ? NLD : 1]) {
    const int64_t in_bytes = w.nrows * R;
    const int64_t base = (ch - w.begin) * CHUNK;
#pragma unroll
    for (int i = 0; i < (NLD > 0 ? NLD : 1); ++i) {
      const int off = (tid + 256 * i) * 16;
      const int64_t g = base + off;
      r[i] = (ch < nchunks && off < CHUNK && g < in_bytes)
                 ? *reinterpret_cast<const u4*>(w.wq + g)
                 : (u4){0u, 0u, 0u, 0u};
    }
  };
  auto store_chunk = [&](const u4 (&r)[NLD > 0 ? NLD : 1]) {
#pragma unroll
    for (int i = 0; i < (NLD > 0 ? NLD : 1); ++i) {
      const int off = (tid + 256 * i) * 16;
      if (off < CHUNK) *reinterpret_cast<u4*>(s_in + off / R * LR + off % R) = r[i];
    }
  };

  u4 pre[NLD > 0 ? NLD : 1];
  int64_t ch = blockIdx.x;
  Cur cur = fetch(ch, 0);
  load_chunk(ch, cur, pre);
  store_chunk(pre);
  __syncthreads();
  for (; ch < nchunks; ch += gridDim.x) {
    const int64_t chn = ch + gridDim.x;
    const Cur nxt = (NJ > 1 && chn >= cur.end && chn < nchunks) ? fetch(chn, cur.j) : cur;
    load_chunk(chn, nxt, pre);  // next chunk, in flight during this one

    const int64_t nrows = cur.nrows;
    uint16_t* __restrict__ out = cur.out;
    const int64_t tile = (ch - cur.begin) * TPB + tl;
    float c;
    if constexpr (PC) {
      // weight row of view row vr: q = vr / vrows_per_ch from a float64
      // estimate (vr < 2^53), corrected by one either way
      const int vpc = jobs.job[cur.j].vrows_per_ch;
      const int64_t vr = tile * 32 + jl < nrows ? tile * 32 + jl : nrows - 1;
      int64_t q = (int64_t)((double)vr * jobs.job[cur.j].inv_vrows_per_ch);
      if (q * vpc > vr) --q;
      if ((q + 1) * vpc <= vr) ++q;
      c = jobs.job[cur.j].s_w[q] * (1.0f / (float)(1 << KS));
    } else {
      c = cur.ct;
    }
    v4i bfr[NB];
#pragma unroll
    for (int ib = 0; ib < NB; ++ib)
      bfr[ib] = *reinterpret_cast<const v4i*>(s_in + (tl * 32 + jl) * LR + 32 * ib + 16 * kh);
    uint8_t* so = s_out[wave];
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
      // lane (jl, kh) holds outputs j = 8a + 4kh + e of view row jl: stage
      // them as bf16 in this wave's LDS rows
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const u2 v = {pack16x2<F16>((float)acc[4 * a + 0] * c, (float)acc[4 * a + 1] * c),
                      pack16x2<F16>((float)acc[4 * a + 2] * c, (float)acc[4 * a + 3] * c)};
        *reinterpret_cast<u2*>(so + jl * OSTR + 2 * (32 * jw + 8 * a + 4 * kh)) = v;
      }
    }
    // (LDS ops of one wave complete in order; keep the compiler from
    // moving the reads below above the writes above)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // coalesced stores: each row's OW outputs are contiguous in the output;
    // lane -> (row, 16-byte piece)
    constexpr int PPR = OW * 2 / 16;  // 16-byte pieces per row
    constexpr int RPI = 64 / PPR;     // rows per store instruction
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = RPI * i + lane / PPR;
      const int pc = lane % PPR;
      const u4 v = *reinterpret_cast<const u4*>(so + row * OSTR + 16 * pc);
      const int64_t vr = tile * 32 + row;
      if (vr < nrows)
        *reinterpret_cast<u4*>(out + vr * R + jq * OW + 8 * pc) = v;
    }
    __syncthreads();  // every wave is done with s_in and its own s_out
    store_chunk(pre);
    __syncthreads();
    cur = nxt;
  }
}

}  // namespace

template <int G, int NJ>
static void launch_g(bool pc, bool f16, int64_t blocks, const DequantJobs<NJ>& jobs,
                     const SignMask& sm, hipStream_t st) {
  auto kern = f16 ? (pc ? dequant_kernel<G, true, true, NJ> : dequant_kernel<G, false, true, NJ>)
                  : (pc ? dequant_kernel<G, true, false, NJ> : dequant_kernel<G, false, false, NJ>);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, st, jobs, sm);
}

// 32-row tiles per block step: one at g = 256 (its 8 output blocks spread
// over the 4 waves), four at g <= 64.
static int tiles_per_step(int g) { return (g > 32 ? g : 32) / 32 >= 4 ? 1 : 4; }

static int64_t dequant_chunks(int64_t n, int64_t k, int g) {
  const int R = g > 32 ? g : 32;
  const int64_t tiles = (n * k / R + 31) / 32;
  const int tpb = tiles_per_step(g);
  return (tiles + tpb - 1) / tpb;
}

// Persistent blocks per CU, as measured: 2 when a block step is one tile
// (g = 256; 4 blocks were 4-18% slower on 3072x3072 .. 13824x5120), 4 when
// it is four (g <= 64, where 2 or 3 were up to 11% slower).
static LaunchPlan plan_chunks(int64_t chunks, int g, int cus) {
  LaunchPlan p;
  p.block = 256;
  p.rows_per_block = tiles_per_step(g);
  const int64_t cap = (int64_t)(cus > 0 ? cus : 1) * (p.rows_per_block == 1 ? 2 : 4);
  p.grid = chunks < cap ? chunks : cap;
  p.passes = p.grid > 0 ? (chunks + p.grid - 1) / p.grid : 0;
  return p;
}

LaunchPlan plan_dequant(int64_t n, int64_t k, int g, int cus) {
  return plan_chunks(dequant_chunks(n, k, g), g, cus);
}

// Launches of up to NJ weights each (NJ = 1 for a single weight).
template <int NJ>
static hipError_t launch_jobs(const DequantJob* job, int njobs, bool sw_per_channel, int g,
                              const SignMask& sm, DType dt, hipStream_t st) {
  const int R = g > 32 ? g : 32;
  const int cus = compute_units();
  for (int j0 = 0; j0 < njobs;) {
    DequantJobs<NJ> jobs;
    jobs.njobs = 0;
    int64_t chunks = 0;
    for (; j0 < njobs && jobs.njobs < NJ; ++j0) {
      const int64_t c = dequant_chunks(job[j0].n, job[j0].k, g);
      if (c == 0) continue;  // an empty weight has nothing to decode
      typename DequantJobs<NJ>::Desc& d = jobs.job[jobs.njobs];
      d.wq = job[j0].wq;
      d.s_w = job[j0].s_w;
      d.w_out = job[j0].w_out;
      d.nrows = job[j0].n * job[j0].k / R;
      d.vrows_per_ch = (int)(job[j0].k / R);  // K % R == 0 for every supported (K, g)
      d.inv_vrows_per_ch = 1.0 / (double)d.vrows_per_ch;
      jobs.chunk_begin[jobs.njobs] = chunks;
      chunks += c;
      ++jobs.njobs;
    }
    if (jobs.njobs == 0) continue;
    jobs.chunk_begin[jobs.njobs] = chunks;
    const int64_t blocks = plan_chunks(chunks, g, cus).grid;
    const bool pc = sw_per_channel, f16 = dt == DType::kF16;
    switch (g) {
      case 4: launch_g<4, NJ>(pc, f16, blocks, jobs, sm, st); break;
      case 16: launch_g<16, NJ>(pc, f16, blocks, jobs, sm, st); break;
      case 64: launch_g<64, NJ>(pc, f16, blocks, jobs, sm, st); break;
      default: launch_g<256, NJ>(pc, f16, blocks, jobs, sm, st); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_dequant_jobs(const DequantJob* job, int njobs, bool sw_per_channel, int g,
                               const SignMask& sm, DType dt, hipStream_t st) {
  return njobs == 1 ? launch_jobs<1>(job, njobs, sw_per_channel, g, sm, dt, st)
                    : launch_jobs<kMaxDequantJobs>(job, njobs, sw_per_channel, g, sm, dt, st);
}

hipError_t launch_dequant(const int8_t* wq, const float* s_w, bool sw_per_channel, int64_t n,
                          int64_t k, int g, const SignMask& sm, uint16_t* w_out, DType dt,
                          hipStream_t st) {
  const DequantJob job{wq, s_w, w_out, n, k};
  return launch_dequant_jobs(&job, 1, sw_per_channel, g, sm, dt, st);
}

}  // namespace convrot

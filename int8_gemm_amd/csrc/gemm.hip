// int8 x int8 -> int32 GEMM with the convrot scaling epilogue (gfx950).
//
// acc[m, n] = sum_k xq[m, k] * wq[n, k] (exact int32: |acc| <= 127^2 K < 2^31)
// y[m, n]   = bf16(RN32(RN32(float(acc) * s_w) * s_x[m]) [+ bias[n] in fp32])
//             (s_w per tensor, or s_w[n] per output channel; bias and y in
//             bf16 or IEEE half)
//
// This is the int8 tensor-core multiply of int8_compute (Invoke docs
// "int8 Compute", introduction: the input is quantized per token and int8 is
// multiplied by int8); the pages run it through Triton on NVIDIA, this is a
// gfx950 design of its own:
//   * block tile BM x BN: 384x192 (K % 128 == 0) with 8 compute waves in a
//     4 x 2 grid, 256x256 with 8 compute waves in a 2 x 4 grid,
//     192x192 with 4 compute waves (2 x 2) plus 4 producer waves, 128x128
//     with 4 waves (2 x 2, two blocks per CU); v_mfma_i32_32x32x32_i8 (on
//     gfx950 it sustains the full int8 rate, the 16x16x64 form about half)
//     with the weight rows in the A operand, so each lane's accumulators
//     come in runs of 4 consecutive output columns;
//   * K-step BK = 128 bytes when K % 128 == 0, else 64; an NS-deep ring of
//     LDS stages filled by global_load_lds_dwordx4 (global -> LDS, no
//     VGPRs); one barrier per K-step, after which the copies of stage s+NS
//     go into the slot of the stage s just read (every wave waits for its
//     LDS reads before the barrier; with 8 waves, the two waves of a SIMD
//     issue theirs at different points of the step). With producer waves,
//     only they issue copies and wait for them;
//   * LDS stage: rows of BK bytes, weights then activations; each copy
//     instruction fills 1024 / BK rows; within a row the 16-byte chunks are
//     XOR-swizzled by row (below), which makes the fragment reads free of
//     bank conflicts;
//   * the block index is remapped so that each XCD (8 on an MI355X; the
//     count follows the device's compute units) gets a contiguous range of
//     tiles, walked in groups of 8 tile rows (L2 reuse).
// Measured on MI355X (rocprofv3 counters): the K-loop is bound by the rate
// at which each CU's vector L1 streams operands from L2 into LDS. A CU keeps
// only some 40-70 L1->L2 requests in flight at ~300 cycles each, so per-CU
// bandwidth is set by the bytes each request carries and by latency: a
// 128-byte K-step turns every request into a whole L2 line (+9-37% over 64
// bytes, even with the ring cut to two stages; on the 192 tile only
// together with four copy-issuing waves). Deeper rings, an L2 prefetch copy
// and non-temporal output stores were all slower. Every round of tiles
// ends with all CUs writing their output tiles at once: with 256 x 256
// tiles at K = 5120 that burst is ~9% of the time (skipping the stores in a
// timing copy saves it). Persistent blocks that issue the next tile's first
// copies before the stores did not hide it (a single vmcnt orders the next
// tile's copy waits behind the stores) and were slower for their register
// use; a 4-wave 256 x 256 layout (128 x 128 per wave, accumulators in
// AGPRs) lost 12% for want of a second wave per SIMD.
// Both operands are K-contiguous ("TN"). K % 64 == 0, N % 16 == 0.

#include "common.h"
#include "internal.h"

namespace convrot {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// s_waitcnt on vmcnt only (expcnt, lgkmcnt left unconstrained); gfx9 encoding
template <int V>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(V >= 0 && V < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((V & 0xF) | (0x7 << 4) | (0xF << 8) | ((V >> 4) << 14));
}

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4, SGPR base
// + 32-bit VGPR offset): lane i writes LDS bytes [lds_base + 16 i, +16).
// Written as inline asm so that the compiler's waitcnt model (which treats the
// LDS write of the builtin form as pending LDS traffic and drains it around
// every later LDS read) stays out of the way; completion is tracked by the
// explicit vmcnt waits of the K-loop. The instruction has no VGPR result.
__device__ __forceinline__ void dma16(const int8_t* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}

// s_waitcnt lgkmcnt(0) only (vmcnt, expcnt left unconstrained)
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those would force vmcnt(0) and drain the in-flight LDS-DMA stages. The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// PC: s_w holds one scale per output column n (per output channel of the
// weight) instead of one for the tensor. F16: bias and y are IEEE half
// instead of bf16.
template <int BM, int BN, int BK, int WM, int WN, int NS, int MINB, int NP, bool PC, bool F16>
__global__ __launch_bounds__(64 * (WM * WN + NP), MINB) void gemm_i8_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ s_x, const int8_t* __restrict__ wq,
    const float* __restrict__ s_w, const uint16_t* __restrict__ bias, int M, int N, int K,
    int tiles_m, int tiles_n, int nx, uint16_t* __restrict__ y, int32_t* __restrict__ acc_out) {
  constexpr int NW = WM * WN;                   // waves: WM along m, WN along n
  constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile (m, n)
  constexpr int NJ = WTM / 32, NI = WTN / 32;   // 32x32 MFMA tiles per wave (m, n)
  constexpr int STAGE = (BM + BN) * BK;         // bytes per LDS stage
  constexpr int RPI = 1024 / BK;                // rows per 1 KB DMA instruction
  constexpr int CPR = BK / 16;                  // 16-byte chunks per row
  // NP == 0: every wave copies its share of each stage and computes.
  // NP > 0: NP extra producer waves issue all copies and wait for them, so
  // a stalled copy issue never holds up a compute wave's MFMAs; the compute
  // (consumer) waves only read LDS and multiply. Both meet at the one
  // barrier per K-step.
  constexpr int DW = NP > 0 ? NP : NW;          // waves that issue copies
  constexpr int LW = (BM + BN) / (RPI * DW);    // DMA instructions per copying wave per stage
  constexpr int H = BK / 32;                    // 32-k slices per K-step
  static_assert(BK == 64 || BK == 128, "K-step");
  // LDS bank swizzle: 16-byte chunk c of stage row r sits in slot c ^ swz(r),
  // swz(r) = (r / RPB) % CPR with RPB = 256 / BK rows per 256-byte bank line
  constexpr int RPB = 256 / BK;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && (BM + BN) % (RPI * DW) == 0, "tile shape");
  // Ring of NS stages. Every consumer wave waits for its own LDS reads before
  // the barrier of step s, so after it nobody reads stage s again (its last
  // slice is in registers): the copies of stage s+NS go into stage s's slot
  // right after that barrier, and NS-1 stages stay in flight during a step.
  constexpr int LA = NS;
  static_assert(NS >= 2, "ring depth");
  static_assert(LA * LW < 64, "copies in flight per wave must fit vmcnt");
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % WN;
  const int wm = wave / WN;
  const int cw = NP > 0 ? wave - NW : wave;  // index among the copying waves

  // ---- tile index: XCD-contiguous ranges (workgroups are dealt to the nx
  // XCDs round-robin), grouped rows ----
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  {
    const int per = (ntiles + nx - 1) / nx;
    const int xcd = bid % nx;
    const int loc = bid / nx;
    const int full = ntiles - (per - 1) * nx;
    bid = (xcd < full) ? xcd * per + loc : full * per + (xcd - full) * (per - 1) + loc;
  }
  constexpr int GROUP = 8;
  const int group_sz = GROUP * tiles_n;
  const int grp = bid / group_sz;
  const int first_m = grp * GROUP;
  const int gm = min(tiles_m - first_m, GROUP);
  const int in_grp = bid - grp * group_sz;
  const int m0 = (first_m + in_grp % gm) * BM;
  const int n0 = (in_grp / gm) * BN;

  // ---- per-lane DMA sources: instruction t of this wave covers combined
  // rows RPI*q .. RPI*q+RPI-1 (weights first, then activations); lane ->
  // row RPI*q + lane/CPR, 16-byte chunk lane%CPR (whole L2 lines for BK=128) ----
  // 32-bit byte offsets from the tile's first weight / activation row
  // (below BM*K <= 384 * 133144 < 2^31); the 64-bit tile base pointer and the
  // K-step offset go in SGPRs. Rows past the matrix edge re-read its last row.
  const int8_t* wtile = wq + (int64_t)n0 * K;
  const int8_t* xtile = xq + (int64_t)m0 * K;
  uint32_t voff[LW];
  bool is_w[LW];
  int ldsoff[LW];
#pragma unroll
  for (int t = 0; t < LW; ++t) {
    const int q = (cw > 0 ? cw : 0) * LW + t;  // consumers of a producer layout never copy
    const int row = RPI * q + lane / CPR;
    const int p = lane % CPR;
    is_w[t] = (RPI * q) < BN;  // whole instruction in one region (BN % RPI == 0)
    // LDS slot p of the row holds global chunk p ^ swz(row) (bank swizzle)
    const uint32_t chunk = (uint32_t)(p ^ ((row / RPB) % CPR));
    if (row < BN) {
      const int n = min(n0 + row, N - 1) - n0;
      voff[t] = (uint32_t)n * (uint32_t)K + 16u * chunk;
    } else {
      const int m = min(m0 + row - BN, M - 1) - m0;
      voff[t] = (uint32_t)m * (uint32_t)K + 16u * chunk;
    }
    ldsoff[t] = q * 1024;
  }
  const int nk = K / BK;
  const uint32_t lds_u32 = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
  // wave-uniform operands of the DMA go through readfirstlane into SGPRs
  auto uniform_ptr = [](const int8_t* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const int8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  };
  auto issue = [&](int s, int slot) {
#pragma unroll
    for (int t = 0; t < LW; ++t) {
      const int8_t* base = uniform_ptr((is_w[t] ? wtile : xtile) + (int64_t)s * BK);
      const uint32_t dst =
          __builtin_amdgcn_readfirstlane(lds_u32 + (uint32_t)(slot * STAGE + ldsoff[t]));
      dma16(base, voff[t], dst);
    }
  };

  v16i acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = (v16i){};

  // a stage's copies are complete when at most the copies of the p later
  // stages are outstanding (copies complete in order)
  auto wait_stage_runtime = [&](int p) {  // p = later stages allowed to stay pending
    if (p >= LA - 1) {
      wait_vmcnt<(LA - 1) * LW>();
      return;
    }
    if constexpr (LA - 1 > 3) {
      if (p == 3) {
        wait_vmcnt<(LA - 1 > 3 ? 3 * LW : 0)>();
        return;
      }
    }
    if constexpr (LA - 1 > 2) {
      if (p == 2) {
        wait_vmcnt<(LA - 1 > 2 ? 2 * LW : 0)>();
        return;
      }
    }
    if constexpr (LA - 1 > 1) {
      if (p == 1) {
        wait_vmcnt<(LA - 1 > 1 ? LW : 0)>();
        return;
      }
    }
    wait_vmcnt<0>();
  };

  // The scaled output tile is staged in LDS (the ring is free after the
  // K-loop) with rows of PITCH bytes; then every wave of the block stores
  // whole tile rows with 16-byte stores, so each 128-byte output line is
  // written once instead of in 16-byte pieces by 8 different instructions.
  constexpr int PITCH = BN * 2 + 16;
  static_assert(BM * PITCH <= 160 * 1024, "staged output tile");
  auto store_tile = [&]() {
    wait_lgkm0();  // this wave's staging writes are done
    lds_barrier();
    constexpr int CPR16 = BN * 2 / 16;  // 16-byte pieces per tile row
#pragma unroll 4
    for (int idx = tid; idx < BM * CPR16; idx += 64 * (NW + NP)) {
      const int r = idx / CPR16;
      const int cc = idx - r * CPR16;
      const int m = m0 + r, n = n0 + 8 * cc;
      if (m < M && n < N)  // N % 16 == 0: a piece is all inside or all outside
        *reinterpret_cast<u4*>(y + (int64_t)m * N + n) =
            *reinterpret_cast<const u4*>(lds + r * PITCH + 16 * cc);
    }
  };

  // The epilogue's row scales (and the per-tensor weight scale), loaded
  // before the first copies instead of after the K-loop, where their
  // latency stood between the last MFMAs and the stores of every tile.
  // Issued ahead of the copies, they complete first (in-order vmcnt), so the
  // stage waits account for them.
  float sx_pre[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int m = m0 + wm * WTM + j * 32 + (lane & 31);
    sx_pre[j] = s_x[m < M ? m : M - 1];
  }
  const float sw_pre = PC ? 0.0f : *s_w;

  if constexpr (NP > 0) {
    if (wave >= NW) {
      // ---- producer: stage s+1 landed before the barrier that ends step
      // s; after it, the slot of stage s-1 (read by every consumer before
      // that barrier) takes stage s+NS-1. Same barrier count as a consumer
      // (one before the loop, one per step).
#pragma unroll
      for (int s = 0; s < LA; ++s)
        if (s < nk) issue(s, s % NS);
      wait_stage_runtime(min(LA - 1, nk - 1));  // stage 0 landed
      lds_barrier();
      for (int s = 0; s + 1 < nk; ++s) {
        wait_stage_runtime(min(LA - 2, nk - 2 - s));  // stage s+1 landed
        lds_barrier();
        if (s + LA < nk) issue(s + LA, (s + LA) % NS);
      }
      lds_barrier();  // the consumers' last-step barrier
      if (y) {
        lds_barrier();  // the consumers' barrier before staging the tile
        store_tile();
      }
      return;
    }
  } else {
#pragma unroll
    for (int s = 0; s < LA; ++s)
      if (s < nk) issue(s, s % NS);
  }

  // 32x32x32 operands: lane -> row lane%32 of a 32-row block, 16-byte
  // half lane/32 of the 32-byte k-slice h of the K-step
  const int fr = lane & 31;
  const int fh = lane >> 5;
  // The 16 lanes that read 16 consecutive rows at one chunk hit 16 distinct
  // 16-byte bank groups (without the swizzle, rows RPB apart share banks).
  // Row blocks start at multiples of 32, so swz(row) = (fr / RPB) % CPR for
  // every fragment of this lane; slice h reads chunk 2h + fh.
  const int swz = (fr / RPB) % CPR;
  int dsw[H];
#pragma unroll
  for (int h = 0; h < H; ++h) dsw[h] = 16 * ((2 * h + fh) ^ swz);
  int aoff[NI], boff[NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i) aoff[i] = (wn * WTN + i * 32 + fr) * BK;
#pragma unroll
  for (int j = 0; j < NJ; ++j) boff[j] = BN * BK + (wm * WTM + j * 32 + fr) * BK;

  // Each K-step is H 32-k slices whose fragments alternate between two
  // register sets X (even slices) and Y (odd slices): while the MFMAs of one
  // slice run, the next slice's fragments are read. Before the last slice of
  // step s, the barrier publishes stage s+1 (and frees the ring slot of stage
  // s-1 for the next DMA), so the last slice's MFMAs overlap the reads of
  // slice 0 of step s+1.
  constexpr int NF = NI + NJ;
  v4i xa[NI], xb[NJ], ya[NI], yb[NJ];
  auto read_slice = [&](int s, int h, v4i (&fa)[NI], v4i (&fb)[NJ]) {
    const uint8_t* base = lds + (s % NS) * STAGE + dsw[h];
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb[j] = *reinterpret_cast<const v4i*>(base + boff[j]);
#pragma unroll
    for (int i = 0; i < NI; ++i) fa[i] = *reinterpret_cast<const v4i*>(base + aoff[i]);
  };
  auto mfma_slice = [&](const v4i (&fa)[NI], const v4i (&fb)[NJ]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  // spread the NF reads of the next slice over the NI*NJ MFMAs of this one
  auto sched_slice = [&]() {
    constexpr int NM = NI * NJ;
    constexpr int PER = NM / NF > 0 ? NM / NF : 1;
    constexpr int NR = NM / PER < NF ? NM / PER : NF;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one DS read
      __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // PER MFMAs
    }
    __builtin_amdgcn_sched_group_barrier(0x100, NF - NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM - NR * PER, 0);
  };
  // the first H-1 slices of step s (slice 0 is already in X)
  auto early_slices = [&](int s) {
#pragma unroll
    for (int h = 0; h + 1 < H; ++h) {
      if (h % 2 == 0) {
        read_slice(s, h + 1, ya, yb);
        mfma_slice(xa, xb);
      } else {
        read_slice(s, h + 1, xa, xb);
        mfma_slice(ya, yb);
      }
      sched_slice();
    }
  };

  // Consume the epilogue's pointer arguments here: their scalar loads then
  // complete before the K-loop. A scalar load still in flight at the loop
  // entry (they return out of order) makes every LDS-read wait in the loop
  // a full lgkmcnt(0) drain.
  asm volatile("" ::"s"(y), "s"(acc_out), "s"(s_x), "s"(s_w), "s"(bias), "s"(sw_pre));
  if constexpr (NP == 0) wait_stage_runtime(min(LA - 1, nk - 1));  // stage 0 landed
  lds_barrier();
  read_slice(0, 0, xa, xb);
  // One uniform loop (no separate tail copy, which would double the live
  // ranges): before the last slice of step s, stage s+1 must have landed;
  // the barrier publishes it and frees the slot of stage s-1 for the copies
  // of stage s+NS-1.
  for (int s = 0; s < nk; ++s) {
    early_slices(s);
    if constexpr (NP == 0) wait_stage_runtime(min(LA - 2, nk - 2 - s));  // stage s+1 landed
    wait_lgkm0();  // this wave's reads of stage s are done before the barrier
    lds_barrier();
    // With 8 waves, waves w and w + 4 share a SIMD: the first four issue
    // their copies right after the barrier, the other four after the MFMAs
    // of the last slice, so one wave of each SIMD keeps its MFMAs going
    // while the other issues (all issuing at once left the MFMA pipes idle
    // for the length of the issue, +1.5-5% measured).
    const bool late = NP == 0 && NW == 8 && wave >= 4;
    if constexpr (NP == 0) {
      if (!late && s + LA < nk) issue(s + LA, (s + LA) % NS);
    }
    // Every step takes the same path, the last one included (its reads of
    // a stale ring slot land in X and are never used): with a branch around
    // the barrier and these reads, the compiler's LDS-wait count for the Y
    // slice below merges the two paths and then waits for the X reads just
    // issued, stalling the MFMAs behind the LDS latency once per step.
    read_slice(s + 1, 0, xa, xb);
    mfma_slice(ya, yb);  // H is even: the last slice sits in Y
    sched_slice();
    if constexpr (NP == 0) {
      if (late && s + LA < nk) issue(s + LA, (s + LA) % NS);
    }
  }

  // ---- epilogue: 32x32 output layout: lane holds m = lane % 32 of the
  // tile and n = 8*a + 4*(lane/32) + e for register 4a + e; the results go
  // to the LDS staging tile, then out by store_tile ----
  if (y) {
    wait_lgkm0();  // every wave's last ring reads are done before the tile is staged
    lds_barrier();
  }
  const float sw = sw_pre;
  // per-channel: the 4 consecutive columns of each (i, a) register group,
  // loaded once for all NJ row blocks
  typedef float f4 __attribute__((ext_vector_type(4)));
  f4 swc[PC ? NI : 1][4];
  if constexpr (PC) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int n = n0 + wn * WTN + i * 32 + 8 * a + 4 * fh;
        swc[i][a] = n < N ? *reinterpret_cast<const f4*>(s_w + n) : (f4){0.f, 0.f, 0.f, 0.f};
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int ml = wm * WTM + j * 32 + fr;  // row within the tile
    const int m = m0 + ml;
    if (m >= M) continue;
    const float sx = sx_pre[j];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int nl = wn * WTN + i * 32 + 8 * a + 4 * fh;  // column within the tile
        const int n = n0 + nl;
        if (n >= N) continue;
        const v16i& v = acc[i][j];
        if (acc_out) {
          *reinterpret_cast<v4i*>(acc_out + (int64_t)m * N + n) =
              (v4i){v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]};
        }
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[e] = (float)v[4 * a + e] * (PC ? swc[PC ? i : 0][a][e] : sw);
          f[e] = f[e] * sx;
        }
        if (bias) {
          const u2 bb = *reinterpret_cast<const u2*>(bias + n);
          f[0] = f[0] + lo16<F16>(bb.x);
          f[1] = f[1] + hi16<F16>(bb.x);
          f[2] = f[2] + lo16<F16>(bb.y);
          f[3] = f[3] + hi16<F16>(bb.y);
        }
        if (y) {
          const u2 o = {pack16x2<F16>(f[0], f[1]), pack16x2<F16>(f[2], f[3])};
          *reinterpret_cast<u2*>(lds + ml * PITCH + 2 * nl) = o;
        }
      }
    }
  }
  if (y) store_tile();
}

struct TileCfg {
  int bm, bn, ns, per_cu;
};

template <bool PC, bool F16, int BM, int BN, int BK, int WM, int WN, int NS, int MINB, int NP = 0>
hipError_t launch_cfg(const int8_t* xq, const float* s_x, const int8_t* wq, const float* s_w,
                      const uint16_t* bias, int m, int n, int k, uint16_t* y, int32_t* acc,
                      int nx, hipStream_t st) {
  // the K-loop's ring, or the staged output tile (rows of 2 BN + 16 bytes)
  constexpr int ring_bytes = NS * (BM + BN) * BK;
  constexpr int tile_bytes = BM * (BN * 2 + 16);
  constexpr int lds_bytes = ring_bytes > tile_bytes ? ring_bytes : tile_bytes;
  static_assert(lds_bytes <= 160 * 1024, "LDS");
  auto kern = gemm_i8_kernel<BM, BN, BK, WM, WN, NS, MINB, NP, PC, F16>;
  static bool attr = false;  // benign race: the call is idempotent
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int tiles_m = (m + BM - 1) / BM;
  const int tiles_n = (n + BN - 1) / BN;
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(64 * (WM * WN + NP)), lds_bytes, st, xq,
                     s_x, wq, s_w, bias, m, n, k, tiles_m, tiles_n, nx, y, acc);
  return hipGetLastError();
}

// Pick the tile whose estimated time is least: rounds of concurrent tiles
// over 256 CUs times the measured duration of one round of that tile
// (relative; the operand stream per CU bounds every tile, so a round's
// duration follows the tile's operand bytes and its L2 behaviour). The
// 384 x 192 tile exists for K % 128 == 0 only.
TileCfg choose_tile(int64_t m, int64_t n, int64_t k, int cus) {
  const TileCfg cands[] = {{384, 192, 2, 1}, {256, 256, 2, 1}, {192, 192, 3, 1}, {128, 128, 2, 2}};
  // duration of one full round relative to the 192 tile's. Measured on MI355X
  // the ratios vary with the shape (384 x 192: 1.71-1.85, 256 x 256:
  // 1.25-1.56 of a 192 round; their ratio 1.18-1.37): the 384 figure is set
  // to 1.2 times the 256 one, which orders the two tiles right on the
  // workload layers and the linear's slices of them (e.g. 5112 x 13824 x
  // 5120: 384 x 192 in 4 rounds 319 us, 256 x 256 in 4 rounds plus 56 tiles
  // 338 us; 4608 x 3072 x 12288: 256 x 256 148 us, 384 x 192 152 us).
  const double round_t[] = {1.6, 1.336, 1.0, 1.0};
  TileCfg best = cands[2];
  double best_t = 1e300;
  for (int c = 0; c < 4; ++c) {
    const TileCfg& t = cands[c];
    if (t.bm == 384 && k % 128 != 0) continue;
    const int64_t tiles = ((m + t.bm - 1) / t.bm) * ((n + t.bn - 1) / t.bn);
    const int64_t slots = (int64_t)(cus > 0 ? cus : 1) * t.per_cu;
    const int64_t rounds = (tiles + slots - 1) / slots;
    // with no more 128 tiles than CUs each block runs alone on its CU:
    // measured 0.92 of the 192 tile's one-round time (1024x3840x3840)
    const double rt = (t.per_cu == 2 && tiles <= cus) ? 0.92 : round_t[c];
    const double time = (double)rounds * rt;
    if (time < best_t * 0.999) {
      best_t = time;
      best = t;
    }
  }
  return best;
}

}  // namespace

// One configuration per tile size. When K allows, every tile streams
// 128-byte K-steps (whole L2 lines per request): a two-stage ring for the
// 384 x 192, 256 and 128 tiles (72, 64 and 32 KB stages), three stages and
// four producer waves for the 192 tile. Otherwise 64-byte K-steps with
// deeper rings (the 384 x 192 tile then does not exist).
template <bool PC, bool F16>
static hipError_t launch_tile(int tile, const int8_t* xq, const float* s_x, const int8_t* wq,
                              const float* s_w, const uint16_t* bias, int M, int N, int K,
                              uint16_t* y, int32_t* acc, int nx, hipStream_t st) {
  switch (tile) {
    case 256:
      if (K % 128 == 0)
        return launch_cfg<PC, F16, 256, 256, 128, 2, 4, 2, 1>(xq, s_x, wq, s_w, bias, M, N, K, y, acc, nx, st);
      return launch_cfg<PC, F16, 256, 256, 64, 2, 4, 4, 1>(xq, s_x, wq, s_w, bias, M, N, K, y, acc, nx, st);
    case 384:  // 384 x 192 (K % 128 == 0 only)
      return launch_cfg<PC, F16, 384, 192, 128, 4, 2, 2, 1>(xq, s_x, wq, s_w, bias, M, N, K, y, acc,
                                                            nx, st);
    case 192:
      if (K % 128 == 0)
        return launch_cfg<PC, F16, 192, 192, 128, 2, 2, 3, 1, 4>(xq, s_x, wq, s_w, bias, M, N, K, y, acc,
                                                          nx, st);
      return launch_cfg<PC, F16, 192, 192, 64, 2, 2, 6, 1, 4>(xq, s_x, wq, s_w, bias, M, N, K, y, acc, nx, st);
    default:
      if (K % 128 == 0)
        return launch_cfg<PC, F16, 128, 128, 128, 2, 2, 2, 2>(xq, s_x, wq, s_w, bias, M, N, K, y, acc, nx, st);
      return launch_cfg<PC, F16, 128, 128, 64, 2, 2, 4, 2>(xq, s_x, wq, s_w, bias, M, N, K, y, acc, nx, st);
  }
}

hipError_t launch_gemm(const int8_t* xq, const float* s_x, const int8_t* wq, const float* s_w,
                       bool sw_per_channel, const uint16_t* bias, int64_t m, int64_t n, int64_t k,
                       uint16_t* y, int32_t* acc, DType dt, hipStream_t st) {
  return launch_gemm_tile(xq, s_x, wq, s_w, sw_per_channel, bias, m, n, k, y, acc, 0, dt, st);
}

LaunchPlan plan_gemm(int64_t m, int64_t n, int64_t k, int tile, int cus) {
  LaunchPlan p;
  if (tile == 0) tile = choose_tile(m, n, k, cus).bm;
  p.tile_m = tile;
  p.tile_n = tile == 384 ? 192 : tile;
  p.block = tile == 192 ? 512 : (tile == 128 ? 256 : 512);
  p.grid = ((m + p.tile_m - 1) / p.tile_m) * ((n + p.tile_n - 1) / p.tile_n);
  p.xcds = xcd_count(cus);
  p.passes = 1;
  return p;
}

hipError_t launch_gemm_tile(const int8_t* xq, const float* s_x, const int8_t* wq,
                            const float* s_w, bool sw_per_channel, const uint16_t* bias,
                            int64_t m, int64_t n, int64_t k, uint16_t* y, int32_t* acc, int tile,
                            DType dt, hipStream_t st) {
  if (m == 0 || n == 0) return hipSuccess;
  const int cus = compute_units();
  const LaunchPlan p = plan_gemm(m, n, k, tile, cus);
  const int M = (int)m, N = (int)n, K = (int)k, nx = p.xcds;
  if (dt == DType::kF16)
    return sw_per_channel
               ? launch_tile<true, true>(p.tile_m, xq, s_x, wq, s_w, bias, M, N, K, y, acc, nx, st)
               : launch_tile<false, true>(p.tile_m, xq, s_x, wq, s_w, bias, M, N, K, y, acc, nx, st);
  return sw_per_channel
             ? launch_tile<true, false>(p.tile_m, xq, s_x, wq, s_w, bias, M, N, K, y, acc, nx, st)
             : launch_tile<false, false>(p.tile_m, xq, s_x, wq, s_w, bias, M, N, K, y, acc, nx, st);
}

}  // namespace convrot

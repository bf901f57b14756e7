// C ABI of the convrot library: argument checks, rotation signs, slicing.
// Every check runs before any HIP call, so argument errors are reported
// (and testable) without a GPU.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <cmath>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/convrot.h"
#include "common.h"
#include "internal.h"

using namespace convrot;

namespace {

thread_local char g_last_error[512] = "";

convrot_status fail(convrot_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
convrot_status fail(convrot_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

convrot_status ok() {
  g_last_error[0] = '\0';
  return CONVROT_OK;
}

convrot_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CONVROT_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014), counter form:
// output i = mix(seed + (i + 1) * golden gamma).
uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

SignMask make_signs(uint64_t seed, int g) {
  SignMask sm;
  memset(&sm, 0, sizeof sm);
  for (int i = 0; i < g; ++i) {
    const uint64_t z = splitmix64_mix(seed + (uint64_t)(i + 1) * 0x9E3779B97F4A7C15ull);
    if (z >> 63) sm.w[i >> 5] |= 1u << (i & 31);
  }
  return sm;
}

bool valid_group(int g) { return g == 4 || g == 16 || g == 64 || g == 256; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x0 = (uintptr_t)a, x1 = x0 + na, y0 = (uintptr_t)b, y1 = y0 + nb;
  return x0 < y1 && y0 < x1;
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxRotK = 16384;
constexpr int64_t kMaxGemmK = 133144;  // 127^2 * K < 2^31

// Checks shared by the rotating entry points (rows x k with group g).
convrot_status check_rot(const char* fn, int64_t rows, int64_t k, int g) {
  if (rows < 0 || k <= 0) return fail(CONVROT_E_INVALID_ARG, "%s: bad dims rows=%lld k=%lld", fn,
                                      (long long)rows, (long long)k);
  if (!valid_group(g)) return fail(CONVROT_E_UNSUPPORTED_GROUP, "%s: g=%d not in {4,16,64,256}",
                                   fn, g);
  if (k % g) return fail(CONVROT_E_UNSUPPORTED_GROUP, "%s: k=%lld not a multiple of g=%d", fn,
                         (long long)k, g);
  if (k % 64 || k > kMaxRotK || rows >= kMaxDim)
    return fail(CONVROT_E_UNSUPPORTED_SHAPE,
                "%s: need k %% 64 == 0, k <= %lld, rows < 2^31 (rows=%lld k=%lld)", fn,
                (long long)kMaxRotK, (long long)rows, (long long)k);
  return CONVROT_OK;
}

convrot_status check_gemm(const char* fn, int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n <= 0 || k <= 0)
    return fail(CONVROT_E_INVALID_ARG, "%s: bad dims m=%lld n=%lld k=%lld", fn, (long long)m,
                (long long)n, (long long)k);
  if (k % 64 || n % 16 || k > kMaxGemmK || m >= kMaxDim || n >= kMaxDim)
    return fail(CONVROT_E_UNSUPPORTED_SHAPE,
                "%s: need k %% 64 == 0, n %% 16 == 0, k <= %lld (m=%lld n=%lld k=%lld)", fn,
                (long long)kMaxGemmK, (long long)m, (long long)n, (long long)k);
  // the smallest block tile is 128 x 128: the tile count must fit the 32-bit grid
  if (((m + 127) / 128) * ((n + 127) / 128) >= kMaxDim)
    return fail(CONVROT_E_UNSUPPORTED_SHAPE, "%s: output too large (m=%lld n=%lld)", fn,
                (long long)m, (long long)n);
  return CONVROT_OK;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// enum arguments of the *_ex entry points
bool dtype_of(int v, DType* dt) {
  if (v != CONVROT_DTYPE_BF16 && v != CONVROT_DTYPE_F16) return false;
  *dt = v == CONVROT_DTYPE_F16 ? DType::kF16 : DType::kBF16;
  return true;
}
bool scale_mode_of(int v, bool* pc) {
  if (v != CONVROT_SCALE_PER_TENSOR && v != CONVROT_SCALE_PER_CHANNEL) return false;
  *pc = v == CONVROT_SCALE_PER_CHANNEL;
  return true;
}

// Per-tensor s_w: one fp32, 4-byte aligned. Per-channel s_w: n fp32, 16-byte
// aligned (the GEMM epilogue reads four consecutive scales at once).
size_t sw_bytes(bool pc, int64_t n) { return pc ? (size_t)n * 4 : 4; }
bool sw_aligned(bool pc, const float* s_w) { return aligned(s_w, pc ? 16 : 4); }

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];  // 0 = not queried yet
std::atomic<int> g_cu_override{0};

}  // namespace

namespace convrot {

int compute_units() {
  const int forced = g_cu_override.load(std::memory_order_relaxed);
  if (forced > 0) return forced;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int cus = g_device_cus[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      return 256;
    g_device_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

}  // namespace convrot

extern "C" {

int convrot_abi_version(void) { return CONVROT_ABI_VERSION; }

convrot_status convrot_set_compute_units(int compute_units_override) {
  if (compute_units_override < 0 || compute_units_override > 1 << 16)
    return fail(CONVROT_E_INVALID_ARG, "convrot_set_compute_units: %d", compute_units_override);
  g_cu_override.store(compute_units_override, std::memory_order_relaxed);
  return ok();
}

int convrot_compute_units(void) { return convrot::compute_units(); }

convrot_status convrot_plan_launch(convrot_kernel kernel, int64_t m, int64_t n, int64_t k, int g,
                                   int compute_units, convrot_launch_plan* out) {
  const char* fn = "convrot_plan_launch";
  if (!out) return fail(CONVROT_E_INVALID_ARG, "%s: null output", fn);
  memset(out, 0, sizeof *out);
  if (compute_units < 0) return fail(CONVROT_E_INVALID_ARG, "%s: compute_units < 0", fn);
  const int cus = compute_units > 0 ? compute_units : convrot::compute_units();
  LaunchPlan p;
  switch (kernel) {
    case CONVROT_KERNEL_ACT_QUANT:
    case CONVROT_KERNEL_ACT_QUANT_DEFERRED:
    case CONVROT_KERNEL_EXACT:
      if (convrot_status s = check_rot(fn, m, k, g)) return s;
      if (m == 0) return ok();
      p = kernel == CONVROT_KERNEL_EXACT
              ? plan_exact(m, (int)k, cus)
              : plan_act_quant(m, (int)k, kernel == CONVROT_KERNEL_ACT_QUANT_DEFERRED, cus);
      break;
    case CONVROT_KERNEL_DEQUANT:
      if (n <= 0) return fail(CONVROT_E_INVALID_ARG, "%s: n=%lld", fn, (long long)n);
      if (convrot_status s = check_rot(fn, n, k, g)) return s;
      p = plan_dequant(n, k, g, cus);
      break;
    case CONVROT_KERNEL_GEMM:
      if (convrot_status s = check_gemm(fn, m, n, k)) return s;
      if (m == 0) return ok();
      p = plan_gemm(m, n, k, 0, cus);
      break;
    default:
      return fail(CONVROT_E_INVALID_ARG, "%s: kernel=%d", fn, (int)kernel);
  }
  out->grid = p.grid;
  out->block = p.block;
  out->rows_per_block = p.rows_per_block;
  out->tile_m = p.tile_m;
  out->tile_n = p.tile_n;
  out->xcds = p.xcds;
  out->passes = p.passes;
  out->compute_units = cus;
  return ok();
}

const char* convrot_status_string(convrot_status s) {
  switch (s) {
    case CONVROT_OK: return "ok";
    case CONVROT_E_INVALID_ARG: return "invalid argument";
    case CONVROT_E_UNSUPPORTED_GROUP: return "unsupported rotation group size";
    case CONVROT_E_UNSUPPORTED_SHAPE: return "unsupported shape";
    case CONVROT_E_MISALIGNED: return "misaligned pointer";
    case CONVROT_E_WORKSPACE: return "workspace too small";
    case CONVROT_E_HIP: return "HIP error";
    case CONVROT_E_SELFCHECK: return "first-call check failed (latched)";
  }
  return "unknown status";
}

const char* convrot_last_error_string(void) { return g_last_error; }

convrot_status convrot_rotation_signs(uint64_t rot_seed, int g, int8_t* d) {
  if (!d) return fail(CONVROT_E_INVALID_ARG, "convrot_rotation_signs: null output");
  if (!valid_group(g))
    return fail(CONVROT_E_UNSUPPORTED_GROUP, "convrot_rotation_signs: g=%d", g);
  const SignMask sm = make_signs(rot_seed, g);
  for (int i = 0; i < g; ++i) d[i] = ((sm.w[i >> 5] >> (i & 31)) & 1u) ? -1 : 1;
  return ok();
}

static convrot_status quantize_weights_impl(const char* fn, bool pc, const uint16_t* w,
                                            int64_t n, int64_t k, int g, uint64_t rot_seed,
                                            int8_t* wq, float* s_w, void* stream) {
  if (!w || !wq || !s_w) return fail(CONVROT_E_INVALID_ARG, "%s: null pointer", fn);
  if (n <= 0) return fail(CONVROT_E_INVALID_ARG, "%s: n=%lld", fn, (long long)n);
  if (convrot_status s = check_rot(fn, n, k, g)) return s;
  if (!aligned(w, 16) || !aligned(wq, 16) || !sw_aligned(pc, s_w))
    return fail(CONVROT_E_MISALIGNED, "%s: misaligned pointer", fn);
  const size_t nsw = sw_bytes(pc, n);
  if (overlap(w, (size_t)(n * k) * 2, wq, (size_t)(n * k)) ||
      overlap(w, (size_t)(n * k) * 2, s_w, nsw) || overlap(wq, (size_t)(n * k), s_w, nsw))
    return fail(CONVROT_E_INVALID_ARG, "%s: overlapping buffers", fn);
  const SignMask sm = make_signs(rot_seed, g);
  // per channel, a weight row is quantized exactly as a token row is
  const hipError_t e =
      pc ? launch_quantize_rows(w, wq, s_w, n, (int)k, g, sm, DType::kBF16, (hipStream_t)stream)
         : launch_quantize_tensor(w, wq, s_w, n, (int)k, g, sm, (hipStream_t)stream);
  return hip_status(e, fn);
}

convrot_status convrot_quantize_weights(const uint16_t* w, int64_t n, int64_t k, int g,
                                        uint64_t rot_seed, int8_t* wq, float* s_w,
                                        void* stream) {
  return quantize_weights_impl("convrot_quantize_weights", false, w, n, k, g, rot_seed, wq, s_w,
                               stream);
}

convrot_status convrot_quantize_weights_per_channel(const uint16_t* w, int64_t n, int64_t k,
                                                    int g, uint64_t rot_seed, int8_t* wq,
                                                    float* s_w, void* stream) {
  return quantize_weights_impl("convrot_quantize_weights_per_channel", true, w, n, k, g, rot_seed,
                               wq, s_w, stream);
}

static convrot_status dequant_impl(const char* fn, bool pc, DType dt, const int8_t* wq,
                                   const float* s_w, int64_t n, int64_t k, int g,
                                   uint64_t rot_seed, uint16_t* w_out, void* stream) {
  if (!wq || !s_w || !w_out) return fail(CONVROT_E_INVALID_ARG, "%s: null pointer", fn);
  if (n <= 0) return fail(CONVROT_E_INVALID_ARG, "%s: n=%lld", fn, (long long)n);
  if (convrot_status s = check_rot(fn, n, k, g)) return s;
  if (!aligned(wq, 16) || !aligned(w_out, 16) || !sw_aligned(pc, s_w))
    return fail(CONVROT_E_MISALIGNED, "%s: misaligned pointer", fn);
  if (overlap(wq, (size_t)(n * k), w_out, (size_t)(n * k) * 2) ||
      overlap(s_w, sw_bytes(pc, n), w_out, (size_t)(n * k) * 2))
    return fail(CONVROT_E_INVALID_ARG, "%s: overlapping buffers", fn);
  const SignMask sm = make_signs(rot_seed, g);
  return hip_status(launch_dequant(wq, s_w, pc, n, k, g, sm, w_out, dt, (hipStream_t)stream),
                    fn);
}

convrot_status convrot_dequant_derotate(const int8_t* wq, const float* s_w, int64_t n, int64_t k,
                                        int g, uint64_t rot_seed, uint16_t* w_out,
                                        void* stream) {
  return dequant_impl("convrot_dequant_derotate", false, DType::kBF16, wq, s_w, n, k, g, rot_seed,
                      w_out, stream);
}

convrot_status convrot_dequant_derotate_per_channel(const int8_t* wq, const float* s_w, int64_t n,
                                                    int64_t k, int g, uint64_t rot_seed,
                                                    uint16_t* w_out, void* stream) {
  return dequant_impl("convrot_dequant_derotate_per_channel", true, DType::kBF16, wq, s_w, n, k, g,
                      rot_seed, w_out, stream);
}

convrot_status convrot_dequant_derotate_ex(const int8_t* wq, const float* s_w,
                                           convrot_scale_mode scale_mode, int64_t n, int64_t k,
                                           int g, uint64_t rot_seed, void* w_out,
                                           convrot_dtype out_dtype, void* stream) {
  const char* fn = "convrot_dequant_derotate_ex";
  bool pc;
  DType dt;
  if (!scale_mode_of(scale_mode, &pc) || !dtype_of(out_dtype, &dt))
    return fail(CONVROT_E_INVALID_ARG, "%s: scale_mode=%d out_dtype=%d", fn, (int)scale_mode,
                (int)out_dtype);
  return dequant_impl(fn, pc, dt, wq, s_w, n, k, g, rot_seed, static_cast<uint16_t*>(w_out),
                      stream);
}

convrot_status convrot_dequant_derotate_batched(const convrot_dequant_job* jobs, int njobs,
                                                convrot_scale_mode scale_mode, int g,
                                                uint64_t rot_seed, convrot_dtype out_dtype,
                                                void* stream) {
  const char* fn = "convrot_dequant_derotate_batched";
  bool pc;
  DType dt;
  if (!scale_mode_of(scale_mode, &pc) || !dtype_of(out_dtype, &dt))
    return fail(CONVROT_E_INVALID_ARG, "%s: scale_mode=%d out_dtype=%d", fn, (int)scale_mode,
                (int)out_dtype);
  if (njobs < 0 || (njobs > 0 && !jobs))
    return fail(CONVROT_E_INVALID_ARG, "%s: njobs=%d, jobs=%p", fn, njobs, (const void*)jobs);
  if (!valid_group(g)) return fail(CONVROT_E_UNSUPPORTED_GROUP, "%s: g=%d", fn, g);
  std::vector<DequantJob> js((size_t)njobs);
  for (int i = 0; i < njobs; ++i) {
    const convrot_dequant_job& jb = jobs[i];
    if (!jb.wq || !jb.s_w || !jb.w_out)
      return fail(CONVROT_E_INVALID_ARG, "%s: job %d: null pointer", fn, i);
    if (jb.n <= 0) return fail(CONVROT_E_INVALID_ARG, "%s: job %d: n=%lld", fn, i, (long long)jb.n);
    if (convrot_status st = check_rot(fn, jb.n, jb.k, g)) return st;
    if (!aligned(jb.wq, 16) || !aligned(jb.w_out, 16) || !sw_aligned(pc, jb.s_w))
      return fail(CONVROT_E_MISALIGNED, "%s: job %d: misaligned pointer", fn, i);
    js[(size_t)i] = DequantJob{jb.wq, jb.s_w, static_cast<uint16_t*>(jb.w_out), jb.n, jb.k};
  }
  // every output is written by its job alone and read by none
  for (int i = 0; i < njobs; ++i) {
    const size_t ob = (size_t)(js[i].n * js[i].k) * 2;
    for (int j = 0; j < njobs; ++j) {
      const size_t nb = (size_t)(js[j].n * js[j].k);
      if (overlap(js[i].w_out, ob, js[j].wq, nb) ||
          overlap(js[i].w_out, ob, js[j].s_w, sw_bytes(pc, js[j].n)) ||
          (j != i && overlap(js[i].w_out, ob, js[j].w_out, nb * 2)))
        return fail(CONVROT_E_INVALID_ARG, "%s: job %d's output overlaps job %d's buffers", fn,
                    i, j);
    }
  }
  if (njobs == 0) return ok();
  const SignMask sm = make_signs(rot_seed, g);
  return hip_status(launch_dequant_jobs(js.data(), njobs, pc, g, sm, dt, (hipStream_t)stream),
                    fn);
}

static convrot_status quantize_activations_impl(const char* fn, bool exact, DType dt,
                                                const uint16_t* x, int64_t m, int64_t k, int g,
                                                uint64_t rot_seed, int8_t* xq, float* s_x,
                                                void* stream) {
  if (convrot_status s = check_rot(fn, m, k, g)) return s;
  if (m == 0) return ok();  // nothing to read or write; the M-sized buffers may be null
  if (!x || !xq || !s_x) return fail(CONVROT_E_INVALID_ARG, "%s: null pointer", fn);
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(s_x, 4))
    return fail(CONVROT_E_MISALIGNED, "%s: misaligned pointer", fn);
  if (overlap(x, (size_t)(m * k) * 2, xq, (size_t)(m * k)) ||
      overlap(x, (size_t)(m * k) * 2, s_x, (size_t)m * 4) ||
      overlap(xq, (size_t)(m * k), s_x, (size_t)m * 4))
    return fail(CONVROT_E_INVALID_ARG, "%s: overlapping buffers", fn);
  if (m == 0) return ok();
  const SignMask sm = make_signs(rot_seed, g);
  hipError_t e = exact ? launch_quantize_rows_exact(x, xq, s_x, m, (int)k, g, sm,
                                                    (hipStream_t)stream)
                       : launch_quantize_rows(x, xq, s_x, m, (int)k, g, sm, dt,
                                              (hipStream_t)stream);
  return hip_status(e, fn);
}

convrot_status convrot_quantize_activations(const uint16_t* x, int64_t m, int64_t k, int g,
                                            uint64_t rot_seed, int8_t* xq, float* s_x,
                                            void* stream) {
  return quantize_activations_impl("convrot_quantize_activations", false, DType::kBF16, x, m, k,
                                   g, rot_seed, xq, s_x, stream);
}

convrot_status convrot_quantize_activations_ex(const void* x, convrot_dtype dtype, int64_t m,
                                               int64_t k, int g, uint64_t rot_seed, int8_t* xq,
                                               float* s_x, void* stream) {
  const char* fn = "convrot_quantize_activations_ex";
  DType dt;
  if (!dtype_of(dtype, &dt)) return fail(CONVROT_E_INVALID_ARG, "%s: dtype=%d", fn, (int)dtype);
  return quantize_activations_impl(fn, false, dt, static_cast<const uint16_t*>(x), m, k, g,
                                   rot_seed, xq, s_x, stream);
}

convrot_status convrot_quantize_activations_exact(const uint16_t* x, int64_t m, int64_t k, int g,
                                                  uint64_t rot_seed, int8_t* xq, float* s_x,
                                                  void* stream) {
  return quantize_activations_impl("convrot_quantize_activations_exact", true, DType::kBF16, x, m,
                                   k, g, rot_seed, xq, s_x, stream);
}

static convrot_status gemm_impl(const char* fn, bool pc, DType dt, const int8_t* xq,
                                const float* s_x,
                                const int8_t* wq, const float* s_w, const uint16_t* bias,
                                int64_t m, int64_t n, int64_t k, uint16_t* y, int32_t* acc,
                                int tile, void* stream) {
  if (tile != 0 && tile != 128 && tile != 192 && tile != 256 && tile != 384)
    return fail(CONVROT_E_INVALID_ARG, "%s: tile=%d not supported", fn, tile);
  if (tile == 384 && k % 128 != 0)
    return fail(CONVROT_E_INVALID_ARG, "%s: the 384 x 192 tile needs k %% 128 == 0", fn);
  if (!wq || !s_w) return fail(CONVROT_E_INVALID_ARG, "%s: null pointer", fn);
  if (convrot_status s = check_gemm(fn, m, n, k)) return s;
  if (m == 0) return ok();  // the M-sized buffers may be null
  if (!xq || !s_x || (!y && !acc)) return fail(CONVROT_E_INVALID_ARG, "%s: null pointer", fn);
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(s_x, 4) || !sw_aligned(pc, s_w) ||
      (bias && !aligned(bias, 8)) || (y && !aligned(y, 16)) || (acc && !aligned(acc, 16)))
    return fail(CONVROT_E_MISALIGNED, "%s: misaligned pointer", fn);
  const size_t ny = (size_t)(m * n) * 2, na = (size_t)(m * n) * 4;
  if (overlap(y, ny, xq, (size_t)(m * k)) || overlap(y, ny, wq, (size_t)(n * k)) ||
      overlap(acc, na, xq, (size_t)(m * k)) || overlap(acc, na, wq, (size_t)(n * k)) ||
      overlap(y, ny, acc, na) || overlap(y, ny, s_w, sw_bytes(pc, n)) ||
      overlap(acc, na, s_w, sw_bytes(pc, n)))
    return fail(CONVROT_E_INVALID_ARG, "%s: overlapping buffers", fn);
  if (m == 0) return ok();
  return hip_status(launch_gemm_tile(xq, s_x, wq, s_w, pc, bias, m, n, k, y, acc, tile, dt,
                                     (hipStream_t)stream),
                    fn);
}

convrot_status convrot_gemm_int8(const int8_t* xq, const float* s_x, const int8_t* wq,
                                 const float* s_w, const uint16_t* bias, int64_t m, int64_t n,
                                 int64_t k, uint16_t* y, int32_t* acc, void* stream) {
  return gemm_impl("convrot_gemm_int8", false, DType::kBF16, xq, s_x, wq, s_w, bias, m, n, k, y, acc, 0,
                   stream);
}

convrot_status convrot_gemm_int8_per_channel(const int8_t* xq, const float* s_x,
                                             const int8_t* wq, const float* s_w,
                                             const uint16_t* bias, int64_t m, int64_t n,
                                             int64_t k, uint16_t* y, int32_t* acc,
                                             void* stream) {
  return gemm_impl("convrot_gemm_int8_per_channel", true, DType::kBF16, xq, s_x, wq, s_w, bias, m, n, k, y, acc,
                   0, stream);
}

convrot_status convrot_gemm_int8_tile(const int8_t* xq, const float* s_x, const int8_t* wq,
                                      const float* s_w, const uint16_t* bias, int64_t m,
                                      int64_t n, int64_t k, uint16_t* y, int32_t* acc, int tile,
                                      void* stream) {
  return gemm_impl("convrot_gemm_int8_tile", false, DType::kBF16, xq, s_x, wq, s_w, bias, m, n, k, y, acc, tile,
                   stream);
}

convrot_status convrot_gemm_int8_per_channel_tile(const int8_t* xq, const float* s_x,
                                                  const int8_t* wq, const float* s_w,
                                                  const uint16_t* bias, int64_t m, int64_t n,
                                                  int64_t k, uint16_t* y, int32_t* acc, int tile,
                                                  void* stream) {
  return gemm_impl("convrot_gemm_int8_per_channel_tile", true, DType::kBF16, xq, s_x, wq, s_w, bias,
                   m, n, k, y, acc, tile, stream);
}

convrot_status convrot_gemm_int8_ex(const int8_t* xq, const float* s_x, const int8_t* wq,
                                    const float* s_w, convrot_scale_mode scale_mode,
                                    const void* bias, int64_t m, int64_t n, int64_t k, void* y,
                                    int32_t* acc, convrot_dtype dtype, int tile, void* stream) {
  const char* fn = "convrot_gemm_int8_ex";
  bool pc;
  DType dt;
  if (!scale_mode_of(scale_mode, &pc) || !dtype_of(dtype, &dt))
    return fail(CONVROT_E_INVALID_ARG, "%s: scale_mode=%d dtype=%d", fn, (int)scale_mode,
                (int)dtype);
  return gemm_impl(fn, pc, dt, xq, s_x, wq, s_w, static_cast<const uint16_t*>(bias), m, n, k,
                   static_cast<uint16_t*>(y), acc, tile, stream);
}

size_t convrot_linear_int8_workspace_for_rows(int64_t rows, int64_t k) {
  if (rows <= 0 || k <= 0) return 0;
  return align_up((size_t)(rows * k), 256) + (size_t)rows * 4;
}

size_t convrot_linear_int8_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n <= 0 || k <= 0) return 0;
  int64_t rows = m < 2 * n ? m : 2 * n;
  if (rows < 1) rows = 1;
  return convrot_linear_int8_workspace_for_rows(rows, k);
}

// Argument checks of the int8_compute forward; on success *slice holds the
// token rows per slice (0 when m == 0: nothing to do).
static convrot_status linear_check(const char* fn, bool pc, const uint16_t* x, const int8_t* wq,
                                   const float* s_w, const uint16_t* bias, int64_t m, int64_t n,
                                   int64_t k, int g, const uint16_t* y, const void* workspace,
                                   size_t workspace_bytes, int64_t* slice) {
  *slice = 0;
  if (!wq || !s_w) return fail(CONVROT_E_INVALID_ARG, "%s: null pointer", fn);
  if (convrot_status s = check_rot(fn, m, k, g)) return s;
  if (convrot_status s = check_gemm(fn, m, n, k)) return s;
  if (m == 0) return ok();  // the M-sized buffers may be null
  if (!x || !y || !workspace) return fail(CONVROT_E_INVALID_ARG, "%s: null pointer", fn);
  if (!aligned(x, 16) || !aligned(wq, 16) || !sw_aligned(pc, s_w) || !aligned(y, 16) ||
      (bias && !aligned(bias, 8)) || !aligned(workspace, 256))
    return fail(CONVROT_E_MISALIGNED, "%s: misaligned pointer", fn);
  // largest slice that fits: align256(r*k) + 4r <= bytes
  int64_t rows_fit = (int64_t)(workspace_bytes / (size_t)(k + 4));
  while (rows_fit > 0 && convrot_linear_int8_workspace_for_rows(rows_fit, k) > workspace_bytes)
    --rows_fit;
  if (rows_fit < 1)
    return fail(CONVROT_E_WORKSPACE, "%s: %zu bytes hold no row (need %zu)", fn, workspace_bytes,
                convrot_linear_int8_workspace_for_rows(1, k));
  const size_t ny = (size_t)(m * n) * 2;
  if (overlap(y, ny, x, (size_t)(m * k) * 2) || overlap(y, ny, wq, (size_t)(n * k)) ||
      overlap(y, ny, workspace, workspace_bytes) ||
      overlap(workspace, workspace_bytes, x, (size_t)(m * k) * 2) ||
      overlap(workspace, workspace_bytes, wq, (size_t)(n * k)) ||
      overlap(y, ny, s_w, sw_bytes(pc, n)) || overlap(workspace, workspace_bytes, s_w, sw_bytes(pc, n)))
    return fail(CONVROT_E_INVALID_ARG, "%s: overlapping buffers", fn);
  // whole GEMM tiles per slice when the workspace allows
  *slice = rows_fit < m ? rows_fit : m;
  if (*slice < m && *slice >= 256) *slice -= *slice % 256;
  return ok();
}

// Launches of the int8_compute forward (arguments already checked); tile 0
// lets the GEMM choose its block tile.
static convrot_status linear_run(const char* fn, bool pc, DType dt, const uint16_t* x,
                                 const int8_t* wq, const float* s_w, const uint16_t* bias,
                                 int64_t m, int64_t n, int64_t k, int g, uint64_t rot_seed,
                                 uint16_t* y, void* workspace, int64_t slice, void* stream,
                                 int tile = 0) {
  const SignMask sm = make_signs(rot_seed, g);
  int8_t* xq = static_cast<int8_t*>(workspace);
  float* sx = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                       align_up((size_t)(slice * k), 256));
  hipStream_t st = (hipStream_t)stream;
  for (int64_t r0 = 0; r0 < m; r0 += slice) {
    const int64_t rows = (m - r0) < slice ? (m - r0) : slice;
    hipError_t e = launch_quantize_rows(x + r0 * k, xq, sx, rows, (int)k, g, sm, dt, st);
    if (e != hipSuccess) return hip_status(e, fn);
    e = launch_gemm_tile(xq, sx, wq, s_w, pc, bias, rows, n, k, y + r0 * n, nullptr, tile, dt,
                         st);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  return ok();
}

static convrot_status linear_impl(const char* fn, bool pc, DType dt, const uint16_t* x,
                                  const int8_t* wq, const float* s_w, const uint16_t* bias,
                                  int64_t m, int64_t n, int64_t k, int g, uint64_t rot_seed,
                                  uint16_t* y, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  int64_t slice;
  if (convrot_status s = linear_check(fn, pc, x, wq, s_w, bias, m, n, k, g, y, workspace,
                                      workspace_bytes, &slice))
    return s;
  if (slice == 0) return ok();
  return linear_run(fn, pc, dt, x, wq, s_w, bias, m, n, k, g, rot_seed, y, workspace, slice,
                    stream);
}

convrot_status convrot_linear_int8(const uint16_t* x, const int8_t* wq, const float* s_w,
                                   const uint16_t* bias, int64_t m, int64_t n, int64_t k, int g,
                                   uint64_t rot_seed, uint16_t* y, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return linear_impl("convrot_linear_int8", false, DType::kBF16, x, wq, s_w, bias, m, n, k, g, rot_seed, y,
                     workspace, workspace_bytes, stream);
}

convrot_status convrot_linear_int8_per_channel(const uint16_t* x, const int8_t* wq,
                                               const float* s_w, const uint16_t* bias, int64_t m,
                                               int64_t n, int64_t k, int g, uint64_t rot_seed,
                                               uint16_t* y, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  return linear_impl("convrot_linear_int8_per_channel", true, DType::kBF16, x, wq, s_w, bias, m, n,
                     k, g, rot_seed, y, workspace, workspace_bytes, stream);
}

convrot_status convrot_linear_int8_ex(const void* x, const int8_t* wq, const float* s_w,
                                      convrot_scale_mode scale_mode, const void* bias, int64_t m,
                                      int64_t n, int64_t k, int g, uint64_t rot_seed, void* y,
                                      convrot_dtype dtype, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  const char* fn = "convrot_linear_int8_ex";
  bool pc;
  DType dt;
  if (!scale_mode_of(scale_mode, &pc) || !dtype_of(dtype, &dt))
    return fail(CONVROT_E_INVALID_ARG, "%s: scale_mode=%d dtype=%d", fn, (int)scale_mode,
                (int)dtype);
  return linear_impl(fn, pc, dt, static_cast<const uint16_t*>(x), wq, s_w,
                     static_cast<const uint16_t*>(bias), m, n, k, g, rot_seed,
                     static_cast<uint16_t*>(y), workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// The int8 forward for callers that cannot allocate: the token slices go
// through a file-scope device array instead of a caller workspace.
// ---------------------------------------------------------------------------

}  // extern "C"

// One slice of int8 activations and their fp32 scales (the workspace layout
// of convrot_linear_int8). Each device holds its own copy of the array from
// the library's load to the end of the process.
static constexpr size_t kScratchBytes = (size_t)CONVROT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// The array's device address per device (the host-side name of a __device__
// variable is only a stand-in), resolved once with that device current.
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

convrot_status scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CONVROT_E_INVALID_ARG, "%s: device %d beyond the %d supported", fn, dev,
                kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e, fn);
      if (!p || !aligned(p, 256))
        return fail(CONVROT_E_HIP, "%s: scratch address %p unusable", fn, p);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return CONVROT_OK;
}

}  // namespace

extern "C" {

convrot_status convrot_linear_int8_noalloc(const void* x, const int8_t* wq, const float* s_w,
                                           convrot_scale_mode scale_mode, const void* bias,
                                           int64_t m, int64_t n, int64_t k, int g,
                                           uint64_t rot_seed, void* y, convrot_dtype dtype,
                                           void* stream) {
  const char* fn = "convrot_linear_int8_noalloc";
  bool pc;
  DType dt;
  if (!scale_mode_of(scale_mode, &pc) || !dtype_of(dtype, &dt))
    return fail(CONVROT_E_INVALID_ARG, "%s: scale_mode=%d dtype=%d", fn, (int)scale_mode,
                (int)dtype);
  // a token row of k int8 plus its scale must fit (always so for k <= 16384)
  if (k > 0 && convrot_linear_int8_workspace_for_rows(1, k) > kScratchBytes)
    return fail(CONVROT_E_WORKSPACE, "%s: a row of k=%lld does not fit the %zu-byte scratch", fn,
                (long long)k, kScratchBytes);
  // argument checks first (nothing touches HIP when they fail); a stand-in
  // address of the right alignment lets linear_check size the slices
  int64_t slice;
  if (convrot_status st = linear_check(fn, pc, static_cast<const uint16_t*>(x), wq, s_w,
                                       static_cast<const uint16_t*>(bias), m, n, k, g,
                                       static_cast<const uint16_t*>(y),
                                       reinterpret_cast<void*>((uintptr_t)256), kScratchBytes,
                                       &slice))
    return st;
  if (slice == 0) return ok();
  void* ws = nullptr;
  if (convrot_status st = scratch_address(fn, &ws)) return st;
  // the real scratch may not overlap the caller's tensors (it never does:
  // it is the library's own memory), but check as for a workspace
  const size_t ny = (size_t)(m * n) * 2;
  if (overlap(ws, kScratchBytes, y, ny) || overlap(ws, kScratchBytes, x, (size_t)(m * k) * 2))
    return fail(CONVROT_E_INVALID_ARG, "%s: buffers overlap the scratch", fn);
  return linear_run(fn, pc, dt, static_cast<const uint16_t*>(x), wq, s_w,
                    static_cast<const uint16_t*>(bias), m, n, k, g, rot_seed,
                    static_cast<uint16_t*>(y), ws, slice, stream);
}

// ---------------------------------------------------------------------------
// Host-streamed int8 layers: a ring of device staging slots. Each call copies
// one layer's int8 weight into the next slot on the streamer's own copy
// stream, and the forward waits for that copy on the caller's stream; the
// next call's copy waits only for its own slot's previous forward, so the
// copies of later layers overlap the forwards of earlier ones.
// ---------------------------------------------------------------------------

struct convrot_streamer {
  int device;
  size_t slot_bytes;
  int nslots;
  int next;
  void* slot[CONVROT_STREAMER_MAX_SLOTS];
  hipEvent_t ready[CONVROT_STREAMER_MAX_SLOTS];     // the slot's copy is done
  hipEvent_t released[CONVROT_STREAMER_MAX_SLOTS];  // the slot's forward is done
  hipStream_t copy;
};

static void streamer_release(convrot_streamer* s) {
  if (s->copy) (void)hipStreamSynchronize(s->copy);
  for (int i = 0; i < s->nslots; ++i) {
    if (s->released[i]) (void)hipEventSynchronize(s->released[i]);
    if (s->slot[i]) (void)hipFree(s->slot[i]);
    if (s->ready[i]) (void)hipEventDestroy(s->ready[i]);
    if (s->released[i]) (void)hipEventDestroy(s->released[i]);
  }
  if (s->copy) (void)hipStreamDestroy(s->copy);
  delete s;
}

convrot_status convrot_streamer_create(size_t slot_bytes, int slots, convrot_streamer** out) {
  const char* fn = "convrot_streamer_create";
  if (!out) return fail(CONVROT_E_INVALID_ARG, "%s: null output", fn);
  *out = nullptr;
  if (slots < 1 || slots > CONVROT_STREAMER_MAX_SLOTS || slot_bytes == 0)
    return fail(CONVROT_E_INVALID_ARG, "%s: slots=%d (1..%d), slot_bytes=%zu", fn, slots,
                CONVROT_STREAMER_MAX_SLOTS, slot_bytes);
  convrot_streamer* s = new convrot_streamer();
  s->slot_bytes = slot_bytes;
  s->nslots = slots;
  hipError_t e = hipGetDevice(&s->device);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&s->copy, hipStreamNonBlocking);
  for (int i = 0; i < slots && e == hipSuccess; ++i) {
    e = hipMalloc(&s->slot[i], align_up(slot_bytes, 256));
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s->ready[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s->released[i], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    streamer_release(s);
    return hip_status(e, fn);
  }
  *out = s;
  return ok();
}

convrot_status convrot_streamer_destroy(convrot_streamer* s) {
  if (!s) return fail(CONVROT_E_INVALID_ARG, "convrot_streamer_destroy: null streamer");
  streamer_release(s);
  return ok();
}

convrot_status convrot_streamer_linear_int8(convrot_streamer* s, const void* x, convrot_dtype dtype,
                                            const int8_t* wq_host, const float* s_w,
                                            convrot_scale_mode scale_mode, const void* bias,
                                            int64_t m, int64_t n, int64_t k, int g,
                                            uint64_t rot_seed, void* y, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  const char* fn = "convrot_streamer_linear_int8";
  bool pc;
  DType dt;
  if (!s) return fail(CONVROT_E_INVALID_ARG, "%s: null streamer", fn);
  if (!scale_mode_of(scale_mode, &pc) || !dtype_of(dtype, &dt))
    return fail(CONVROT_E_INVALID_ARG, "%s: scale_mode=%d dtype=%d", fn, (int)scale_mode,
                (int)dtype);
  if (!wq_host) return fail(CONVROT_E_INVALID_ARG, "%s: null weight", fn);
  if (n > 0 && k > 0 && (size_t)n * (size_t)k > s->slot_bytes)
    return fail(CONVROT_E_WORKSPACE, "%s: weight of %lld bytes exceeds the %zu-byte slots", fn,
                (long long)(n * k), s->slot_bytes);
  const int i = s->next;
  const int8_t* wq = static_cast<const int8_t*>(s->slot[i]);
  int64_t slice;
  if (convrot_status st = linear_check(fn, pc, static_cast<const uint16_t*>(x), wq, s_w,
                                       static_cast<const uint16_t*>(bias), m, n, k, g,
                                       static_cast<const uint16_t*>(y), workspace,
                                       workspace_bytes, &slice))
    return st;
  if (slice == 0) return ok();
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev != s->device)
    return fail(CONVROT_E_INVALID_ARG, "%s: current device %d, streamer made on device %d", fn,
                dev, s->device);
  hipStream_t st = (hipStream_t)stream;
  e = hipStreamWaitEvent(s->copy, s->released[i], 0);
  if (e == hipSuccess)
    e = hipMemcpyAsync(s->slot[i], wq_host, (size_t)(n * k), hipMemcpyDefault, s->copy);
  if (e == hipSuccess) e = hipEventRecord(s->ready[i], s->copy);
  if (e == hipSuccess) e = hipStreamWaitEvent(st, s->ready[i], 0);
  if (e != hipSuccess) return hip_status(e, fn);
  s->next = (i + 1) % s->nslots;
  if (convrot_status r = linear_run(fn, pc, dt, static_cast<const uint16_t*>(x), wq, s_w,
                                    static_cast<const uint16_t*>(bias), m, n, k, g, rot_seed,
                                    static_cast<uint16_t*>(y), workspace, slice, stream))
    return r;
  return hip_status(hipEventRecord(s->released[i], st), fn);
}

// ---------------------------------------------------------------------------
// Sessions: first-call tile tuning and check against the default path.
// ---------------------------------------------------------------------------

namespace {

// One device buffer per session: written whole before each timed tile run
// (256 MB, the MI355X MALL), then reused for the check.
constexpr size_t kSessionScratch = (size_t)256 << 20;
constexpr int kCheckRows = 256;
constexpr size_t kPartialBytes = (size_t)kCheckRows * 2 * sizeof(double);

struct SessionEntry {
  int tile;
  double err;
};

using SessionKey = std::tuple<int64_t, int64_t, int, int, int, int>;

int token_bucket(int64_t m) {
  int b = 0;
  while (b < 62 && ((int64_t)1 << b) < m) ++b;
  return b;  // ceil(log2 m)
}

// Weight rows per check chunk: partial sums, y_ref [kCheckRows, nc] fp32 and
// W_hat [nc, k] in 16-bit must fit the session buffer; a multiple of 64
// (k <= 16384 gives nc >= 7936).
int64_t check_chunk_rows(int64_t n, int64_t k) {
  int64_t nc = (int64_t)((kSessionScratch - kPartialBytes - 256) /
                         (size_t)(2 * k + 4 * kCheckRows)) / 64 * 64;
  return nc < n ? nc : n;
}

}  // namespace

struct convrot_session {
  int device = -1;
  double tol = 0.1;
  bool latched = false;
  std::string latch_reason;
  std::map<SessionKey, SessionEntry> entries;
  std::map<SessionKey, int> preset;  // imported tiles for keys without a first call
  std::mutex mu;
  void* scratch = nullptr;  // kSessionScratch bytes on `device`
  hipEvent_t e0 = nullptr, e1 = nullptr;
  double host[2 * kCheckRows];
  ~convrot_session() {
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (scratch) (void)hipFree(scratch);
  }
};

convrot_status convrot_session_create(double check_tolerance, convrot_session** out) {
  const char* fn = "convrot_session_create";
  if (!out) return fail(CONVROT_E_INVALID_ARG, "%s: null output", fn);
  *out = nullptr;
  if (std::isnan(check_tolerance))
    return fail(CONVROT_E_INVALID_ARG, "%s: tolerance is NaN", fn);
  convrot_session* s = new convrot_session();
  s->tol = check_tolerance > 0 ? check_tolerance : 0.1;
  hipError_t e = hipGetDevice(&s->device);
  if (e == hipSuccess) e = hipMalloc(&s->scratch, kSessionScratch);
  if (e == hipSuccess) e = hipEventCreate(&s->e0);
  if (e == hipSuccess) e = hipEventCreate(&s->e1);
  if (e != hipSuccess) {
    delete s;
    return hip_status(e, fn);
  }
  *out = s;
  return ok();
}

convrot_status convrot_session_destroy(convrot_session* s) {
  if (!s) return fail(CONVROT_E_INVALID_ARG, "convrot_session_destroy: null session");
  delete s;
  return ok();
}

// The first call for a key: tune, run, check, in the session's buffer and
// events (nothing allocated). Returns the status; on success *entry holds the
// kept tile and the check's error.
static convrot_status session_first_call(const char* fn, convrot_session* s, bool pc, DType dt,
                                         const uint16_t* x, const int8_t* wq, const float* s_w,
                                         const uint16_t* bias, int64_t m, int64_t n, int64_t k,
                                         int g, uint64_t rot_seed, uint16_t* y, void* workspace,
                                         int64_t slice, hipStream_t st, int preset_tile,
                                         SessionEntry* entry) {
  const SignMask sm = make_signs(rot_seed, g);
  int8_t* xq = static_cast<int8_t*>(workspace);
  float* sx = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                       align_up((size_t)(slice * k), 256));
  const int64_t rows0 = slice < m ? slice : m;
  hipError_t e = hipSuccess;
  // 1. time every tile that exists for k on the first slice, caches flushed
  // (an imported tile skips this)
  int best = preset_tile;
  float best_ms = 0.0f;
  if (best == 0) e = launch_quantize_rows(x, xq, sx, rows0, (int)k, g, sm, dt, st);
  const int cands[] = {384, 256, 192, 128};
  for (int c : cands) {
    if (preset_tile != 0) break;
    if (e != hipSuccess) break;
    if (c == 384 && k % 128 != 0) continue;
    for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {
      e = launch_flush(s->scratch, kSessionScratch, st);
      if (e == hipSuccess) e = hipEventRecord(s->e0, st);
      if (e == hipSuccess)
        e = launch_gemm_tile(xq, sx, wq, s_w, pc, bias, rows0, n, k, y, nullptr, c, dt, st);
      if (e == hipSuccess) e = hipEventRecord(s->e1, st);
      if (e == hipSuccess) e = hipEventSynchronize(s->e1);
      float ms = 0.0f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, s->e0, s->e1);
      if (e == hipSuccess && (best == 0 || ms < best_ms)) {
        best = c;
        best_ms = ms;
      }
    }
  }
  if (e != hipSuccess) return hip_status(e, fn);
  // 2. the forward with the kept tile
  if (convrot_status r = linear_run(fn, pc, dt, x, wq, s_w, bias, m, n, k, g, rot_seed, y,
                                    workspace, slice, st, best))
    return r;
  // 3. the check against the default path on the first rows, over chunks of
  // weight rows: W_hat of the chunk, then y_ref of its columns
  const int rows = (int)(m < kCheckRows ? m : kCheckRows);
  const int64_t nc = check_chunk_rows(n, k);
  uint8_t* buf = static_cast<uint8_t*>(s->scratch);
  double* partial = reinterpret_cast<double*>(buf);
  float* y_ref = reinterpret_cast<float*>(buf + align_up(kPartialBytes, 256));
  uint16_t* w_hat = reinterpret_cast<uint16_t*>(
      buf + align_up(kPartialBytes, 256) + align_up((size_t)kCheckRows * (size_t)nc * 4, 256));
  for (int64_t n0 = 0; n0 < n && e == hipSuccess; n0 += nc) {
    const int64_t nn = n - n0 < nc ? n - n0 : nc;
    e = launch_dequant(wq + n0 * k, pc ? s_w + n0 : s_w, pc, nn, k, g, sm, w_hat, dt, st);
    if (e == hipSuccess)
      e = launch_check_rows(x, w_hat, bias ? bias + n0 : nullptr, y + n0, n, rows, (int)nn,
                            (int)k, dt, n0 > 0, y_ref, partial, st);
  }
  if (e == hipSuccess)
    e = hipMemcpyAsync(s->host, partial, (size_t)rows * 2 * sizeof(double),
                       hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_status(e, fn);
  double d2 = 0.0, r2 = 0.0;
  for (int r = 0; r < rows; ++r) {
    d2 += s->host[2 * r];
    r2 += s->host[2 * r + 1];
  }
  entry->tile = best;
  entry->err = r2 > 0.0 ? std::sqrt(d2 / r2) : (d2 == 0.0 ? 0.0 : INFINITY);
  return ok();
}

convrot_status convrot_session_linear_int8(convrot_session* s, const void* x, convrot_dtype dtype,
                                           const int8_t* wq, const float* s_w,
                                           convrot_scale_mode scale_mode, const void* bias,
                                           int64_t m, int64_t n, int64_t k, int g,
                                           uint64_t rot_seed, void* y, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  const char* fn = "convrot_session_linear_int8";
  bool pc;
  DType dt;
  if (!s) return fail(CONVROT_E_INVALID_ARG, "%s: null session", fn);
  if (!scale_mode_of(scale_mode, &pc) || !dtype_of(dtype, &dt))
    return fail(CONVROT_E_INVALID_ARG, "%s: scale_mode=%d dtype=%d", fn, (int)scale_mode,
                (int)dtype);
  std::lock_guard<std::mutex> lock(s->mu);
  if (s->latched)
    return fail(CONVROT_E_SELFCHECK, "%s: latched (%s); use the default path", fn,
                s->latch_reason.c_str());
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* bb = static_cast<const uint16_t*>(bias);
  uint16_t* yb = static_cast<uint16_t*>(y);
  int64_t slice;
  if (convrot_status st = linear_check(fn, pc, xb, wq, s_w, bb, m, n, k, g, yb, workspace,
                                       workspace_bytes, &slice))
    return st;
  if (slice == 0) return ok();
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev != s->device)
    return fail(CONVROT_E_INVALID_ARG, "%s: current device %d, session made on device %d", fn,
                dev, s->device);
  const SessionKey key{n, k, token_bucket(m), g, (int)dt, pc ? 1 : 0};
  auto it = s->entries.find(key);
  if (it != s->entries.end())
    return linear_run(fn, pc, dt, xb, wq, s_w, bb, m, n, k, g, rot_seed, yb, workspace, slice,
                      stream, it->second.tile);
  SessionEntry entry{0, 0.0};
  const auto pre = s->preset.find(key);
  const int preset_tile = pre != s->preset.end() ? pre->second : 0;
  const convrot_status r = session_first_call(fn, s, pc, dt, xb, wq, s_w, bb, m, n, k, g, rot_seed,
                                              yb, workspace, slice, (hipStream_t)stream,
                                              preset_tile, &entry);
  char why[256];
  if (r != CONVROT_OK) {
    snprintf(why, sizeof why, "first call for n=%lld k=%lld failed: %s", (long long)n,
             (long long)k, g_last_error);
    s->latched = true;
    s->latch_reason = why;
    return fail(CONVROT_E_SELFCHECK, "%s: %s", fn, why);
  }
  s->entries[key] = entry;
  if (pre != s->preset.end()) s->preset.erase(pre);
  if (!(entry.err <= s->tol)) {
    snprintf(why, sizeof why,
             "first result for n=%lld k=%lld (token bucket 2^%d) is %.4g away from the default "
             "path, tolerance %.4g",
             (long long)n, (long long)k, token_bucket(m), entry.err, s->tol);
    s->latched = true;
    s->latch_reason = why;
    return fail(CONVROT_E_SELFCHECK, "%s: %s", fn, why);
  }
  return ok();
}

convrot_status convrot_session_lookup(convrot_session* s, int64_t m, int64_t n, int64_t k, int g,
                                      convrot_dtype dtype, convrot_scale_mode scale_mode,
                                      int* tile, double* check_error, int* latched) {
  const char* fn = "convrot_session_lookup";
  bool pc;
  DType dt;
  if (!s) return fail(CONVROT_E_INVALID_ARG, "%s: null session", fn);
  if (!scale_mode_of(scale_mode, &pc) || !dtype_of(dtype, &dt))
    return fail(CONVROT_E_INVALID_ARG, "%s: scale_mode=%d dtype=%d", fn, (int)scale_mode,
                (int)dtype);
  std::lock_guard<std::mutex> lock(s->mu);
  if (latched) *latched = s->latched ? 1 : 0;
  auto it = s->entries.find(SessionKey{n, k, token_bucket(m), g, (int)dt, pc ? 1 : 0});
  if (it == s->entries.end()) return fail(CONVROT_E_INVALID_ARG, "%s: no first call yet", fn);
  if (tile) *tile = it->second.tile;
  if (check_error) *check_error = it->second.err;
  return ok();
}

static const char kTilesHeader[] = "convrot-session-tiles 1";

size_t convrot_session_export(convrot_session* s, char* buf, size_t buf_bytes) {
  if (!s) {
    (void)fail(CONVROT_E_INVALID_ARG, "convrot_session_export: null session");
    return 0;
  }
  std::string text = std::string(kTilesHeader) + "\n";
  {
    std::lock_guard<std::mutex> lock(s->mu);
    std::map<SessionKey, int> all(s->preset);
    for (const auto& kv : s->entries) all[kv.first] = kv.second.tile;
    char line[160];
    for (const auto& kv : all) {
      const SessionKey& key = kv.first;
      snprintf(line, sizeof line, "%lld %lld %d %d %d %d %d\n", (long long)std::get<0>(key),
               (long long)std::get<1>(key), std::get<2>(key), std::get<3>(key), std::get<4>(key),
               std::get<5>(key), kv.second);
      text += line;
    }
  }
  if (buf_bytes > 0 && buf) {
    const size_t len = text.size() < buf_bytes - 1 ? text.size() : buf_bytes - 1;
    memcpy(buf, text.data(), len);
    buf[len] = '\0';
  }
  return text.size() + 1;
}

convrot_status convrot_session_import(convrot_session* s, const char* text) {
  const char* fn = "convrot_session_import";
  if (!s || !text) return fail(CONVROT_E_INVALID_ARG, "%s: null argument", fn);
  std::map<SessionKey, int> got;
  int lineno = 0;
  const char* p = text;
  while (*p) {
    const char* eol = strchr(p, '\n');
    const size_t len = eol ? (size_t)(eol - p) : strlen(p);
    std::string line(p, len);
    p += len + (eol ? 1 : 0);
    ++lineno;
    if (!line.empty() && line.back() == '\r') line.pop_back();
    if (lineno == 1) {
      if (line != kTilesHeader)
        return fail(CONVROT_E_INVALID_ARG, "%s: line 1 is not \"%s\"", fn, kTilesHeader);
      continue;
    }
    if (line.empty()) continue;
    long long n = 0, k = 0;
    int bucket = 0, g = 0, dtype = 0, mode = 0, tile = 0, used = 0;
    const int got_fields = sscanf(line.c_str(), "%lld %lld %d %d %d %d %d %n", &n, &k, &bucket,
                                  &g, &dtype, &mode, &tile, &used);
    DType dt;
    bool pc;
    const bool ok_line =
        got_fields == 7 && used == (int)line.size() && n >= 16 && n % 16 == 0 && k >= 64 &&
        k % 64 == 0 && k <= kMaxRotK && (g == 4 || g == 16 || g == 64 || g == 256) &&
        k % g == 0 && bucket >= 0 && bucket <= 62 && dtype_of(dtype, &dt) &&
        scale_mode_of(mode, &pc) &&
        (tile == 128 || tile == 192 || tile == 256 || (tile == 384 && k % 128 == 0));
    if (!ok_line) return fail(CONVROT_E_INVALID_ARG, "%s: line %d is not a valid entry", fn, lineno);
    got[SessionKey{(int64_t)n, (int64_t)k, bucket, g, (int)dt, pc ? 1 : 0}] = tile;
  }
  if (lineno == 0) return fail(CONVROT_E_INVALID_ARG, "%s: empty text", fn);
  std::lock_guard<std::mutex> lock(s->mu);
  for (const auto& kv : got)
    if (s->entries.find(kv.first) == s->entries.end()) s->preset[kv.first] = kv.second;
  return ok();
}

}  // extern "C"

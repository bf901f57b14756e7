/* Compile-and-link check of include/convrot.h from plain C99: every entry
 * point is referenced with arguments of the declared types. Nothing here is
 * executed. */
#include <stddef.h>
#include <stdint.h>

#include "convrot.h"

int convrot_header_c99_check(void* p, int i) {
  convrot_status s = CONVROT_OK;
  convrot_streamer* st = NULL;
  convrot_session* se = NULL;
  const uint16_t* x = (const uint16_t*)p;
  int8_t* q = (int8_t*)p;
  float* f = (float*)p;
  int32_t* a = (int32_t*)p;
  uint16_t* y = (uint16_t*)p;
  int tile = 0, latched = 0;
  double err = 0.0;
  if (i == 1) {
    s = convrot_quantize_weights(x, 1, 64, 4, 1u, q, f, p);
    s = convrot_quantize_weights_per_channel(x, 1, 64, 4, 1u, q, f, p);
    s = convrot_dequant_derotate(q, f, 1, 64, 4, 1u, y, p);
    s = convrot_dequant_derotate_per_channel(q, f, 1, 64, 4, 1u, y, p);
    s = convrot_quantize_activations(x, 1, 64, 4, 1u, q, f, p);
    s = convrot_quantize_activations_exact(x, 1, 64, 4, 1u, q, f, p);
    s = convrot_gemm_int8(q, f, q, f, x, 1, 16, 64, y, a, p);
    s = convrot_gemm_int8_tile(q, f, q, f, x, 1, 16, 64, y, a, 128, p);
    s = convrot_gemm_int8_per_channel(q, f, q, f, x, 1, 16, 64, y, a, p);
    s = convrot_gemm_int8_per_channel_tile(q, f, q, f, x, 1, 16, 64, y, a, 192, p);
    s = convrot_linear_int8(x, q, f, x, 1, 16, 64, 4, 1u, y, p, 64, p);
    s = convrot_linear_int8_per_channel(x, q, f, x, 1, 16, 64, 4, 1u, y, p, 64, p);
    s = convrot_quantize_activations_ex(p, CONVROT_DTYPE_F16, 1, 64, 4, 1u, q, f, p);
    s = convrot_dequant_derotate_ex(q, f, CONVROT_SCALE_PER_CHANNEL, 1, 64, 4, 1u, p,
                                    CONVROT_DTYPE_BF16, p);
    s = convrot_gemm_int8_ex(q, f, q, f, CONVROT_SCALE_PER_TENSOR, p, 1, 16, 64, p, a,
                             CONVROT_DTYPE_F16, 0, p);
    s = convrot_linear_int8_ex(p, q, f, CONVROT_SCALE_PER_TENSOR, p, 1, 16, 64, 4, 1u, p,
                               CONVROT_DTYPE_BF16, p, 64, p);
    s = convrot_streamer_create((size_t)1 << 20, CONVROT_STREAMER_MAX_SLOTS, &st);
    s = convrot_streamer_linear_int8(st, p, CONVROT_DTYPE_BF16, q, f, CONVROT_SCALE_PER_TENSOR,
                                     p, 1, 16, 64, 4, 1u, p, p, 64, p);
    s = convrot_streamer_destroy(st);
    s = convrot_session_create(0.1, &se);
    s = convrot_session_linear_int8(se, p, CONVROT_DTYPE_F16, q, f, CONVROT_SCALE_PER_CHANNEL, p,
                                    1, 16, 64, 4, 1u, p, p, 64, p);
    s = convrot_session_lookup(se, 1, 16, 64, 4, CONVROT_DTYPE_F16, CONVROT_SCALE_PER_CHANNEL,
                               &tile, &err, &latched);
    {
      char text[256];
      tile += (int)convrot_session_export(se, text, sizeof text);
      s = convrot_session_import(se, text);
    }
    s = convrot_session_destroy(se);
    s = convrot_rotation_signs(1u, 4, q);
    (void)convrot_linear_int8_workspace_for_rows(1, 64);
    (void)convrot_linear_int8_workspace_size(1, 16, 64);
    (void)convrot_status_string(CONVROT_E_SELFCHECK);
    (void)convrot_last_error_string();
    {
      convrot_launch_plan plan;
      s = convrot_plan_launch(CONVROT_KERNEL_GEMM, 1, 16, 64, 4, 256, &plan);
      s = convrot_set_compute_units(0);
      tile += (int)plan.grid + convrot_compute_units();
      s = convrot_linear_int8_noalloc(p, q, f, CONVROT_SCALE_PER_TENSOR, p, 1, 16, 64, 4, 1u, p,
                                      CONVROT_DTYPE_BF16, p);
    }
    {
      convrot_dequant_job job;
      job.wq = q;
      job.s_w = f;
      job.w_out = p;
      job.n = 1;
      job.k = 64;
      s = convrot_dequant_derotate_batched(&job, 1, CONVROT_SCALE_PER_TENSOR, 4, 1u,
                                           CONVROT_DTYPE_BF16, p);
    }
  }
  return (int)s + convrot_abi_version() + (int)CONVROT_ABI_VERSION + tile + latched + (int)err;
}

// Stand-ins for the kernel launchers behind the C ABI, for a host-only build of
// the validation layer (ncattn_api.hip compiled as plain C++ under AddressSanitizer
// and UndefinedBehaviorSanitizer).  Each launcher records what it was asked to
// do and enqueues nothing; driver.cpp checks the records.
#include "stubs.hpp"

#include <string.h>

LaunchRecord g_last;

static void rec(const char *fn, int B, int T, int H, int KV, int D, int window, float scale) {
  g_last.fn = fn;
  g_last.B = B;
  g_last.T = T;
  g_last.H = H;
  g_last.KV = KV;
  g_last.D = D;
  g_last.window = window;
  g_last.scale = scale;
  ++g_last.count;
}

extern "C" const char *hipGetErrorString(hipError_t) { return "stub HIP error"; }

namespace ncattn {

hipError_t launch_qknorm_rope(void *, void *, int B, int T, int H, int KV, int D, const int32_t *, const double *inv,
                              float, float, bool, hipStream_t, float *rstd, long long rstd_stride, int rstd_k_off) {
  rec("qknorm_rope", B, T, H, KV, D, 0, (float)inv[D / 2 - 1]);
  g_last.T_max = rstd ? (int)rstd_stride : -1;  // the 1/r layout, if any
  g_last.stages = rstd ? rstd_k_off : -1;
  return hipSuccess;
}

hipError_t launch_qknorm_rope_bwd(void *, void *, const void *, const void *, int B, int T, int H, int KV, int D,
                                  const int32_t *, const double *inv, float, float, bool, hipStream_t,
                                  const float *rstd, long long rstd_stride, int rstd_k_off) {
  rec("qknorm_rope_bwd", B, T, H, KV, D, 0, (float)inv[D / 2 - 1]);
  g_last.T_max = rstd ? (int)rstd_stride : -1;
  g_last.stages = rstd ? rstd_k_off : -1;
  return hipSuccess;
}

hipError_t launch_fwd_bf16(const void *, const void *, const void *, void *, float *, const AttnShape &sh,
                           hipStream_t) {
  rec("fwd_bf16", sh.B, sh.T, sh.H, sh.KV, sh.D, sh.window, sh.scale);
  return hipSuccess;
}

hipError_t launch_fwd_fp8(const void *, const void *, const void *, float qd, float kd, float vd, void *, float *,
                          const AttnShape &sh, hipStream_t) {
  rec("fwd_fp8", sh.B, sh.T, sh.H, sh.KV, sh.D, sh.window, sh.scale * qd * kd * vd);
  return hipSuccess;
}

hipError_t launch_fwd_bf16_qknorm_rope(void *, const void *, const void *, void *, float *, const AttnShape &sh,
                                       const int32_t *, const double *, float, float, hipStream_t, float *,
                                       long long) {
  rec("fwd_bf16_qknorm_rope", sh.B, sh.T, sh.H, sh.KV, sh.D, sh.window, sh.scale);
  return hipSuccess;
}

hipError_t launch_fwd_bf16_rows(const void *, const void *, const void *, void *, float *, const int32_t *, int B,
                                int Tq, int, int H, int KV, int D, int W, float scale, hipStream_t) {
  rec("fwd_bf16_rows", B, Tq, H, KV, D, W, scale);
  return hipSuccess;
}

hipError_t launch_bwd_bf16(const void *, const void *, const void *, const void *, const float *, const void *,
                           void *, void *, void *, void *, const AttnShape &sh, int stages, hipStream_t) {
  rec("bwd_bf16", sh.B, sh.T, sh.H, sh.KV, sh.D, sh.window, sh.scale);
  g_last.stages = stages;
  return hipSuccess;
}

hipError_t launch_bwd_bf16_qknorm_rope(const void *, const void *, const void *, const void *, const float *,
                                       const void *, const float *, void *, void *, void *, void *,
                                       const AttnShape &sh, const int32_t *, const double *inv, float,
                                       hipStream_t) {
  rec("bwd_bf16_qknorm_rope", sh.B, sh.T, sh.H, sh.KV, sh.D, sh.window, sh.scale);
  g_last.stages = (int)(inv[sh.D / 2 - 1] * 1e9);
  return hipSuccess;
}

hipError_t launch_fwd_f32(const float *, const float *, const float *, float *, float *, const AttnShape &sh,
                          hipStream_t) {
  rec("fwd_f32", sh.B, sh.T, sh.H, sh.KV, sh.D, sh.window, sh.scale);
  return hipSuccess;
}

hipError_t launch_bwd_f32(const float *, const float *, const float *, const float *, const float *, const float *,
                          float *, float *, float *, float *, const AttnShape &sh, int stages, hipStream_t) {
  rec("bwd_f32", sh.B, sh.T, sh.H, sh.KV, sh.D, sh.window, sh.scale);
  g_last.stages = stages;
  return hipSuccess;
}

hipError_t launch_decode_bf16(const void *, const void *, const void *, void *, void *, const int32_t *, void *,
                              float *, int B, int T_max, int H, int KV, int D, int window, float scale, void *ws,
                              hipStream_t) {
  rec("decode_bf16", B, T_max, H, KV, D, window, scale);
  g_last.workspace = ws;
  return hipSuccess;
}

char g_fake_scratch[16];

hipError_t decode_scratch_ptr(void **out) {
  *out = g_fake_scratch;
  return hipSuccess;
}

hipError_t launch_cache_replicate(const void *, const void *, const int32_t *, void *, void *, int32_t *, int N,
                                  int T_src, int T_max, int row_pieces, hipStream_t) {
  rec("cache_replicate", N, T_src, 0, 0, row_pieces, T_max, 0.f);
  return hipSuccess;
}

hipError_t launch_prefill_bf16(const void *, const void *, const void *, void *, void *, const int32_t *, void *,
                               float *, int B, int Tn, int T_max, int H, int KV, int D, int window, float scale,
                               hipStream_t) {
  rec("prefill_bf16", B, Tn, H, KV, D, window, scale);
  g_last.T_max = T_max;
  return hipSuccess;
}

}  // namespace ncattn

void *fake_scratch() { return ncattn::g_fake_scratch; }

// Host-only exercise of the C ABI's validation and sizing under AddressSanitizer
// and UndefinedBehaviorSanitizer: every entry point with invalid arguments, with
// extreme sizes (INT_MAX windows, lengths and counts), and with valid arguments
// that reach the stand-in launchers of stubs.cpp, whose records are checked.
// Nothing here touches a GPU; the pointers are never dereferenced.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ncattn.h"
#include "stubs.hpp"

static int g_checks = 0, g_fail = 0;

#define CHECK(cond)                                                         \
  do {                                                                      \
    ++g_checks;                                                             \
    if (!(cond)) {                                                          \
      ++g_fail;                                                             \
      fprintf(stderr, "FAILED line %d: %s (%s)\n", __LINE__, #cond, ncattn_last_error()); \
    }                                                                       \
  } while (0)

alignas(256) static char g_mem[4096];
static void *P(int i) { return g_mem + 256 * i; }               // distinct, 16-byte aligned
static void *MIS(int i) { return g_mem + 256 * i + 2; }         // misaligned
static float *F(int i) { return (float *)P(i); }

static bool err_ok() {
  const char *e = ncattn_last_error();
  return e != nullptr && strlen(e) > 0 && strlen(e) < 512;
}

static int fwd(void *q, void *k, void *v, void *o, float *lse, int B, int T, int H, int KV, int D, int wl, int wr,
               float sc, int dt) {
  return ncattn_fwd(q, k, v, o, lse, B, T, H, KV, D, wl, wr, sc, dt, nullptr);
}

static void test_fwd() {
  CHECK(fwd(nullptr, P(1), P(2), P(3), F(4), 1, 64, 2, 2, 128, -1, 0, 0, NCATTN_BF16) == NCATTN_EINVAL && err_ok());
  CHECK(fwd(P(0), MIS(1), P(2), P(3), F(4), 1, 64, 2, 2, 128, -1, 0, 0, NCATTN_BF16) == NCATTN_EINVAL && err_ok());
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 0, 64, 2, 2, 128, -1, 0, 0, NCATTN_BF16) == NCATTN_EINVAL);
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 1, INT_MIN, 2, 2, 128, -1, 0, 0, NCATTN_BF16) == NCATTN_EINVAL);
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 1, 64, 6, 4, 128, -1, 0, 0, NCATTN_BF16) == NCATTN_EINVAL);
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 1, 64, 2, 2, 128, INT_MIN, 0, 0, NCATTN_BF16) == NCATTN_EINVAL);
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 1, 64, 2, 2, 128, -1, 1, 0, NCATTN_BF16) == NCATTN_EINVAL);
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 1, 64, 2, 2, 128, -1, 0, 0, 7) == NCATTN_EINVAL);
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 1, 64, 2, 2, 96, -1, 0, 0, NCATTN_BF16) == NCATTN_EUNSUPPORTED);
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 1, 64, 2, 2, 256, -1, 0, 0, NCATTN_F32) == NCATTN_EUNSUPPORTED);
  CHECK(fwd(P(0), P(1), P(2), P(0), F(4), 1, 64, 2, 2, 128, -1, 0, 0, NCATTN_BF16) == NCATTN_EINVAL);
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 1, 64, 2, 2, 128, -1, 0, NAN, NCATTN_BF16) == NCATTN_EINVAL);
  // every size at INT_MAX: refused as too large, no overflow on the way
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, -1, 0, 0, NCATTN_BF16) ==
        NCATTN_EINVAL);
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 1, INT_MAX, 1, 1, 128, -1, 0, 0, NCATTN_BF16) == NCATTN_EUNSUPPORTED);
  // windows reaching every key become -1; the scale resolves to 1 / sqrt(D)
  const int T = 300;
  for (int W : {T - 1, T, T + 1, INT_MAX - 64, INT_MAX}) {
    CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 2, T, 4, 2, 64, W, 0, 0, NCATTN_BF16) == NCATTN_OK);
    CHECK(strcmp(g_last.fn, "fwd_bf16") == 0 && g_last.window == -1 && g_last.D == 64);
  }
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 2, T, 4, 2, 128, T - 2, 0, 0, NCATTN_F32) == NCATTN_OK);
  CHECK(strcmp(g_last.fn, "fwd_f32") == 0 && g_last.window == T - 2);
  CHECK(fabsf(g_last.scale - 1.0f / sqrtf(128.f)) < 1e-7f);
  CHECK(fwd(P(0), P(1), P(2), P(3), F(4), 2, T, 4, 2, 128, 0, 0, 0.25f, NCATTN_BF16) == NCATTN_OK);
  CHECK(g_last.window == 0 && g_last.scale == 0.25f);
}

static int fwd8(void *q, void *k, void *v, float qd, float kd, float vd, void *o, float *lse, int B, int T, int H,
                int KV, int D, int wl, int wr, float sc) {
  return ncattn_fwd_fp8(q, k, v, qd, kd, vd, o, lse, B, T, H, KV, D, wl, wr, sc, nullptr);
}

static void test_fwd_fp8() {
  CHECK(fwd8(nullptr, P(1), P(2), 1, 1, 1, P(3), F(4), 1, 64, 2, 2, 128, -1, 0, 0) == NCATTN_EINVAL && err_ok());
  CHECK(fwd8(P(0), P(1), MIS(2), 1, 1, 1, P(3), F(4), 1, 64, 2, 2, 128, -1, 0, 0) == NCATTN_EINVAL);
  CHECK(fwd8(P(0), P(1), P(2), 1, 1, 1, P(3), F(4), 1, 64, 2, 2, 64, -1, 0, 0) == NCATTN_EUNSUPPORTED);
  CHECK(fwd8(P(0), P(1), P(2), 1, 1, 1, P(3), F(4), 1, 64, 6, 4, 128, -1, 0, 0) == NCATTN_EINVAL);
  CHECK(fwd8(P(0), P(1), P(2), 0.f, 1, 1, P(3), F(4), 1, 64, 2, 2, 128, -1, 0, 0) == NCATTN_EINVAL);
  CHECK(fwd8(P(0), P(1), P(2), 1, -1.f, 1, P(3), F(4), 1, 64, 2, 2, 128, -1, 0, 0) == NCATTN_EINVAL);
  CHECK(fwd8(P(0), P(1), P(2), 1, 1, NAN, P(3), F(4), 1, 64, 2, 2, 128, -1, 0, 0) == NCATTN_EINVAL);
  CHECK(fwd8(P(0), P(1), P(2), 1, 1, INFINITY, P(3), F(4), 1, 64, 2, 2, 128, -1, 0, 0) == NCATTN_EINVAL);
  CHECK(fwd8(P(0), P(1), P(2), 1, 1, 1, P(1), F(4), 1, 64, 2, 2, 128, -1, 0, 0) == NCATTN_EINVAL);
  CHECK(fwd8(P(0), P(1), P(2), 1, 1, 1, P(3), F(4), 1, 64, 2, 2, 128, -1, 1, 0) == NCATTN_EINVAL);
  CHECK(fwd8(P(0), P(1), P(2), 1, 1, 1, P(3), F(4), INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, -1, 0, 0) ==
        NCATTN_EINVAL);
  CHECK(fwd8(P(0), P(1), P(2), 1, 1, 1, P(3), F(4), 1, INT_MAX, 1, 1, 128, -1, 0, 0) == NCATTN_EUNSUPPORTED);
  CHECK(fwd8(P(0), P(1), P(2), 0.5f, 0.25f, 2.f, P(3), F(4), 2, 300, 4, 2, 128, INT_MAX, 0, 0) == NCATTN_OK);
  CHECK(strcmp(g_last.fn, "fwd_fp8") == 0 && g_last.window == -1 && g_last.D == 128);
  CHECK(fabsf(g_last.scale - 0.25f / sqrtf(128.f)) < 1e-7f);
}

static void test_qknorm() {
  double dummy = 0;
  (void)dummy;
  CHECK(ncattn_qknorm_rope(nullptr, P(1), 1, 4, 2, 2, 128, nullptr, 1e5f, 1e-6f, 1.f, 0, nullptr) == NCATTN_EINVAL);
  CHECK(ncattn_qknorm_rope(P(0), P(1), 1, 4, 2, 2, 96, nullptr, 1e5f, 1e-6f, 1.f, 0, nullptr) == NCATTN_EUNSUPPORTED);
  CHECK(ncattn_qknorm_rope(P(0), P(1), 1, 4, 2, 2, 128, nullptr, 1.0f, 1e-6f, 1.f, 0, nullptr) == NCATTN_EINVAL);
  CHECK(ncattn_qknorm_rope(P(0), P(1), 1, 4, 2, 2, 128, nullptr, INFINITY, 1e-6f, 1.f, 0, nullptr) == NCATTN_EINVAL);
  CHECK(ncattn_qknorm_rope(P(0), P(1), 1, 4, 2, 2, 128, nullptr, 1e5f, -1.f, 1.f, 0, nullptr) == NCATTN_EINVAL);
  CHECK(ncattn_qknorm_rope(P(0), P(1), 1, 4, 2, 2, 128, nullptr, 1e5f, 1e-6f, NAN, 0, nullptr) == NCATTN_EINVAL);
  CHECK(ncattn_qknorm_rope(P(0), P(1), 1, 4, 2, 2, 128, (const int32_t *)MIS(2), 1e5f, 1e-6f, 1.f, 0, nullptr) ==
        NCATTN_EINVAL);
  CHECK(ncattn_qknorm_rope(P(0), P(1), INT_MAX, INT_MAX, INT_MAX, 1, 128, nullptr, 1e5f, 1e-6f, 1.f, 0, nullptr) ==
        NCATTN_EINVAL);
  for (int D : {64, 128}) {
    CHECK(ncattn_qknorm_rope(P(0), P(1), 1, 4, 2, 2, D, nullptr, 1e5f, 1e-6f, 1.f, 0, nullptr) == NCATTN_OK);
    // the last frequency base^(-2 (D/2 - 1) / D), recorded by the stand-in
    CHECK(fabs(g_last.scale - pow(1e5, -2.0 * (D / 2 - 1) / D)) < 1e-9);
  }
  CHECK(ncattn_qknorm_rope_bwd(P(0), P(1), P(0), P(3), 1, 4, 2, 2, 128, nullptr, 1e5f, 1e-6f, 1.f, 0, nullptr) ==
        NCATTN_EINVAL);
  CHECK(ncattn_qknorm_rope_bwd(P(0), P(0), P(2), P(3), 1, 4, 2, 2, 128, nullptr, 1e5f, 1e-6f, 1.f, 0, nullptr) ==
        NCATTN_EINVAL);
  CHECK(ncattn_qknorm_rope_bwd(P(0), P(1), P(2), P(3), 1, 4, 2, 2, 64, nullptr, 1e5f, 1e-6f, 1.f, 1, nullptr) ==
        NCATTN_OK);
  CHECK(ncattn_fwd_qknorm_rope(P(0), P(0), P(2), P(3), F(4), nullptr, 1, 4, 2, 2, 128, nullptr, 1e5f, 1e-6f, 1.f,
                               -1, 0, 0, 0, nullptr) == NCATTN_EINVAL);
  CHECK(ncattn_fwd_qknorm_rope(P(0), P(1), P(2), P(3), F(4), (float *)MIS(5), 1, 4, 2, 2, 128, nullptr, 1e5f, 1e-6f,
                               1.f, -1, 0, 0, 0, nullptr) == NCATTN_EINVAL);
  CHECK(ncattn_fwd_qknorm_rope(P(0), P(1), P(2), P(3), F(4), F(5), 1, 40, 2, 2, 64, nullptr, 1e5f, 1e-6f, 1.f,
                               INT_MAX, 0, 0, 0, nullptr) == NCATTN_OK);
  CHECK(strcmp(g_last.fn, "fwd_bf16_qknorm_rope") == 0 && g_last.window == -1);
  // the variant that also stores 1/r per row
  CHECK(ncattn_qknorm_rope_rstd(P(0), P(1), nullptr, 1, 4, 2, 2, 128, nullptr, 1e5f, 1e-6f, 1.f, 0, nullptr) ==
        NCATTN_EINVAL);
  CHECK(ncattn_qknorm_rope_rstd(P(0), P(1), (float *)MIS(2), 1, 4, 2, 2, 128, nullptr, 1e5f, 1e-6f, 1.f, 0,
                                nullptr) == NCATTN_EINVAL);
  CHECK(ncattn_qknorm_rope_rstd(P(0), P(1), F(2), 1, 4, 6, 2, 128, nullptr, 1e5f, 1e-6f, 1.f, 0, nullptr) ==
        NCATTN_OK);
  CHECK(strcmp(g_last.fn, "qknorm_rope") == 0 && g_last.T_max == 8 && g_last.stages == 6);  // stride, k offset
}

static int bwd(int (*f)(const void *, const void *, const void *, const void *, const float *, const void *, void *,
                        void *, void *, int, int, int, int, int, int, int, float, int, void *, size_t, void *),
               int B, int T, int H, int KV, int D, int wl, int dt, void *ws, size_t wsb, void *dq = P(6)) {
  return f(P(0), P(1), P(2), P(3), F(4), P(5), dq, P(7), P(8), B, T, H, KV, D, wl, 0, 0.f, dt, ws, wsb, nullptr);
}

static void test_bwd() {
  const size_t need = ncattn_bwd_workspace_bytes(2, 300, 4, 2, 128, -1, NCATTN_BF16);
  CHECK(need == 2 * (((size_t)2 * 4 * 300 * 4 + 255) / 256 * 256));
  CHECK(ncattn_bwd_workspace_bytes(2, 300, 4, 2, 128, -1, NCATTN_F32) == need / 2);
  CHECK(ncattn_bwd_workspace_bytes(0, 300, 4, 2, 128, -1, NCATTN_BF16) == 0);
  CHECK(ncattn_bwd_workspace_bytes(2, 300, 4, 2, 128, -2, NCATTN_BF16) == 0);
  // absurd shapes: 0 (the calls refuse them), never a wrapped size
  CHECK(ncattn_bwd_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 1, 128, -1, NCATTN_BF16) == 0);
  CHECK(ncattn_bwd_workspace_bytes(1 << 20, 1 << 20, 1 << 10, 1, 128, INT_MAX, NCATTN_BF16) == 0);
  for (int W : {-1, 0, 299, INT_MAX})
    CHECK(ncattn_bwd_workspace_bytes(2, 300, 4, 2, 128, W, NCATTN_BF16) == need);
  CHECK(bwd(ncattn_bwd, 2, 300, 4, 2, 128, -1, NCATTN_BF16, P(9), need - 1) == NCATTN_EWORKSPACE);
  CHECK(bwd(ncattn_bwd, 2, 300, 4, 2, 128, -1, NCATTN_BF16, nullptr, need) == NCATTN_EWORKSPACE);
  CHECK(bwd(ncattn_bwd, 2, 300, 4, 2, 128, -1, NCATTN_BF16, MIS(9), need) == NCATTN_EINVAL);
  CHECK(bwd(ncattn_bwd, 2, 300, 4, 2, 128, -1, NCATTN_BF16, P(9), need, P(0)) == NCATTN_EINVAL);  // dq aliases q
  CHECK(bwd(ncattn_bwd, 2, 300, 4, 2, 128, -1, NCATTN_BF16, P(9), need, P(7)) == NCATTN_EINVAL);  // dq == dk
  CHECK(bwd(ncattn_bwd, 2, 300, 4, 2, 96, -1, NCATTN_BF16, P(9), need) == NCATTN_EUNSUPPORTED);
  CHECK(bwd(ncattn_bwd, INT_MAX, INT_MAX, INT_MAX, 1, 128, -1, NCATTN_BF16, P(9), SIZE_MAX) == NCATTN_EINVAL);
  struct {
    int (*f)(const void *, const void *, const void *, const void *, const float *, const void *, void *, void *,
             void *, int, int, int, int, int, int, int, float, int, void *, size_t, void *);
    int stages;
  } calls[] = {{ncattn_bwd, 7}, {ncattn_bwd_preprocess, 1}, {ncattn_bwd_dkdv, 2}, {ncattn_bwd_dq, 4}};
  for (auto &c : calls) {
    CHECK(bwd(c.f, 2, 300, 4, 2, 64, INT_MAX, NCATTN_BF16, P(9), need) == NCATTN_OK);
    CHECK(strcmp(g_last.fn, "bwd_bf16") == 0 && g_last.stages == c.stages && g_last.window == -1);
  }
  CHECK(bwd(ncattn_bwd, 2, 300, 4, 2, 64, 17, NCATTN_F32, P(9), need) == NCATTN_OK);
  CHECK(strcmp(g_last.fn, "bwd_f32") == 0 && g_last.window == 17);

  // the fused QK-norm + RoPE backward: the backward's checks, the norm's, and
  // no gradient aliasing the raw rows
  auto fb = [&](const void *rs, void *dq, float base, int D, int wl, int dt, void *ws, size_t wsb) {
    return ncattn_bwd_qknorm_rope(P(0), P(1), P(2), P(3), F(4), P(5), (const float *)rs, nullptr, base, 1.f, dq,
                                  P(7), P(8), 2, 300, 4, 2, D, wl, 0, 0.f, dt, ws, wsb, nullptr);
  };
  CHECK(fb(nullptr, P(6), 1e5f, 128, -1, NCATTN_BF16, P(9), need) == NCATTN_EINVAL);
  CHECK(fb(MIS(10), P(6), 1e5f, 128, -1, NCATTN_BF16, P(9), need) == NCATTN_EINVAL);
  CHECK(fb(P(10), P(10), 1e5f, 128, -1, NCATTN_BF16, P(9), need) == NCATTN_EINVAL);   // dq aliases rstd
  CHECK(fb(P(10), P(0), 1e5f, 128, -1, NCATTN_BF16, P(9), need) == NCATTN_EINVAL);    // dq aliases q
  CHECK(fb(P(10), P(6), 0.5f, 128, -1, NCATTN_BF16, P(9), need) == NCATTN_EINVAL);    // rope base
  CHECK(fb(P(10), P(6), 1e5f, 96, -1, NCATTN_BF16, P(9), need) == NCATTN_EUNSUPPORTED);
  CHECK(fb(P(10), P(6), 1e5f, 128, -1, NCATTN_BF16, P(9), need - 1) == NCATTN_EWORKSPACE);
  const long before = g_last.count;
  CHECK(fb(P(10), P(6), 1e5f, 128, -2, NCATTN_BF16, P(9), need) == NCATTN_EINVAL);
  CHECK(g_last.count == before);  // nothing launched on a refusal
  CHECK(fb(P(10), P(6), 1e5f, 64, INT_MAX, NCATTN_BF16, P(9), need) == NCATTN_OK);
  CHECK(strcmp(g_last.fn, "bwd_bf16_qknorm_rope") == 0 && g_last.window == -1 && g_last.D == 64);
  CHECK(g_last.stages == (int)(pow(1e5, -2.0 * 31 / 64) * 1e9));
  CHECK(fb(P(10), P(6), 1e5f, 128, 5, NCATTN_F32, P(9), need) == NCATTN_OK);
  CHECK(strcmp(g_last.fn, "qknorm_rope_bwd") == 0 && g_last.count == before + 3);  // bwd_f32, then the norm's
  CHECK(g_last.T_max == 6 && g_last.stages == 4);  // from y: 1/r with stride n_head + n_kv_head, k rows after q
}

static int dec(bool noalloc, int B, int Tm, int H, int KV, int D, int wl, int dt, void *ws, size_t wsb,
               const void *lens = P(5), void *kc = P(3), void *o = P(6)) {
  if (noalloc)
    return ncattn_decode_noalloc(P(0), P(1), P(2), kc, P(4), (const int32_t *)lens, o, nullptr, B, Tm, H, KV, D, wl,
                                 0.f, dt, nullptr);
  return ncattn_decode(P(0), P(1), P(2), kc, P(4), (const int32_t *)lens, o, nullptr, B, Tm, H, KV, D, wl, 0.f, dt,
                       ws, wsb, nullptr);
}

static void test_decode() {
  const size_t full = ncattn_decode_workspace_bytes(64, 8320, 10, 10, 128, -1);
  const size_t win = ncattn_decode_workspace_bytes(64, 8320, 10, 10, 128, 1024);
  CHECK(full == (size_t)64 * 10 * 65 * 130 * 4 + 256 && win == (size_t)64 * 10 * 9 * 130 * 4 + 256);
  CHECK(ncattn_decode_workspace_bytes(64, 8320, 10, 10, 64, -1) == (size_t)64 * 10 * 65 * 66 * 4 + 256);
  for (int W : {8319, 8320, INT_MAX}) CHECK(ncattn_decode_workspace_bytes(64, 8320, 10, 10, 128, W) == full);
  CHECK(ncattn_decode_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 1, 128, -1) == 0);
  for (bool na : {false, true}) {
    CHECK(dec(na, 4, 512, 2, 2, 128, -1, NCATTN_F32, P(9), full) == NCATTN_EUNSUPPORTED);
    CHECK(dec(na, 4, 512, 2, 2, 96, -1, NCATTN_BF16, P(9), full) == NCATTN_EUNSUPPORTED);
    CHECK(dec(na, 4, 512, 2, 2, 128, -2, NCATTN_BF16, P(9), full) == NCATTN_EINVAL);
    CHECK(dec(na, 4, 512, 2, 2, 128, -1, NCATTN_BF16, P(9), full, MIS(5)) == NCATTN_EINVAL);
    CHECK(dec(na, 4, 512, 2, 2, 128, -1, NCATTN_BF16, P(9), full, nullptr) == NCATTN_EINVAL);
    CHECK(dec(na, 4, 512, 2, 2, 128, -1, NCATTN_BF16, P(9), full, P(5), P(4)) == NCATTN_EINVAL);  // k_cache == v_cache
    CHECK(dec(na, 4, 512, 2, 2, 128, -1, NCATTN_BF16, P(9), full, P(5), P(3), P(0)) == NCATTN_EINVAL);
    CHECK(dec(na, INT_MAX, INT_MAX, INT_MAX, 1, 128, -1, NCATTN_BF16, P(9), SIZE_MAX) == NCATTN_EINVAL);
    CHECK(dec(na, 4, 512, 2, 2, 64, INT_MAX, NCATTN_BF16, P(9), full) == NCATTN_OK);
    CHECK(strcmp(g_last.fn, "decode_bf16") == 0 && g_last.window == -1 && g_last.D == 64);
    CHECK(g_last.workspace == (na ? fake_scratch() : P(9)));
  }
  CHECK(dec(false, 4, 512, 2, 2, 128, -1, NCATTN_BF16, P(9), 0) == NCATTN_EWORKSPACE);
  // the no-alloc scratch boundary: the largest full-causal T_max whose partials fit
  const size_t cap = NCATTN_DECODE_SCRATCH_BYTES;
  int fit = 0;
  for (int Tm = 128; Tm <= (1 << 20); Tm += 128)
    if (ncattn_decode_workspace_bytes(16, Tm, 16, 16, 128, -1) <= cap) fit = Tm;
  CHECK(fit > 0);
  CHECK(dec(true, 16, fit, 16, 16, 128, -1, NCATTN_BF16, nullptr, 0) == NCATTN_OK);
  CHECK(dec(true, 16, fit + 1, 16, 16, 128, -1, NCATTN_BF16, nullptr, 0) == NCATTN_EWORKSPACE && err_ok());
}

static void test_prefill() {
  auto pf = [](int Tn, int Tm, int D, int wl, int dt, const void *lens = P(5)) {
    return ncattn_prefill(P(0), P(1), P(2), P(3), P(4), (const int32_t *)lens, P(6), nullptr, 2, Tn, Tm, 2, 2, D, wl,
                          0.f, dt, nullptr);
  };
  CHECK(pf(0, 64, 128, -1, NCATTN_BF16) == NCATTN_EINVAL);
  CHECK(pf(65, 64, 128, -1, NCATTN_BF16) == NCATTN_EINVAL);
  CHECK(pf(INT_MAX, INT_MAX, 128, -1, NCATTN_BF16) == NCATTN_EUNSUPPORTED);
  CHECK(pf(8, 64, 128, -1, NCATTN_F32) == NCATTN_EUNSUPPORTED);
  CHECK(pf(8, 64, 96, -1, NCATTN_BF16) == NCATTN_EUNSUPPORTED);
  CHECK(pf(8, 64, 128, -1, NCATTN_BF16, MIS(5)) == NCATTN_EINVAL);
  CHECK(pf(8, 64, 64, 63, NCATTN_BF16) == NCATTN_OK);
  CHECK(strcmp(g_last.fn, "prefill_bf16") == 0 && g_last.window == -1 && g_last.T_max == 64 && g_last.D == 64);
  CHECK(pf(8, 64, 128, 62, NCATTN_BF16) == NCATTN_OK && g_last.window == 62);
}

static void test_replicate() {
  auto rp = [](int N, int Ts, int Tm, int KV, int D, int dt, void *kd = P(3)) {
    return ncattn_cache_replicate(P(0), P(1), (const int32_t *)P(2), kd, P(4), (int32_t *)P(5), N, Ts, Tm, KV, D, dt,
                                  nullptr);
  };
  CHECK(rp(0, 16, 32, 2, 128, NCATTN_BF16) == NCATTN_EINVAL);
  CHECK(rp(4, 33, 32, 2, 128, NCATTN_BF16) == NCATTN_EINVAL);
  CHECK(rp(4, 16, 32, 1, 4, NCATTN_BF16) == NCATTN_EINVAL);    // 8-byte rows
  CHECK(rp(4, 16, 32, 2, 128, NCATTN_BF16, P(4)) == NCATTN_EINVAL);
  // every size at INT_MAX: refused, no overflow in the row or total sizes
  CHECK(rp(INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, NCATTN_F32) == NCATTN_EINVAL);
  CHECK(rp(INT_MAX, 1, INT_MAX, 1 << 16, 1 << 16, NCATTN_BF16) == NCATTN_EINVAL);
  CHECK(rp(4, 16, 32, 2, 128, NCATTN_BF16) == NCATTN_OK);
  CHECK(strcmp(g_last.fn, "cache_replicate") == 0 && g_last.D == 2 * 128 * 2 / 16);
  CHECK(rp(3, 9, 9, 1, 4, NCATTN_F32) == NCATTN_OK && g_last.D == 1);
}

int main() {
  test_fwd();
  test_fwd_fp8();
  test_qknorm();
  test_bwd();
  test_decode();
  test_prefill();
  test_replicate();
  CHECK(strcmp(ncattn_version(), "") != 0);
  printf("checks=%d failures=%d launches=%ld\n", g_checks, g_fail, g_last.count);
  return g_fail != 0;
}

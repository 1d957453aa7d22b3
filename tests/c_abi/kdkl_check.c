/* Host-side checks of the loss library's C ABI (include/kdkl.h), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer (host code only) by
 * tests/test_host_sanitized.py.
 *
 * 1. kd_workspace_size over a product of shapes at and beyond every domain limit
 *    the header states, for each op and dtype: a problem is accepted exactly when
 *    the header's domain holds (a predicate written here from the header text), a
 *    problem with one kind of fault gets that fault's status, and the size of an
 *    accepted problem is positive and a multiple of 256 bytes.  The 64-bit size
 *    arithmetic runs at the largest shapes under UBSan's overflow checks.
 * 2. Every entry point's argument errors.  Each call here has at least one bad
 *    argument, so none gets past validation: no device work is ever requested,
 *    with or without a GPU.
 * 3. Status strings, the version and an empty profiling session.
 *
 * usage: kdkl_check; prints "ok <checks>" and exits 0, or names the first failed
 * check and exits 1. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kdkl.h"

static long n_checks = 0;

#define CHECK(cond, ...)                                     \
  do {                                                       \
    ++n_checks;                                              \
    if (!(cond)) {                                           \
      fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                          \
      fprintf(stderr, "\n");                                 \
      exit(1);                                               \
    }                                                        \
  } while (0)

static int64_t up256(int64_t x) { return (x + 255) / 256 * 256; }

/* the header's domain, one flag per kind of fault */
static void domain(kd_op op, const kd_problem* p, int* shape_ok, int* dtype_ok, int* tau_ok) {
  const int x = p->x_dtype, v = p->val_dtype, h = p->dh_dtype;
  *dtype_ok = (x == KD_BF16 || x == KD_F32) && v == x && (op != KD_OP_KL_BWD || h == KD_F32 || h == KD_BF16);
  const int64_t kmax = p->vocab < 65535 ? p->vocab : 65535;
  int ok = p->n_tokens >= 0 && p->n_tokens <= ((int64_t)1 << 31) - 256;
  ok = ok && p->d_model >= 8 && p->d_model % 8 == 0 && p->d_model <= ((int64_t)1 << 20);
  ok = ok && p->vocab >= 1 && p->vocab <= 2097088;
  ok = ok && p->k >= 1 && p->k <= kmax && (op != KD_OP_TOPK_BUILD || p->k <= 4096);
  ok = ok && p->chunk_tokens >= 0;
  if (ok && p->chunk_tokens > 0) {
    /* the defaults are far below the limit, so only an explicit chunk can pass it */
    int64_t used = up256(p->chunk_tokens);
    const int64_t cap = up256(p->n_tokens > 1 ? p->n_tokens : 1);
    if (used > cap) used = cap;
    ok = used <= 2096896;
  }
  *shape_ok = ok;
  *tau_ok = op == KD_OP_TOPK_BUILD || (isfinite(p->tau) && p->tau > 0.f);
}

static void workspace_sweep(void) {
  const kd_op ops[] = {KD_OP_TOPK_BUILD, KD_OP_KL_FWD, KD_OP_KL_BWD};
  const int64_t ns[] = {-1, 0, 1, 255, 256, 257, 16384, 131072, 2096896, 2096897, ((int64_t)1 << 31) - 256,
                        ((int64_t)1 << 31) - 255, INT64_MAX};
  const int64_t ds[] = {0, 7, 8, 12, 4096, (int64_t)1 << 20, ((int64_t)1 << 20) + 8, INT64_MAX - 7};
  const int64_t vs[] = {0, 1, 257, 128256, 2097088, 2097089, INT64_MAX};
  const int32_t ks[] = {-1, 0, 1, 100, 4096, 4097, 65535, 65536, INT32_MAX};
  const int32_t chunks[] = {-1, 0, 1, 16384, 2096896, 2096897, INT32_MAX};
  const float taus[] = {1.f, 0.f, -1.f, INFINITY, NAN};
  const int32_t dts[][3] = {{KD_BF16, KD_BF16, KD_F32}, {KD_BF16, KD_BF16, KD_BF16}, {KD_F32, KD_F32, KD_F32},
                            {KD_F32, KD_BF16, KD_F32},  {KD_BF16, KD_BF16, 7},       {9, 9, KD_F32}};
#define COUNT(a) (sizeof(a) / sizeof((a)[0]))
  long accepted = 0;
  for (size_t o = 0; o < COUNT(ops); ++o)
    for (size_t di = 0; di < COUNT(ds); ++di)
      for (size_t vi = 0; vi < COUNT(vs); ++vi)
        for (size_t ki = 0; ki < COUNT(ks); ++ki)
          for (size_t ci = 0; ci < COUNT(chunks); ++ci)
            for (size_t ti = 0; ti < COUNT(taus); ++ti)
              for (size_t xi = 0; xi < COUNT(dts); ++xi) {
                for (size_t ni = 0; ni < COUNT(ns); ++ni) {
                  kd_problem p;
                  memset(&p, 0, sizeof p);
                  p.n_tokens = ns[ni];
                  p.d_model = ds[di];
                  p.vocab = vs[vi];
                  p.k = ks[ki];
                  p.tau = taus[ti];
                  p.x_dtype = dts[xi][0];
                  p.val_dtype = dts[xi][1];
                  p.dh_dtype = dts[xi][2];
                  p.chunk_tokens = chunks[ci];
                  int s_ok, d_ok, t_ok;
                  domain(ops[o], &p, &s_ok, &d_ok, &t_ok);
                  size_t bytes = 12345;
                  const kd_status st = kd_workspace_size(ops[o], &p, &bytes);
                  const char* what = "op %d N %lld d %lld V %lld K %d chunk %d tau %g dtypes %d/%d/%d: status %d";
#define ARGS (int)ops[o], (long long)p.n_tokens, (long long)p.d_model, (long long)p.vocab, p.k, p.chunk_tokens, \
             (double)p.tau, p.x_dtype, p.val_dtype, p.dh_dtype, (int)st
                  if (s_ok && d_ok && t_ok) {
                    CHECK(st == KD_OK, what, ARGS);
                    CHECK(bytes > 0 && bytes % 256 == 0, what, ARGS);
                    ++accepted;
                  } else {
                    CHECK(st != KD_OK, what, ARGS);
                    CHECK(bytes == 12345, what, ARGS);   /* nothing written on an error */
                    if (!s_ok && d_ok && t_ok) CHECK(st == KD_ERR_BAD_SHAPE, what, ARGS);
                    if (s_ok && !d_ok && t_ok) CHECK(st == KD_ERR_BAD_DTYPE, what, ARGS);
                    if (s_ok && d_ok && !t_ok) CHECK(st == KD_ERR_BAD_TAU, what, ARGS);
                    if (!(s_ok && d_ok && t_ok))
                      CHECK(st == KD_ERR_BAD_SHAPE || st == KD_ERR_BAD_DTYPE || st == KD_ERR_BAD_TAU, what, ARGS);
                  }
#undef ARGS
                }
              }
  CHECK(accepted > 10000, "only %ld accepted problems in the sweep", accepted);
  kd_problem p;
  memset(&p, 0, sizeof p);
  p.n_tokens = 64;
  p.d_model = 128;
  p.vocab = 1000;
  p.k = 8;
  p.tau = 1.f;
  size_t bytes = 0;
  CHECK(kd_workspace_size(KD_OP_KL_FWD, NULL, &bytes) == KD_ERR_NULL_POINTER, "workspace: NULL problem");
  CHECK(kd_workspace_size(KD_OP_KL_FWD, &p, NULL) == KD_ERR_NULL_POINTER, "workspace: NULL out");
  CHECK(kd_workspace_size((kd_op)7, &p, &bytes) == KD_ERR_BAD_SHAPE, "workspace: unknown op");
#undef COUNT
}

/* host buffers standing in for device ones: no call below reaches the device */
static _Alignas(256) unsigned char buf[8][1 << 16];

static void call_errors(void) {
  kd_problem p;
  memset(&p, 0, sizeof p);
  p.n_tokens = 64;
  p.d_model = 128;
  p.vocab = 1000;
  p.k = 8;
  p.tau = 1.f;
  p.x_dtype = KD_BF16;
  p.val_dtype = KD_BF16;
  p.dh_dtype = KD_F32;
  size_t need = 0;
  CHECK(kd_workspace_size(KD_OP_KL_FWD, &p, &need) == KD_OK, "workspace of the base problem");
  const size_t small = need - 1;   /* one byte short: every call below stops at validation */
  void *h = buf[0], *w = buf[1], *val = buf[3], *ws = buf[7];
  int32_t* idx = (int32_t*)buf[2];
  float *loss = (float*)buf[4], *lse = (float*)buf[5], *rows = (float*)buf[6];
  unsigned char* odd = buf[0] + 4;   /* 4-byte but not 16-byte aligned */

  /* forward */
  CHECK(kd_chunked_kl_fwd(NULL, h, w, idx, val, loss, lse, rows, ws, need, NULL) == KD_ERR_NULL_POINTER, "fwd p");
  CHECK(kd_chunked_kl_fwd(&p, NULL, w, idx, val, loss, lse, rows, ws, need, NULL) == KD_ERR_NULL_POINTER, "fwd h");
  CHECK(kd_chunked_kl_fwd(&p, h, NULL, idx, val, loss, lse, rows, ws, need, NULL) == KD_ERR_NULL_POINTER, "fwd w");
  CHECK(kd_chunked_kl_fwd(&p, h, w, NULL, val, loss, lse, rows, ws, need, NULL) == KD_ERR_NULL_POINTER, "fwd idx");
  CHECK(kd_chunked_kl_fwd(&p, h, w, idx, NULL, loss, lse, rows, ws, need, NULL) == KD_ERR_NULL_POINTER, "fwd val");
  CHECK(kd_chunked_kl_fwd(&p, h, w, idx, val, NULL, lse, rows, ws, need, NULL) == KD_ERR_NULL_POINTER, "fwd loss");
  CHECK(kd_chunked_kl_fwd(&p, h, w, idx, val, loss, NULL, rows, ws, need, NULL) == KD_ERR_NULL_POINTER, "fwd lse");
  CHECK(kd_chunked_kl_fwd(&p, h, w, idx, val, loss, lse, rows, NULL, need, NULL) == KD_ERR_NULL_POINTER, "fwd ws");
  CHECK(kd_chunked_kl_fwd(&p, odd, w, idx, val, loss, lse, rows, ws, need, NULL) == KD_ERR_MISALIGNED, "fwd odd h");
  CHECK(kd_chunked_kl_fwd(&p, h, w, idx, val, loss, lse, (float*)odd, ws, need, NULL) == KD_ERR_MISALIGNED,
        "fwd odd rows");
  CHECK(kd_chunked_kl_fwd(&p, h, w, idx, val, loss, lse, rows, ws, small, NULL) == KD_ERR_WORKSPACE_TOO_SMALL,
        "fwd small workspace");
  kd_problem bad = p;
  bad.tau = NAN;
  CHECK(kd_chunked_kl_fwd(&bad, h, w, idx, val, loss, lse, rows, ws, need, NULL) == KD_ERR_BAD_TAU, "fwd tau");

  /* loss options */
  kd_loss_opts o = {(const int32_t*)buf[6], -100, 0.5f, KD_STUDENT_FULL};
  const float bad_weights[] = {-0.01f, 1.01f, NAN, INFINITY};
  for (size_t i = 0; i < sizeof bad_weights / sizeof bad_weights[0]; ++i) {
    o.ce_weight = bad_weights[i];
    CHECK(kd_chunked_kl_fwd_ex(&p, &o, h, w, idx, val, loss, lse, rows, ws, small, NULL) == KD_ERR_BAD_OPTION,
          "fwd_ex weight %g", (double)bad_weights[i]);
    CHECK(kd_chunked_kl_bwd_ex(&p, &o, h, w, idx, val, lse, NULL, buf[3], (float*)buf[4], ws, small, NULL) ==
              KD_ERR_BAD_OPTION,
          "bwd_ex weight %g", (double)bad_weights[i]);
  }
  o.ce_weight = 0.5f;
  o.labels = NULL;
  CHECK(kd_chunked_kl_fwd_ex(&p, &o, h, w, idx, val, loss, lse, rows, ws, small, NULL) == KD_ERR_BAD_OPTION,
        "fwd_ex mix without labels");
  o.labels = (const int32_t*)(buf[6] + 2);
  CHECK(kd_chunked_kl_fwd_ex(&p, &o, h, w, idx, val, loss, lse, rows, ws, small, NULL) == KD_ERR_MISALIGNED,
        "fwd_ex misaligned labels");
  o.labels = (const int32_t*)(buf[6] + 4);   /* labels need only 4-byte alignment: the small workspace stops it */
  CHECK(kd_chunked_kl_fwd_ex(&p, &o, h, w, idx, val, loss, lse, rows, ws, small, NULL) ==
            KD_ERR_WORKSPACE_TOO_SMALL,
        "fwd_ex 4-byte aligned labels");
  o.labels = NULL;
  o.ce_weight = 0.f;
  CHECK(kd_chunked_kl_fwd_ex(&p, &o, h, w, idx, val, loss, lse, rows, ws, small, NULL) ==
            KD_ERR_WORKSPACE_TOO_SMALL,
        "fwd_ex plain options");
  CHECK(kd_chunked_kl_fwd_ex(&p, NULL, h, w, idx, val, loss, lse, rows, ws, small, NULL) ==
            KD_ERR_WORKSPACE_TOO_SMALL,
        "fwd_ex NULL options");
  /* the student normaliser: only the two kd_student values, and no mix with the renormalised one */
  const int32_t bad_students[] = {-1, 2, 1000};
  for (size_t i = 0; i < sizeof bad_students / sizeof bad_students[0]; ++i) {
    o.student = bad_students[i];
    CHECK(kd_chunked_kl_fwd_ex(&p, &o, h, w, idx, val, loss, lse, rows, ws, need, NULL) == KD_ERR_BAD_OPTION,
          "fwd_ex student %d", (int)bad_students[i]);
    CHECK(kd_chunked_kl_bwd_ex(&p, &o, h, w, idx, val, lse, NULL, buf[3], (float*)buf[4], ws, small, NULL) ==
              KD_ERR_BAD_OPTION,
          "bwd_ex student %d", (int)bad_students[i]);
  }
  o.student = KD_STUDENT_RENORM;
  o.labels = (const int32_t*)buf[6];
  o.ce_weight = 0.25f;
  CHECK(kd_chunked_kl_fwd_ex(&p, &o, h, w, idx, val, loss, lse, rows, ws, need, NULL) == KD_ERR_BAD_OPTION,
        "fwd_ex renormalised student with a mix");
  o.ce_weight = 0.f;
  CHECK(kd_chunked_kl_fwd_ex(&p, &o, h, w, idx, val, loss, lse, rows, ws, small, NULL) ==
            KD_ERR_WORKSPACE_TOO_SMALL,
        "fwd_ex renormalised student");
  o.student = KD_STUDENT_FULL;
  o.labels = NULL;

  /* backward */
  size_t need_b = 0;
  CHECK(kd_workspace_size(KD_OP_KL_BWD, &p, &need_b) == KD_OK, "backward workspace");
  void* dh = buf[3];
  float* dw = (float*)buf[4];
  const float* g = (const float*)buf[5];
  CHECK(kd_chunked_kl_bwd(&p, h, w, idx, val, lse, g, dh, NULL, ws, need_b, NULL) == KD_ERR_NULL_POINTER, "bwd dw");
  CHECK(kd_chunked_kl_bwd(&p, h, w, idx, val, NULL, g, dh, dw, ws, need_b, NULL) == KD_ERR_NULL_POINTER, "bwd lse");
  CHECK(kd_chunked_kl_bwd(&p, h, w, idx, val, lse, g, NULL, dw, ws, need_b, NULL) == KD_ERR_NULL_POINTER, "bwd dh");
  CHECK(kd_chunked_kl_bwd(&p, h, w, idx, val, lse, g, odd, dw, ws, need_b, NULL) == KD_ERR_MISALIGNED, "bwd odd dh");
  CHECK(kd_chunked_kl_bwd(&p, h, w, idx, val, lse, g, dh, dw, ws, need_b - 1, NULL) == KD_ERR_WORKSPACE_TOO_SMALL,
        "bwd small workspace");
  bad = p;
  bad.dh_dtype = 5;
  CHECK(kd_chunked_kl_bwd(&bad, h, w, idx, val, lse, g, dh, dw, ws, need_b, NULL) == KD_ERR_BAD_DTYPE, "bwd dtype");

  /* cache build */
  size_t need_t = 0;
  CHECK(kd_workspace_size(KD_OP_TOPK_BUILD, &p, &need_t) == KD_OK, "cache build workspace");
  CHECK(kd_topk_cache_build(&p, h, NULL, idx, val, ws, need_t, NULL) == KD_ERR_NULL_POINTER, "build w_t");
  CHECK(kd_topk_cache_build(&p, h, w, NULL, val, ws, need_t, NULL) == KD_ERR_NULL_POINTER, "build idx");
  CHECK(kd_topk_cache_build(&p, h, w, idx, val, NULL, need_t, NULL) == KD_ERR_NULL_POINTER, "build ws");
  CHECK(kd_topk_cache_build(&p, h, w, (int32_t*)odd, val, ws, need_t, NULL) == KD_ERR_MISALIGNED, "build odd idx");
  CHECK(kd_topk_cache_build(&p, h, w, idx, val, ws, need_t - 1, NULL) == KD_ERR_WORKSPACE_TOO_SMALL,
        "build small workspace");
  bad = p;
  bad.k = 4097;
  bad.vocab = 10000;
  CHECK(kd_topk_cache_build(&bad, h, w, idx, val, ws, need_t, NULL) == KD_ERR_BAD_SHAPE, "build K > 4096");
}

static void strings_and_hooks(void) {
  for (int s = -3; s < 40; ++s) {
    const char* t = kd_status_string((kd_status)s);
    CHECK(t != NULL && strlen(t) > 0 && strlen(t) < 200, "status string %d", s);
  }
  CHECK(strcmp(kd_status_string(KD_OK), kd_status_string(KD_ERR_LAUNCH)) != 0, "distinct status strings");
  CHECK(kd_version() >= 100, "version %d", kd_version());
  kd_kernel_stat st[4];
  int n = -1;
  CHECK(kd_profile_begin() == KD_OK, "profile begin");
  CHECK(kd_profile_end(st, 4, &n) == KD_OK && n == 0, "empty profile session gives %d kinds", n);
  CHECK(kd_profile_end(NULL, 0, NULL) == KD_OK, "profile end with no outputs");
}

int main(void) {
  workspace_sweep();
  call_errors();
  strings_and_hooks();
  printf("ok %ld checks\n", n_checks);
  return 0;
}

/*
 * Plain-C client of the kdkl C ABI (include/kdkl.h), linked against libkdkl.so and
 * the HIP runtime's C API only.  It reads a problem file, builds the teacher's
 * top-K cache, runs the forward and the backward, and writes the results.  It
 * then writes the cache to two shard files in DIR (include/kdcache.h), streams them
 * back to the device with the loader and runs the forward again on that copy.
 * It also streams the device cache to shards with the streaming writer (two puts,
 * shards of N/2 + 1 rows) and compares what kd_cache_read returns with it.
 * Last, the loss options (kd_loss_opts): labels[i] = -100 (ignored) when
 * i % 7 == 3, else (131 i) mod V, with a cross-entropy weight of 0.25, through the
 * _ex forward and backward:
 *
 *   kd_client IN OUT DIR
 *   IN : int64 N, d, V; int32 K; float tau; then H [N*d], W [V*d], W_T [V*d] as bf16
 *        bits (uint16), teacher hidden states = H
 *   OUT: int32 status; then idx [N*K] int32, val [N*K] bf16 bits, loss float,
 *        lse [N] float, dH [N*d] float, dW [V*d] float, loss from the reloaded cache float,
 *        then with the options: loss float, dH [N*d] float, dW [V*d] float,
 *        then int32 writer_ok (1 when the writer's shards hold the cache exactly)
 *
 * Exit status 0 on success; on a library error the kd_status is printed with
 * kd_status_string() and the exit status is 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kdcache.h"
#include "kdkl.h"

#define HIP_OK(x)                                                             \
  do {                                                                        \
    if ((x) != hipSuccess) {                                                  \
      fprintf(stderr, "kd_client: HIP call failed: %s\n", #x);                \
      return 2;                                                               \
    }                                                                         \
  } while (0)

#define KD_OK_OR_FAIL(x)                                                      \
  do {                                                                        \
    kd_status s_ = (x);                                                       \
    if (s_ != KD_OK) {                                                        \
      fprintf(stderr, "kd_client: %s -> %s\n", #x, kd_status_string(s_));     \
      return 1;                                                               \
    }                                                                         \
  } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }
static int write_all(FILE* f, const void* p, size_t n) { return fwrite(p, 1, n, f) == n; }

int main(int argc, char** argv) {
  if (argc != 4) {
    fprintf(stderr, "usage: kd_client IN OUT DIR\n");
    return 2;
  }
  FILE* fi = fopen(argv[1], "rb");
  if (!fi) return 2;
  int64_t dims[3];
  int32_t K;
  float tau;
  if (!read_all(fi, dims, sizeof dims) || !read_all(fi, &K, sizeof K) || !read_all(fi, &tau, sizeof tau)) return 2;
  const int64_t N = dims[0], d = dims[1], V = dims[2];
  const size_t nh = (size_t)(N * d), nw = (size_t)(V * d), nk = (size_t)(N * K);
  uint16_t* h = malloc(2 * nh);
  uint16_t* w = malloc(2 * nw);
  uint16_t* wt = malloc(2 * nw);
  if (!h || !w || !wt) return 2;
  if (!read_all(fi, h, 2 * nh) || !read_all(fi, w, 2 * nw) || !read_all(fi, wt, 2 * nw)) return 2;
  fclose(fi);

  kd_problem p = {N, d, V, K, tau, KD_BF16, KD_BF16, KD_F32, 0};
  size_t ws_bytes = 0, b = 0;
  KD_OK_OR_FAIL(kd_workspace_size(KD_OP_TOPK_BUILD, &p, &b));
  if (b > ws_bytes) ws_bytes = b;
  KD_OK_OR_FAIL(kd_workspace_size(KD_OP_KL_FWD, &p, &b));
  if (b > ws_bytes) ws_bytes = b;
  KD_OK_OR_FAIL(kd_workspace_size(KD_OP_KL_BWD, &p, &b));
  if (b > ws_bytes) ws_bytes = b;

  void *dh_in, *dw_in, *dwt_in, *didx, *dval, *dloss, *dlse, *ddh, *ddw, *dws;
  HIP_OK(hipMalloc(&dh_in, 2 * nh));
  HIP_OK(hipMalloc(&dw_in, 2 * nw));
  HIP_OK(hipMalloc(&dwt_in, 2 * nw));
  HIP_OK(hipMalloc(&didx, 4 * nk + 16));
  HIP_OK(hipMalloc(&dval, 2 * nk + 16));
  HIP_OK(hipMalloc(&dloss, 16));
  HIP_OK(hipMalloc(&dlse, 4 * (size_t)N + 16));
  HIP_OK(hipMalloc(&ddh, 4 * nh + 16));
  HIP_OK(hipMalloc(&ddw, 4 * nw));
  HIP_OK(hipMalloc(&dws, ws_bytes ? ws_bytes : 16));
  HIP_OK(hipMemcpy(dh_in, h, 2 * nh, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dw_in, w, 2 * nw, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dwt_in, wt, 2 * nw, hipMemcpyHostToDevice));

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  KD_OK_OR_FAIL(kd_topk_cache_build(&p, dh_in, dwt_in, (int32_t*)didx, dval, dws, ws_bytes, st));
  KD_OK_OR_FAIL(kd_chunked_kl_fwd(&p, dh_in, dw_in, (const int32_t*)didx, dval, (float*)dloss, (float*)dlse,
                                  NULL, dws, ws_bytes, st));
  KD_OK_OR_FAIL(kd_chunked_kl_bwd(&p, dh_in, dw_in, (const int32_t*)didx, dval, (const float*)dlse, NULL, ddh,
                                  (float*)ddw, dws, ws_bytes, st));
  HIP_OK(hipStreamSynchronize(st));

  int32_t* idx = malloc(4 * nk + 4);
  uint16_t* val = malloc(2 * nk + 2);
  float* lse = malloc(4 * (size_t)N + 4);
  float* dhh = malloc(4 * nh + 4);
  float* dwh = malloc(4 * nw);
  float loss = 0.f;
  if (!idx || !val || !lse || !dhh || !dwh) return 2;
  HIP_OK(hipMemcpy(idx, didx, 4 * nk, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(val, dval, 2 * nk, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&loss, dloss, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse, dlse, 4 * (size_t)N, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dhh, ddh, 4 * nh, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dwh, ddw, 4 * nw, hipMemcpyDeviceToHost));

  /* the cache through two shard files and the loader, then the forward again */
  char path0[4096], path1[4096];
  snprintf(path0, sizeof path0, "%s/c0.kdc", argv[3]);
  snprintf(path1, sizeof path1, "%s/c1.kdc", argv[3]);
  const int64_t half = N / 2;
  kd_cache_info ci0 = {half, V, K, 0, KD_BF16};
  kd_cache_info ci1 = {N - half, V, K, 0, KD_BF16};
  KD_OK_OR_FAIL(kd_cache_write(path0, &ci0, idx, val));
  KD_OK_OR_FAIL(kd_cache_write(path1, &ci1, idx + half * K, val + half * K));
  void *didx2, *dval2, *dloss2;
  HIP_OK(hipMalloc(&didx2, 4 * nk + 16));
  HIP_OK(hipMalloc(&dval2, 2 * nk + 16));
  HIP_OK(hipMalloc(&dloss2, 16));
  const char* paths[2] = {path0, path1};
  kd_cache_loader* ld = NULL;
  const int64_t batch = N / 3 + 1;
  KD_OK_OR_FAIL(kd_cache_loader_open(paths, 2, batch, 2, &ld));
  int64_t row = 0, rows = 0;
  do {
    KD_OK_OR_FAIL(kd_cache_loader_next(ld, (int32_t*)didx2 + row * K, (uint16_t*)dval2 + row * K, &rows, st));
    row += rows;
  } while (rows > 0);
  HIP_OK(hipStreamSynchronize(st));
  KD_OK_OR_FAIL(kd_cache_loader_close(ld));
  if (row != N) {
    fprintf(stderr, "kd_client: loader returned %lld rows, expected %lld\n", (long long)row, (long long)N);
    return 1;
  }
  KD_OK_OR_FAIL(kd_chunked_kl_fwd(&p, dh_in, dw_in, (const int32_t*)didx2, dval2, (float*)dloss2, (float*)dlse,
                                  NULL, dws, ws_bytes, st));
  HIP_OK(hipStreamSynchronize(st));
  float loss2 = 0.f;
  HIP_OK(hipMemcpy(&loss2, dloss2, 4, hipMemcpyDeviceToHost));

  /* the loss options: a padding mask and a hard-label mix */
  int32_t* lab = malloc(4 * (size_t)N + 4);
  if (!lab) return 2;
  for (int64_t i = 0; i < N; ++i) lab[i] = (i % 7 == 3) ? -100 : (int32_t)((131 * i) % V);
  void* dlab;
  HIP_OK(hipMalloc(&dlab, 4 * (size_t)N + 16));
  HIP_OK(hipMemcpy(dlab, lab, 4 * (size_t)N, hipMemcpyHostToDevice));
  const kd_loss_opts opts = {(const int32_t*)dlab, -100, 0.25f, KD_STUDENT_FULL};
  KD_OK_OR_FAIL(kd_chunked_kl_fwd_ex(&p, &opts, dh_in, dw_in, (const int32_t*)didx, dval, (float*)dloss2,
                                     (float*)dlse, NULL, dws, ws_bytes, st));
  KD_OK_OR_FAIL(kd_chunked_kl_bwd_ex(&p, &opts, dh_in, dw_in, (const int32_t*)didx, dval, (const float*)dlse, NULL,
                                     ddh, (float*)ddw, dws, ws_bytes, st));
  HIP_OK(hipStreamSynchronize(st));
  float loss3 = 0.f;
  float* dhh3 = malloc(4 * nh + 4);
  float* dwh3 = malloc(4 * nw);
  if (!dhh3 || !dwh3) return 2;
  HIP_OK(hipMemcpy(&loss3, dloss2, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dhh3, ddh, 4 * nh, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dwh3, ddw, 4 * nw, hipMemcpyDeviceToHost));

  /* the streaming writer: the device cache in two puts, shards of N/2 + 1 rows */
  int32_t writer_ok = 0;
  {
    char wprefix[4096];
    snprintf(wprefix, sizeof wprefix, "%s/w", argv[3]);
    kd_cache_info shard = {N / 2 + 1, V, K, 0, KD_BF16};
    kd_cache_writer* wr = NULL;
    KD_OK_OR_FAIL(kd_cache_writer_open(wprefix, &shard, N - N / 2, 2, &wr));
    KD_OK_OR_FAIL(kd_cache_writer_put(wr, (const int32_t*)didx, dval, N / 2, st));
    KD_OK_OR_FAIL(kd_cache_writer_put(wr, (const int32_t*)didx + (N / 2) * K, (const uint16_t*)dval + (N / 2) * K,
                                      N - N / 2, st));
    int64_t n_shards = 0;
    KD_OK_OR_FAIL(kd_cache_writer_close(wr, &n_shards));
    int32_t* ridx = malloc(4 * nk + 4);
    uint16_t* rval = malloc(2 * nk + 2);
    if (!ridx || !rval) return 2;
    int64_t row = 0;
    for (int64_t i = 0; i < n_shards; ++i) {
      char path[4200];
      snprintf(path, sizeof path, "%s_%05lld.kdc", wprefix, (long long)i);
      kd_cache_info si;
      KD_OK_OR_FAIL(kd_cache_info_read(path, &si));
      KD_OK_OR_FAIL(kd_cache_read(path, 0, si.n_tokens, ridx + row * K, rval + row * K));
      row += si.n_tokens;
    }
    writer_ok = n_shards == 2 && row == N && memcmp(ridx, idx, 4 * nk) == 0 && memcmp(rval, val, 2 * nk) == 0;
    free(ridx);
    free(rval);
  }

  FILE* fo = fopen(argv[2], "wb");
  if (!fo) return 2;
  const int32_t ok = 0;
  if (!write_all(fo, &ok, 4) || !write_all(fo, idx, 4 * nk) || !write_all(fo, val, 2 * nk) ||
      !write_all(fo, &loss, 4) || !write_all(fo, lse, 4 * (size_t)N) || !write_all(fo, dhh, 4 * nh) ||
      !write_all(fo, dwh, 4 * nw) || !write_all(fo, &loss2, 4) || !write_all(fo, &loss3, 4) ||
      !write_all(fo, dhh3, 4 * nh) || !write_all(fo, dwh3, 4 * nw) || !write_all(fo, &writer_ok, 4))
    return 2;
  fclose(fo);
  printf("kd_client: N=%lld d=%lld V=%lld K=%d loss=%.6f (kd_version %d)\n", (long long)N, (long long)d,
         (long long)V, K, loss, kd_version());
  HIP_OK(hipStreamDestroy(st));
  return 0;
}

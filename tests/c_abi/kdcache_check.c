/* Host-only checks of the teacher-cache C ABI (include/kdcache.h), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_cache_sanitized.py:
 * round trips over both index widths and value types, partial reads, every
 * argument error, corrupted and truncated shard files (each header field and the
 * file size), and the argument errors and release paths of the loader and the
 * writer.  Without a device their open calls stop at the pinned-buffer
 * allocation; with one they open and are closed again.
 *
 * usage: kdcache_check <scratch directory>; prints "ok <checks>" and exits 0, or
 * names the first failed check and exits 1. */
#include <dirent.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/stat.h>

#include "kdcache.h"

static int n_checks = 0;
static const char* dir = ".";

#define CHECK(cond, ...)                                  \
  do {                                                    \
    ++n_checks;                                           \
    if (!(cond)) {                                        \
      fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                       \
      fprintf(stderr, "\n");                              \
      exit(1);                                            \
    }                                                     \
  } while (0)

static void path_of(char* out, size_t n, const char* name) { snprintf(out, n, "%s/%s", dir, name); }

static int64_t file_size(const char* p) {
  struct stat st;
  return stat(p, &st) == 0 ? (int64_t)st.st_size : -1;
}

static unsigned char* slurp(const char* p, int64_t* n) {
  FILE* f = fopen(p, "rb");
  if (!f) return NULL;
  *n = file_size(p);
  unsigned char* b = (unsigned char*)malloc((size_t)(*n > 0 ? *n : 1));
  if (b && *n > 0 && fread(b, 1, (size_t)*n, f) != (size_t)*n) {
    free(b);
    b = NULL;
  }
  fclose(f);
  return b;
}

static void spit(const char* p, const unsigned char* b, int64_t n) {
  FILE* f = fopen(p, "wb");
  CHECK(f != NULL, "cannot create %s", p);
  if (n > 0) CHECK(fwrite(b, 1, (size_t)n, f) == (size_t)n, "short write %s", p);
  fclose(f);
}

static void put32(unsigned char* p, uint32_t v) {
  for (int i = 0; i < 4; ++i) p[i] = (unsigned char)(v >> (8 * i));
}
static void put64(unsigned char* p, uint64_t v) {
  for (int i = 0; i < 8; ++i) p[i] = (unsigned char)(v >> (8 * i));
}

static int64_t expected_size(int64_t n, int32_t k, int bits, int vdt) {
  const int64_t idx_end = 64 + n * k * (bits / 8);
  const int64_t val_off = (idx_end + 63) / 64 * 64;
  return val_off + n * k * (vdt == KD_F32 ? 4 : 2);
}

/* one shard written, its header read back, then the whole and parts of it */
static void round_trip(int64_t n, int64_t vocab, int32_t k, int32_t bits, int32_t vdt) {
  char p[512];
  path_of(p, sizeof p, "rt.kdc");
  const int64_t total = n * k;
  const size_t vb = vdt == KD_F32 ? 4 : 2;
  int32_t* idx = (int32_t*)malloc((size_t)(total > 0 ? total : 1) * 4);
  unsigned char* val = (unsigned char*)malloc((size_t)(total > 0 ? total : 1) * vb);
  for (int64_t e = 0; e < total; ++e) {
    idx[e] = (int32_t)((e * 7919 + e / k * 31) % vocab);
    for (size_t b = 0; b < vb; ++b) val[e * (int64_t)vb + (int64_t)b] = (unsigned char)(e * 13 + (int64_t)b * 101);
  }
  if (total > 0) idx[total - 1] = (int32_t)(vocab - 1);   /* the largest index survives narrowing */
  kd_cache_info in = {n, vocab, k, bits, vdt};
  CHECK(kd_cache_write(p, &in, idx, val) == KD_OK, "write n=%lld V=%lld k=%d bits=%d", (long long)n,
        (long long)vocab, k, bits);
  const int on_disk = bits ? bits : (vocab <= 65536 ? 16 : 32);
  CHECK(file_size(p) == expected_size(n, k, on_disk, vdt), "file size n=%lld k=%d", (long long)n, k);
  kd_cache_info got;
  memset(&got, 0, sizeof got);
  CHECK(kd_cache_info_read(p, &got) == KD_OK, "info_read");
  CHECK(got.n_tokens == n && got.vocab == vocab && got.k == k && got.idx_bits == on_disk && got.val_dtype == vdt,
        "header fields");
  int32_t* ri = (int32_t*)malloc((size_t)(total > 0 ? total : 1) * 4);
  unsigned char* rv = (unsigned char*)malloc((size_t)(total > 0 ? total : 1) * vb);
  const int64_t cuts[][2] = {{0, n}, {0, n / 2}, {n / 3, n - n / 3}, {n, 0}, {n > 0 ? n - 1 : 0, n > 0 ? 1 : 0}};
  for (size_t c = 0; c < sizeof cuts / sizeof cuts[0]; ++c) {
    const int64_t r0 = cuts[c][0], m = cuts[c][1];
    memset(ri, 0xAB, (size_t)(total > 0 ? total : 1) * 4);
    CHECK(kd_cache_read(p, r0, m, ri, rv) == KD_OK, "read rows [%lld, +%lld)", (long long)r0, (long long)m);
    CHECK(memcmp(ri, idx + r0 * k, (size_t)(m * k) * 4) == 0, "indices of rows [%lld, +%lld)", (long long)r0,
          (long long)m);
    CHECK(memcmp(rv, val + r0 * k * (int64_t)vb, (size_t)(m * k) * vb) == 0, "values of rows [%lld, +%lld)",
          (long long)r0, (long long)m);
  }
  CHECK(kd_cache_read(p, 0, n + 1, ri, rv) == KD_ERR_BAD_SHAPE, "read past the end");
  CHECK(kd_cache_read(p, -1, 1, ri, rv) == KD_ERR_BAD_SHAPE, "negative first row");
  CHECK(kd_cache_read(p, 0, -1, ri, rv) == KD_ERR_BAD_SHAPE, "negative row count");
  CHECK(kd_cache_read(p, INT64_MAX, 1, ri, rv) == KD_ERR_BAD_SHAPE, "first row near INT64_MAX");
  CHECK(kd_cache_read(p, 0, 0, NULL, NULL) == KD_OK, "empty read with no buffers");
  if (n > 0) CHECK(kd_cache_read(p, 0, 1, NULL, rv) == KD_ERR_NULL_POINTER, "read into NULL");
  free(idx);
  free(val);
  free(ri);
  free(rv);
}

static void write_errors(void) {
  char p[512];
  path_of(p, sizeof p, "err.kdc");
  int32_t idx[12] = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11};
  uint16_t val[12] = {0};
  kd_cache_info ok = {3, 100, 4, 0, KD_BF16};
  CHECK(kd_cache_write(NULL, &ok, idx, val) == KD_ERR_NULL_POINTER, "NULL path");
  CHECK(kd_cache_write(p, NULL, idx, val) == KD_ERR_NULL_POINTER, "NULL info");
  CHECK(kd_cache_write(p, &ok, NULL, val) == KD_ERR_NULL_POINTER, "NULL idx");
  CHECK(kd_cache_write(p, &ok, idx, NULL) == KD_ERR_NULL_POINTER, "NULL val");
  const kd_cache_info bad_shapes[] = {
      {-1, 100, 4, 0, KD_BF16},        {3, 0, 1, 0, KD_BF16},     {3, 4194305, 4, 0, KD_BF16},
      {3, 100, 0, 0, KD_BF16},         {3, 100, 101, 0, KD_BF16}, {3, 100000, 65536, 0, KD_BF16},
      {3, 70000, 4, 16, KD_BF16},      {3, 100, 4, 8, KD_BF16},   {((int64_t)1 << 40) / 4 + 1, 100, 4, 0, KD_BF16},
  };
  for (size_t i = 0; i < sizeof bad_shapes / sizeof bad_shapes[0]; ++i)
    CHECK(kd_cache_write(p, &bad_shapes[i], idx, val) == KD_ERR_BAD_SHAPE, "bad shape %zu", i);
  kd_cache_info bad_dt = {3, 100, 4, 0, 7};
  CHECK(kd_cache_write(p, &bad_dt, idx, val) == KD_ERR_BAD_DTYPE, "bad value dtype");
  idx[5] = 100;
  CHECK(kd_cache_write(p, &ok, idx, val) == KD_ERR_IDX_OUT_OF_RANGE, "index == V");
  idx[5] = -1;
  CHECK(kd_cache_write(p, &ok, idx, val) == KD_ERR_IDX_OUT_OF_RANGE, "index -1");
  CHECK(file_size(p) < 0, "a rejected write leaves no file");
  idx[5] = 5;
  char q[600];
  snprintf(q, sizeof q, "%s/no_such_dir/x.kdc", dir);
  CHECK(kd_cache_write(q, &ok, idx, val) == KD_ERR_IO, "write into a missing directory");
  kd_cache_info got;
  CHECK(kd_cache_info_read(p, NULL) == KD_ERR_NULL_POINTER, "info_read into NULL");
  CHECK(kd_cache_info_read(NULL, &got) == KD_ERR_NULL_POINTER, "info_read of NULL path");
  CHECK(kd_cache_info_read(p, &got) == KD_ERR_IO, "info_read of a missing file");
  CHECK(kd_cache_read(p, 0, 0, NULL, NULL) == KD_ERR_IO, "read of a missing file");
}

/* every header field and the file size, each broken on its own */
static void corrupt_files(void) {
  char good[512], bad[512];
  path_of(good, sizeof good, "good.kdc");
  path_of(bad, sizeof bad, "bad.kdc");
  int32_t idx[30];
  float val[30];
  for (int i = 0; i < 30; ++i) {
    idx[i] = (i * 11) % 1000;
    val[i] = (float)i;
  }
  kd_cache_info in = {10, 1000, 3, 0, KD_F32};
  CHECK(kd_cache_write(good, &in, idx, val) == KD_OK, "write the good shard");
  int64_t n = 0;
  unsigned char* g = slurp(good, &n);
  CHECK(g != NULL && n == expected_size(10, 3, 16, KD_F32), "good shard size");
  unsigned char* b = (unsigned char*)malloc((size_t)n + 64);

  struct {
    int off, width;
    uint64_t v;
    const char* what;
  } fields[] = {
      {0, 1, 'X', "magic"},
      {8, 4, 2, "version"},
      {12, 4, 65, "header bytes"},
      {16, 8, 11, "row count one more than the file holds"},
      {16, 8, (uint64_t)1 << 63, "negative row count"},
      {16, 8, (uint64_t)1 << 50, "row count past the overflow bound"},
      {24, 8, 0, "vocabulary 0"},
      {24, 8, 4194305, "vocabulary over the limit"},
      {24, 8, 70000, "vocabulary too large for 16-bit indices"},
      {32, 4, 0, "k 0"},
      {32, 4, 0xFFFFFFFFu, "k -1"},
      {32, 4, 1001, "k > V"},
      {36, 4, 8, "index width 8"},
      {36, 4, 32, "index width 32 with a 16-bit file"},
      {40, 4, 9, "value dtype"},
      {40, 4, KD_BF16, "value dtype bf16 with an f32 file"},
      {44, 4, 1, "reserved field"},
      {48, 8, 0, "index offset"},
      {56, 8, 64, "value offset"},
  };
  kd_cache_info got;
  int32_t ri[30];
  float rv[30];
  for (size_t f = 0; f < sizeof fields / sizeof fields[0]; ++f) {
    memcpy(b, g, (size_t)n);
    if (fields[f].width == 1) b[fields[f].off] = (unsigned char)fields[f].v;
    else if (fields[f].width == 4) put32(b + fields[f].off, (uint32_t)fields[f].v);
    else put64(b + fields[f].off, fields[f].v);
    spit(bad, b, n);
    CHECK(kd_cache_info_read(bad, &got) == KD_ERR_BAD_FORMAT, "header: %s", fields[f].what);
    CHECK(kd_cache_read(bad, 0, 1, ri, rv) == KD_ERR_BAD_FORMAT, "read with header: %s", fields[f].what);
  }
  const int64_t sizes[] = {0, 10, 63, 64, n - 1, n + 1, n + 64};
  for (size_t s = 0; s < sizeof sizes / sizeof sizes[0]; ++s) {
    memcpy(b, g, (size_t)n);
    memset(b + n, 0, 64);
    spit(bad, b, sizes[s]);
    CHECK(kd_cache_info_read(bad, &got) == KD_ERR_BAD_FORMAT, "file of %lld bytes", (long long)sizes[s]);
  }
  /* the good shard still reads */
  CHECK(kd_cache_read(good, 0, 10, ri, rv) == KD_OK && memcmp(ri, idx, sizeof idx) == 0 &&
            memcmp(rv, val, sizeof val) == 0,
        "good shard after the corrupt ones");
  free(g);
  free(b);
}

static void loader_and_writer_errors(void) {
  char a[512], c[512], bad[512], missing[512], prefix[512];
  path_of(a, sizeof a, "la.kdc");
  path_of(c, sizeof c, "lc.kdc");
  path_of(bad, sizeof bad, "bad.kdc");
  path_of(missing, sizeof missing, "missing.kdc");
  path_of(prefix, sizeof prefix, "w");
  int32_t idx[8] = {1, 2, 3, 4, 5, 6, 7, 0};
  uint16_t val[8] = {0};
  kd_cache_info ia = {2, 50, 4, 0, KD_BF16}, ic = {4, 50, 2, 0, KD_BF16};
  CHECK(kd_cache_write(a, &ia, idx, val) == KD_OK && kd_cache_write(c, &ic, idx, val) == KD_OK, "loader shards");
  kd_cache_loader* L = (kd_cache_loader*)1;
  const char* one[] = {a};
  const char* mixed[] = {a, c};
  const char* with_bad[] = {a, bad};
  const char* with_missing[] = {a, missing};
  CHECK(kd_cache_loader_open(NULL, 1, 4, 2, &L) == KD_ERR_NULL_POINTER, "loader: NULL paths");
  CHECK(kd_cache_loader_open(one, 1, 4, 2, NULL) == KD_ERR_NULL_POINTER, "loader: NULL out");
  CHECK(kd_cache_loader_open(one, 0, 4, 2, &L) == KD_ERR_BAD_SHAPE && L == NULL, "loader: no shards");
  CHECK(kd_cache_loader_open(one, 1, 0, 2, &L) == KD_ERR_BAD_SHAPE, "loader: batch 0");
  CHECK(kd_cache_loader_open(one, 1, 4, 1, &L) == KD_ERR_BAD_SHAPE, "loader: prefetch 1");
  CHECK(kd_cache_loader_open(one, 1, 4, 65, &L) == KD_ERR_BAD_SHAPE, "loader: prefetch 65");
  CHECK(kd_cache_loader_open(mixed, 2, 4, 2, &L) == KD_ERR_BAD_FORMAT && L == NULL, "loader: shards disagree on k");
  CHECK(kd_cache_loader_open(with_bad, 2, 4, 2, &L) == KD_ERR_BAD_FORMAT, "loader: a corrupt shard");
  CHECK(kd_cache_loader_open(with_missing, 2, 4, 2, &L) == KD_ERR_IO, "loader: a missing shard");
  const kd_status lo = kd_cache_loader_open(one, 1, 4, 3, &L);
  CHECK(lo == KD_OK || lo == KD_ERR_NO_DEVICE, "loader: valid open gives %d", (int)lo);
  if (lo == KD_OK) {
    kd_cache_info li;
    CHECK(kd_cache_loader_info(L, &li) == KD_OK && li.n_tokens == 2 && li.idx_bits == 32, "loader info");
    CHECK(kd_cache_loader_close(L) == KD_OK, "loader close");
  } else {
    CHECK(L == NULL, "loader: no handle after an error");
  }
  CHECK(kd_cache_loader_close(NULL) == KD_OK, "loader: close NULL");
  CHECK(kd_cache_loader_info(NULL, NULL) == KD_ERR_NULL_POINTER, "loader: info of NULL");
  int64_t rows = -1;
  CHECK(kd_cache_loader_next(NULL, NULL, NULL, &rows, NULL) == KD_ERR_NULL_POINTER, "loader: next of NULL");

  kd_cache_writer* W = (kd_cache_writer*)1;
  kd_cache_info ws = {16, 50, 4, 0, KD_BF16};
  CHECK(kd_cache_writer_open(NULL, &ws, 8, 2, &W) == KD_ERR_NULL_POINTER, "writer: NULL prefix");
  CHECK(kd_cache_writer_open(prefix, NULL, 8, 2, &W) == KD_ERR_NULL_POINTER, "writer: NULL shape");
  CHECK(kd_cache_writer_open(prefix, &ws, 8, 2, NULL) == KD_ERR_NULL_POINTER, "writer: NULL out");
  CHECK(kd_cache_writer_open(prefix, &ws, 0, 2, &W) == KD_ERR_BAD_SHAPE && W == NULL, "writer: batch 0");
  CHECK(kd_cache_writer_open(prefix, &ws, 8, 1, &W) == KD_ERR_BAD_SHAPE, "writer: depth 1");
  CHECK(kd_cache_writer_open(prefix, &ws, 8, 65, &W) == KD_ERR_BAD_SHAPE, "writer: depth 65");
  kd_cache_info w0 = ws, wk = ws, wd = ws;
  w0.n_tokens = 0;
  wk.k = 51;
  wd.val_dtype = 5;
  CHECK(kd_cache_writer_open(prefix, &w0, 8, 2, &W) == KD_ERR_BAD_SHAPE, "writer: shards of 0 rows");
  CHECK(kd_cache_writer_open(prefix, &wk, 8, 2, &W) == KD_ERR_BAD_SHAPE, "writer: k > V");
  CHECK(kd_cache_writer_open(prefix, &wd, 8, 2, &W) == KD_ERR_BAD_DTYPE, "writer: value dtype");
  CHECK(kd_cache_writer_open(prefix, &ws, ((int64_t)1 << 40) / 4 + 1, 2, &W) == KD_ERR_BAD_SHAPE,
        "writer: batch past the overflow bound");
  const kd_status wo = kd_cache_writer_open(prefix, &ws, 8, 2, &W);
  CHECK(wo == KD_OK || wo == KD_ERR_NO_DEVICE, "writer: valid open gives %d", (int)wo);
  if (wo == KD_OK) {
    CHECK(kd_cache_writer_put(W, NULL, NULL, 0, NULL) == KD_OK, "writer: empty put");
    CHECK(kd_cache_writer_put(W, NULL, NULL, 9, NULL) == KD_ERR_BAD_SHAPE, "writer: put over the batch size");
    int64_t shards = -1;
    CHECK(kd_cache_writer_close(W, &shards) == KD_OK && shards == 0, "writer: close with nothing put");
  } else {
    CHECK(W == NULL, "writer: no handle after an error");
  }
  CHECK(kd_cache_writer_put(NULL, NULL, NULL, 1, NULL) == KD_ERR_NULL_POINTER, "writer: put to NULL");
  CHECK(kd_cache_writer_close(NULL, NULL) == KD_OK, "writer: close NULL");
}

/* nothing but the files written on purpose: no temporaries, no empty writer shards */
static void no_stray_files(void) {
  DIR* d = opendir(dir);
  CHECK(d != NULL, "open the scratch directory");
  const char* allowed[] = {"rt.kdc", "good.kdc", "bad.kdc", "la.kdc", "lc.kdc", NULL};
  struct dirent* e;
  while ((e = readdir(d)) != NULL) {
    if (e->d_name[0] == '.') continue;
    int ok = 0;
    for (int i = 0; allowed[i]; ++i) ok = ok || strcmp(e->d_name, allowed[i]) == 0;
    CHECK(ok, "unexpected file %s", e->d_name);
  }
  closedir(d);
}

int main(int argc, char** argv) {
  if (argc > 1) dir = argv[1];
  const int64_t ns[] = {0, 1, 37};
  const struct {
    int64_t vocab;
    int32_t k;
  } shapes[] = {{1, 1}, {7, 5}, {65536, 3}, {65537, 4}, {4194304, 2}};
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
    for (size_t i = 0; i < sizeof ns / sizeof ns[0]; ++i)
      for (int vdt = 0; vdt < 2; ++vdt) {
        round_trip(ns[i], shapes[s].vocab, shapes[s].k, 0, vdt);
        round_trip(ns[i], shapes[s].vocab, shapes[s].k, 32, vdt);
        if (shapes[s].vocab <= 65536) round_trip(ns[i], shapes[s].vocab, shapes[s].k, 16, vdt);
      }
  write_errors();
  corrupt_files();
  loader_and_writer_errors();
  no_stray_files();
  printf("ok %d checks\n", n_checks);
  return 0;
}

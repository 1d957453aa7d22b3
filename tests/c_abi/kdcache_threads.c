/* The cache writer's and loader's background threads under ThreadSanitizer (and,
 * built again, AddressSanitizer), linked with tests/c_abi/hip_host_stub.cpp in place
 * of the HIP runtime, by tests/test_host_sanitized.py:
 *   - the writer: batches of uneven sizes handed over, shards of a fixed row count
 *     read back exactly;
 *   - the loader: the shards streamed back in batches that cross shard boundaries;
 *   - the writer's failure path: an out-of-range index stops it, and only the
 *     shards before the failed one are on disk;
 *   - a loader closed while its thread still reads ahead;
 *   - four writer/loader pairs at once, in four threads.
 *
 * usage: kdcache_threads <scratch directory>; prints "ok <checks>" and exits 0, or
 * names the first failed check and exits 1. */
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/stat.h>

#include "kdcache.h"

static const char* dir = ".";
static long n_checks = 0;
static pthread_mutex_t count_mu = PTHREAD_MUTEX_INITIALIZER;

#define CHECK(cond, ...)                                     \
  do {                                                       \
    pthread_mutex_lock(&count_mu);                           \
    ++n_checks;                                              \
    pthread_mutex_unlock(&count_mu);                         \
    if (!(cond)) {                                           \
      fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                          \
      fprintf(stderr, "\n");                                 \
      exit(1);                                               \
    }                                                        \
  } while (0)

enum { VOCAB = 50000, K = 8 };

static int32_t idx_of(int64_t row, int j, int seed) { return (int32_t)((row * 131 + j * 7919 + seed * 17) % VOCAB); }
static uint16_t val_of(int64_t row, int j, int seed) { return (uint16_t)(row * 3 + j + seed * 1000); }

/* writes `rows` rows in uneven batches through a writer; returns the shard count */
static int64_t write_all(const char* prefix, int64_t rows, int64_t shard, int seed, int64_t bad_row) {
  kd_cache_info in = {shard, VOCAB, K, 0, KD_BF16};
  kd_cache_writer* W = NULL;
  CHECK(kd_cache_writer_open(prefix, &in, 300, 3, &W) == KD_OK && W, "writer open %s", prefix);
  int32_t* bi = (int32_t*)malloc(300 * K * 4);
  uint16_t* bv = (uint16_t*)malloc(300 * K * 2);
  kd_status first_error = KD_OK;
  int64_t r0 = 0;
  for (int b = 0; r0 < rows; ++b) {
    int64_t m = 1 + (b * 97) % 300;
    if (m > rows - r0) m = rows - r0;
    for (int64_t r = 0; r < m; ++r)
      for (int j = 0; j < K; ++j) {
        bi[r * K + j] = r0 + r == bad_row && j == 3 ? VOCAB : idx_of(r0 + r, j, seed);
        bv[r * K + j] = val_of(r0 + r, j, seed);
      }
    const kd_status st = kd_cache_writer_put(W, bi, bv, m, NULL);
    if (st != KD_OK) {
      first_error = st;
      break;
    }
    r0 += m;
  }
  int64_t n = -1;
  const kd_status cs = kd_cache_writer_close(W, &n);
  if (bad_row < 0) {
    CHECK(first_error == KD_OK && cs == KD_OK, "writer %s: put %d close %d", prefix, (int)first_error, (int)cs);
    CHECK(n == (rows + shard - 1) / shard, "writer %s: %lld shards", prefix, (long long)n);
  } else {
    CHECK(cs == KD_ERR_IDX_OUT_OF_RANGE, "writer %s: close gives %d", prefix, (int)cs);
    CHECK(n == bad_row / shard, "writer %s: %lld shards before the failed one", prefix, (long long)n);
  }
  free(bi);
  free(bv);
  return n;
}

static void shard_path(char* out, size_t len, const char* prefix, int64_t i) {
  snprintf(out, len, "%s_%05lld.kdc", prefix, (long long)i);
}

/* reads the shards back through the loader; `stop_after` > 0 closes it early */
static void load_all(const char* prefix, int64_t n_shards, int64_t rows, int seed, int64_t batch, int stop_after) {
  char** paths = (char**)malloc(sizeof(char*) * (size_t)n_shards);
  for (int64_t i = 0; i < n_shards; ++i) {
    paths[i] = (char*)malloc(600);
    shard_path(paths[i], 600, prefix, i);
  }
  kd_cache_loader* L = NULL;
  CHECK(kd_cache_loader_open((const char* const*)paths, (int32_t)n_shards, batch, 3, &L) == KD_OK && L,
        "loader open %s", prefix);
  kd_cache_info li;
  CHECK(kd_cache_loader_info(L, &li) == KD_OK && li.n_tokens == rows && li.k == K, "loader info %s", prefix);
  int32_t* di = (int32_t*)malloc((size_t)(batch * K * 4));
  uint16_t* dv = (uint16_t*)malloc((size_t)(batch * K * 2));
  int64_t r0 = 0;
  int calls = 0;
  for (;;) {
    if (stop_after > 0 && calls == stop_after) break;
    int64_t got = -1;
    CHECK(kd_cache_loader_next(L, di, dv, &got, NULL) == KD_OK, "loader next %s", prefix);
    ++calls;
    if (got == 0) break;
    for (int64_t r = 0; r < got; ++r)
      for (int j = 0; j < K; ++j) {
        if (di[r * K + j] != idx_of(r0 + r, j, seed) || dv[r * K + j] != val_of(r0 + r, j, seed)) {
          CHECK(0, "loader %s: row %lld entry %d", prefix, (long long)(r0 + r), j);
        }
      }
    r0 += got;
  }
  if (stop_after <= 0) CHECK(r0 == rows, "loader %s: %lld rows", prefix, (long long)r0);
  CHECK(kd_cache_loader_close(L) == KD_OK, "loader close %s", prefix);
  for (int64_t i = 0; i < n_shards; ++i) free(paths[i]);
  free(paths);
  free(di);
  free(dv);
}

struct job {
  int seed;
};

static void* pair(void* arg) {
  const int seed = ((struct job*)arg)->seed;
  char prefix[512];
  snprintf(prefix, sizeof prefix, "%s/t%d", dir, seed);
  const int64_t rows = 2500 + 100 * seed;
  const int64_t n = write_all(prefix, rows, 700, seed, -1);
  load_all(prefix, n, rows, seed, 211, 0);
  return NULL;
}

int main(int argc, char** argv) {
  if (argc > 1) dir = argv[1];
  char prefix[512];

  /* one writer, then one loader over its shards */
  snprintf(prefix, sizeof prefix, "%s/a", dir);
  const int64_t n = write_all(prefix, 5000, 1000, 0, -1);
  load_all(prefix, n, 5000, 0, 333, 0);
  load_all(prefix, n, 5000, 0, 5000, 0);

  /* a loader closed while its thread reads ahead */
  load_all(prefix, n, 5000, 0, 64, 3);

  /* the failure path: the bad index is in the third shard of 1,000 rows */
  snprintf(prefix, sizeof prefix, "%s/bad", dir);
  write_all(prefix, 5000, 1000, 1, 2345);
  char p[600];
  struct stat st;
  shard_path(p, sizeof p, prefix, 1);
  CHECK(stat(p, &st) == 0, "shard 1 before the failure is on disk");
  shard_path(p, sizeof p, prefix, 2);
  CHECK(stat(p, &st) != 0, "no shard 2 (the failed one)");
  shard_path(p, sizeof p, prefix, 3);
  CHECK(stat(p, &st) != 0, "no shard 3 after the failure");

  /* four writer/loader pairs at once */
  pthread_t th[4];
  struct job jobs[4];
  for (int i = 0; i < 4; ++i) {
    jobs[i].seed = 10 + i;
    CHECK(pthread_create(&th[i], NULL, pair, &jobs[i]) == 0, "thread %d", i);
  }
  for (int i = 0; i < 4; ++i) pthread_join(th[i], NULL);

  printf("ok %ld checks\n", n_checks);
  return 0;
}

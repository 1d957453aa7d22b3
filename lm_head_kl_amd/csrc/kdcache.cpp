// On-disk teacher cache shards and the streaming loader (C ABI in include/kdcache.h).
//
// The cache holds K (vocabulary index, logit) pairs per token row (the offline
// teacher pass writes it once; training reads it sequentially).  A shard stores
// the index and value arrays separately, in the [rows, K] layouts the loss takes,
// so reading a batch is two sequential reads and an upload.  16-bit indices halve
// the index bytes when the vocabulary has at most 65,536 entries; the reader widens
// them to int32 on the host.
#include <hip/hip_runtime.h>

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "kdcache.h"

namespace {

constexpr char kMagic[8] = {'K', 'D', 'C', 'A', 'C', 'H', 'E', '1'};
constexpr uint32_t kVersion = 1;
constexpr int64_t kHeader = 64;
constexpr int64_t kMaxVocab = 4194304;
constexpr int32_t kMaxK = 65535;
constexpr int64_t kIoBlock = int64_t(1) << 24;   // bytes per read/write call and per widening pass

int64_t round64(int64_t x) { return (x + 63) & ~int64_t(63); }

int val_bytes(int32_t dt) { return dt == KD_F32 ? 4 : 2; }

// Shape checks shared by the writer and the header parser.
kd_status check_shape(int64_t n, int64_t vocab, int32_t k, int32_t idx_bits, int32_t val_dtype) {
  if (n < 0 || vocab < 1 || vocab > kMaxVocab || k < 1 || k > kMaxK || k > vocab) return KD_ERR_BAD_SHAPE;
  if (idx_bits != 16 && idx_bits != 32) return KD_ERR_BAD_SHAPE;
  if (idx_bits == 16 && vocab > 65536) return KD_ERR_BAD_SHAPE;
  if (val_dtype != KD_F32 && val_dtype != KD_BF16) return KD_ERR_BAD_DTYPE;
  if (n > (int64_t(1) << 40) / k) return KD_ERR_BAD_SHAPE;   // keeps every byte count far from overflow
  return KD_OK;
}

struct Layout {
  int64_t idx_off, val_off, end;
};

Layout layout_of(int64_t n, int32_t k, int32_t idx_bits, int32_t val_dtype) {
  Layout l;
  l.idx_off = kHeader;
  l.val_off = round64(l.idx_off + n * k * (idx_bits / 8));
  l.end = l.val_off + n * k * val_bytes(val_dtype);
  return l;
}

void put32(unsigned char* p, uint32_t v) {
  for (int i = 0; i < 4; ++i) p[i] = (unsigned char)(v >> (8 * i));
}
void put64(unsigned char* p, uint64_t v) {
  for (int i = 0; i < 8; ++i) p[i] = (unsigned char)(v >> (8 * i));
}
uint32_t get32(const unsigned char* p) {
  uint32_t v = 0;
  for (int i = 0; i < 4; ++i) v |= uint32_t(p[i]) << (8 * i);
  return v;
}
uint64_t get64(const unsigned char* p) {
  uint64_t v = 0;
  for (int i = 0; i < 8; ++i) v |= uint64_t(p[i]) << (8 * i);
  return v;
}

bool write_all(int fd, const void* buf, int64_t bytes) {
  const char* p = (const char*)buf;
  while (bytes > 0) {
    const ssize_t w = ::write(fd, p, (size_t)std::min(bytes, kIoBlock));
    if (w <= 0) return false;
    p += w;
    bytes -= w;
  }
  return true;
}

bool read_at(int fd, void* buf, int64_t bytes, int64_t off) {
  char* p = (char*)buf;
  while (bytes > 0) {
    const ssize_t r = ::pread(fd, p, (size_t)std::min(bytes, kIoBlock), (off_t)off);
    if (r <= 0) return false;
    p += r;
    bytes -= r;
    off += r;
  }
  return true;
}

// An open, validated shard.
struct Shard {
  int fd = -1;
  kd_cache_info info{};
  Layout lay{};
};

kd_status open_shard(const char* path, Shard* s) {
  if (!path) return KD_ERR_NULL_POINTER;
  const int fd = ::open(path, O_RDONLY | O_CLOEXEC);
  if (fd < 0) return KD_ERR_IO;
  unsigned char h[kHeader];
  struct stat st;
  if (!read_at(fd, h, kHeader, 0) || ::fstat(fd, &st) != 0) {
    ::close(fd);
    return KD_ERR_BAD_FORMAT;   // shorter than a header
  }
  kd_cache_info in{};
  in.n_tokens = (int64_t)get64(h + 16);
  in.vocab = (int64_t)get64(h + 24);
  in.k = (int32_t)get32(h + 32);
  in.idx_bits = (int32_t)get32(h + 36);
  in.val_dtype = (int32_t)get32(h + 40);
  bool ok = std::memcmp(h, kMagic, 8) == 0 && get32(h + 8) == kVersion && get32(h + 12) == kHeader &&
            get32(h + 44) == 0 && check_shape(in.n_tokens, in.vocab, in.k, in.idx_bits, in.val_dtype) == KD_OK;
  Layout lay{};
  if (ok) {
    lay = layout_of(in.n_tokens, in.k, in.idx_bits, in.val_dtype);
    ok = (int64_t)get64(h + 48) == lay.idx_off && (int64_t)get64(h + 56) == lay.val_off &&
         (int64_t)st.st_size == lay.end;
  }
  if (!ok) {
    ::close(fd);
    return KD_ERR_BAD_FORMAT;
  }
  s->fd = fd;
  s->info = in;
  s->lay = lay;
  return KD_OK;
}

// Rows [row0, row0 + rows) of an open shard into host buffers (int32 indices).
kd_status read_rows(const Shard& s, int64_t row0, int64_t rows, int32_t* idx, void* val) {
  const int64_t k = s.info.k;
  if (rows == 0) return KD_OK;
  if (s.info.idx_bits == 32) {
    if (!read_at(s.fd, idx, rows * k * 4, s.lay.idx_off + row0 * k * 4)) return KD_ERR_IO;
  } else {
    // widen in blocks, front to back
    std::vector<uint16_t> tmp;
    const int64_t total = rows * k;
    const int64_t blk = std::min<int64_t>(total, kIoBlock / 2);
    try {
      tmp.resize((size_t)blk);
    } catch (const std::bad_alloc&) {
      return KD_ERR_IO;
    }
    for (int64_t e = 0; e < total; e += blk) {
      const int64_t m = std::min(blk, total - e);
      if (!read_at(s.fd, tmp.data(), m * 2, s.lay.idx_off + (row0 * k + e) * 2)) return KD_ERR_IO;
      for (int64_t i = 0; i < m; ++i) idx[e + i] = (int32_t)tmp[(size_t)i];
    }
  }
  const int vb = val_bytes(s.info.val_dtype);
  if (!read_at(s.fd, val, rows * k * vb, s.lay.val_off + row0 * k * vb)) return KD_ERR_IO;
  return KD_OK;
}

}  // namespace

extern "C" kd_status kd_cache_write(const char* path, const kd_cache_info* info, const int32_t* idx,
                                    const void* val) {
  if (!path || !info) return KD_ERR_NULL_POINTER;
  const int64_t n = info->n_tokens, vocab = info->vocab;
  const int32_t k = info->k;
  int32_t bits = info->idx_bits;
  if (bits == 0) bits = vocab <= 65536 ? 16 : 32;
  const kd_status sh = check_shape(n, vocab, k, bits, info->val_dtype);
  if (sh != KD_OK) return sh;
  const int64_t total = n * k;
  if (total > 0 && (!idx || !val)) return KD_ERR_NULL_POINTER;
  for (int64_t i = 0; i < total; ++i)
    if (idx[i] < 0 || idx[i] >= vocab) return KD_ERR_IDX_OUT_OF_RANGE;

  const Layout lay = layout_of(n, k, bits, info->val_dtype);
  unsigned char h[kHeader];
  std::memset(h, 0, sizeof(h));
  std::memcpy(h, kMagic, 8);
  put32(h + 8, kVersion);
  put32(h + 12, kHeader);
  put64(h + 16, (uint64_t)n);
  put64(h + 24, (uint64_t)vocab);
  put32(h + 32, (uint32_t)k);
  put32(h + 36, (uint32_t)bits);
  put32(h + 40, (uint32_t)info->val_dtype);
  put64(h + 48, (uint64_t)lay.idx_off);
  put64(h + 56, (uint64_t)lay.val_off);

  // unique per process and per call, so concurrent writers never share a temporary
  static std::atomic<unsigned long> serial{0};
  const std::string tmp = std::string(path) + ".tmp." + std::to_string((long)::getpid()) + "." +
                          std::to_string(serial.fetch_add(1));
  const int fd = ::open(tmp.c_str(), O_WRONLY | O_CREAT | O_TRUNC | O_CLOEXEC, 0644);
  if (fd < 0) return KD_ERR_IO;
  bool ok = write_all(fd, h, kHeader);
  if (ok && bits == 32) {
    ok = write_all(fd, idx, total * 4);
  } else if (ok) {
    std::vector<uint16_t> narrow;
    const int64_t blk = std::min<int64_t>(total, kIoBlock / 2);
    try {
      narrow.resize((size_t)std::max<int64_t>(blk, 1));
    } catch (const std::bad_alloc&) {
      ok = false;
    }
    for (int64_t e = 0; ok && e < total; e += blk) {
      const int64_t m = std::min(blk, total - e);
      for (int64_t i = 0; i < m; ++i) narrow[(size_t)i] = (uint16_t)idx[e + i];
      ok = write_all(fd, narrow.data(), m * 2);
    }
  }
  const int64_t pad = lay.val_off - (lay.idx_off + total * (bits / 8));
  if (ok && pad > 0) {
    const unsigned char zero[64] = {0};
    ok = write_all(fd, zero, pad);
  }
  if (ok) ok = write_all(fd, val, total * val_bytes(info->val_dtype));
  if (::close(fd) != 0) ok = false;
  if (!ok || ::rename(tmp.c_str(), path) != 0) {
    ::unlink(tmp.c_str());
    return KD_ERR_IO;
  }
  return KD_OK;
}

extern "C" kd_status kd_cache_info_read(const char* path, kd_cache_info* out) {
  if (!out) return KD_ERR_NULL_POINTER;
  Shard s;
  const kd_status st = open_shard(path, &s);
  if (st != KD_OK) return st;
  *out = s.info;
  ::close(s.fd);
  return KD_OK;
}

extern "C" kd_status kd_cache_read(const char* path, int64_t row0, int64_t rows, int32_t* idx, void* val) {
  Shard s;
  const kd_status st = open_shard(path, &s);
  if (st != KD_OK) return st;
  kd_status r = KD_OK;
  if (row0 < 0 || rows < 0 || row0 > s.info.n_tokens - rows) r = KD_ERR_BAD_SHAPE;
  else if (rows > 0 && (!idx || !val)) r = KD_ERR_NULL_POINTER;
  else r = read_rows(s, row0, rows, idx, val);
  ::close(s.fd);
  return r;
}

// ---- streaming loader

struct kd_cache_loader {
  std::vector<Shard> shards;
  std::vector<int64_t> first;   // first global row of each shard
  kd_cache_info info{};         // n_tokens = total rows
  int64_t batch = 0, n_batches = 0;
  int nslots = 0;
  struct Slot {
    int32_t* idx = nullptr;
    void* val = nullptr;
    int64_t rows = 0;
    hipEvent_t done = nullptr;
    bool pending = false;       // copies enqueued from this slot, maybe not finished
  };
  std::vector<Slot> slots;
  std::thread producer;
  std::mutex mu;
  std::condition_variable cv;
  int64_t produced = 0, consumed = 0;
  bool stop = false;
  kd_status err = KD_OK;

  // rows [g0, g0 + rows) of the concatenated shards into slot s
  kd_status fill(Slot& s, int64_t g0, int64_t rows) {
    const int64_t k = info.k;
    int64_t done = 0;
    size_t i = std::upper_bound(first.begin(), first.end(), g0) - first.begin() - 1;
    while (done < rows) {
      const Shard& sh = shards[i];
      const int64_t r0 = g0 + done - first[i];
      const int64_t m = std::min(rows - done, sh.info.n_tokens - r0);
      if (m > 0) {
        const kd_status st =
            read_rows(sh, r0, m, s.idx + done * k, (char*)s.val + done * k * val_bytes(info.val_dtype));
        if (st != KD_OK) return st;
        done += m;
      }
      ++i;
    }
    s.rows = rows;
    return KD_OK;
  }

  void run() {
    for (int64_t b = 0; b < n_batches; ++b) {
      Slot& s = slots[(size_t)(b % nslots)];
      {
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return stop || b - consumed < nslots; });
        if (stop) return;
      }
      // the consumer has handed this slot's previous batch to the device: wait for
      // those copies before overwriting the pinned buffers
      if (s.pending) {
        if (hipEventSynchronize(s.done) != hipSuccess) {
          std::lock_guard<std::mutex> lk(mu);
          err = KD_ERR_LAUNCH;
          cv.notify_all();
          return;
        }
        s.pending = false;
      }
      const int64_t g0 = b * batch;
      const kd_status st = fill(s, g0, std::min(batch, info.n_tokens - g0));
      std::lock_guard<std::mutex> lk(mu);
      if (st != KD_OK) {
        err = st;
        cv.notify_all();
        return;
      }
      ++produced;
      cv.notify_all();
    }
  }

  void release() {
    for (auto& s : slots) {
      if (s.done) {
        if (s.pending) (void)hipEventSynchronize(s.done);
        (void)hipEventDestroy(s.done);
      }
      if (s.idx) (void)hipHostFree(s.idx);
      if (s.val) (void)hipHostFree(s.val);
    }
    slots.clear();
    for (auto& sh : shards)
      if (sh.fd >= 0) ::close(sh.fd);
    shards.clear();
  }
};

extern "C" kd_status kd_cache_loader_open(const char* const* paths, int32_t n_paths, int64_t batch_tokens,
                                          int32_t prefetch, kd_cache_loader** out) {
  if (!paths || !out) return KD_ERR_NULL_POINTER;
  *out = nullptr;
  if (n_paths < 1 || batch_tokens < 1 || prefetch < 2 || prefetch > 64) return KD_ERR_BAD_SHAPE;
  kd_cache_loader* L = new (std::nothrow) kd_cache_loader;
  if (!L) return KD_ERR_IO;
  kd_status st = KD_OK;
  int64_t total = 0;
  for (int32_t i = 0; i < n_paths && st == KD_OK; ++i) {
    Shard s;
    st = open_shard(paths[i], &s);
    if (st != KD_OK) break;
    L->shards.push_back(s);
    const kd_cache_info& a = L->shards[0].info;
    if (s.info.vocab != a.vocab || s.info.k != a.k || s.info.val_dtype != a.val_dtype) st = KD_ERR_BAD_FORMAT;
    L->first.push_back(total);
    total += s.info.n_tokens;
  }
  if (st == KD_OK && total > (int64_t(1) << 40) / L->shards[0].info.k) st = KD_ERR_BAD_SHAPE;
  if (st == KD_OK) {
    L->info = L->shards[0].info;
    L->info.n_tokens = total;
    L->info.idx_bits = 32;   // as handed out
    L->batch = std::min<int64_t>(batch_tokens, std::max<int64_t>(total, 1));
    L->n_batches = (total + L->batch - 1) / L->batch;
    L->nslots = prefetch;
    L->slots.resize((size_t)prefetch);
    const size_t ib = (size_t)(L->batch * L->info.k * 4);
    const size_t vb = (size_t)(L->batch * L->info.k * val_bytes(L->info.val_dtype));
    for (auto& s : L->slots) {
      if (hipHostMalloc((void**)&s.idx, ib, hipHostMallocDefault) != hipSuccess ||
          hipHostMalloc(&s.val, vb, hipHostMallocDefault) != hipSuccess ||
          hipEventCreateWithFlags(&s.done, hipEventDisableTiming) != hipSuccess) {
        st = KD_ERR_NO_DEVICE;
        break;
      }
    }
  }
  if (st != KD_OK) {
    L->release();
    delete L;
    return st;
  }
  try {
    L->producer = std::thread([L] { L->run(); });
  } catch (...) {
    L->release();
    delete L;
    return KD_ERR_IO;
  }
  *out = L;
  return KD_OK;
}

extern "C" kd_status kd_cache_loader_info(const kd_cache_loader* L, kd_cache_info* out) {
  if (!L || !out) return KD_ERR_NULL_POINTER;
  *out = L->info;
  return KD_OK;
}

extern "C" kd_status kd_cache_loader_next(kd_cache_loader* L, int32_t* idx_dev, void* val_dev, int64_t* rows,
                                          void* stream) {
  if (!L || !rows) return KD_ERR_NULL_POINTER;
  *rows = 0;
  std::unique_lock<std::mutex> lk(L->mu);
  if (L->consumed == L->n_batches) return KD_OK;
  if (!idx_dev || !val_dev) return KD_ERR_NULL_POINTER;
  L->cv.wait(lk, [&] { return L->produced > L->consumed || L->err != KD_OK; });
  if (L->produced <= L->consumed) return L->err;
  auto& s = L->slots[(size_t)(L->consumed % L->nslots)];
  lk.unlock();
  const hipStream_t st = (hipStream_t)stream;
  const int64_t k = L->info.k;
  if (hipMemcpyAsync(idx_dev, s.idx, (size_t)(s.rows * k * 4), hipMemcpyHostToDevice, st) != hipSuccess ||
      hipMemcpyAsync(val_dev, s.val, (size_t)(s.rows * k * val_bytes(L->info.val_dtype)), hipMemcpyHostToDevice,
                     st) != hipSuccess ||
      hipEventRecord(s.done, st) != hipSuccess)
    return KD_ERR_LAUNCH;
  lk.lock();
  s.pending = true;
  *rows = s.rows;
  ++L->consumed;
  L->cv.notify_all();
  return KD_OK;
}

extern "C" kd_status kd_cache_loader_close(kd_cache_loader* L) {
  if (!L) return KD_OK;
  {
    std::lock_guard<std::mutex> lk(L->mu);
    L->stop = true;
    L->cv.notify_all();
  }
  if (L->producer.joinable()) L->producer.join();
  L->release();
  delete L;
  return KD_OK;
}

// ---- streaming writer

struct kd_cache_writer {
  std::string prefix;
  kd_cache_info info{};          // n_tokens = rows per full shard
  int64_t max_batch = 0;
  int nslots = 0;
  struct Slot {
    int32_t* idx = nullptr;
    void* val = nullptr;
    int64_t rows = 0;
    hipEvent_t done = nullptr;
  };
  std::vector<Slot> slots;
  std::vector<int32_t> sidx;     // the shard being assembled
  std::vector<unsigned char> sval;
  int64_t srows = 0;
  int64_t shards_written = 0;
  std::thread worker;
  std::mutex mu;
  std::condition_variable cv;
  int64_t queued = 0, drained = 0;   // batches put / batches moved into shards
  bool closing = false;
  kd_status err = KD_OK;

  std::string shard_path(int64_t i) const {
    char num[32];
    std::snprintf(num, sizeof num, "_%05lld.kdc", (long long)i);
    return prefix + num;
  }

  kd_status flush() {
    if (srows == 0) return KD_OK;
    kd_cache_info in = info;
    in.n_tokens = srows;
    const kd_status st = kd_cache_write(shard_path(shards_written).c_str(), &in, sidx.data(), sval.data());
    if (st == KD_OK) ++shards_written;
    srows = 0;
    return st;
  }

  // rows of one slot into the shard buffer, writing every shard that fills up
  kd_status take(const Slot& s) {
    const int64_t k = info.k, vb = val_bytes(info.val_dtype);
    int64_t done = 0;
    while (done < s.rows) {
      const int64_t m = std::min(s.rows - done, info.n_tokens - srows);
      std::memcpy(sidx.data() + srows * k, s.idx + done * k, (size_t)(m * k * 4));
      std::memcpy(sval.data() + srows * k * vb, (const char*)s.val + done * k * vb, (size_t)(m * k * vb));
      srows += m;
      done += m;
      if (srows == info.n_tokens) {
        const kd_status st = flush();
        if (st != KD_OK) return st;
      }
    }
    return KD_OK;
  }

  // After the first error no further shard is written (a failed shard leaves no
  // file), so the shards on disk are always the leading rows, complete and in order;
  // later batches are only drained.
  void run() {
    bool failed = false;
    for (;;) {
      int64_t b;
      {
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return queued > drained || closing; });
        if (queued == drained) break;   // closing, nothing left
        b = drained;
      }
      Slot& s = slots[(size_t)(b % nslots)];
      kd_status st = hipEventSynchronize(s.done) == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
      if (st == KD_OK && !failed) st = take(s);
      failed = failed || st != KD_OK;
      std::lock_guard<std::mutex> lk(mu);
      if (st != KD_OK && err == KD_OK) err = st;
      ++drained;
      cv.notify_all();
    }
    const kd_status st = failed ? KD_OK : flush();
    std::lock_guard<std::mutex> lk(mu);
    if (st != KD_OK && err == KD_OK) err = st;
  }

  void release() {
    for (auto& s : slots) {
      if (s.done) (void)hipEventDestroy(s.done);
      if (s.idx) (void)hipHostFree(s.idx);
      if (s.val) (void)hipHostFree(s.val);
    }
    slots.clear();
  }
};

extern "C" kd_status kd_cache_writer_open(const char* prefix, const kd_cache_info* shard, int64_t max_batch_tokens,
                                          int32_t depth, kd_cache_writer** out) {
  if (!prefix || !shard || !out) return KD_ERR_NULL_POINTER;
  *out = nullptr;
  kd_cache_info in = *shard;
  if (in.idx_bits == 0) in.idx_bits = in.vocab <= 65536 ? 16 : 32;
  if (in.n_tokens < 1 || max_batch_tokens < 1 || depth < 2 || depth > 64) return KD_ERR_BAD_SHAPE;
  const kd_status sh = check_shape(in.n_tokens, in.vocab, in.k, in.idx_bits, in.val_dtype);
  if (sh != KD_OK) return sh;
  if (max_batch_tokens > (int64_t(1) << 40) / in.k) return KD_ERR_BAD_SHAPE;
  kd_cache_writer* W = new (std::nothrow) kd_cache_writer;
  if (!W) return KD_ERR_IO;
  W->prefix = prefix;
  W->info = in;
  W->max_batch = max_batch_tokens;
  W->nslots = depth;
  kd_status st = KD_OK;
  try {
    W->sidx.resize((size_t)(in.n_tokens * in.k));
    W->sval.resize((size_t)(in.n_tokens * in.k * val_bytes(in.val_dtype)));
  } catch (const std::bad_alloc&) {
    st = KD_ERR_IO;
  }
  W->slots.resize((size_t)depth);
  const size_t ib = (size_t)(max_batch_tokens * in.k * 4);
  const size_t vb = (size_t)(max_batch_tokens * in.k * val_bytes(in.val_dtype));
  for (auto& s : W->slots) {
    if (st != KD_OK) break;
    if (hipHostMalloc((void**)&s.idx, ib, hipHostMallocDefault) != hipSuccess ||
        hipHostMalloc(&s.val, vb, hipHostMallocDefault) != hipSuccess ||
        hipEventCreateWithFlags(&s.done, hipEventDisableTiming) != hipSuccess)
      st = KD_ERR_NO_DEVICE;
  }
  if (st == KD_OK) {
    try {
      W->worker = std::thread([W] { W->run(); });
    } catch (...) {
      st = KD_ERR_IO;
    }
  }
  if (st != KD_OK) {
    W->release();
    delete W;
    return st;
  }
  *out = W;
  return KD_OK;
}

extern "C" kd_status kd_cache_writer_put(kd_cache_writer* W, const int32_t* idx_dev, const void* val_dev,
                                         int64_t rows, void* stream) {
  if (!W) return KD_ERR_NULL_POINTER;
  if (rows < 0 || rows > W->max_batch) return KD_ERR_BAD_SHAPE;
  if (rows == 0) return KD_OK;
  if (!idx_dev || !val_dev) return KD_ERR_NULL_POINTER;
  std::unique_lock<std::mutex> lk(W->mu);
  if (W->err != KD_OK) return W->err;
  // a slot is free once the worker has moved its previous batch into a shard
  W->cv.wait(lk, [&] { return W->queued - W->drained < W->nslots || W->err != KD_OK; });
  if (W->err != KD_OK) return W->err;
  auto& s = W->slots[(size_t)(W->queued % W->nslots)];
  lk.unlock();
  const hipStream_t st = (hipStream_t)stream;
  const int64_t k = W->info.k;
  if (hipMemcpyAsync(s.idx, idx_dev, (size_t)(rows * k * 4), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(s.val, val_dev, (size_t)(rows * k * val_bytes(W->info.val_dtype)), hipMemcpyDeviceToHost,
                     st) != hipSuccess ||
      hipEventRecord(s.done, st) != hipSuccess)
    return KD_ERR_LAUNCH;
  s.rows = rows;
  lk.lock();
  ++W->queued;
  W->cv.notify_all();
  return KD_OK;
}

extern "C" kd_status kd_cache_writer_close(kd_cache_writer* W, int64_t* n_shards) {
  if (!W) return KD_OK;
  {
    std::lock_guard<std::mutex> lk(W->mu);
    W->closing = true;
    W->cv.notify_all();
  }
  if (W->worker.joinable()) W->worker.join();
  const kd_status st = W->err;
  if (n_shards) *n_shards = W->shards_written;
  W->release();
  delete W;
  return st;
}

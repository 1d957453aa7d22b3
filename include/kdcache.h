/*
 * kdcache.h - C ABI of the on-disk teacher cache, its streaming writer and its
 * streaming loader: the storage side of offline top-K distillation, next to the
 * loss in kdkl.h.
 *
 * Sources (web pages about arXiv 2608.03796):
 *   [wiki] llm-wiki study note "LLM 지식 증류 효율화 ...":
 *          "핵심 아이디어 1: Offline Top-K Logits": the teacher runs once and K
 *          (vocabulary index, logit) pairs per token position are stored;
 *          "운영 적용 가이드", "사전 계산(Pre-computation) 파이프라인": the cache is
 *          written once after the teacher pass; 16-bit indices with bf16 values
 *          are the suggested format; "캐시 크기 추정": size = tokens x K x
 *          (index bytes + value bytes); "실용 팁": 16-bit indices suffice when the
 *          vocabulary has fewer than 65,536 entries, the cache is read
 *          sequentially, and loading should prefetch ahead of training.
 *   [mv]   mind-verse.de, section "1. Offline-Destillation": one cache serves
 *          many training runs.
 *
 * Shard file (all integers little-endian; one shard = a contiguous range of token
 * rows; a cache is one or more shards read in order):
 *   offset  size  field
 *        0     8  magic "KDCACHE1"
 *        8     4  version (1)
 *       12     4  header bytes (64)
 *       16     8  n_tokens  (rows in this shard, >= 0)
 *       24     8  vocab     (V, 1 <= V <= 4194304)
 *       32     4  k         (entries per row, 1 <= k <= min(V, 65535))
 *       36     4  idx_bits  (16: uint16 indices, needs V <= 65536; 32: int32)
 *       40     4  val_dtype (kd_dtype: KD_F32 or KD_BF16)
 *       44     4  reserved (0)
 *       48     8  idx offset (64)
 *       56     8  val offset (idx offset + n_tokens*k*idx_bits/8, rounded up to 64)
 *   then the [n_tokens, k] index array and the [n_tokens, k] value array, both
 *   row-major, i.e. exactly the idx [N, K] and val [N, K] inputs of kdkl.h.  The
 *   file is 64 + N*K*idx_bytes, padded to 64, + N*K*val_bytes long.
 *
 * Conventions:
 *   - Paths are NUL-terminated; host buffers are plain pointers owned by the
 *     caller; the loader's device buffers are the caller's too.
 *   - Every call returns a kd_status (kdkl.h): KD_ERR_IO when a file cannot be
 *     opened, read or written; KD_ERR_BAD_FORMAT when a header or a file size does
 *     not match the layout above (or shards of one loader disagree on vocab, k or
 *     val_dtype); KD_ERR_IDX_OUT_OF_RANGE when a written index is outside [0, V).
 *     Nothing aborts, prints or throws.
 */
#ifndef KDCACHE_H
#define KDCACHE_H

#include <stddef.h>
#include <stdint.h>

#include "kdkl.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Shape of one shard. */
typedef struct {
  int64_t n_tokens;   /* rows */
  int64_t vocab;      /* V */
  int32_t k;          /* entries per row */
  int32_t idx_bits;   /* 16 or 32 on disk (0 in kd_cache_write: 16 when V <= 65536, else 32) */
  int32_t val_dtype;  /* KD_F32 or KD_BF16 */
} kd_cache_info;

/* Writes one shard ([wiki] "사전 계산(Pre-computation) 파이프라인", step 3).
 *   idx [n_tokens, k] int32 host, every value in [0, vocab);
 *   val [n_tokens, k] host, val_dtype elements (bf16 as its 16-bit pattern).
 * The file is written under a temporary name and renamed when complete, so a
 * reader never sees a partial shard. */
kd_status kd_cache_write(const char* path, const kd_cache_info* info, const int32_t* idx, const void* val);

/* Reads and validates a shard header (and the file size) into *out. */
kd_status kd_cache_info_read(const char* path, kd_cache_info* out);

/* Reads rows [row0, row0 + rows) of a shard into host buffers: idx as int32
 * (16-bit indices are widened), val in the shard's val_dtype. */
kd_status kd_cache_read(const char* path, int64_t row0, int64_t rows, int32_t* idx, void* val);

/* Streaming loader ([wiki] "실용 팁": sequential reads, prefetch ahead of
 * training).  It reads the shards in order as one sequence of rows and hands it
 * out in batches of batch_tokens rows (the last one may be shorter; batches cross
 * shard boundaries).  A background thread fills a ring of `prefetch` (>= 2)
 * batches in pinned host memory (hipHostMalloc; the loader allocates no device
 * memory).  Not thread-safe: one consumer per loader. */
typedef struct kd_cache_loader kd_cache_loader;

kd_status kd_cache_loader_open(const char* const* paths, int32_t n_paths, int64_t batch_tokens,
                               int32_t prefetch, kd_cache_loader** out);

/* Shape shared by the loader's shards: n_tokens is their total, idx_bits 32 (the
 * loader hands indices out as int32). */
kd_status kd_cache_loader_info(const kd_cache_loader* loader, kd_cache_info* out);

/* Next batch: enqueues the copies of its rows to the device buffers idx_dev
 * [batch_tokens, k] int32 and val_dev [batch_tokens, k] val_dtype on `stream`
 * (hipStream_t; NULL = default) and writes the row count to *rows (0 once every
 * row has been handed out).  It waits only for the background thread to have
 * read that batch; the thread refills a slot after the copies out of it have
 * completed.  Errors of the background thread's reads are returned here. */
kd_status kd_cache_loader_next(kd_cache_loader* loader, int32_t* idx_dev, void* val_dev, int64_t* rows,
                               void* stream);

/* Stops the background thread and frees the loader (NULL is accepted). */
kd_status kd_cache_loader_close(kd_cache_loader* loader);

/* Streaming writer: the storing end of the teacher pass ([wiki] "사전 계산
 * (Pre-computation) 파이프라인", steps 2-3: the teacher runs over the whole dataset
 * and the top-K pairs of every position are stored).  Batches of rows that are on
 * the device (such as kd_topk_cache_build's outputs) are handed over as they are
 * produced; a background thread assembles them into shards of shard->n_tokens rows
 * and writes each one as with kd_cache_write, named <prefix>_00000.kdc,
 * <prefix>_00001.kdc, ... (the last shard holds the remaining rows).
 *   shard    vocab, k, idx_bits (0: 16 when V <= 65536, else 32), val_dtype, and
 *            n_tokens = rows per shard (>= 1);
 *   max_batch_tokens  the most rows one kd_cache_writer_put may hand over;
 *   depth    pinned host batch buffers in flight (2..64).
 * Host memory: depth pinned buffers of max_batch_tokens rows plus one shard of
 * rows; the writer allocates no device memory.  Not thread-safe: one producer per
 * writer. */
typedef struct kd_cache_writer kd_cache_writer;

kd_status kd_cache_writer_open(const char* prefix, const kd_cache_info* shard, int64_t max_batch_tokens,
                               int32_t depth, kd_cache_writer** out);

/* Hands over `rows` rows (0 <= rows <= max_batch_tokens): idx_dev [rows, k] int32
 * and val_dev [rows, k] val_dtype, device buffers that must stay unchanged until
 * the copies enqueued on `stream` (hipStream_t; NULL = default) have run.  The
 * call waits only for a free host buffer, never for the copies or the disk.
 * Indices are checked when their shard is written; an error of the background
 * thread (KD_ERR_IO, KD_ERR_IDX_OUT_OF_RANGE, ...) is returned by the next put and
 * by close. */
kd_status kd_cache_writer_put(kd_cache_writer* writer, const int32_t* idx_dev, const void* val_dev, int64_t rows,
                              void* stream);

/* Writes the last shard, stops the thread, frees the writer (NULL is accepted)
 * and returns the first error of any shard write; *n_shards (may be NULL) gets
 * the number of shards written.  After an error no further shard is written, so
 * the n_shards files on disk always hold the first n_shards * shard->n_tokens
 * rows handed over, complete and in order. */
kd_status kd_cache_writer_close(kd_cache_writer* writer, int64_t* n_shards);

#ifdef __cplusplus
}
#endif
#endif /* KDCACHE_H */

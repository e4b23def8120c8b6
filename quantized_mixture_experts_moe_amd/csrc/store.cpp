// Expert store on local storage: the per-expert blobs of every layer in one
// file, read on demand with bounded-parallel pread into page-locked host
// buffers, bypassing the page cache.
//
// The pages stream each token's missing experts from SSD with parallel pread
// calls into buffers the GPU reads directly, rather than through mmap, whose
// page faults made a cold expert cost about 10 ms against 2.8-3 ms
// (hndistilled.com, "Enfoque tecnico (MoE + transmision desde SSD)";
// yodev.dev, "Por que pread y no mmap"; es.news.hada.io, "Proceso de
// generacion de tokens").  Here the buffers are pinned host memory, and the
// pool copies them into its HBM slots.
#include "store.h"

#include <errno.h>
#include <fcntl.h>
#include <stdlib.h>
#include <string.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

namespace moe {

size_t store_stride(int D, int F) {
  const size_t b = blob_layout(D, F).total;
  return (b + kStoreAlign - 1) / kStoreAlign * kStoreAlign;
}

}  // namespace moe

// A fixed set of reader threads; a batch of (offset, length, destination)
// pieces is spread over them, and the caller waits for the batch.
struct moe_store {
  int fd = -1;
  int n_layers = 0, E = 0, D = 0, F = 0;
  size_t stride = 0, blob = 0;
  bool direct = false;
  const uint8_t *map = nullptr;  // MOE_STORE_MMAP: the whole file mapped
  size_t file_bytes = 0;
  moe_store_stats stats{};

  struct Piece {
    off_t off;
    size_t len;
    uint8_t *dst;
  };
  std::vector<std::thread> workers;
  std::mutex mu;
  std::condition_variable cv_work, cv_done;
  std::vector<Piece> queue;
  size_t next = 0, pending = 0;
  int failed = 0;
  bool stop = false;
  std::vector<uint8_t> inline_scratch;  // bounce buffer of the calling thread (one reader)

  // Direct reads land in a bounce buffer of the reading thread (then copied
  // out) once a destination has refused them: memory that the kernel cannot
  // pin for the device's DMA, such as page-locked buffers that the GPU driver
  // mapped, fails direct I/O with EFAULT or EINVAL.
  std::atomic<bool> bounce{false};

  static int pread_all(int fd, uint8_t *dst, size_t len, off_t off) {
    size_t done = 0;
    while (done < len) {
      const ssize_t r = pread(fd, dst + done, len - done, off + (off_t)done);
      if (r < 0) {
        if (errno == EINTR) continue;
        return errno ? errno : EIO;
      }
      if (r == 0) return EIO;  // past the end of the file
      done += (size_t)r;
    }
    return 0;
  }

  // One piece: pread until it is complete (or mapped memory copied).
  // `scratch` is the calling thread's bounce buffer.
  int read_piece(const Piece &p, std::vector<uint8_t> &scratch) {
    if (map) {
      memcpy(p.dst, map + p.off, p.len);
      return 0;
    }
    if (direct && !bounce.load(std::memory_order_relaxed)) {
      const int err = pread_all(fd, p.dst, p.len, p.off);
      if (err != EFAULT && err != EINVAL) return err;
      bounce.store(true, std::memory_order_relaxed);
    }
    if (!direct) return pread_all(fd, p.dst, p.len, p.off);
    constexpr size_t A = moe::kStoreAlign;
    if (scratch.size() < p.len + A) scratch.resize(p.len + A);
    uint8_t *b = scratch.data() + (A - (uintptr_t)scratch.data() % A) % A;
    const int err = pread_all(fd, b, p.len, p.off);
    if (err) return err;
    memcpy(p.dst, b, p.len);
    return 0;
  }

  void worker() {
    std::vector<uint8_t> scratch;
    std::unique_lock<std::mutex> lock(mu);
    for (;;) {
      cv_work.wait(lock, [&] { return stop || next < queue.size(); });
      if (stop) return;
      const Piece p = queue[next++];
      lock.unlock();
      const int err = read_piece(p, scratch);
      lock.lock();
      if (err && !failed) failed = err;
      if (--pending == 0) cv_done.notify_all();
    }
  }

  // Runs the pieces on the readers (or inline with one reader); 0 or errno.
  int run(std::vector<Piece> &&pieces) {
    if (pieces.empty()) return 0;
    if (workers.empty()) {
      for (const auto &p : pieces) {
        const int err = read_piece(p, inline_scratch);
        if (err) return err;
      }
      return 0;
    }
    std::unique_lock<std::mutex> lock(mu);
    queue = std::move(pieces);
    next = 0;
    pending = queue.size();
    failed = 0;
    cv_work.notify_all();
    cv_done.wait(lock, [&] { return pending == 0; });
    queue.clear();
    next = 0;
    return failed;
  }
};

namespace moe {

moe_status store_read(moe_store *st, int layer, const int32_t *experts, int n,
                      void *const *dst, size_t chunk) {
  if (!st || !experts || !dst || n < 0 || layer < 0 || layer >= st->n_layers)
    return MOE_E_INVALID;
  if (chunk == 0) chunk = st->stride;
  chunk = (chunk + kStoreAlign - 1) / kStoreAlign * kStoreAlign;
  std::vector<moe_store::Piece> pieces;
  pieces.reserve((size_t)n * (st->stride / chunk + 1));
  for (int i = 0; i < n; ++i) {
    const int e = experts[i];
    if (e < 0 || e >= st->E || !dst[i]) return MOE_E_INVALID;
    if (st->direct && ((uintptr_t)dst[i] % kStoreAlign)) return MOE_E_INVALID;
    const off_t base = (off_t)(((size_t)layer * st->E + e) * st->stride);
    // direct I/O reads whole aligned pieces (the stride is aligned); a
    // buffered read takes the blob's own bytes only
    const size_t total = st->direct ? st->stride : st->blob;
    for (size_t o = 0; o < total; o += chunk) {
      const size_t len = o + chunk <= total ? chunk : total - o;
      pieces.push_back({base + (off_t)o, len, (uint8_t *)dst[i] + o});
    }
  }
  const auto t0 = std::chrono::steady_clock::now();
  const int err = st->run(std::move(pieces));
  const auto t1 = std::chrono::steady_clock::now();
  if (err) {
    st->stats.errors += 1;
    st->stats.last_errno = (uint64_t)err;
    return MOE_E_POOL;
  }
  st->stats.bounced = st->bounce.load() ? 1 : 0;
  st->stats.blobs += (uint64_t)n;
  st->stats.bytes += (uint64_t)n * st->blob;
  st->stats.ns += (uint64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(t1 - t0).count();
  return MOE_OK;
}

size_t store_blob_bytes(const moe_store *st) { return st->blob; }
size_t store_stride_of(const moe_store *st) { return st->stride; }
int store_layers(const moe_store *st) { return st->n_layers; }
int store_E(const moe_store *st) { return st->E; }
int store_D(const moe_store *st) { return st->D; }
int store_F(const moe_store *st) { return st->F; }
bool store_direct(const moe_store *st) { return st->direct; }

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_store_stride(int32_t D, int32_t F) {
  if (D < 64 || F < 64 || D % 64 || F % 64) return 0;
  return store_stride(D, F);
}

moe_status moe_store_open(moe_store **out, const char *path, int32_t n_layers, int32_t E,
                          int32_t D, int32_t F, int32_t flags, int32_t threads) {
  if (!out || !path || n_layers < 1 || E < 1 || D < 64 || F < 64 || D % 64 || F % 64 ||
      threads < 1 || threads > kStoreMaxThreads)
    return MOE_E_INVALID;
  if (flags & ~(MOE_STORE_DIRECT | MOE_STORE_MMAP)) return MOE_E_INVALID;
  if ((flags & MOE_STORE_DIRECT) && (flags & MOE_STORE_MMAP)) return MOE_E_INVALID;
  *out = nullptr;
  moe_store *st = new (std::nothrow) moe_store;
  if (!st) return MOE_E_POOL;
  st->n_layers = n_layers;
  st->E = E;
  st->D = D;
  st->F = F;
  st->stride = store_stride(D, F);
  st->blob = blob_layout(D, F).total;
  const size_t need = (size_t)n_layers * E * st->stride;
  int fd = -1;
  if (flags & MOE_STORE_DIRECT) {
    fd = open(path, O_RDONLY | O_DIRECT);
    st->direct = fd >= 0;  // file systems without direct I/O: buffered reads
  }
  if (fd < 0) fd = open(path, O_RDONLY);
  if (fd < 0) {
    delete st;
    return MOE_E_INVALID;
  }
  st->fd = fd;
  struct stat sb;
  if (fstat(fd, &sb) != 0 || (size_t)sb.st_size < need) {
    close(fd);
    delete st;
    return MOE_E_INVALID;
  }
  st->file_bytes = (size_t)sb.st_size;
  if (flags & MOE_STORE_MMAP) {
    void *m = mmap(nullptr, st->file_bytes, PROT_READ, MAP_SHARED, fd, 0);
    if (m == MAP_FAILED) {
      close(fd);
      delete st;
      return MOE_E_POOL;
    }
    st->map = (const uint8_t *)m;
  }
  if (threads > 1) {
    try {
      for (int i = 0; i < threads; ++i) st->workers.emplace_back([st] { st->worker(); });
    } catch (...) {
      moe_store_close(st);
      return MOE_E_POOL;
    }
  }
  *out = st;
  return MOE_OK;
}

moe_status moe_store_read(moe_store *st, int32_t layer, const int32_t *experts, int32_t n,
                          void *const *dst, size_t chunk_bytes) {
  return store_read(st, layer, experts, n, dst, chunk_bytes);
}

moe_status moe_store_get_stats(const moe_store *st, moe_store_stats *out) {
  if (!st || !out) return MOE_E_INVALID;
  *out = st->stats;
  return MOE_OK;
}

moe_status moe_store_close(moe_store *st) {
  if (!st) return MOE_E_INVALID;
  {
    std::lock_guard<std::mutex> lock(st->mu);
    st->stop = true;
  }
  st->cv_work.notify_all();
  for (auto &w : st->workers) w.join();
  if (st->map) munmap((void *)st->map, st->file_bytes);
  if (st->fd >= 0) close(st->fd);
  delete st;
  return MOE_OK;
}

}  // extern "C"

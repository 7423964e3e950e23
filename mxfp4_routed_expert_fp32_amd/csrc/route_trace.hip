// Router trace: the authoritative routed ids and the fp32 bits of their
// combine weights, one line per (layer, token), and the reader that counts a
// trace's experts per layer for offline cache warming.
//
// After "How the native runtime works", section "Router tracing and offline
// expert warming" (a buffered trace of the 16 routed ids and fp32 weight bits
// after routing; a synchronous mode that flushes each pass; symlinks refused;
// a size cap), and "Deltafin's custom compiled runtime", section "Router
// traces and cache warming" (regular non-symlink files, bounded lines, an
// 8 GiB limit on the whole trace; a warmer that parses the exact traces and
// ranks experts).  Tracing only reads routes the layer already produced: it
// never changes a route or an output.
//
// Line format (one per traced token, at most kMaxLine bytes):
//   {"layer":L,"pos":P,"ids":[i0,...,ik-1],"w":["xxxxxxxx",...]}
// with L, P and the ids in decimal and each weight as the 8 lowercase hex
// digits of its fp32 bit pattern.
#include <errno.h>
#include <fcntl.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <new>
#include <string>
#include <vector>

#include "moe_mxfp4.h"

namespace {

constexpr size_t kMaxLine = 4096;
constexpr size_t kBufferBytes = size_t(1) << 20;
constexpr uint64_t kDefaultCap = uint64_t(8) << 30;

bool write_all(int fd, const char* p, size_t n) {
  while (n > 0) {
    const ssize_t w = write(fd, p, n);
    if (w < 0) {
      if (errno == EINTR) continue;
      return false;
    }
    p += w;
    n -= (size_t)w;
  }
  return true;
}

}  // namespace

struct moe_trace {
  int fd = -1;
  int mode = MOE_TRACE_BUFFERED;
  uint64_t cap = 0, written = 0;
  std::vector<char> buf;
  bool failed = false;

  bool flush() {
    if (buf.empty()) return true;
    const bool ok = write_all(fd, buf.data(), buf.size());
    buf.clear();
    return ok;
  }
};

extern "C" {

moe_status moe_trace_open(const char* path, int32_t mode, uint64_t max_bytes, moe_trace** out) {
  if (!path || !out) return MOE_ERR_NULL;
  *out = nullptr;
  if (mode != MOE_TRACE_BUFFERED && mode != MOE_TRACE_SYNC) return MOE_ERR_UNSUPPORTED;
  // the final path component must not be a symlink (O_NOFOLLOW), and the
  // file must be a regular file
  const int fd = open(path, O_WRONLY | O_CREAT | O_TRUNC | O_NOFOLLOW | O_CLOEXEC, 0644);
  if (fd < 0) return MOE_ERR_IO;
  struct stat st;
  if (fstat(fd, &st) != 0 || !S_ISREG(st.st_mode)) {
    close(fd);
    return MOE_ERR_IO;
  }
  moe_trace* t = new (std::nothrow) moe_trace;
  if (!t) {
    close(fd);
    return MOE_ERR_IO;
  }
  t->fd = fd;
  t->mode = mode;
  t->cap = max_bytes ? max_bytes : kDefaultCap;
  if (mode == MOE_TRACE_BUFFERED) t->buf.reserve(kBufferBytes);
  *out = t;
  return MOE_OK;
}

moe_status moe_trace_record(moe_trace* t, int32_t layer, int64_t position, int32_t n_tokens, int32_t k,
                            const int32_t* ids, const float* w) {
  if (!t || !ids || !w) return MOE_ERR_NULL;
  if (t->failed) return MOE_ERR_IO;
  if (layer < 0 || position < 0 || n_tokens < 1 || k < 1 || k > 64) return MOE_ERR_SHAPE;
  std::string lines;
  char tmp[64];
  for (int32_t tok = 0; tok < n_tokens; ++tok) {
    const size_t start = lines.size();
    snprintf(tmp, sizeof tmp, "{\"layer\":%d,\"pos\":%lld,\"ids\":[", layer, (long long)(position + tok));
    lines += tmp;
    for (int j = 0; j < k; ++j) {
      snprintf(tmp, sizeof tmp, j ? ",%d" : "%d", ids[(size_t)tok * k + j]);
      lines += tmp;
    }
    lines += "],\"w\":[";
    for (int j = 0; j < k; ++j) {
      uint32_t b;
      memcpy(&b, &w[(size_t)tok * k + j], 4);
      snprintf(tmp, sizeof tmp, j ? ",\"%08x\"" : "\"%08x\"", b);
      lines += tmp;
    }
    lines += "]}\n";
    if (lines.size() - start > kMaxLine) return MOE_ERR_SHAPE;
  }
  if (t->written + lines.size() > t->cap) {  // the trace's size limit: refuse, keep what is written
    t->failed = true;
    t->flush();
    return MOE_ERR_IO;
  }
  t->written += lines.size();
  if (t->mode == MOE_TRACE_SYNC) {  // each completed pass reaches the file before returning
    if (!write_all(t->fd, lines.data(), lines.size()) || fdatasync(t->fd) != 0) {
      t->failed = true;
      return MOE_ERR_IO;
    }
    return MOE_OK;
  }
  if (t->buf.size() + lines.size() > kBufferBytes && !t->flush()) {
    t->failed = true;
    return MOE_ERR_IO;
  }
  if (lines.size() > kBufferBytes) {
    if (!write_all(t->fd, lines.data(), lines.size())) {
      t->failed = true;
      return MOE_ERR_IO;
    }
  } else {
    t->buf.insert(t->buf.end(), lines.begin(), lines.end());
  }
  return MOE_OK;
}

moe_status moe_trace_close(moe_trace* t) {
  if (!t) return MOE_OK;
  bool ok = !t->failed && t->flush();
  if (close(t->fd) != 0) ok = false;
  delete t;
  return ok ? MOE_OK : MOE_ERR_IO;
}

moe_status moe_trace_count(const char* path, int32_t n_layers, int32_t n_experts, int64_t* counts,
                           int64_t* n_records) {
  if (!path || !counts || !n_records) return MOE_ERR_NULL;
  if (n_layers < 1 || n_experts < 1 || (int64_t)n_layers * n_experts > (int64_t{1} << 31)) return MOE_ERR_SHAPE;
  const int fd = open(path, O_RDONLY | O_NOFOLLOW | O_CLOEXEC);
  if (fd < 0) return MOE_ERR_IO;
  struct stat st;
  FILE* f = nullptr;
  if (fstat(fd, &st) != 0 || !S_ISREG(st.st_mode) || (uint64_t)st.st_size > kDefaultCap || !(f = fdopen(fd, "r"))) {
    close(fd);
    return MOE_ERR_IO;
  }
  memset(counts, 0, sizeof(int64_t) * (size_t)n_layers * (size_t)n_experts);
  std::vector<char> line(kMaxLine + 2);
  int64_t recs = 0;
  moe_status rc = MOE_OK;
  while (fgets(line.data(), (int)line.size(), f)) {
    const char* p = line.data();
    const size_t len = strlen(p);
    if (len == 0 || p[len - 1] != '\n') { rc = MOE_ERR_IO; break; }  // unterminated or too long
    int layer = -1, used = 0;
    long long pos = -1;
    if (sscanf(p, "{\"layer\":%d,\"pos\":%lld,\"ids\":[%n", &layer, &pos, &used) != 2 || used == 0 || layer < 0 ||
        layer >= n_layers || pos < 0) {
      rc = MOE_ERR_IO;
      break;
    }
    p += used;
    int nid = 0;
    while (true) {
      int id = -1, u = 0;
      if (sscanf(p, "%d%n", &id, &u) != 1 || id < 0 || id >= n_experts) { rc = MOE_ERR_IO; break; }
      counts[(size_t)layer * n_experts + id] += 1;
      ++nid;
      p += u;
      if (*p == ',') { ++p; continue; }
      if (*p == ']') { ++p; break; }
      rc = MOE_ERR_IO;
      break;
    }
    if (rc != MOE_OK) break;
    if (strncmp(p, ",\"w\":[", 6) != 0) { rc = MOE_ERR_IO; break; }
    p += 6;
    for (int j = 0; j < nid; ++j) {  // one 8-digit hex weight per id
      if (p[0] != '"') { rc = MOE_ERR_IO; break; }
      for (int d = 1; d <= 8; ++d)
        if (!((p[d] >= '0' && p[d] <= '9') || (p[d] >= 'a' && p[d] <= 'f'))) rc = MOE_ERR_IO;
      if (rc != MOE_OK || p[9] != '"') { rc = MOE_ERR_IO; break; }
      p += 10;
      if (j + 1 < nid) {
        if (*p != ',') { rc = MOE_ERR_IO; break; }
        ++p;
      }
    }
    if (rc != MOE_OK) break;
    if (strcmp(p, "]}\n") != 0) { rc = MOE_ERR_IO; break; }
    ++recs;
  }
  if (rc == MOE_OK && ferror(f)) rc = MOE_ERR_IO;
  fclose(f);
  *n_records = recs;
  return rc;
}

}  // extern "C"

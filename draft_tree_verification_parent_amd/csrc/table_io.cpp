// Successor-table checkpoint: the table is the round's only state besides
// the KV cache, and a warmed table is kept across rounds (Graft page,
// arXiv:2605.20104 write-up, section 6: warm-up fills the table and later
// rounds keep updating it).  File: a 32-byte header (the 8 bytes
// "GRAFTTB1", V and k as little-endian int64, the 64-bit FNV-1a hash of the
// payload), then the [V, k] int32 rows, little-endian, row-major.
#include <cerrno>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "common.h"

namespace {

constexpr char kMagic[8] = {'G', 'R', 'A', 'F', 'T', 'T', 'B', '1'};
constexpr size_t kHeader = 32;

// FNV-1a, 64-bit (offset basis and prime from the published definition)
uint64_t fnv1a64(const unsigned char *p, size_t n) {
  uint64_t h = 14695981039346656037ull;
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

void put64(unsigned char *d, uint64_t v) {
  for (int i = 0; i < 8; ++i) d[i] = static_cast<unsigned char>(v >> (8 * i));
}
uint64_t get64(const unsigned char *s) {
  uint64_t v = 0;
  for (int i = 0; i < 8; ++i) v |= static_cast<uint64_t>(s[i]) << (8 * i);
  return v;
}

bool shape_ok(int V, int k) { return V > 0 && k >= 1 && k <= GRAFT_MAX_K; }

}  // namespace

extern "C" int graft_table_save(const char *path, int V, int k, const int32_t *table, graft_stream stream) {
  using graft::fail;
  if (!path || !table || !shape_ok(V, k))
    return fail(GRAFT_EINVAL, "table_save: path=%p V=%d k=%d table=%p", static_cast<const void *>(path), V, k,
                static_cast<const void *>(table));
  graft::clear_error();
  const size_t n = static_cast<size_t>(V) * k * sizeof(int32_t);
  std::vector<unsigned char> buf(kHeader + n);
  hipStream_t s = graft::as_stream(stream);
  hipError_t e = hipMemcpyAsync(buf.data() + kHeader, table, n, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(GRAFT_EHIP, "table_save: copy from the device: %s", hipGetErrorString(e));
  std::memcpy(buf.data(), kMagic, 8);
  put64(buf.data() + 8, static_cast<uint64_t>(V));
  put64(buf.data() + 16, static_cast<uint64_t>(k));
  put64(buf.data() + 24, fnv1a64(buf.data() + kHeader, n));
  // written whole under a temporary name, then renamed over the target
  const std::string tmp = std::string(path) + ".tmp";
  FILE *f = std::fopen(tmp.c_str(), "wb");
  if (!f) return fail(GRAFT_EIO, "table_save: cannot create %s: %s", tmp.c_str(), std::strerror(errno));
  const bool wrote = std::fwrite(buf.data(), 1, buf.size(), f) == buf.size();
  const bool closed = std::fclose(f) == 0;
  if (!wrote || !closed) {
    std::remove(tmp.c_str());
    return fail(GRAFT_EIO, "table_save: writing %s failed", tmp.c_str());
  }
  if (std::rename(tmp.c_str(), path) != 0) {
    std::remove(tmp.c_str());
    return fail(GRAFT_EIO, "table_save: cannot rename %s to %s: %s", tmp.c_str(), path, std::strerror(errno));
  }
  return GRAFT_OK;
}

extern "C" int graft_table_load(const char *path, int V, int k, int32_t *table, graft_stream stream) {
  using graft::fail;
  if (!path || !table || !shape_ok(V, k))
    return fail(GRAFT_EINVAL, "table_load: path=%p V=%d k=%d table=%p", static_cast<const void *>(path), V, k,
                static_cast<void *>(table));
  graft::clear_error();
  FILE *f = std::fopen(path, "rb");
  if (!f) return fail(GRAFT_EIO, "table_load: cannot open %s: %s", path, std::strerror(errno));
  const size_t n = static_cast<size_t>(V) * k * sizeof(int32_t);
  std::vector<unsigned char> buf(kHeader + n + 1);
  const size_t got = std::fread(buf.data(), 1, buf.size(), f);  // one byte more: a longer file is caught
  std::fclose(f);
  if (got < kHeader || std::memcmp(buf.data(), kMagic, 8) != 0)
    return fail(GRAFT_EINVAL, "table_load: %s is not a table file", path);
  const uint64_t fV = get64(buf.data() + 8), fk = get64(buf.data() + 16);
  if (fV != static_cast<uint64_t>(V) || fk != static_cast<uint64_t>(k))
    return fail(GRAFT_EINVAL, "table_load: %s holds a %llu x %llu table, not %d x %d", path,
                static_cast<unsigned long long>(fV), static_cast<unsigned long long>(fk), V, k);
  if (got != kHeader + n)
    return fail(GRAFT_EINVAL, "table_load: %s has %zu payload bytes, not %zu", path, got - kHeader, n);
  if (get64(buf.data() + 24) != fnv1a64(buf.data() + kHeader, n))
    return fail(GRAFT_EINVAL, "table_load: %s: payload checksum mismatch", path);
  for (size_t i = 0; i < static_cast<size_t>(V) * k; ++i) {
    int32_t t;
    std::memcpy(&t, buf.data() + kHeader + 4 * i, 4);
    if (t < 0 || t >= V)
      return fail(GRAFT_EINVAL, "table_load: %s: entry %zu = %d is not a token id below %d", path, i, t, V);
  }
  hipStream_t s = graft::as_stream(stream);
  hipError_t e = hipMemcpyAsync(table, buf.data() + kHeader, n, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(GRAFT_EHIP, "table_load: copy to the device: %s", hipGetErrorString(e));
  return GRAFT_OK;
}

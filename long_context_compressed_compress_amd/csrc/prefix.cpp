// Prefix reuse: one sequence of a decode cache to and from a file (host I/O
// around the path; the CSDN page's section on shared-prefix reuse keeps
// compressed entries on disk and offers full, periodic or no caching of the
// uncompressed window KV).  Every check of a file is made before the cache is
// written; both calls synchronise the caller's stream.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/libcsa.h"

namespace csa {
int abi_decode_cache_status(const csa_decode_cache* c);
int abi_hip_status(hipError_t e);
}  // namespace csa

namespace {

constexpr char kMagic[8] = {'C', 'S', 'A', 'P', 'F', 'X', '0', '1'};
constexpr uint32_t kVersion = 2;  // 2: the header carries a checksum of its own fields
constexpr int kRow = CSA_MIXED_ROW_BYTES;
constexpr int kCsaRing = 8, kHcaRing = 128;  // compressor ring rows of the decode cache
constexpr int kSections = 10;

// Sections in file order; the first four belong to ENTRIES, the rest to RINGS.
enum Section { S_CSA_KV, S_CSA_KEYS, S_CSA_SCALES, S_HCA_KV, S_CSA_RAW, S_CSA_LOG, S_HCA_RAW, S_HCA_LOG,
               S_CSA_WIN, S_HCA_WIN };

struct Header {          // 144 bytes, little-endian as written
  char magic[8];
  uint32_t version;
  uint32_t parts;
  int64_t pos;           // tokens 0 .. pos-1 are in the snapshot
  int64_t csa_count;
  int64_t hca_count;
  int64_t win_rows;
  int32_t idx_dim;
  int32_t row_bytes;
  uint64_t sum[kSections];
  uint64_t head_sum;     // checksum of every byte above (a damaged position or count is caught too)
};
static_assert(sizeof(Header) == 144, "header layout");  // 56 bytes of fields + 10 section checksums + 1

// 64-bit checksum of a byte run (word-wise multiply-rotate; detects truncation
// and damage, not tampering).
uint64_t checksum(const uint8_t* p, size_t n) {
  uint64_t h = 0x9E3779B97F4A7C15ull ^ n;
  size_t i = 0;
  for (; i + 8 <= n; i += 8) {
    uint64_t w;
    std::memcpy(&w, p + i, 8);
    h = (h ^ (w * 0xBF58476D1CE4E5B9ull)) * 0x94D049BB133111EBull;
    h = (h << 29) | (h >> 35);
  }
  uint64_t w = 0;
  std::memcpy(&w, p + i, n - i);
  h = (h ^ (w * 0xBF58476D1CE4E5B9ull) ^ (n - i)) * 0x94D049BB133111EBull;
  return h ^ (h >> 31);
}

// Where each section of sequence `seq` lives in the cache, and its full size.
struct Span {
  uint8_t* dev;
  size_t row;   // bytes per row (entries) or 0 for fixed-size rings
  size_t bytes;
};
Span span(const csa_decode_cache& c, int32_t seq, Section s, int64_t csa_n, int64_t hca_n) {
  const size_t b = (size_t)seq;
  const size_t kb = (size_t)c.idx_dim / 2, sb = (size_t)c.idx_dim / 32;
  switch (s) {
    case S_CSA_KV: return {c.csa_kv + b * c.csa_cap * kRow, kRow, (size_t)csa_n * kRow};
    case S_CSA_KEYS: return {c.csa_keys + b * c.csa_cap * kb, kb, (size_t)csa_n * kb};
    case S_CSA_SCALES: return {c.csa_key_scales + b * c.csa_cap * sb, sb, (size_t)csa_n * sb};
    case S_HCA_KV: return {c.hca_kv + b * c.hca_cap * kRow, kRow, (size_t)hca_n * kRow};
    case S_CSA_RAW: return {reinterpret_cast<uint8_t*>(c.csa_raw + b * kCsaRing * CSA_DIM), 0, kCsaRing * CSA_DIM * 2};
    case S_CSA_LOG: return {reinterpret_cast<uint8_t*>(c.csa_logits + b * kCsaRing * CSA_DIM), 0, kCsaRing * CSA_DIM * 4};
    case S_HCA_RAW: return {reinterpret_cast<uint8_t*>(c.hca_raw + b * kHcaRing * CSA_DIM), 0, kHcaRing * CSA_DIM * 2};
    case S_HCA_LOG: return {reinterpret_cast<uint8_t*>(c.hca_logits + b * kHcaRing * CSA_DIM), 0, kHcaRing * CSA_DIM * 4};
    case S_CSA_WIN: return {c.csa_win + b * c.win_rows * kRow, 0, (size_t)c.win_rows * kRow};
    default: return {c.hca_win + b * c.win_rows * kRow, 0, (size_t)c.win_rows * kRow};
  }
}
// Paged entries: the physical pages of sequence seq's entry sections, read
// from the device tables (empty when the cache is contiguous).
struct SeqPages {
  std::vector<int32_t> csa, hca;
};
int read_pages(const csa_decode_cache& c, int32_t seq, hipStream_t s, SeqPages& out) {
  if (c.page_entries == 0) return CSA_OK;
  const int64_t tc = c.csa_cap / c.page_entries, th = c.hca_cap / c.page_entries;
  out.csa.resize((size_t)tc);
  out.hca.resize((size_t)th);
  hipError_t e = hipMemcpyAsync(out.csa.data(), c.csa_pages + seq * tc, tc * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(out.hca.data(), c.hca_pages + seq * th, th * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? CSA_OK : csa::abi_hip_status(e);
}
// The pages that n entries occupy must be inside the pool (the kernels clamp a
// bad id; a host copy refuses it instead).
bool pages_ok(const std::vector<int32_t>& tab, int64_t n, int64_t P, int32_t pool) {
  for (int64_t i = 0; i * P < n; ++i)
    if (tab[(size_t)i] < 0 || tab[(size_t)i] >= pool) return false;
  return true;
}
// Copy an entry section of n rows between the host buffer and the cache, a
// page at a time when paged (the pool is the section's array, the sequence's
// rows are page-sized runs at the pages its table names).
hipError_t copy_entries(const csa_decode_cache& c, const SeqPages& pg, const Span& sp, Section k, int64_t n,
                        uint8_t* host, bool to_device, hipStream_t s) {
  if (c.page_entries == 0) {
    if (!sp.bytes) return hipSuccess;
    return to_device ? hipMemcpyAsync(sp.dev, host, sp.bytes, hipMemcpyHostToDevice, s)
                     : hipMemcpyAsync(host, sp.dev, sp.bytes, hipMemcpyDeviceToHost, s);
  }
  uint8_t* pool = k == S_CSA_KV ? c.csa_kv : k == S_CSA_KEYS ? c.csa_keys : k == S_CSA_SCALES ? c.csa_key_scales : c.hca_kv;
  const std::vector<int32_t>& tab = k == S_HCA_KV ? pg.hca : pg.csa;
  const int64_t P = c.page_entries;
  hipError_t e = hipSuccess;
  for (int64_t i = 0; i * P < n && e == hipSuccess; ++i) {
    const int64_t rows = n - i * P < P ? n - i * P : P;
    uint8_t* dev = pool + (int64_t)tab[(size_t)i] * P * (int64_t)sp.row;
    uint8_t* h = host + i * P * (int64_t)sp.row;
    const size_t bytes = (size_t)(rows * (int64_t)sp.row);
    e = to_device ? hipMemcpyAsync(dev, h, bytes, hipMemcpyHostToDevice, s)
                  : hipMemcpyAsync(h, dev, bytes, hipMemcpyDeviceToHost, s);
  }
  return e;
}

inline bool in_parts(int s, uint32_t parts) {
  return s <= S_HCA_KV ? (parts & CSA_PREFIX_ENTRIES) != 0 : (parts & CSA_PREFIX_RINGS) != 0;
}

struct File {
  FILE* f = nullptr;
  ~File() {
    if (f) std::fclose(f);
  }
};

int check_common(const csa_decode_cache* cache, int32_t seq, const char* path, int32_t parts) {
  const int st = csa::abi_decode_cache_status(cache);
  if (st != CSA_OK) return st;
  if (!path) return CSA_ERR_NULL;
  if (seq < 0 || seq >= cache->batch) return CSA_ERR_SHAPE;
  if (parts <= 0 || (parts & ~(CSA_PREFIX_ENTRIES | CSA_PREFIX_RINGS))) return CSA_ERR_SHAPE;
  return CSA_OK;
}

int prefix_save_impl(const csa_decode_cache* cache, int32_t seq, const char* path, int32_t parts, void* stream) {
  int st = check_common(cache, seq, path, parts);
  if (st != CSA_OK) return st;
  const csa_decode_cache& c = *cache;
  const hipStream_t s = (hipStream_t)stream;
  int64_t pos = 0;
  int32_t nc = 0, nh = 0;
  hipError_t e = hipMemcpyAsync(&pos, c.pos + seq, 8, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&nc, c.csa_entries + seq, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&nh, c.hca_entries + seq, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return csa::abi_hip_status(e);
  if (pos < 0 || nc < 0 || nh < 0 || nc > c.csa_cap || nh > c.hca_cap) return CSA_ERR_RANGE;  // inactive or corrupt
  SeqPages pg;
  if ((parts & CSA_PREFIX_ENTRIES) && (st = read_pages(c, seq, s, pg)) != CSA_OK) return st;
  if ((parts & CSA_PREFIX_ENTRIES) && c.page_entries &&
      (!pages_ok(pg.csa, nc, c.page_entries, c.csa_pool_pages) || !pages_ok(pg.hca, nh, c.page_entries, c.hca_pool_pages)))
    return CSA_ERR_RANGE;

  Header h;
  std::memset(&h, 0, sizeof h);
  std::memcpy(h.magic, kMagic, 8);
  h.version = kVersion;
  h.parts = (uint32_t)parts;
  h.pos = pos;
  h.csa_count = nc;
  h.hca_count = nh;
  h.win_rows = c.win_rows;
  h.idx_dim = c.idx_dim;
  h.row_bytes = kRow;
  std::vector<std::vector<uint8_t>> data(kSections);
  for (int k = 0; k < kSections; ++k) {
    if (!in_parts(k, h.parts)) continue;
    const Span sp = span(c, seq, (Section)k, nc, nh);
    data[k].resize(sp.bytes);
    if (k <= S_HCA_KV)
      e = copy_entries(c, pg, sp, (Section)k, k == S_HCA_KV ? nh : nc, data[k].data(), false, s);
    else if (sp.bytes)
      e = hipMemcpyAsync(data[k].data(), sp.dev, sp.bytes, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return csa::abi_hip_status(e);
  }
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return csa::abi_hip_status(e);
  for (int k = 0; k < kSections; ++k) h.sum[k] = in_parts(k, h.parts) ? checksum(data[k].data(), data[k].size()) : 0;
  h.head_sum = checksum(reinterpret_cast<const uint8_t*>(&h), offsetof(Header, head_sum));

  File f;
  f.f = std::fopen(path, "wb");
  if (!f.f) return CSA_ERR_IO;
  if (std::fwrite(&h, sizeof h, 1, f.f) != 1) return CSA_ERR_IO;
  for (int k = 0; k < kSections; ++k)
    if (!data[k].empty() && std::fwrite(data[k].data(), 1, data[k].size(), f.f) != data[k].size()) return CSA_ERR_IO;
  const int rc = std::fclose(f.f);
  f.f = nullptr;
  return rc == 0 ? CSA_OK : CSA_ERR_IO;
}

int prefix_load_impl(const csa_decode_cache* cache, int32_t seq, const char* path, int32_t parts, int64_t prefix_len,
                     int64_t* prime_from, void* stream) {
  int st = check_common(cache, seq, path, parts);
  if (st != CSA_OK) return st;
  const csa_decode_cache& c = *cache;
  File f;
  f.f = std::fopen(path, "rb");
  if (!f.f) return CSA_ERR_IO;
  Header h;
  if (std::fread(&h, sizeof h, 1, f.f) != 1) return CSA_ERR_FORMAT;
  if (checksum(reinterpret_cast<const uint8_t*>(&h), offsetof(Header, head_sum)) != h.head_sum) return CSA_ERR_FORMAT;
  if (std::memcmp(h.magic, kMagic, 8) != 0 || h.version != kVersion || h.row_bytes != kRow) return CSA_ERR_FORMAT;
  if (h.parts == 0 || (h.parts & ~(uint32_t)(CSA_PREFIX_ENTRIES | CSA_PREFIX_RINGS))) return CSA_ERR_FORMAT;
  if ((uint32_t)parts & ~h.parts) return CSA_ERR_FORMAT;  // asked for a part the file does not hold
  // sizes the header claims must fit the file before anything is allocated
  if (std::fseek(f.f, 0, SEEK_END) != 0) return CSA_ERR_IO;
  const long fsize = std::ftell(f.f);
  if (fsize < 0 || std::fseek(f.f, (long)sizeof h, SEEK_SET) != 0) return CSA_ERR_IO;
  const int64_t max_rows = (int64_t)fsize / kRow;
  if (h.pos < 0 || h.csa_count < 0 || h.hca_count < 0 || h.csa_count > h.pos / 4 || h.hca_count > h.pos / 128 ||
      h.win_rows < 1 || h.csa_count > max_rows || h.hca_count > max_rows ||
      ((h.parts & CSA_PREFIX_RINGS) && h.win_rows > max_rows))  // window rows are in the file only with rings
    return CSA_ERR_FORMAT;
  if (h.idx_dim != c.idx_dim) return CSA_ERR_FORMAT;
  if ((parts & CSA_PREFIX_RINGS) && h.win_rows != c.win_rows) return CSA_ERR_FORMAT;

  const int64_t p = h.pos;
  const int64_t L = prefix_len < 0 ? p : prefix_len;
  if (prefix_len < -1) return CSA_ERR_RANGE;
  if ((parts & CSA_PREFIX_ENTRIES) && L > p) return CSA_ERR_RANGE;  // the file does not cover the prefix
  if ((parts & CSA_PREFIX_RINGS) && L < p) return CSA_ERR_RANGE;    // its rings hold tokens past the prefix
  const int64_t nc = (parts & CSA_PREFIX_ENTRIES) ? (h.csa_count < L / 4 ? h.csa_count : L / 4) : 0;
  const int64_t nh = (parts & CSA_PREFIX_ENTRIES) ? (h.hca_count < L / 128 ? h.hca_count : L / 128) : 0;
  if (nc > c.csa_cap || nh > c.hca_cap) return CSA_ERR_RANGE;

  // read and verify every section the file holds (sizes from the header: the
  // sections follow each other), keep those asked for
  std::vector<std::vector<uint8_t>> data(kSections);
  csa_decode_cache file_shape = c;
  file_shape.win_rows = h.win_rows;
  for (int k = 0; k < kSections; ++k) {
    if (!in_parts(k, h.parts)) continue;
    const size_t bytes = span(file_shape, 0, (Section)k, h.csa_count, h.hca_count).bytes;
    data[k].resize(bytes);
    if (bytes && std::fread(data[k].data(), 1, bytes, f.f) != bytes) return CSA_ERR_FORMAT;
    if (checksum(data[k].data(), bytes) != h.sum[k]) return CSA_ERR_FORMAT;
  }
  uint8_t extra;
  if (std::fread(&extra, 1, 1, f.f) != 0) return CSA_ERR_FORMAT;  // trailing bytes: not this format

  // the pages the prefix's entries go to (paged caches), checked before any write
  const hipStream_t s = (hipStream_t)stream;
  SeqPages pg;
  if ((parts & CSA_PREFIX_ENTRIES) && (st = read_pages(c, seq, s, pg)) != CSA_OK) return st;
  if ((parts & CSA_PREFIX_ENTRIES) && c.page_entries &&
      (!pages_ok(pg.csa, nc, c.page_entries, c.csa_pool_pages) || !pages_ok(pg.hca, nh, c.page_entries, c.hca_pool_pages)))
    return CSA_ERR_RANGE;
  // the cache: rows of the prefix, rings, then position and counts
  hipError_t e = hipSuccess;
  for (int k = 0; k < kSections && e == hipSuccess; ++k) {
    if (!in_parts(k, (uint32_t)parts)) continue;
    const Span sp = span(c, seq, (Section)k, nc, nh);
    if (k <= S_HCA_KV)
      e = copy_entries(c, pg, sp, (Section)k, k == S_HCA_KV ? nh : nc, data[k].data(), true, s);
    else if (sp.bytes)
      e = hipMemcpyAsync(sp.dev, data[k].data(), sp.bytes, hipMemcpyHostToDevice, s);
  }
  const int64_t pos = L;
  const int32_t c32 = (int32_t)nc, h32 = (int32_t)nh;
  if (e == hipSuccess) e = hipMemcpyAsync(c.pos + seq, &pos, 8, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && (parts & CSA_PREFIX_ENTRIES))
    e = hipMemcpyAsync(c.csa_entries + seq, &c32, 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && (parts & CSA_PREFIX_ENTRIES))
    e = hipMemcpyAsync(c.hca_entries + seq, &h32, 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return csa::abi_hip_status(e);
  if (prime_from) {
    const int64_t need = c.win_rows > kHcaRing ? c.win_rows : kHcaRing;
    int64_t from = L - need > 0 ? L - need : 0;
    if ((parts & CSA_PREFIX_RINGS) && p > from) from = p;
    *prime_from = from;
  }
  return CSA_OK;
}

}  // namespace

extern "C" {

// No exception crosses the C ABI (host buffers are the only allocations).
int prefix_save(const csa_decode_cache* cache, int32_t seq, const char* path, int32_t parts, void* stream) {
  try {
    return prefix_save_impl(cache, seq, path, parts, stream);
  } catch (...) {
    return CSA_ERR_IO;
  }
}

int prefix_load(const csa_decode_cache* cache, int32_t seq, const char* path, int32_t parts, int64_t prefix_len,
                int64_t* prime_from, void* stream) {
  try {
    return prefix_load_impl(cache, seq, path, parts, prefix_len, prime_from, stream);
  } catch (...) {
    return CSA_ERR_IO;
  }
}

}  // extern "C"

// W12 checkpoint files and the streamed load with the load-time check overlapped.
//
// SpecPilot summary page, result bullet of section 4.1: converted layers are checked bit for
// bit when they are loaded.  A file holds encoded tensors in this library's physical layout;
// loading streams them from the file through two pinned host staging halves into device
// memory and enqueues the bit-for-bit check of each tensor against its BF16 source as soon as
// its planes are enqueued, so the GPU checks tensor i while the host reads tensor i + 1.
//
// File layout (little-endian):
//   header   64 bytes: magic "W12CKPT1", uint32 version (1), uint32 count, 48 bytes zero
//   index    count entries of 128 bytes: name (64 bytes, NUL-padded), int32 N, int32 K,
//            int32 layout, int32 reserved (0), int64 num_escapes, uint64 data offset,
//            uint64 data bytes, 24 bytes zero
//   data     per tensor, at its offset: base [N], esc_ptr [N+1] u32, esc [E] u32, hi, lo;
//            every section starts on a 256-byte boundary of the file
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "w12_device.h"
#include "w12_kernels.h"

namespace w12 {

namespace {

constexpr char kMagic[8] = {'W', '1', '2', 'C', 'K', 'P', 'T', '1'};
constexpr uint32_t kVersion = 1;
constexpr uint64_t kAlign = 256;
constexpr size_t kHeaderBytes = 64;
constexpr size_t kEntryBytes = 128;

uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Sections {
  uint64_t off[5];     // base, esc_ptr, esc, hi, lo (relative to the tensor's data offset)
  uint64_t bytes[5];
  uint64_t total;
};

Sections sections_of(int32_t N, int32_t K, int64_t E) {
  Sections s;
  const uint64_t chunks = (uint64_t)num_row_blocks(N) * (uint64_t)num_chunks(K);
  s.bytes[0] = (uint64_t)N;
  s.bytes[1] = ((uint64_t)N + 1) * 4;
  s.bytes[2] = (uint64_t)E * 4;
  s.bytes[3] = chunks * kHiChunkBytes;
  s.bytes[4] = chunks * kLoChunkBytes;
  uint64_t o = 0;
  for (int i = 0; i < 5; ++i) {
    s.off[i] = o;
    o = align_up(o + s.bytes[i]);
  }
  s.total = o;
  return s;
}

void put32(uint8_t* p, uint32_t v) { memcpy(p, &v, 4); }
void put64(uint8_t* p, uint64_t v) { memcpy(p, &v, 8); }
uint32_t get32(const uint8_t* p) { uint32_t v; memcpy(&v, p, 4); return v; }
uint64_t get64(const uint8_t* p) { uint64_t v; memcpy(&v, p, 8); return v; }

struct File {
  FILE* f = nullptr;
  ~File() { if (f) fclose(f); }
};

}  // namespace

uint64_t file_tensor_bytes(int32_t N, int32_t K, int64_t E) { return sections_of(N, K, E).total; }

// Writes header, index and data; every array of host_tensors[i] is host memory.
int file_write(const char* path, int32_t count, const char* const* names, const w12_tensor* t, char* err, size_t errn) {
  File fh;
  fh.f = fopen(path, "wb");
  if (!fh.f) { snprintf(err, errn, "cannot open %s for writing", path); return -1; }
  std::vector<uint8_t> head(kHeaderBytes + (size_t)count * kEntryBytes, 0);
  memcpy(head.data(), kMagic, 8);
  put32(head.data() + 8, kVersion);
  put32(head.data() + 12, (uint32_t)count);
  uint64_t off = align_up(head.size());
  std::vector<uint64_t> offs(count);
  for (int i = 0; i < count; ++i) {
    uint8_t* e = head.data() + kHeaderBytes + (size_t)i * kEntryBytes;
    const size_t nl = strnlen(names[i], 63);
    memcpy(e, names[i], nl);
    put32(e + 64, (uint32_t)t[i].N);
    put32(e + 68, (uint32_t)t[i].K);
    put32(e + 72, (uint32_t)t[i].layout);
    put64(e + 80, (uint64_t)t[i].num_escapes);
    const uint64_t bytes = sections_of(t[i].N, t[i].K, t[i].num_escapes).total;
    put64(e + 88, off);
    put64(e + 96, bytes);
    offs[i] = off;
    off += bytes;
  }
  if (fwrite(head.data(), 1, head.size(), fh.f) != head.size()) { snprintf(err, errn, "short write of the index"); return -1; }
  std::vector<uint8_t> zeros(kAlign, 0);
  uint64_t pos = head.size();
  auto pad_to = [&](uint64_t target) -> bool {
    while (pos < target) {
      const size_t n = (size_t)std::min<uint64_t>(target - pos, kAlign);
      if (fwrite(zeros.data(), 1, n, fh.f) != n) return false;
      pos += n;
    }
    return true;
  };
  for (int i = 0; i < count; ++i) {
    const Sections s = sections_of(t[i].N, t[i].K, t[i].num_escapes);
    const void* src[5] = {t[i].base, t[i].esc_ptr, t[i].esc, t[i].hi, t[i].lo};
    for (int k = 0; k < 5; ++k) {
      if (!pad_to(offs[i] + s.off[k])) { snprintf(err, errn, "short write (padding)"); return -1; }
      if (s.bytes[k] && fwrite(src[k], 1, s.bytes[k], fh.f) != s.bytes[k]) {
        snprintf(err, errn, "short write of tensor %d", i);
        return -1;
      }
      pos += s.bytes[k];
    }
    if (!pad_to(offs[i] + s.total)) { snprintf(err, errn, "short write (padding)"); return -1; }
  }
  if (fflush(fh.f) != 0) { snprintf(err, errn, "flush failed"); return -1; }
  return 0;
}

int file_index(const char* path, int32_t* count, w12_file_entry* entries, int32_t max_entries, char* err, size_t errn) {
  File fh;
  fh.f = fopen(path, "rb");
  if (!fh.f) { snprintf(err, errn, "cannot open %s", path); return -1; }
  uint8_t h[kHeaderBytes];
  if (fread(h, 1, kHeaderBytes, fh.f) != kHeaderBytes || memcmp(h, kMagic, 8) != 0 || get32(h + 8) != kVersion) {
    snprintf(err, errn, "%s is not a version-1 W12 checkpoint", path);
    return -1;
  }
  const uint32_t n = get32(h + 12);
  *count = (int32_t)n;
  if (!entries) return 0;
  if ((int64_t)n > max_entries) { snprintf(err, errn, "file holds %u tensors, room for %d", n, max_entries); return -1; }
  for (uint32_t i = 0; i < n; ++i) {
    uint8_t e[kEntryBytes];
    if (fread(e, 1, kEntryBytes, fh.f) != kEntryBytes) { snprintf(err, errn, "truncated index"); return -1; }
    w12_file_entry& x = entries[i];
    memset(&x, 0, sizeof(x));
    memcpy(x.name, e, 63);
    x.N = (int32_t)get32(e + 64);
    x.K = (int32_t)get32(e + 68);
    x.layout = (int32_t)get32(e + 72);
    x.num_escapes = (int64_t)get64(e + 80);
    x.offset = get64(e + 88);
    x.bytes = get64(e + 96);
    if (x.bytes != sections_of(x.N, x.K, x.num_escapes).total) {
      snprintf(err, errn, "index entry %u is inconsistent", i);
      return -1;
    }
  }
  return 0;
}

// Streams the listed tensors into their device descriptors.  staging: pinned host memory cut
// in two halves; the host fills one half from the file while the other half's copy runs.
int file_load(const char* path, int32_t count, const int32_t* which, const w12_tensor* dst, void* staging,
              uint64_t staging_bytes, const uint16_t* const* refs, const int64_t* ldr, unsigned long long* d_results,
              hipStream_t stream, char* err, size_t errn) {
  std::vector<w12_file_entry> idx;
  int32_t n = 0;
  if (file_index(path, &n, nullptr, 0, err, errn)) return -1;
  idx.resize(n);
  if (file_index(path, &n, idx.data(), n, err, errn)) return -1;
  File fh;
  fh.f = fopen(path, "rb");
  if (!fh.f) { snprintf(err, errn, "cannot open %s", path); return -1; }
  const uint64_t half = staging_bytes / 2 / kAlign * kAlign;
  uint8_t* buf[2] = {reinterpret_cast<uint8_t*>(staging), reinterpret_cast<uint8_t*>(staging) + half};
  hipEvent_t ev[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  int rc = 0;
  int cur = 0;
  for (int b = 0; b < 2; ++b) {
    if (hipEventCreateWithFlags(&ev[b], hipEventDisableTiming) != hipSuccess) {
      snprintf(err, errn, "hipEventCreate failed");
      rc = -2;
    }
  }
  for (int i = 0; i < count && rc == 0; ++i) {
    const w12_file_entry& e = idx[which[i]];
    const Sections s = sections_of(e.N, e.K, e.num_escapes);
    void* dptr[5] = {dst[i].base, dst[i].esc_ptr, dst[i].esc, dst[i].hi, dst[i].lo};
    for (int k = 0; k < 5 && rc == 0; ++k) {
      uint64_t done = 0;
      while (done < s.bytes[k]) {
        const uint64_t nb = std::min(half, s.bytes[k] - done);
        if (pending[cur] && hipEventSynchronize(ev[cur]) != hipSuccess) {   // this half's last copy
          snprintf(err, errn, "hipEventSynchronize failed");
          rc = -2;
          break;
        }
        pending[cur] = false;
        if (fseeko(fh.f, (off_t)(e.offset + s.off[k] + done), SEEK_SET) != 0 ||
            fread(buf[cur], 1, nb, fh.f) != nb) {
          snprintf(err, errn, "short read of tensor %d (%s)", which[i], e.name);
          rc = -1;
          break;
        }
        if (hipMemcpyAsync(reinterpret_cast<uint8_t*>(dptr[k]) + done, buf[cur], nb, hipMemcpyHostToDevice, stream) !=
                hipSuccess ||
            hipEventRecord(ev[cur], stream) != hipSuccess) {
          snprintf(err, errn, "host-to-device copy failed");
          rc = -2;
          break;
        }
        pending[cur] = true;
        cur ^= 1;
        done += nb;
      }
    }
    if (rc == 0 && refs && refs[i]) {
      const hipError_t he = launch_verify(&dst[i], refs[i], ldr[i], d_results + 2 * i, stream);
      if (he != hipSuccess) {
        snprintf(err, errn, "verify launch failed: %s", hipGetErrorString(he));
        rc = -2;
      }
    }
  }
  // the staging buffer belongs to the caller again only once its copies have drained
  for (int b = 0; b < 2; ++b) {
    if (pending[b]) (void)hipEventSynchronize(ev[b]);
    if (ev[b]) (void)hipEventDestroy(ev[b]);
  }
  return rc;
}

}  // namespace w12

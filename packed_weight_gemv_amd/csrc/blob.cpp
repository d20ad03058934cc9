// The packed-blob header: format version, shape, layout and a checksum of the
// logical values, so that a reader can check that a packed blob holds the
// matrix it claims before using it, whatever its packing (page "The Neutrino
// Engine", sections "The same weights take four execution paths" and "What
// ships": every path reads the same stored values, and a converted pack must
// match the engine).  Plain host C++; the layout is in pwg.h.
//
// The checksum is FNV-1a 64 (Fowler, Noll, Vo) over the logical matrix as
// int8, row-major: the 2-bit and the base-3 packings of one matrix, as stored
// or as arranged for the device, carry the same value.
#include <cstddef>
#include <cstring>

#include "pwg_internal.h"

static_assert(sizeof(pwg_blob_header) == 64, "the header is 64 bytes");

namespace {

constexpr uint64_t kFnvOffset = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

struct Fnv {
  uint64_t h = kFnvOffset;
  void add(uint8_t b) { h = (h ^ b) * kFnvPrime; }
  void add_bytes(const void* p, size_t n) {
    const uint8_t* c = static_cast<const uint8_t*>(p);
    for (size_t i = 0; i < n; ++i) add(c[i]);
  }
};

bool shape_ok(int32_t layout, int64_t rows, int64_t cols) {
  if (rows < 1 || rows > (int64_t{1} << 30) || cols < 1 || cols > PWG_MAX_COLS) return false;
  switch (layout) {
    case PWG_BLOB_T2: return cols % 64 == 0;
    case PWG_BLOB_T2_TILED: return cols % 256 == 0;
    case PWG_BLOB_B3:
    case PWG_BLOB_B3_TILED: return true;
    default: return false;
  }
}

size_t payload_size(int32_t layout, int64_t rows, int64_t cols) {
  if (!shape_ok(layout, rows, cols)) return 0;
  const size_t r = static_cast<size_t>(rows);
  switch (layout) {
    case PWG_BLOB_T2: return r * static_cast<size_t>(cols / 4);
    case PWG_BLOB_T2_TILED: return (r + 15) / 16 * 16 * static_cast<size_t>(cols / 4);
    case PWG_BLOB_B3: return r * static_cast<size_t>((cols + 4) / 5);
    case PWG_BLOB_B3_TILED: {
      const size_t windows = static_cast<size_t>(((cols + 4) / 5 + 5) / 6 + 7) / 8;
      return (r + 15) / 16 * windows * 768;
    }
    default: return 0;
  }
}

uint64_t header_sum(const pwg_blob_header& h) {
  Fnv f;
  f.add_bytes(&h, offsetof(pwg_blob_header, header_fnv1a));
  return f.h;
}

// Byte m of row r of the stored form, read from the payload in `layout`.
uint8_t stored_byte(int32_t layout, const uint8_t* p, int64_t r, int64_t m, int64_t cols) {
  switch (layout) {
    case PWG_BLOB_T2: return p[r * (cols / 4) + m];
    case PWG_BLOB_T2_TILED: {
      // 16-row x 64-byte tiles; inside a tile the byte of row i, column
      // 16 q + b of the tile's window is at 256 q + 16 i + b
      const int64_t T = cols / 4 / 64, c = m % 64;
      return p[((r / 16) * T + m / 64) * 1024 + (c / 16) * 256 + (r % 16) * 16 + c % 16];
    }
    case PWG_BLOB_B3: return p[r * ((cols + 4) / 5) + m];
    default: {  // PWG_BLOB_B3_TILED: lane 16 g + i holds groups 8 t + g, 8 t + 4 + g of row i
      const int64_t windows = (((cols + 4) / 5 + 5) / 6 + 7) / 8;
      const int64_t q = m / 6, t = q / 8, w = q % 8;
      const int64_t lane = 16 * (w % 4) + r % 16;
      return p[((r / 16) * windows + t) * 768 + 12 * lane + 6 * (w / 4) + m % 6];
    }
  }
}

// FNV-1a of the logical values a payload holds; false on an invalid code.
bool logical_sum(int32_t layout, const uint8_t* p, int64_t rows, int64_t cols, uint64_t* out, int64_t* bad_r,
                 int64_t* bad_k) {
  Fnv f;
  const bool t2 = layout == PWG_BLOB_T2 || layout == PWG_BLOB_T2_TILED;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t k = 0; k < cols; ++k) {
      int v;
      if (t2) {
        // byte b of a 16-weight word holds weights 2b, 2b+1 (low nibble) and
        // 8+2b, 9+2b (high nibble), lower index in the lower bits
        const int64_t word = k / 16, mw = k % 16;
        const int64_t byte = 4 * word + (mw % 8) / 2;
        const int shift = 4 * static_cast<int>(mw / 8) + 2 * static_cast<int>(mw % 2);
        const unsigned code = (stored_byte(layout, p, r, byte, cols) >> shift) & 3u;
        if (code == 2u) {
          *bad_r = r;
          *bad_k = k;
          return false;
        }
        v = code == 3u ? -1 : static_cast<int>(code);
      } else {
        unsigned code = stored_byte(layout, p, r, k / 5, cols);
        if (code > 242u) {
          *bad_r = r;
          *bad_k = k;
          return false;
        }
        for (int64_t i = 0; i < k % 5; ++i) code /= 3;
        v = static_cast<int>(code % 3) - 1;
      }
      f.add(static_cast<uint8_t>(static_cast<int8_t>(v)));
    }
  }
  *out = f.h;
  return true;
}

}  // namespace

using pwg::fail;

extern "C" size_t pwg_blob_payload_bytes(int32_t layout, int64_t rows, int64_t cols) {
  return payload_size(layout, rows, cols);
}

extern "C" int pwg_blob_header_init(int32_t layout, const int8_t* w_host, int64_t rows, int64_t cols,
                                    pwg_blob_header* out) {
  const char* fn = "pwg_blob_header_init";
  if (!w_host || !out) return fail(PWG_ERR_ARG, "%s: null pointer", fn);
  if (!shape_ok(layout, rows, cols))
    return fail(PWG_ERR_ARG, "%s: layout %d does not take a %lld x %lld matrix", fn, layout, (long long)rows,
                (long long)cols);
  Fnv f;
  const size_t n = static_cast<size_t>(rows) * static_cast<size_t>(cols);
  for (size_t i = 0; i < n; ++i) {
    if (w_host[i] < -1 || w_host[i] > 1)
      return fail(PWG_ERR_VALUE, "%s: value %d at (row %lld, col %lld) is not in {-1, 0, 1}", fn, (int)w_host[i],
                  (long long)(i / cols), (long long)(i % cols));
    f.add(static_cast<uint8_t>(w_host[i]));
  }
  pwg_blob_header h;
  std::memset(&h, 0, sizeof h);
  h.magic = PWG_BLOB_MAGIC;
  h.version = PWG_BLOB_VERSION;
  h.layout = static_cast<uint16_t>(layout);
  h.rows = rows;
  h.cols = cols;
  h.payload_bytes = payload_size(layout, rows, cols);
  h.logical_fnv1a = f.h;
  h.header_fnv1a = header_sum(h);
  *out = h;
  return PWG_OK;
}

extern "C" int pwg_blob_header_check(const pwg_blob_header* h, size_t payload_bytes) {
  const char* fn = "pwg_blob_header_check";
  if (!h) return fail(PWG_ERR_ARG, "%s: null header", fn);
  if (h->magic != PWG_BLOB_MAGIC) return fail(PWG_ERR_VALUE, "%s: not a packed-blob header (magic %08x)", fn, h->magic);
  if (h->version != PWG_BLOB_VERSION)
    return fail(PWG_ERR_VALUE, "%s: header version %u, this library reads %u", fn, (unsigned)h->version,
                (unsigned)PWG_BLOB_VERSION);
  if (header_sum(*h) != h->header_fnv1a) return fail(PWG_ERR_VALUE, "%s: the header's checksum does not match", fn);
  if (h->reserved[0] != 0 || h->reserved[1] != 0) return fail(PWG_ERR_VALUE, "%s: reserved words are not zero", fn);
  if (!shape_ok(h->layout, h->rows, h->cols))
    return fail(PWG_ERR_VALUE, "%s: layout %u with %lld x %lld is not a valid blob", fn, (unsigned)h->layout,
                (long long)h->rows, (long long)h->cols);
  const size_t need = payload_size(h->layout, h->rows, h->cols);
  if (h->payload_bytes != need)
    return fail(PWG_ERR_VALUE, "%s: header says %llu payload bytes, the layout needs %zu", fn,
                (unsigned long long)h->payload_bytes, need);
  if (payload_bytes != need)
    return fail(PWG_ERR_SIZE, "%s: payload of %zu bytes, the header needs %zu", fn, payload_bytes, need);
  return PWG_OK;
}

extern "C" int pwg_blob_verify(const pwg_blob_header* h, const void* payload_host, size_t payload_bytes) {
  const char* fn = "pwg_blob_verify";
  TRY(pwg_blob_header_check(h, payload_bytes));
  if (!payload_host) return fail(PWG_ERR_ARG, "%s: null payload", fn);
  uint64_t sum = 0;
  int64_t br = 0, bk = 0;
  if (!logical_sum(h->layout, static_cast<const uint8_t*>(payload_host), h->rows, h->cols, &sum, &br, &bk))
    return fail(PWG_ERR_VALUE, "%s: invalid code for the weight at (row %lld, col %lld)", fn, (long long)br,
                (long long)bk);
  if (sum != h->logical_fnv1a)
    return fail(PWG_ERR_VALUE, "%s: the payload's logical values do not match the header's checksum", fn);
  return PWG_OK;
}

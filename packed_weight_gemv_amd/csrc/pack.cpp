// Host packer for the T2 ternary format (2 bits per weight).
//
// The page "The Neutrino Engine", section "The same weights take four
// execution paths", has the loader arrange the same stored values for each
// device at load time; this is that arrangement for gfx950.  Layout (also in
// pwg.h): row-major rows of cols/4 bytes; each little-endian 32-bit word holds
// 16 weights; byte b of a word holds weights 2b, 2b+1 in its low nibble and
// 8+2b, 9+2b in its high nibble, two bits each, lower index in lower bits;
// the code is w in 2-bit two's complement.
//
// The nibble interleave exists for the GEMV kernels: masking a word with
// 0xCCCCCCCC (and, after a 2-bit left shift, again) leaves eight 4-bit lanes
// holding 0b0100 / 0b1100 / 0 for w = +1 / -1 / 0, the FP4 (e2m1) values
// +2 / -2 / 0 that the matrix-core instructions take as their A operand.
//
// Also here: the base-3 format (five weights per byte), packed and unpacked
// on the host; its device arrangement is tile.hip's.
#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

#include "pwg_internal.h"

namespace {

// Packs rows [r0, r1); returns the first flat index of an invalid value or -1.
int64_t pack_rows(const int8_t* w, int64_t cols, int64_t r0, int64_t r1, uint8_t* out) {
  const int64_t words = cols / 16;
  for (int64_t r = r0; r < r1; ++r) {
    const int8_t* row = w + r * cols;
    uint8_t* dst = out + r * (cols / 4);
    for (int64_t j = 0; j < words; ++j) {
      const int8_t* g = row + 16 * j;
      bool ok = true;
      for (int m = 0; m < 16; ++m) ok &= static_cast<uint8_t>(g[m] + 1) <= 2;
      if (!ok) {
        for (int m = 0; m < 16; ++m)
          if (static_cast<uint8_t>(g[m] + 1) > 2) return r * cols + 16 * j + m;
      }
      for (int b = 0; b < 4; ++b) {
        const unsigned c0 = static_cast<unsigned>(g[2 * b]) & 3u;
        const unsigned c1 = static_cast<unsigned>(g[2 * b + 1]) & 3u;
        const unsigned c2 = static_cast<unsigned>(g[8 + 2 * b]) & 3u;
        const unsigned c3 = static_cast<unsigned>(g[9 + 2 * b]) & 3u;
        dst[4 * j + b] = static_cast<uint8_t>(c0 | (c1 << 2) | (c2 << 4) | (c3 << 6));
      }
    }
  }
  return -1;
}

int64_t unpack_rows(const uint8_t* in, int64_t cols, int64_t r0, int64_t r1, int8_t* w) {
  static const int8_t kValue[4] = {0, 1, 127, -1};  // 0b10 is invalid (marked 127)
  const int64_t words = cols / 16;
  for (int64_t r = r0; r < r1; ++r) {
    const uint8_t* src = in + r * (cols / 4);
    int8_t* row = w + r * cols;
    for (int64_t j = 0; j < words; ++j) {
      for (int b = 0; b < 4; ++b) {
        const unsigned byte = src[4 * j + b];
        const int8_t v[4] = {kValue[byte & 3u], kValue[(byte >> 2) & 3u], kValue[(byte >> 4) & 3u],
                             kValue[(byte >> 6) & 3u]};
        const int idx[4] = {2 * b, 2 * b + 1, 8 + 2 * b, 9 + 2 * b};
        for (int q = 0; q < 4; ++q) {
          if (v[q] == 127) return r * cols + 16 * j + idx[q];
          row[16 * j + idx[q]] = v[q];
        }
      }
    }
  }
  return -1;
}

template <class F>
int64_t parallel_rows(int64_t rows, int64_t cols, F&& fn) {
  const int64_t work = rows * cols;
  unsigned hw = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  const int64_t nthreads = work < (int64_t{1} << 22) ? 1 : std::min<int64_t>(hw, rows);
  if (nthreads <= 1) return fn(0, rows);
  std::vector<int64_t> bad(nthreads, -1);
  std::vector<std::thread> pool;
  const int64_t per = (rows + nthreads - 1) / nthreads;
  for (int64_t t = 0; t < nthreads; ++t) {
    const int64_t r0 = t * per, r1 = std::min(rows, r0 + per);
    if (r0 >= r1) break;
    pool.emplace_back([&, t, r0, r1] { bad[t] = fn(r0, r1); });
  }
  for (auto& th : pool) th.join();
  for (int64_t b : bad)
    if (b >= 0) return b;  // threads own increasing row ranges: first hit is the lowest
  return -1;
}

bool valid_shape(int64_t rows, int64_t cols) { return rows >= 1 && cols >= 64 && cols % 64 == 0; }

// Base-3: row r is ceil(cols / 5) bytes; byte m holds weights 5 m + i as
// digits w + 1 (first weight least significant); padding weights are 0.
int64_t b3_row(int64_t cols) { return (cols + 4) / 5; }
bool b3_valid_shape(int64_t rows, int64_t cols) { return rows >= 1 && cols >= 1 && cols <= PWG_MAX_COLS; }

int64_t pack_rows_b3(const int8_t* w, int64_t cols, int64_t r0, int64_t r1, uint8_t* out) {
  const int64_t B = b3_row(cols);
  for (int64_t r = r0; r < r1; ++r) {
    const int8_t* row = w + r * cols;
    uint8_t* dst = out + r * B;
    for (int64_t m = 0; m < B; ++m) {
      unsigned code = 0, place = 1;
      for (int i = 0; i < 5; ++i, place *= 3) {
        const int64_t k = 5 * m + i;
        const int v = k < cols ? row[k] : 0;
        if (v < -1 || v > 1) return r * cols + k;
        code += static_cast<unsigned>(v + 1) * place;
      }
      dst[m] = static_cast<uint8_t>(code);
    }
  }
  return -1;
}

// Returns the flat index (row * B + byte) of the first invalid byte or -1.
int64_t unpack_rows_b3(const uint8_t* in, int64_t cols, int64_t r0, int64_t r1, int8_t* w) {
  const int64_t B = b3_row(cols);
  for (int64_t r = r0; r < r1; ++r) {
    const uint8_t* src = in + r * B;
    int8_t* row = w + r * cols;
    for (int64_t m = 0; m < B; ++m) {
      unsigned code = src[m];
      if (code > 242) return r * B + m;
      for (int i = 0; i < 5; ++i, code /= 3) {
        const int64_t k = 5 * m + i;
        if (k < cols) row[k] = static_cast<int8_t>(static_cast<int>(code % 3) - 1);
      }
    }
  }
  return -1;
}

}  // namespace

extern "C" size_t pwg_packed_size(int64_t rows, int64_t cols) {
  if (!valid_shape(rows, cols)) return 0;
  return static_cast<size_t>(rows) * static_cast<size_t>(cols) / 4;
}

extern "C" int pwg_pack_weights(const int8_t* w_host, int64_t rows, int64_t cols, void* out_host,
                                size_t out_capacity, size_t* out_bytes) {
  using pwg::fail;
  if (!w_host || !out_host) return fail(PWG_ERR_ARG, "pwg_pack_weights: null pointer");
  if (!valid_shape(rows, cols))
    return fail(PWG_ERR_ARG, "pwg_pack_weights: need rows >= 1 and cols a positive multiple of 64 (got %lld x %lld)",
                (long long)rows, (long long)cols);
  const size_t need = pwg_packed_size(rows, cols);
  if (out_capacity < need)
    return fail(PWG_ERR_SIZE, "pwg_pack_weights: output capacity %zu < %zu bytes", out_capacity, need);
  uint8_t* out = static_cast<uint8_t*>(out_host);
  const int64_t bad = parallel_rows(rows, cols, [&](int64_t r0, int64_t r1) {
    return pack_rows(w_host, cols, r0, r1, out);
  });
  if (bad >= 0)
    return fail(PWG_ERR_VALUE, "pwg_pack_weights: value %d at (row %lld, col %lld) is not in {-1, 0, 1}",
                (int)w_host[bad], (long long)(bad / cols), (long long)(bad % cols));
  if (out_bytes) *out_bytes = need;
  return PWG_OK;
}

extern "C" int pwg_unpack_weights(const void* packed_host, int64_t rows, int64_t cols, int8_t* w_out_host) {
  using pwg::fail;
  if (!packed_host || !w_out_host) return fail(PWG_ERR_ARG, "pwg_unpack_weights: null pointer");
  if (!valid_shape(rows, cols))
    return fail(PWG_ERR_ARG, "pwg_unpack_weights: need rows >= 1 and cols a positive multiple of 64");
  const uint8_t* in = static_cast<const uint8_t*>(packed_host);
  const int64_t bad = parallel_rows(rows, cols, [&](int64_t r0, int64_t r1) {
    return unpack_rows(in, cols, r0, r1, w_out_host);
  });
  if (bad >= 0)
    return fail(PWG_ERR_VALUE, "pwg_unpack_weights: invalid code 0b10 at (row %lld, col %lld)",
                (long long)(bad / cols), (long long)(bad % cols));
  return PWG_OK;
}

extern "C" size_t pwg_b3_packed_size(int64_t rows, int64_t cols) {
  if (!b3_valid_shape(rows, cols)) return 0;
  return static_cast<size_t>(rows) * static_cast<size_t>(b3_row(cols));
}

extern "C" int pwg_pack_weights_b3(const int8_t* w_host, int64_t rows, int64_t cols, void* out_host,
                                   size_t out_capacity, size_t* out_bytes) {
  using pwg::fail;
  const char* fn = "pwg_pack_weights_b3";
  if (!w_host || !out_host) return fail(PWG_ERR_ARG, "%s: null pointer", fn);
  if (!b3_valid_shape(rows, cols))
    return fail(PWG_ERR_ARG, "%s: need rows >= 1 and cols in [1, %d] (got %lld x %lld)", fn, PWG_MAX_COLS,
                (long long)rows, (long long)cols);
  const size_t need = pwg_b3_packed_size(rows, cols);
  if (out_capacity < need) return fail(PWG_ERR_SIZE, "%s: output capacity %zu < %zu bytes", fn, out_capacity, need);
  uint8_t* out = static_cast<uint8_t*>(out_host);
  const int64_t bad = parallel_rows(rows, cols, [&](int64_t r0, int64_t r1) {
    return pack_rows_b3(w_host, cols, r0, r1, out);
  });
  if (bad >= 0)
    return fail(PWG_ERR_VALUE, "%s: value %d at (row %lld, col %lld) is not in {-1, 0, 1}", fn, (int)w_host[bad],
                (long long)(bad / cols), (long long)(bad % cols));
  if (out_bytes) *out_bytes = need;
  return PWG_OK;
}

extern "C" int pwg_unpack_weights_b3(const void* packed_host, int64_t rows, int64_t cols, int8_t* w_out_host) {
  using pwg::fail;
  const char* fn = "pwg_unpack_weights_b3";
  if (!packed_host || !w_out_host) return fail(PWG_ERR_ARG, "%s: null pointer", fn);
  if (!b3_valid_shape(rows, cols))
    return fail(PWG_ERR_ARG, "%s: need rows >= 1 and cols in [1, %d] (got %lld x %lld)", fn, PWG_MAX_COLS,
                (long long)rows, (long long)cols);
  const uint8_t* in = static_cast<const uint8_t*>(packed_host);
  const int64_t B = b3_row(cols);
  const int64_t bad = parallel_rows(rows, cols, [&](int64_t r0, int64_t r1) {
    return unpack_rows_b3(in, cols, r0, r1, w_out_host);
  });
  if (bad >= 0)
    return fail(PWG_ERR_VALUE, "%s: byte %u at (row %lld, byte %lld) is not a base-3 code (0..242)", fn,
                (unsigned)in[bad], (long long)(bad / B), (long long)(bad % B));
  return PWG_OK;
}

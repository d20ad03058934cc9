// Host-only driver for a sanitizer build (AddressSanitizer + UndefinedBehavior
// Sanitizer) of the library's CPU code: the T2 packer and unpacker and the
// host checks of a step description (buffer aliasing, plan fingerprints).
// Built and run by tests/test_host_sanitizers.py with g++; exits 0 when every
// check holds, prints the first failure otherwise.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../../packed_weight_gemv_amd/csrc/pwg_internal.h"

#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                   \
    }                                                                 \
  } while (0)

static void pack_round_trips() {
  std::mt19937 rng(7);
  const int64_t shapes[][2] = {{1, 64}, {3, 128}, {17, 192}, {1, 4096}, {64, 1024}, {300, 4096}, {5, 16384}, {2049, 128}};
  for (const auto& sh : shapes) {
    const int64_t rows = sh[0], cols = sh[1];
    std::vector<int8_t> w(static_cast<size_t>(rows * cols));
    for (auto& v : w) v = static_cast<int8_t>(static_cast<int>(rng() % 3) - 1);
    const size_t need = pwg_packed_size(rows, cols);
    CHECK(need == static_cast<size_t>(rows * cols / 4));
    std::vector<unsigned char> blob(need);  // exactly sized: any overrun is caught
    size_t wrote = 0;
    CHECK(pwg_pack_weights(w.data(), rows, cols, blob.data(), need, &wrote) == PWG_OK);
    CHECK(wrote == need);
    std::vector<int8_t> back(w.size());
    CHECK(pwg_unpack_weights(blob.data(), rows, cols, back.data()) == PWG_OK);
    CHECK(std::memcmp(back.data(), w.data(), w.size()) == 0);
    CHECK(pwg_pack_weights(w.data(), rows, cols, blob.data(), need - 1, nullptr) == PWG_ERR_SIZE);
    w.back() = 2;  // the last weight out of range
    CHECK(pwg_pack_weights(w.data(), rows, cols, blob.data(), need, nullptr) == PWG_ERR_VALUE);
    CHECK(std::strstr(pwg_last_error(), "row") != nullptr);
    blob[need - 1] = 0xAA;  // code 0b10 in every field of the last byte
    CHECK(pwg_unpack_weights(blob.data(), rows, cols, back.data()) == PWG_ERR_VALUE);
  }
  CHECK(pwg_packed_size(0, 64) == 0 && pwg_packed_size(4, 60) == 0 && pwg_packed_size(-1, 64) == 0);
  int8_t one = 0;
  unsigned char out[16];
  CHECK(pwg_pack_weights(nullptr, 1, 64, out, 16, nullptr) == PWG_ERR_ARG);
  CHECK(pwg_pack_weights(&one, 1, 63, out, 16, nullptr) == PWG_ERR_ARG);
  CHECK(pwg_unpack_weights(nullptr, 1, 64, &one) == PWG_ERR_ARG);
}

// Base-3 packing and the blob header on exactly sized buffers.
static void base3_and_header_checks() {
  std::mt19937 rng(11);
  const int64_t shapes[][2] = {{1, 1}, {3, 7}, {17, 240}, {5, 1001}, {33, 4096}, {2, 12288}, {3, 16384}};
  for (const auto& sh : shapes) {
    const int64_t rows = sh[0], cols = sh[1];
    std::vector<int8_t> w(static_cast<size_t>(rows * cols));
    for (auto& v : w) v = static_cast<int8_t>(static_cast<int>(rng() % 3) - 1);
    const size_t need = pwg_b3_packed_size(rows, cols);
    CHECK(need == static_cast<size_t>(rows * ((cols + 4) / 5)));
    std::vector<unsigned char> blob(need);
    size_t wrote = 0;
    CHECK(pwg_pack_weights_b3(w.data(), rows, cols, blob.data(), need, &wrote) == PWG_OK && wrote == need);
    std::vector<int8_t> back(w.size());
    CHECK(pwg_unpack_weights_b3(blob.data(), rows, cols, back.data()) == PWG_OK);
    CHECK(std::memcmp(back.data(), w.data(), w.size()) == 0);
    CHECK(pwg_pack_weights_b3(w.data(), rows, cols, blob.data(), need - 1, nullptr) == PWG_ERR_SIZE);
    pwg_blob_header h;
    CHECK(pwg_blob_header_init(PWG_BLOB_B3, w.data(), rows, cols, &h) == PWG_OK);
    CHECK(pwg_blob_verify(&h, blob.data(), need) == PWG_OK);
    CHECK(pwg_blob_verify(&h, blob.data(), need - 1) == PWG_ERR_SIZE);
    blob[need - 1] = 243;  // not a base-3 code
    CHECK(pwg_unpack_weights_b3(blob.data(), rows, cols, back.data()) == PWG_ERR_VALUE);
    CHECK(pwg_blob_verify(&h, blob.data(), need) == PWG_ERR_VALUE);
    if (cols % 64 == 0) {  // the same matrix as T2 carries the same logical checksum
      std::vector<unsigned char> t2(pwg_packed_size(rows, cols));
      CHECK(pwg_pack_weights(w.data(), rows, cols, t2.data(), t2.size(), nullptr) == PWG_OK);
      pwg_blob_header h2;
      CHECK(pwg_blob_header_init(PWG_BLOB_T2, w.data(), rows, cols, &h2) == PWG_OK);
      CHECK(h2.logical_fnv1a == h.logical_fnv1a);
      CHECK(pwg_blob_verify(&h2, t2.data(), t2.size()) == PWG_OK);
    }
  }
  pwg_blob_header h;
  int8_t one = 1;
  CHECK(pwg_blob_header_init(PWG_BLOB_T2, &one, 1, 1, &h) == PWG_ERR_ARG);
  CHECK(pwg_blob_header_init(7, &one, 1, 1, &h) == PWG_ERR_ARG);
  CHECK(pwg_blob_header_init(PWG_BLOB_B3, &one, 1, 1, &h) == PWG_OK);
  h.header_fnv1a ^= 1u;
  CHECK(pwg_blob_header_check(&h, 1) == PWG_ERR_VALUE);
  CHECK(pwg_blob_header_check(nullptr, 1) == PWG_ERR_ARG);
}

static uintptr_t slot(int k) { return (uintptr_t{1} << 36) + static_cast<uintptr_t>(k) * (uintptr_t{1} << 24); }
template <typename T>
static T* P(int k) { return reinterpret_cast<T*>(slot(k)); }

static void step_checks() {
  pwg_level lv[3] = {};
  for (int i = 0; i < 3; ++i) {
    lv[i].w_packed = P<void>(20 + 4 * i);
    lv[i].row_scale = P<float>(21 + 4 * i);
    lv[i].x = P<float>(22 + 4 * i);
    lv[i].y = P<float>(23 + 4 * i);
    lv[i].rows = 100;
    lv[i].cols = 4096;
  }
  pwg_step_desc d = {};
  d.n_levels = 3;
  d.schedule = PWG_SCHEDULE_STREAM;
  d.weight_layout = PWG_LAYOUT_TILED;
  d.levels = lv;
  d.vocab = 1000;
  d.hidden = 4096;
  d.h = P<float>(2);
  d.emb_row_out = P<int8_t>(7);
  d.emb_scale_out = P<float>(8);
  d.logits_out = P<float>(9);
  d.workspace = P<void>(10);
  d.workspace_bytes = 1 << 20;
  CHECK(pwg::check_unordered_aliasing(&d, "t") == PWG_OK);
  lv[2].x = lv[1].y;
  CHECK(pwg::check_unordered_aliasing(&d, "t") == PWG_ERR_UNSUPPORTED);
  CHECK(std::strstr(pwg_last_error(), "x of level 2 overlaps y of level 1") != nullptr);
  lv[2].x = reinterpret_cast<const float*>(reinterpret_cast<uintptr_t>(lv[1].y) + 100 * 4);  // just past y1
  CHECK(pwg::check_unordered_aliasing(&d, "t") == PWG_OK);
  d.batch = 4;  // y1 now spans 4 vectors: the same x starts inside it
  CHECK(pwg::check_unordered_aliasing(&d, "t") == PWG_ERR_UNSUPPORTED);
  d.batch = 0;
  lv[2].x = P<float>(30);
  d.h = reinterpret_cast<const float*>(slot(9) + 3996);  // overlaps the logits' last float
  CHECK(pwg::check_unordered_aliasing(&d, "t") == PWG_ERR_UNSUPPORTED);
  d.h = P<float>(2);

  // plan fingerprints: keyed by workspace, sensitive to every pointer and shape
  CHECK(pwg::plan_check(&d, "t") == PWG_ERR_ARG);  // never planned
  pwg::plan_record(&d);
  CHECK(pwg::plan_check(&d, "t") == PWG_OK);
  const uint64_t f0 = pwg::step_fingerprint(&d);
  lv[1].x = P<float>(31);
  CHECK(pwg::step_fingerprint(&d) != f0 && pwg::plan_check(&d, "t") == PWG_ERR_ARG);
  lv[1].x = P<float>(26);
  CHECK(pwg::plan_check(&d, "t") == PWG_OK);
  lv[0].rows = 101;
  CHECK(pwg::plan_check(&d, "t") == PWG_ERR_ARG);
  lv[0].rows = 100;
  lv[0].in.op = PWG_INPUT_SWIGLU;
  CHECK(pwg::plan_check(&d, "t") == PWG_ERR_ARG);
  lv[0].in.op = PWG_INPUT_GIVEN;
  pwg_step_desc other = d;
  other.workspace = P<void>(11);  // another workspace: no plan of its own
  CHECK(pwg::plan_check(&other, "t") == PWG_ERR_ARG);
  pwg::plan_forget(&d);
  CHECK(pwg::plan_check(&d, "t") == PWG_ERR_ARG);
}

int main() {
  pack_round_trips();
  base3_and_header_checks();
  step_checks();
  std::printf("host checks ok\n");
  return 0;
}

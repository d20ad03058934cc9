// Host-side checks of a step description that need no device (plain C++, no
// HIP): buffer aliasing on the schedules that do not order their levels, and
// the fingerprint that ties a workspace's device plan to the description it
// was planned for.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "pwg_internal.h"

namespace pwg {
namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  const char* what;
  int index;         // level, or -1
};

Range range_of(const void* p, size_t bytes, const char* what, int index) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes, what, index};
}

// A 64-bit mix of every field (each field zero-extended to 8 bytes).
struct Hasher {
  uint64_t h = 1469598103934665603ull;
  template <typename T>
  void add(const T& v) {
    static_assert(sizeof(T) <= 8, "one word per field");
    uint64_t u = 0;
    std::memcpy(&u, &v, sizeof(T));
    h ^= u + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
    h *= 0xFF51AFD7ED558CCDull;
    h ^= h >> 33;
  }
  void add_input(const pwg_input& in) {
    add(in.op);
    add(in.head_dim);
    add(in.group);
    add(in.eps);
    add(in.src);
    add(in.resid);
    add(in.gamma);
    add(in.resid_out);
  }
};

std::mutex g_mu;
std::unordered_map<uintptr_t, uint64_t>& plans() {
  static std::unordered_map<uintptr_t, uint64_t> m;
  return m;
}

}  // namespace

int check_unordered_aliasing(const pwg_step_desc* d, const char* fn) {
  const size_t nb = d->batch > 1 ? static_cast<size_t>(d->batch) : 1u;
  std::vector<Range> in, out;
  for (int i = 0; i < d->n_levels; ++i) {
    const pwg_level& L = d->levels[i];
    in.push_back(range_of(L.x, static_cast<size_t>(L.cols) * 4 * nb, "x", i));
    out.push_back(range_of(L.y, static_cast<size_t>(L.rows) * 4 * nb, "y", i));
  }
  in.push_back(range_of(d->h, static_cast<size_t>(d->hidden) * 4 * nb, "h", -1));
  if (d->logits_out) out.push_back(range_of(d->logits_out, static_cast<size_t>(d->vocab) * 4 * nb, "logits_out", -1));
  out.push_back(range_of(d->emb_row_out, static_cast<size_t>(d->hidden) * nb, "emb_row_out", -1));
  out.push_back(range_of(d->emb_scale_out, 4 * nb, "emb_scale_out", -1));
  if (d->emb_deq_out) out.push_back(range_of(d->emb_deq_out, static_cast<size_t>(d->hidden) * 4 * nb, "emb_deq_out", -1));
  auto name = [](const Range& r, char* buf, size_t n) {
    if (r.index >= 0) std::snprintf(buf, n, "%s of level %d", r.what, r.index);
    else std::snprintf(buf, n, "%s", r.what);
  };
  // sweep over the ranges by start address: an input overlaps an output iff
  // one of them starts before the other ends; keep the output (and the
  // input) that reaches furthest so far
  struct Ev {
    Range r;
    bool input;
  };
  std::vector<Ev> ev;
  ev.reserve(in.size() + out.size());
  for (const Range& r : in)
    if (r.lo != r.hi) ev.push_back({r, true});
  for (const Range& r : out)
    if (r.lo != r.hi) ev.push_back({r, false});
  std::sort(ev.begin(), ev.end(), [](const Ev& a, const Ev& b) { return a.r.lo < b.r.lo; });
  const Range* far_in = nullptr;
  const Range* far_out = nullptr;
  for (const Ev& e : ev) {
    const Range* other = e.input ? far_out : far_in;
    if (other && other->hi > e.r.lo) {
      char na[48], nb2[48];
      name(e.input ? e.r : *other, na, sizeof na);
      name(e.input ? *other : e.r, nb2, sizeof nb2);
      return fail(PWG_ERR_UNSUPPORTED,
                  "%s: %s overlaps %s; this schedule runs levels in no fixed order, so an input may not share "
                  "memory with anything the step writes (use the levels schedule for chained levels)",
                  fn, na, nb2);
    }
    const Range*& far = e.input ? far_in : far_out;
    if (!far || e.r.hi > far->hi) far = &e.r;
  }
  return PWG_OK;
}

uint64_t step_fingerprint(const pwg_step_desc* d) {
  Hasher h;
  h.add(d->n_levels);
  h.add(d->schedule);
  h.add(d->weight_layout);
  h.add(d->batch);
  for (int i = 0; i < d->n_levels; ++i) {
    const pwg_level& L = d->levels[i];
    h.add(L.w_packed);
    h.add(L.row_scale);
    h.add(L.x);
    h.add(L.y);
    h.add(L.rows);
    h.add(L.cols);
    h.add_input(L.in);
  }
  h.add(d->out_table);
  h.add(d->out_scale);
  h.add(d->h);
  h.add(d->vocab);
  h.add(d->hidden);
  h.add(d->emb_table);
  h.add(d->emb_scale);
  h.add(d->token_in);
  h.add(d->token_out);
  h.add(d->emb_row_out);
  h.add(d->emb_scale_out);
  h.add(d->emb_deq_out);
  h.add(d->logits_out);
  h.add(d->workspace);
  h.add(d->workspace_bytes);
  h.add_input(d->h_in);
  return h.h;
}

void plan_record(const pwg_step_desc* d) {
  std::lock_guard<std::mutex> lk(g_mu);
  plans()[reinterpret_cast<uintptr_t>(d->workspace)] = step_fingerprint(d);
}

void plan_forget(const pwg_step_desc* d) {
  std::lock_guard<std::mutex> lk(g_mu);
  plans().erase(reinterpret_cast<uintptr_t>(d->workspace));
}

int plan_check(const pwg_step_desc* d, const char* fn) {
  const uint64_t f = step_fingerprint(d);
  std::lock_guard<std::mutex> lk(g_mu);
  const auto it = plans().find(reinterpret_cast<uintptr_t>(d->workspace));
  if (it == plans().end())
    return fail(PWG_ERR_ARG, "%s: this workspace holds no plan; call pwg_step_plan with this description first", fn);
  if (it->second != f)
    return fail(PWG_ERR_ARG,
                "%s: the description differs from the one this workspace was planned for (a pointer, shape or "
                "input op changed); call pwg_step_plan again",
                fn);
  return PWG_OK;
}

}  // namespace pwg

// Randomised requests against the library's host-side validation and
// planning (plan.cpp): tree checks, ancestor sets, the re-root plan and the
// attention tiling. Built by tests/test_host_sanitize.py with g++ and the
// address and undefined-behaviour sanitizers; every array handed to the
// library is a heap block of exactly the size the call may touch, so a read
// or write past it is reported. Valid requests must succeed and produce
// outputs with the invariants checked here; corrupted ones must be refused
// with a status, never crash.
//
// Usage: host_plan_fuzz [iterations]   (exit status 0 when every check holds)
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <random>
#include <vector>

#include "plan.h"

using namespace ta;

namespace {

int g_failures = 0;
long g_ok_bits = 0, g_ok_reroot = 0, g_ok_attn = 0;  // accepted requests, by kind

#define CHECK(cond)                                                            \
  do {                                                                         \
    if (!(cond)) {                                                             \
      if (g_failures < 20) std::fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #cond); \
      ++g_failures;                                                            \
    }                                                                          \
  } while (0)

// A heap block of exactly n elements (null for n == 0), so that the
// sanitizer sees any access past the end.
template <typename T>
std::unique_ptr<T[]> block(int n) {
  return n > 0 ? std::unique_ptr<T[]>(new T[n]) : nullptr;
}

std::mt19937_64 rng(12345);
int uni(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }

// A random forest in the library's convention: parent[i] in {-1} U [0, i).
std::vector<int32_t> random_tree(int n) {
  std::vector<int32_t> p(n);
  for (int i = 0; i < n; ++i) p[i] = (i == 0 || uni(0, 3) == 0) ? -1 : uni(0, i - 1);
  return p;
}

int depth_of(const std::vector<int32_t>& p, int i) {
  int d = 0;
  for (; i >= 0; i = p[i]) ++d;
  return d;
}

void fuzz_ancestor_bits() {
  const int n = uni(-2, TA_MAX_TREE + 3);
  const int m = n > 0 ? n : 0;
  std::vector<int32_t> tree = random_tree(m);
  const bool corrupt = m > 0 && uni(0, 3) == 0;
  if (corrupt) tree[uni(0, m - 1)] = uni(-3, m + 3);
  auto parent = block<int32_t>(m);
  for (int i = 0; i < m; ++i) parent[i] = tree[i];
  auto lo = block<uint64_t>(m);
  const bool with_hi = uni(0, 4) != 0;
  auto hi = with_hi ? block<uint64_t>(m) : nullptr;
  const ta_status st = ancestor_bits(parent.get(), n, lo.get(), hi.get());
  bool valid = n >= 0 && n <= TA_MAX_TREE;
  for (int i = 0; valid && i < m; ++i) valid = tree[i] == -1 || (tree[i] >= 0 && tree[i] < i);
  if (!valid || (n > 64 && !with_hi)) {
    CHECK(st != TA_OK);
    return;
  }
  CHECK(st == TA_OK);
  if (st != TA_OK) return;
  ++g_ok_bits;
  for (int i = 0; i < m; ++i) {
    const uint64_t self_lo = i < 64 ? uint64_t{1} << i : 0, self_hi = i >= 64 ? uint64_t{1} << (i - 64) : 0;
    CHECK((lo[i] & self_lo) == self_lo);
    const int bits = __builtin_popcountll(lo[i]) + (with_hi ? __builtin_popcountll(hi[i]) : 0);
    CHECK(bits == depth_of(tree, i));
    if (with_hi) CHECK((hi[i] & self_hi) == self_hi);
    if (tree[i] >= 0) {
      CHECK((lo[i] & lo[tree[i]]) == lo[tree[i]]);
      if (with_hi) CHECK((hi[i] & hi[tree[i]]) == hi[tree[i]]);
    }
  }
}

void fuzz_reroot_plan() {
  const int n = uni(0, TA_MAX_TREE);
  std::vector<int32_t> tree = random_tree(n);
  // A valid request: a chain from a first-level node, then every (or a
  // random subset of the closed-downward) descendant of its last node.
  std::vector<int32_t> path, surv;
  if (n > 0 && uni(0, 4) != 0) {
    std::vector<int32_t> roots;
    for (int i = 0; i < n; ++i)
      if (tree[i] == -1) roots.push_back(i);
    int at = roots[uni(0, static_cast<int>(roots.size()) - 1)];
    path.push_back(at);
    for (;;) {
      std::vector<int32_t> kids;
      for (int i = at + 1; i < n; ++i)
        if (tree[i] == at) kids.push_back(i);
      if (kids.empty() || uni(0, 2) == 0) break;
      at = kids[uni(0, static_cast<int>(kids.size()) - 1)];
      path.push_back(at);
    }
  }
  const int last = path.empty() ? -1 : path.back();
  std::vector<char> keep(n, 0);
  for (int i = 0; i < n; ++i) {
    const int p = tree[i];
    const bool hangs = p == last || (p >= 0 && keep[p]);
    bool on_path = false;
    for (int a : path) on_path |= a == i;
    if (hangs && !on_path && uni(0, 3) != 0) keep[i] = 1;
  }
  for (int i = 0; i < n; ++i)
    if (keep[i]) surv.push_back(i);
  const int P = uni(0, 1 << 20);
  int capacity = P + n + uni(0, 64);
  // corruptions, one at a time
  const int what = uni(0, 9);
  bool valid = true;
  if (what == 0 && surv.size() >= 2) {
    std::swap(surv[0], surv[1]);
    valid = false;
  } else if (what == 1 && !path.empty() && n > 0) {
    surv.insert(surv.begin(), path[0]);
    valid = false;
  } else if (what == 2) {
    surv.push_back(n + uni(0, 3));
    valid = false;
  } else if (what == 3 && path.size() >= 2) {
    std::swap(path[0], path[1]);
    valid = false;
  } else if (what == 4) {
    capacity = P + n - 1 - uni(0, 3);  // too small (or negative)
    valid = false;
  } else if (what == 5 && n > 0) {
    tree[uni(0, n - 1)] = n + 5;
    valid = false;
  }
  if (static_cast<int64_t>(P) + n > capacity) valid = false;
  const int np = static_cast<int>(path.size()), ns = static_cast<int>(surv.size());
  auto parent = block<int32_t>(n);
  for (int i = 0; i < n; ++i) parent[i] = tree[i];
  auto pa = block<int32_t>(np);
  for (int i = 0; i < np; ++i) pa[i] = path[i];
  auto su = block<int32_t>(ns);
  for (int i = 0; i < ns; ++i) su[i] = surv[i];
  auto src = block<int32_t>(np + ns);
  auto npar = block<int32_t>(ns);
  int32_t new_prefix = -7;
  const ta_status st = plan_kv_reroot(P, capacity, parent.get(), n, pa.get(), np, su.get(), ns, src.get(),
                                      npar.get(), &new_prefix);
  if (!valid) {
    CHECK(st != TA_OK);
    return;
  }
  CHECK(st == TA_OK);
  if (st != TA_OK) return;
  ++g_ok_reroot;
  CHECK(new_prefix == P + np);
  for (int k = 0; k < np + ns; ++k) {
    CHECK(src[k] >= P + k);                   // a row never moves to a later slot
    if (k > 0) CHECK(src[k] > src[k - 1]);    // strictly ascending: the in-place copy is safe
  }
  for (int k = 0; k < ns; ++k) {
    CHECK(npar[k] >= -1 && npar[k] < k);
    const int p = tree[surv[k]];
    if (p == last) CHECK(npar[k] == -1);
    else CHECK(npar[k] >= 0 && surv[npar[k]] == p);
  }
}

void fuzz_reroot_arguments() {
  // Counts and pointers that do not fit: refused, nothing read past the
  // blocks actually given.
  const int n = uni(0, 8);
  std::vector<int32_t> tree = random_tree(n);
  auto parent = block<int32_t>(n);
  for (int i = 0; i < n; ++i) parent[i] = tree[i];
  auto one = block<int32_t>(1);
  one[0] = 0;
  int32_t np_out = 0;
  auto npar = block<int32_t>(1);
  CHECK(plan_kv_reroot(5, 100, parent.get(), n, nullptr, 1, nullptr, 0, nullptr, npar.get(), &np_out) != TA_OK);
  CHECK(plan_kv_reroot(5, 100, parent.get(), n, one.get(), -1, nullptr, 0, nullptr, npar.get(), &np_out) != TA_OK);
  CHECK(plan_kv_reroot(-1, 100, parent.get(), n, nullptr, 0, nullptr, 0, nullptr, npar.get(), &np_out) != TA_OK);
  // prefix_len + n_tree past the capacity near the top of the int32 range
  CHECK((plan_kv_reroot(2147483647 - 2, 2147483647, parent.get(), n, nullptr, 0, nullptr, 0, nullptr, npar.get(),
                        &np_out) != TA_OK) == (n > 2));
  CHECK(plan_kv_reroot(5, 100, parent.get(), n, nullptr, 0, one.get(), n + 1, nullptr, npar.get(), &np_out) != TA_OK);
  CHECK(plan_kv_reroot(5, 100, parent.get(), n, nullptr, 0, nullptr, 0, nullptr, npar.get(), nullptr) != TA_OK);
}

void fuzz_attn_plan() {
  ta_kv_cache c{};
  c.k = nullptr;
  c.v = nullptr;
  const int pick = uni(0, 9);
  c.dtype = pick == 0 ? uni(-1, 3) : uni(0, 1);
  c.head_dim = pick == 1 ? uni(0, 300) : (uni(0, 1) ? 64 : 128);
  c.n_layers = pick == 2 ? uni(-1, 1) : uni(1, 80);
  c.n_kv_heads = pick == 3 ? uni(-1, 1) : (1 << uni(0, 4));
  const int group = uni(1, 20);
  const int n_q_heads = pick == 5 ? uni(-3, 40) : c.n_kv_heads * group;
  const int n_tree = pick == 6 ? uni(-3, TA_MAX_TREE + 3) : uni(0, TA_MAX_TREE);
  const int q_first = pick == 7 ? uni(-3, n_tree + 3) : (n_tree > 0 ? uni(0, n_tree) : 0);
  // prefixes from empty to the top of the int32 range, most of them short
  const int prefix_len = pick == 8 ? uni(-5, 5)
                         : uni(0, 2) ? uni(0, 1 << uni(0, 24))
                                     : uni(0, 2147483647 - TA_MAX_TREE);
  const int64_t room = static_cast<int64_t>(prefix_len) + (n_tree > 0 ? n_tree : 0) + uni(0, 1000);
  c.capacity = pick == 4 ? uni(-5, 5) : static_cast<int32_t>(room < 2147483647 ? room : 2147483647);
  if (pick == 9) c.capacity = uni(1, 2147483647);
  AttnPlan p;
  const ta_status st = plan_tree_attn(&c, n_q_heads, prefix_len, n_tree, q_first, &p);
  const bool shape_ok = (c.dtype == TA_F32 || c.dtype == TA_BF16) && (c.head_dim == 64 || c.head_dim == 128) &&
                        c.n_layers >= 1 && c.n_kv_heads >= 1 && c.capacity >= 1 && n_tree >= 0 &&
                        n_tree <= TA_MAX_TREE && prefix_len >= 0 && q_first >= 0 && q_first <= n_tree &&
                        n_q_heads >= 1 && n_q_heads % c.n_kv_heads == 0 && n_q_heads / c.n_kv_heads <= 16 &&
                        static_cast<int64_t>(prefix_len) + n_tree <= c.capacity;
  if (!shape_ok) {
    CHECK(st != TA_OK);
    return;
  }
  if (st != TA_OK) return;  // refused for a range limit of the kernels: fine
  ++g_ok_attn;
  CHECK(p.group == n_q_heads / c.n_kv_heads);
  CHECK(p.rows_per_head == p.group * (n_tree - q_first));
  CHECK(p.total_keys == prefix_len + n_tree);
  const int64_t bytes = static_cast<int64_t>(p.total_keys) * c.head_dim * (c.dtype == TA_F32 ? 4 : 2);
  CHECK(bytes < 2147483647);  // the kernels' 32-bit buffer ranges
  if (p.rows_per_head == 0) return;
  // 128-row blocks, or 64 (bf16 only: always for heads of at most 64 rows)
  CHECK(p.block_rows == 128 || (p.block_rows == 64 && c.dtype == TA_BF16));
  if (c.dtype == TA_BF16 && p.rows_per_head <= 64) CHECK(p.block_rows == 64);
  CHECK(p.row_blocks == (p.rows_per_head + p.block_rows - 1) / p.block_rows);
  CHECK(p.splits >= 1 && p.splits <= kMaxSplits);
  CHECK(p.splits <= p.n_tiles);  // every split has at least one stage
  CHECK(p.n_units == c.n_kv_heads * p.row_blocks * p.splits && p.n_units < kMaxUnits);
  if (p.splits > 1) {
    CHECK(p.ws_cnt_offset == 0 && p.ws_ml_offset >= kCounterBytes);
    CHECK(p.ws_o_offset % 256 == 0 && p.ws_o_offset >= p.ws_ml_offset + static_cast<size_t>(p.n_units) * 128 * 8);
    CHECK(p.ws_bytes >= p.ws_o_offset + static_cast<size_t>(p.n_units) * 128 * c.head_dim * 4);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::strtol(argv[1], nullptr, 10) : 10000;
  for (long i = 0; i < iters; ++i) {
    fuzz_ancestor_bits();
    fuzz_reroot_plan();
    fuzz_attn_plan();
    if (i % 64 == 0) fuzz_reroot_arguments();
  }
  std::printf("%ld iterations, %d failed checks; accepted: %ld ancestor sets, %ld re-root plans, %ld attention plans\n",
              iters, g_failures, g_ok_bits, g_ok_reroot, g_ok_attn);
  return g_failures == 0 ? 0 : 1;
}

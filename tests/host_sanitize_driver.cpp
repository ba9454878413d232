// Drives the host-only part of libpop (pop_host.cpp: status strings, the
// last-error buffer, region counts, top-k counts and the index-list check)
// through its whole argument range, for a build under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Self-checks the results against the
// definitions restated here in the plainest form; prints "ok <cases>" and
// exits 0 when every check held.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "pop.h"

static int g_failures = 0;
static long g_cases = 0;

#define EXPECT(cond, ...)                      \
  do {                                         \
    ++g_cases;                                 \
    if (!(cond)) {                             \
      if (++g_failures <= 20) {                \
        fprintf(stderr, "FAIL %s: ", #cond);   \
        fprintf(stderr, __VA_ARGS__);          \
        fprintf(stderr, "\n");                 \
      }                                        \
    }                                          \
  } while (0)

// splitmix64: a small counter-based generator for the random cases
static uint64_t g_state = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64() {
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
static int32_t uniform_int(int32_t lo, int32_t hi) {  // [lo, hi]
  return lo + (int32_t)(next_u64() % (uint64_t)((int64_t)hi - lo + 1));
}
static double uniform01() { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

static int64_t cut(double p, int32_t n) { return (int64_t)round(std::min(std::max(p, 0.0), 1.0) * n); }

static void check_counts() {
  const double special[] = {0.0, 0.25, 0.5, 0.75, 1.0 / 3.0, 0.999999, 1e-12};
  for (int trial = 0; trial < 20000; ++trial) {
    const int32_t n = trial < 64 ? (trial % 2 ? POP_MAX_D_FF : 1 + trial) : uniform_int(1, POP_MAX_D_FF);
    const double r = trial % 5 == 0 ? special[trial / 5 % 7] : uniform01() * 0.999;
    const double g = trial % 7 == 0 ? special[trial / 7 % 7] : uniform01() * 0.999;
    pop_counts c;
    memset(&c, 0xff, sizeof(c));
    EXPECT(pop_partition_counts(n, r, g, &c) == POP_OK, "n=%d r=%g g=%g", n, r, g);
    const int64_t lo = cut(r - g, n), hi = cut(r + g, n), live = (int64_t)round((1.0 - r) * n);
    EXPECT(c.d_ff == n && c.c_low == lo && c.c_high == hi && c.n_live == live, "n=%d r=%g g=%g", n, r, g);
    EXPECT(c.n_P + c.n_C + c.n_R == n && c.n_P >= 0 && c.n_C >= 0 && c.n_R >= 0, "n=%d", n);
    EXPECT(c.k >= 0 && c.k <= c.n_C, "k=%d n_C=%d", c.k, c.n_C);
    int32_t k = -1;
    EXPECT(pop_decode_topk_count(n, r, c.n_R, c.n_C, &k) == POP_OK && k == c.k, "k=%d c.k=%d", k, c.k);
  }
  pop_counts c;
  EXPECT(pop_partition_counts(0, 0.5, 0.1, &c) == POP_ERR_BAD_SHAPE, "d_ff=0");
  EXPECT(pop_partition_counts(POP_MAX_D_FF + 1, 0.5, 0.1, &c) == POP_ERR_BAD_SHAPE, "d_ff too large");
  EXPECT(pop_partition_counts(16, NAN, 0.1, &c) == POP_ERR_INVALID_ARGUMENT, "r=nan");
  EXPECT(pop_partition_counts(16, 0.5, INFINITY, &c) == POP_ERR_INVALID_ARGUMENT, "gamma=inf");
  EXPECT(pop_partition_counts(16, 0.5, 0.1, nullptr) == POP_ERR_INVALID_ARGUMENT, "out=NULL");
  EXPECT(strlen(pop_last_error()) > 0, "an error message is set");
  int32_t k;
  EXPECT(pop_decode_topk_count(16, 0.5, 10, 10, &k) == POP_ERR_INVALID_ARGUMENT, "n_R + n_C > d_ff");
  EXPECT(pop_decode_topk_count(16, 0.5, INT32_MAX, INT32_MAX, &k) == POP_ERR_INVALID_ARGUMENT, "int32 overflow");
  EXPECT(pop_decode_topk_count(16, 0.5, -1, 0, &k) == POP_ERR_INVALID_ARGUMENT, "negative n_R");
  EXPECT(pop_decode_topk_count(16, 0.5, 0, 0, nullptr) == POP_ERR_INVALID_ARGUMENT, "k=NULL");
}

// The plain definition pop_check_lists follows: each list strictly ascending
// in [0, d_ff), no channel twice, total count at most d_ff.
static bool lists_valid(const std::vector<int32_t>* l, int32_t d_ff) {
  std::vector<int> seen((size_t)d_ff, 0);
  int64_t total = 0;
  for (int j = 0; j < 3; ++j) {
    total += (int64_t)l[j].size();
    for (size_t i = 0; i < l[j].size(); ++i) {
      const int32_t c = l[j][i];
      if (c < 0 || c >= d_ff || (i > 0 && c <= l[j][i - 1]) || seen[(size_t)c]++) return false;
    }
  }
  return total <= d_ff;
}

static void check_lists() {
  for (int trial = 0; trial < 20000; ++trial) {
    const int32_t d_ff = trial < 8 ? POP_MAX_D_FF : uniform_int(1, trial % 10 == 0 ? 4096 : 64);
    std::vector<int32_t> l[3];
    for (int32_t c = 0; c < d_ff; ++c) {
      const int owner = uniform_int(-1, 2);
      if (owner >= 0) l[owner].push_back(c);
    }
    const int j = uniform_int(0, 2);
    std::vector<int32_t>& a = l[j];
    switch (uniform_int(0, 6)) {  // plant at most one mistake
      case 1: if (a.size() >= 2) std::swap(a[a.size() / 2 - 1], a[a.size() / 2]); break;
      case 2: if (!a.empty()) a.insert(a.begin() + a.size() / 2, a[a.size() / 2]); break;
      case 3: if (!a.empty()) { l[(j + 1) % 3].push_back(a.back()); std::sort(l[(j + 1) % 3].begin(), l[(j + 1) % 3].end()); } break;
      case 4: a.insert(a.begin(), -uniform_int(1, 1 << 30)); break;
      case 5: a.push_back(d_ff + uniform_int(0, 1 << 30)); break;
      case 6: a.push_back(INT32_MIN); break;
      default: break;
    }
    // exact-size heap copies, so that any read past a list's end is caught
    std::vector<int32_t*> h(3, nullptr);
    for (int q = 0; q < 3; ++q)
      if (!l[q].empty()) {
        h[q] = new int32_t[l[q].size()];
        std::copy(l[q].begin(), l[q].end(), h[q]);
      }
    const pop_status s = pop_check_lists(h[0], (int32_t)l[0].size(), h[1], (int32_t)l[1].size(), h[2],
                                         (int32_t)l[2].size(), d_ff);
    const bool ok = lists_valid(l, d_ff);
    EXPECT(s == (ok ? POP_OK : POP_ERR_INVALID_ARGUMENT), "d_ff=%d status=%d expected ok=%d (%s)", d_ff, (int)s,
           (int)ok, pop_last_error());
    EXPECT(ok == (pop_last_error()[0] == '\0'), "error message set iff the check failed");
    for (int q = 0; q < 3; ++q) delete[] h[q];
  }
  const int32_t one = 0;
  EXPECT(pop_check_lists(nullptr, 3, nullptr, 0, nullptr, 0, 8) == POP_ERR_INVALID_ARGUMENT, "NULL R");
  EXPECT(pop_check_lists(&one, 1, nullptr, 1, nullptr, 0, 8) == POP_ERR_INVALID_ARGUMENT, "NULL C");
  EXPECT(pop_check_lists(&one, INT32_MAX, &one, INT32_MAX, &one, INT32_MAX, POP_MAX_D_FF) == POP_ERR_INVALID_ARGUMENT,
         "counts past d_ff are rejected before any read");
  EXPECT(pop_check_lists(&one, -1, nullptr, 0, nullptr, 0, 8) == POP_ERR_INVALID_ARGUMENT, "negative count");
  EXPECT(pop_check_lists(nullptr, 0, nullptr, 0, nullptr, 0, 0) == POP_ERR_BAD_SHAPE, "d_ff=0");
  EXPECT(pop_check_lists(nullptr, 0, nullptr, 0, nullptr, 0, INT32_MIN) == POP_ERR_BAD_SHAPE, "d_ff<0");
}

static void check_strings() {
  for (int s = -3; s < 16; ++s) {
    const char* t = pop_status_string((pop_status)s);
    EXPECT(t != nullptr && strncmp(t, "POP_", 4) == 0, "status %d", s);
  }
  // a message longer than the error buffer is truncated, not overrun
  std::vector<int32_t> big(POP_MAX_D_FF);
  for (int32_t i = 0; i < POP_MAX_D_FF; ++i) big[(size_t)i] = POP_MAX_D_FF - 1 - i;
  EXPECT(pop_check_lists(big.data(), POP_MAX_D_FF, nullptr, 0, nullptr, 0, POP_MAX_D_FF) == POP_ERR_INVALID_ARGUMENT,
         "descending list");
  EXPECT(strlen(pop_last_error()) < 4096, "bounded message");
}

int main() {
  check_counts();
  check_lists();
  check_strings();
  if (g_failures) {
    fprintf(stderr, "%d of %ld checks failed\n", g_failures, g_cases);
    return 1;
  }
  printf("ok %ld\n", g_cases);
  return 0;
}

// Brute-force check of the split-KV partition arithmetic (partition.h) on the
// host: every page of every sequence lands in exactly one range, the slot of
// each (range, sequence) piece is unique, and the combine's search for the
// ranges of a sequence finds exactly the ranges that hold its pages.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "../../latent_kv_cache_mla_amd/csrc/partition.h"

using namespace mla;

static int fails = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL %s at line %d\n", #c, __LINE__); ++fails; return; } } while (0)

static void check_case(const std::vector<int64_t>& lens, int64_t G) {
  const int64_t B = static_cast<int64_t>(lens.size());
  std::vector<int64_t> start(B + 1, 0);
  for (int64_t b = 0; b < B; ++b) start[b + 1] = start[b] + pages_of(lens[b]);
  const int64_t P = start[B];
  if (P == 0) return;
  // range_of_page agrees with a linear scan
  for (int64_t x = 0; x < P; ++x) {
    int64_t want = -1;
    for (int64_t g = 0; g < G; ++g) if (range_begin(g, P, G) <= x) want = g;
    CHECK(range_of_page(x, P, G) == want);
    CHECK(range_begin(want, P, G) <= x && x < range_begin(want + 1, P, G));
  }
  // pieces as the decode kernel enumerates them
  std::set<int64_t> slots;
  std::vector<std::set<int64_t>> ranges_of(B);
  std::vector<int64_t> covered(P, 0);
  for (int64_t g = 0; g < G; ++g) {
    const int64_t pb = range_begin(g, P, G), pe = range_begin(g + 1, P, G);
    if (pb >= pe) continue;
    int64_t lo = 0, hi = B - 1;
    while (lo < hi) { int64_t mid = (lo + hi) / 2; if (start[mid + 1] > pb) hi = mid; else lo = mid + 1; }
    for (int64_t b = lo; b < B && start[b] < pe; ++b) {
      if (start[b + 1] == start[b]) continue;
      const int64_t a0 = start[b] > pb ? start[b] : pb, a1 = start[b + 1] < pe ? start[b + 1] : pe;
      CHECK(a0 < a1);
      for (int64_t x = a0; x < a1; ++x) covered[x]++;
      CHECK(slots.insert(slot_of(g, b)).second);
      CHECK(slot_of(g, b) < G + B);
      ranges_of[b].insert(g);
    }
  }
  for (int64_t x = 0; x < P; ++x) CHECK(covered[x] == 1);
  // the combine's enumeration finds the same ranges
  for (int64_t b = 0; b < B; ++b) {
    std::set<int64_t> found;
    if (start[b + 1] > start[b]) {
      const int64_t glo = range_of_page(start[b], P, G), ghi = range_of_page(start[b + 1] - 1, P, G);
      for (int64_t g = glo; g <= ghi; ++g)
        if (range_begin(g + 1, P, G) != range_begin(g, P, G)) found.insert(g);
    }
    CHECK(found == ranges_of[b]);
  }
}

int main() {
  std::srand(12345);
  int cases = 0;
  for (int it = 0; it < 3000; ++it) {
    const int B = 1 + std::rand() % 12;
    std::vector<int64_t> lens(B);
    for (auto& s : lens) s = (std::rand() % 4 == 0) ? 0 : std::rand() % 700;
    const int64_t G = 1 + std::rand() % 40;
    check_case(lens, G);
    ++cases;
  }
  check_case(std::vector<int64_t>(32, 4096), 256);
  check_case(std::vector<int64_t>(4, 32768), 256);
  check_case(std::vector<int64_t>(128, 8192), 128);
  std::printf("%d cases, %d failures\n", cases + 3, fails);
  return fails ? 1 : 0;
}

// Walks the split-KV decode launch plan (grouped_query_attention_amd/csrc/
// decode_plan.h, the same code the library's launcher calls) on the host and
// replays each persistent workgroup's load/read order as decode_splitkv_kernel
// runs it:
//   * DC_STAGES - 1 tiles are issued before the loop;
//   * at each tile the workgroup waits for it, and at an item's first tile
//     reads the item's query slot, then issues the next tile;
//   * issuing an item's first tile also issues its query load into slot
//     (item ordinal % slots).
// A query load is taken to land the moment it is issued (the worst case), so
// a slot read finds another item's queries exactly when some later item's
// first tile was issued into the same slot before the read.
//
// Usage: decode_plan_walk <query slots> <n_cu> <B> <kv_len> [<B> <kv_len> ...]
//        decode_plan_walk <query slots> <n_cu> sweep <B_max> <kv_max>
// <query slots> "plan" takes the kernel's own count (DC_QSLOTS); a number
// replays the plan with that many slots instead.
// Prints one line per shape with a clobbered read ("clobber B kv_len ...")
// and a final "shapes N clobbered M".
#include <cstdio>
#include <cstdlib>
#include <string_view>
#include <vector>

#include "decode_plan.h"

using namespace gqa;

constexpr int N_KV = 8;

// Number of query-slot reads that would see another item's queries.
static long long walk(int slots, int n_cu, int B, int kv_len) {
  const DecodePlan p = decode_plan(B, kv_len, N_KV, n_cu);
  long long bad = 0;
  for (int wg = 0; wg < p.grid; ++wg) {
    std::vector<int> tiles;
    for (int item = wg; item < p.n_items; item += p.grid)
      tiles.push_back(decode_item_tiles(p, kv_len, item));
    const int n = (int)tiles.size();
    int total = 0;
    for (int t : tiles) total += t;
    std::vector<int> owner(slots, -1);
    int ld_j = 0, ld_t = 0, issued = 0;
    auto issue = [&]() {
      if (ld_t == 0) owner[ld_j % slots] = ld_j;
      if (++ld_t == tiles[ld_j]) { ld_t = 0; ++ld_j; }
      ++issued;
    };
    for (int s = 0; s < DC_STAGES - 1; ++s)
      if (issued < total) issue();
    for (int j = 0; j < n; ++j) {
      for (int t = 0; t < tiles[j]; ++t) {
        if (t == 0 && owner[j % slots] != j) ++bad;
        if (issued < total) issue();
      }
    }
  }
  return bad;
}

int main(int argc, char** argv) {
  if (argc < 5) {
    std::fprintf(stderr, "usage: %s slots n_cu (B kv_len)... | slots n_cu sweep B_max kv_max\n",
                 argv[0]);
    return 2;
  }
  const int slots = std::string_view(argv[1]) == "plan" ? DC_QSLOTS : std::atoi(argv[1]);
  const int n_cu = std::atoi(argv[2]);
  long long shapes = 0, clobbered = 0;
  auto one = [&](int B, int kv) {
    const long long bad = walk(slots, n_cu, B, kv);
    ++shapes;
    if (bad) {
      ++clobbered;
      std::printf("clobber B %d kv_len %d reads %lld\n", B, kv, bad);
    }
  };
  if (std::string_view(argv[3]) == "sweep") {
    const int bmax = std::atoi(argv[4]), kvmax = argc > 5 ? std::atoi(argv[5]) : 2048;
    for (int B = 1; B <= bmax; ++B)
      for (int kv = 1; kv <= kvmax; ++kv) one(B, kv);
  } else {
    for (int i = 3; i + 1 < argc; i += 2) one(std::atoi(argv[i]), std::atoi(argv[i + 1]));
  }
  std::printf("shapes %lld clobbered %lld\n", shapes, clobbered);
  return 0;
}

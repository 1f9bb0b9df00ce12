// Checks the causal prefill launch plan (grouped_query_attention_amd/csrc/
// flash_plan.h, the same code the library's launcher calls) on the host,
// against what flash_fwd_kernel and flash_merge_kernel assume of it:
//   * 2 <= bins <= FA_MAX_BINS, and the grid (bins x B x 8) fits the CUs the
//     plan balances over, so every bin runs at once;
//   * bin_start runs from 0 up to n_ent <= FA_MAX_ENT without going back;
//   * each entry names a query tile of the launch and a non-empty key range
//     inside that tile's causal range, and its fields fit their 8 bits;
//   * the entries of each query tile cover its key tiles exactly once;
//   * a tile with one entry writes H (slot FA_DIRECT); a cut tile has one
//     merge record, at most FA_MERGE_MAXP pieces, and its pieces hold the
//     record's consecutive slots in key order; slots are never shared and
//     n_slots < FA_DIRECT, n_merge <= FA_MAX_MERGE;
//   * in the plan's own cost model (an entry costs its key tiles plus
//     FA_ENTRY_COST, one workgroup per CU), the costliest bin takes no longer
//     than the plain launch (one workgroup per query tile, longest first, each
//     to the first free CU).
//
// Usage: flash_plan_walk <mode> <B> <T> <q_pos0> [<B> <T> <q_pos0> ...]
//        flash_plan_walk <mode> sweep <B_max> <T_max> <q_pos0> [<q_pos0> ...]
// kv_len is q_pos0 + T (a prefill chunk after q_pos0 cached positions).
// <mode> "plan" checks the plan as made; "drop" first removes the last key
// tile of the plan's last entry (or the entry itself), which every check run
// must then flag; "info" also prints "info B T q_pos0 planned n_slots" per
// shape. Prints one line per shape that breaks a rule and a final
// "shapes N planned P broken M worst_ratio R" (R: costliest bin over the
// plain launch's time, largest over planned shapes).
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <queue>
#include <string>
#include <string_view>
#include <vector>

#include "flash_plan.h"

using namespace gqa;

constexpr int N_KV = 8;

// Time of the plain causal launch in the cost model: workgroups in order of
// decreasing query tile, each to the CU that frees first.
static long long plain_time(int B, int nq, int kv_len, int q_pos0) {
  std::priority_queue<long long, std::vector<long long>, std::greater<long long>> cu;
  for (int i = 0; i < FA_PLAN_CUS; ++i) cu.push(0);
  long long end = 0;
  for (int qt = nq - 1; qt >= 0; --qt) {
    const long long c = flash_key_tiles(qt, kv_len, q_pos0) + FA_ENTRY_COST;
    for (int r = 0; r < B * N_KV; ++r) {
      const long long t = cu.top() + c;
      cu.pop();
      cu.push(t);
      end = std::max(end, t);
    }
  }
  return end;
}

// Returns the first broken rule, or an empty string.
static std::string check(const FlashPlan& p, int B, int T, int kv_len, int q_pos0,
                         double* ratio) {
  const int nq = (T + FA_BQ - 1) / FA_BQ;
  if (p.n_bins < 2 || p.n_bins > FA_MAX_BINS) return "bin count";
  if ((long long)p.n_bins * B * N_KV > FA_PLAN_CUS) return "grid exceeds the CUs";
  if (p.n_ent < 1 || p.n_ent > FA_MAX_ENT) return "entry count";
  if (p.bin_start[0] != 0 || p.bin_start[p.n_bins] != p.n_ent) return "bin_start ends";
  for (int s = 0; s < p.n_bins; ++s)
    if (p.bin_start[s + 1] < p.bin_start[s]) return "bin_start goes back";
  if (p.n_merge < 0 || p.n_merge > FA_MAX_MERGE) return "merge count";
  if (p.n_slots < 0 || p.n_slots >= FA_DIRECT) return "slot count";

  struct Piece { int kt0, kt1, slot; };
  std::vector<std::vector<Piece>> of(nq);
  long long worst_bin = 0;
  for (int s = 0; s < p.n_bins; ++s) {
    long long cost = 0;
    for (int i = p.bin_start[s]; i < p.bin_start[s + 1]; ++i) {
      const unsigned e = p.ent[i];
      const int qt = e & 255, kt0 = (e >> 8) & 255, kt1 = (e >> 16) & 255, slot = e >> 24;
      if (qt >= nq) return "entry query tile out of range";
      if (kt0 >= kt1) return "empty key range";
      if (kt1 > flash_key_tiles(qt, kv_len, q_pos0)) return "key range past the causal end";
      if (slot != FA_DIRECT && slot >= p.n_slots) return "slot out of range";
      of[qt].push_back({kt0, kt1, slot});
      cost += FA_ENTRY_COST + (kt1 - kt0);
    }
    worst_bin = std::max(worst_bin, cost);
  }
  std::vector<int> merges_of(nq, 0), slot_used(p.n_slots, 0);
  for (int m = 0; m < p.n_merge; ++m) {
    const unsigned r = p.mrg[m];
    const int qt = r & 255, slot0 = (r >> 8) & 255, pieces = r >> 16;
    if (qt >= nq) return "merge query tile out of range";
    if (++merges_of[qt] > 1) return "two merge records for one tile";
    if (pieces < 2 || pieces > FA_MERGE_MAXP) return "merge piece count";
    if (slot0 + pieces > p.n_slots) return "merge slots out of range";
    for (int j = 0; j < pieces; ++j)
      if (slot_used[slot0 + j]++) return "slot shared by two merges";
    std::vector<Piece> v = of[qt];
    std::sort(v.begin(), v.end(), [](const Piece& a, const Piece& b) { return a.kt0 < b.kt0; });
    if ((int)v.size() != pieces) return "merge pieces differ from the tile's entries";
    for (int j = 0; j < pieces; ++j)
      if (v[j].slot != slot0 + j) return "pieces not in consecutive slots in key order";
  }
  for (int qt = 0; qt < nq; ++qt) {
    std::vector<Piece> v = of[qt];
    if (v.empty()) return "query tile without entries";
    std::sort(v.begin(), v.end(), [](const Piece& a, const Piece& b) { return a.kt0 < b.kt0; });
    int next = 0;
    for (const Piece& pc : v) {
      if (pc.kt0 != next) return pc.kt0 < next ? "key tiles covered twice" : "key tiles missed";
      next = pc.kt1;
    }
    if (next != flash_key_tiles(qt, kv_len, q_pos0)) return "key tiles missed at the end";
    if (v.size() == 1 && (v[0].slot != FA_DIRECT || merges_of[qt]))
      return "whole tile not written directly";
    if (v.size() > 1 && !merges_of[qt]) return "cut tile without merge record";
  }
  const long long plain = plain_time(B, nq, kv_len, q_pos0);
  *ratio = (double)worst_bin / (double)plain;
  if (worst_bin > plain) return "plan slower than the plain launch";
  return "";
}

int main(int argc, char** argv) {
  if (argc < 5) {
    std::fprintf(stderr, "usage: %s plan|drop (B T q_pos0)... | plan|drop sweep B_max T_max q_pos0...\n",
                 argv[0]);
    return 2;
  }
  const bool drop = std::string_view(argv[1]) == "drop";
  const bool info = std::string_view(argv[1]) == "info";
  long long shapes = 0, planned = 0, broken = 0;
  double worst = 0.0;
  auto one = [&](int B, int T, int q_pos0) {
    const int kv_len = q_pos0 + T;
    FlashPlan p;
    ++shapes;
    const bool ok = flash_plan(B, T, kv_len, q_pos0, 1, N_KV, p);
    if (info) std::printf("info %d %d %d %d %d\n", B, T, q_pos0, ok ? 1 : 0, ok ? p.n_slots : 0);
    if (!ok) return;
    ++planned;
    if (drop) {
      unsigned& e = p.ent[p.n_ent - 1];
      const unsigned kt0 = (e >> 8) & 255, kt1 = (e >> 16) & 255;
      if (kt1 > kt0 + 1) {
        e = (e & 0xff00ffffu) | (kt1 - 1) << 16;
      } else {
        --p.n_ent;
        for (int s = 0; s <= p.n_bins; ++s)
          if (p.bin_start[s] > p.n_ent) p.bin_start[s] = (unsigned short)p.n_ent;
      }
    }
    double ratio = 0.0;
    const std::string why = check(p, B, T, kv_len, q_pos0, &ratio);
    worst = std::max(worst, ratio);
    if (!why.empty()) {
      ++broken;
      std::printf("broken B %d T %d q_pos0 %d: %s\n", B, T, q_pos0, why.c_str());
    }
  };
  if (std::string_view(argv[2]) == "sweep") {
    const int bmax = std::atoi(argv[3]), tmax = std::atoi(argv[4]);
    for (int a = 5; a < argc; ++a)
      for (int B = 1; B <= bmax; ++B)
        for (int T = 1; T <= tmax; ++T) one(B, T, std::atoi(argv[a]));
  } else {
    for (int a = 2; a + 2 < argc; a += 3)
      one(std::atoi(argv[a]), std::atoi(argv[a + 1]), std::atoi(argv[a + 2]));
  }
  std::printf("shapes %lld planned %lld broken %lld worst_ratio %.4f\n", shapes, planned, broken,
              worst);
  return 0;
}

// Launch plan of the causal prefill attention (host side, plain C++).
//
// Causal work balance. With few query tiles (B * 8 * tiles under two per CU),
// the longest workgroup (the last query tile attends to every key tile) sets
// the time: at T = 2048 it does 32 key tiles while the mean is 16.5. Such
// launches are planned on the host, stream-K style: per (sequence, KV head)
// the query tiles are laid out in the order last, first, second-to-last,
// second, ... (so a long tile is followed by a short one), their key tiles are
// concatenated, and the stream is cut into bins of equal cost (key tiles plus a
// fixed overhead per piece); workgroup (bin, b, g) runs the pieces of its bin
// one after the other. A query tile cut across two or more bins is computed in
// pieces; a piece writes an unnormalised fp32 partial (O, running max, running
// sum) per query row, and flash_merge_kernel combines the pieces of each cut
// tile, exactly as the online softmax combines key tiles.
//
// Causal means the mask of the model.py excerpt on the Grouped-query attention
// page: the query at position q_pos0 + i sees keys 0 .. q_pos0 + i.
//
// Everything here is plain C++ (no HIP types) so that a host-only program can
// walk the same plan the kernel runs.
#pragma once

namespace gqa {

constexpr int FA_BQ = 64;          // query positions per workgroup
constexpr int FA_BN = 64;          // keys per staged tile
constexpr int FA_MAX_ENT = 256;    // (query tile, key range) entries of a plan
constexpr int FA_MAX_BINS = 256;   // bins per (sequence, KV head)
constexpr int FA_MAX_MERGE = 128;  // cut query tiles of a plan
constexpr int FA_PLAN_CUS = 256;   // CUs the plan balances over (MI355X)
constexpr int FA_MIN_PIECE = 4;    // key tiles: bins never hold fewer
constexpr int FA_ENTRY_COST = 4;   // key-tile trips an entry costs beyond its tiles (plan balance)
constexpr int FA_DIRECT = 255;     // slot value of an entry that writes H itself
constexpr int FA_MERGE_MAXP = 4;   // pieces per cut query tile (flash_merge_kernel)

// A plan for one launch; the same for every (sequence, KV head). Bin s holds
// entries bin_start[s] .. bin_start[s + 1] - 1; an entry is
//   query tile | first key tile << 8 | end key tile << 16 | slot << 24,
// slot FA_DIRECT when the entry is the whole query tile (it writes H), else
// the partial slot of the piece. A merge record is
//   query tile | first slot << 8 | pieces << 16
// (the tile's pieces sit in consecutive slots, in key order).
struct FlashPlan {
  int n_bins = 0, n_ent = 0, n_merge = 0, n_slots = 0;
  unsigned short bin_start[FA_MAX_BINS + 1];
  unsigned ent[FA_MAX_ENT];
  unsigned mrg[FA_MAX_MERGE];
};

// Key tiles query tile qt attends to (causal).
inline int flash_key_tiles(int qt, int kv_len, int q_pos0) {
  const long long last = (long long)q_pos0 + (long long)(qt + 1) * FA_BQ;
  const long long kv_end = kv_len < last ? kv_len : last;
  return (int)((kv_end + FA_BN - 1) / FA_BN);
}

// Time of the plain causal launch in the plan's cost model (an entry costs its
// key tiles plus FA_ENTRY_COST, one workgroup per CU): one workgroup per query
// tile and (sequence, KV head), longest first, each to the CU that frees
// first. cu[] holds the CUs' free times in ascending order; the B * n_kv
// workgroups of one query tile take the earliest ones, and the two sorted runs
// are merged back.
inline long long flash_plain_cost(int B, int nq, int kv_len, int q_pos0, int n_kv) {
  long long cu[FA_PLAN_CUS], nxt[FA_PLAN_CUS];
  for (int i = 0; i < FA_PLAN_CUS; ++i) cu[i] = 0;
  long long end = 0;
  const int per_tile = B * n_kv;
  for (int qt = nq - 1; qt >= 0; --qt) {
    const long long c = flash_key_tiles(qt, kv_len, q_pos0) + FA_ENTRY_COST;
    for (int done = 0; done < per_tile;) {
      const int take = per_tile - done < FA_PLAN_CUS ? per_tile - done : FA_PLAN_CUS;
      if (cu[take - 1] + c > end) end = cu[take - 1] + c;
      int i = 0, j = take, n = 0;
      while (i < take && j < FA_PLAN_CUS) nxt[n++] = cu[i] + c <= cu[j] ? cu[i++] + c : cu[j++];
      while (i < take) nxt[n++] = cu[i++] + c;
      while (j < FA_PLAN_CUS) nxt[n++] = cu[j++];
      for (int k = 0; k < FA_PLAN_CUS; ++k) cu[k] = nxt[k];
      done += take;
    }
  }
  return end;
}

// Plans a causal launch with too few query tiles to balance; returns false
// (plain launch: one workgroup per query tile) when no plan applies, when it
// would not fit its tables, or when its costliest bin would take as long as
// the plain launch in the cost model (a few short query tiles in more bins than
// tiles: every cut adds an entry's cost).
inline bool flash_plan(int B, int T, int kv_len, int q_pos0, int causal, int n_kv,
                       FlashPlan& p) {
  p = FlashPlan{};
  if (!causal || B < 1 || T < 1 || kv_len < 1) return false;
  const int nq = (T + FA_BQ - 1) / FA_BQ;
  if ((long long)B * n_kv * nq >= 2LL * FA_PLAN_CUS || nq > 255) return false;
  // zigzag order of query tiles and the unit (key tile) stream per (b, g)
  int order[256], len[256];
  long long U = 0;
  int longest = 0;
  for (int i = 0; i < nq; ++i) {
    order[i] = (i & 1) ? i / 2 : nq - 1 - i / 2;
    len[i] = flash_key_tiles(order[i], kv_len, q_pos0);
    U += len[i];
    if (len[i] > longest) longest = len[i];
  }
  if (longest > 255) return false;
  int bins = FA_PLAN_CUS / (B * n_kv);
  if ((long long)bins > U / FA_MIN_PIECE) bins = (int)(U / FA_MIN_PIECE);
  if (bins > FA_MAX_BINS) bins = FA_MAX_BINS;
  if (bins < 2) return false;
  // worth it only when the longest tile exceeds a bin by a quarter or more
  // (a chunk of 2048 positions after 2048 cached ones: 64 key tiles against a
  // mean of 48.5 per bin; the whole chunk step 314 -> 306 us)
  if (4 * (long long)longest * bins < 5 * U) return false;
  // Bins are filled greedily in stream order up to a cost C, where an entry
  // costs its key tiles plus FA_ENTRY_COST (the wait for its queries and first
  // tiles, its output write and the re-synchronisation of the waves); C is the
  // smallest cost at which the stream fits in `bins` bins (feasibility is
  // monotone in C, so it is found by bisection). fill returns the number of
  // entries at cost C (recording the first `cap`: key tiles taken and bin), or
  // -1 when the stream does not fit.
  auto fill = [&](long long C, int cap, int* take_out, int* bin_out) -> int {
    int qi = 0, kt = 0, n = 0;
    for (int s = 0; s < bins && qi < nq; ++s) {
      long long cost = 0;
      while (qi < nq && cost + FA_ENTRY_COST + 1 <= C) {
        const long long room = C - cost - FA_ENTRY_COST;
        const int take = len[qi] - kt < room ? len[qi] - kt : (int)room;
        if (n < cap) { take_out[n] = take; bin_out[n] = s; }
        ++n;
        cost += FA_ENTRY_COST + take;
        kt += take;
        if (kt == len[qi]) { ++qi; kt = 0; }
      }
    }
    return qi == nq ? n : -1;
  };
  long long lo = (U + bins - 1) / bins, hi = U + FA_ENTRY_COST;   // one bin holds all at hi
  while (lo < hi) {
    const long long mid = (lo + hi) / 2;
    if (fill(mid, 0, nullptr, nullptr) >= 0) hi = mid; else lo = mid + 1;
  }
  if (lo >= flash_plain_cost(B, nq, kv_len, q_pos0, n_kv)) return false;
  int take_of[FA_MAX_ENT], bin_of[FA_MAX_ENT];
  const int n_ent = fill(lo, FA_MAX_ENT, take_of, bin_of);
  if (n_ent < 0 || n_ent > FA_MAX_ENT) return false;
  // pass 1: pieces per query tile; pass 2: entries, slots, merges
  int pieces_of[256];
  for (int pass = 0; pass < 2; ++pass) {
    int qi = 0, kt = 0, n = 0;   // current query tile (order index), key tile; entry
    int next_slot[256];
    if (pass == 1) {
      p.n_slots = 0;
      for (int i = 0; i < nq; ++i) {
        next_slot[i] = FA_DIRECT;
        if (pieces_of[i] > 1) {
          if (pieces_of[i] > FA_MERGE_MAXP || p.n_merge >= FA_MAX_MERGE) return false;
          next_slot[i] = p.n_slots;
          p.mrg[p.n_merge++] = (unsigned)order[i] | (unsigned)p.n_slots << 8 |
                               (unsigned)pieces_of[i] << 16;
          p.n_slots += pieces_of[i];
        }
      }
      if (p.n_slots >= FA_DIRECT) return false;
    } else {
      for (int i = 0; i < nq; ++i) pieces_of[i] = 0;
    }
    for (int s = 0; s < bins; ++s) {
      if (pass == 1) p.bin_start[s] = (unsigned short)p.n_ent;
      while (n < n_ent && bin_of[n] == s) {
        const int take = take_of[n++];
        if (pass == 0) {
          ++pieces_of[qi];
        } else {
          const int slot = next_slot[qi] == FA_DIRECT ? FA_DIRECT : next_slot[qi]++;
          p.ent[p.n_ent++] = (unsigned)order[qi] | (unsigned)kt << 8 |
                             (unsigned)(kt + take) << 16 | (unsigned)slot << 24;
        }
        kt += take;
        if (kt == len[qi]) { ++qi; kt = 0; }
      }
    }
    if (pass == 1) p.bin_start[bins] = (unsigned short)p.n_ent;
  }
  p.n_bins = bins;
  return true;
}

}  // namespace gqa

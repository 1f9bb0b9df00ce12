// Launch plan of the split-KV decode attention (host side, plain C++).
//
// One decode step attends one new query per sequence over keys
// 0 .. kv_len-1 of a cache [B][S_max][8][128] (Grouped-query attention page,
// "All 13 steps" at a single position, with the causal-mask excerpt's cache
// comment). The key range of each sequence is cut into chunks; an item is
// (sequence b, half of the KV heads, key chunk). Persistent workgroups take
// items blockIdx.x, blockIdx.x + G, ... (G = grid size) and stream the 16-key
// tiles of their items, in item order, through an LDS ring of DC_STAGES
// tiles; each item's four queries per KV head travel into LDS together with
// its first tile, into query slot (item ordinal % DC_QSLOTS).
//
// Everything here is plain C++ (no HIP types) so that a host-only program can
// walk the same plan the kernel runs.
#pragma once

namespace gqa {

constexpr int DC_BN = 16;          // keys per staged tile
constexpr int DC_HG = 4;           // KV heads per workgroup (a 1 KiB slice of each 2 KiB cache row)
constexpr int DC_STAGES = 4;       // tiles in the LDS ring
constexpr int DC_TARGET_ITEMS = 512;   // items per launch the chunking aims for
// Query slots in LDS. While the workgroup reads item j's queries (at its first
// tile, before it issues the next load), the ring holds loads for tiles up to
// DC_STAGES - 2 beyond the current one, and every item has at least one tile:
// at most DC_STAGES - 2 later items have had their queries issued. Their slots
// must differ from item j's, so DC_QSLOTS >= DC_STAGES - 1 suffices; one per
// stage keeps the rule obvious.
constexpr int DC_QSLOTS = DC_STAGES;
static_assert(DC_QSLOTS >= DC_STAGES - 1, "a query slot would be refilled before it is read");

// Key chunks per sequence: enough items to balance the persistent workgroups,
// never chunks shorter than one tile. Monotone in kv_len.
inline int decode_n_split(int B, int kv_len, int n_kv) {
  const int tiles = (kv_len + DC_BN - 1) / DC_BN;
  const int per_seq = B * (n_kv / DC_HG);
  const int want = (DC_TARGET_ITEMS + per_seq - 1) / per_seq;
  return want < 1 ? 1 : (want > tiles ? tiles : want);
}

struct DecodePlan {
  int n_split;   // key chunks per (sequence, head half) after dropping empty ones
  int chunk;     // keys per chunk (a multiple of DC_BN)
  int n_items;   // B * (n_kv / DC_HG) * n_split
  int grid;      // persistent workgroups: min(n_items, n_cu)
};

inline DecodePlan decode_plan(int B, int kv_len, int n_kv, int n_cu) {
  DecodePlan p{};
  const int split = decode_n_split(B, kv_len, n_kv);
  const int tiles = (kv_len + DC_BN - 1) / DC_BN;
  p.chunk = ((tiles + split - 1) / split) * DC_BN;
  p.n_split = (kv_len + p.chunk - 1) / p.chunk;
  p.n_items = B * (n_kv / DC_HG) * p.n_split;
  p.grid = p.n_items < n_cu ? p.n_items : n_cu;
  return p;
}

// 16-key tiles of an item (its chunk, the last one possibly short).
inline int decode_item_tiles(const DecodePlan& p, int kv_len, int item) {
  const int k0 = (item % p.n_split) * p.chunk;
  const int keys = kv_len - k0 < p.chunk ? kv_len - k0 : p.chunk;
  return (keys + DC_BN - 1) / DC_BN;
}

}  // namespace gqa

// Grouped attention kernels of the GQA block (gfx950).
//
// Grouped-query attention page, "All 13 steps": K_G[h] = K_r[floor(h/4)] and
// V_G[h] = V[floor(h/4)]; S = Q_r·K_Gᵀ; S_s = S/sqrt(128); S_m = S_s + M;
// A = softmax over keys; H = A·V_G; H merged with feature 128*h + d. The mask
// follows the model.py excerpt: key j is masked for the query at position p
// when j > p.
//
// Prefill (flash_fwd_kernel): one workgroup per (64-position query tile, KV
// head g, sequence b) runs 8 waves: wave w takes query head 4g + (w & 3) and
// 32 of the 64 positions. Every 64-key tile of K_r and V is loaded into LDS
// once (straight from HBM, through a 4-stage ring) and used by all four heads
// of the group. Waves w and w+4 share a SIMD and are offset by half a tile, so
// one's MFMAs run while the other computes its softmax. Scores are computed
// transposed (keys down the MFMA rows, queries across the lanes), so each lane
// owns one query: the running max needs only in-lane work plus one swap with
// the lane 32 away, and the bf16 probabilities feed the P·V MFMA straight from
// the score accumulator. V is read with transposing LDS loads, in the key
// order the accumulator holds. The softmax is the online (running max /
// running sum) form in base 2 with a lazily moved reference max; the factor
// log2(e)/sqrt(128) is either folded into one multiply-add per score or, in
// the block paths, carried by the queries themselves (the QKV epilogue
// applies it), whose score MFMA chain then starts from minus the row's
// reference. The division by the row sum happens once, at the end, in fp32.
// Causal launches with too few query tiles to fill the chip follow a host-made
// plan that cuts the key-tile stream of each (sequence, KV head) into bins of
// equal cost (flash_plan.h); flash_merge_kernel combines the pieces of cut
// query tiles.
//
// Decode (decode_splitkv_kernel + decode_merge_kernel): the key range of each
// sequence is split into chunks; persistent workgroups of 4 waves (one per KV
// head of a half of the 8) stream their chunks' cache rows through LDS and
// write one unnormalised partial (max, sum, O[4][128]) per (chunk, KV head);
// the merge kernel rescales and sums the partials. The launch plan is in
// decode_plan.h.

#include "decode_plan.h"
#include "flash_plan.h"
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {

constexpr float LOG2E = 1.4426950408889634f;
// log2(e) / sqrt(128): one multiply turns a raw score into the base-2 exponent.
constexpr float SCALE_LOG2 = QK_SCALE_LOG2;
constexpr float SQRT_DH = 11.313708498984761f;
constexpr float NEG_INF = -__builtin_inff();

// ----------------------------------------------------------------------------
// Prefill
// ----------------------------------------------------------------------------

constexpr int FA_THREADS = 512;  // 8 waves: 4 heads x 2 blocks of 32 positions
constexpr int FA_STAGES = 4;     // K/V tiles resident: t-1 (V, lagging waves), t, t+1, t+2
constexpr int FA_TILE = FA_BN * D_HEAD;   // elements of one K or V tile (16 KiB)
constexpr int FA_NI_W = 4;       // 1-KiB direct-to-LDS loads per wave per tile (16 K + 16 V over 8 waves)
// Lazy rescaling: the reference max of a row only moves when a score exceeds it
// by 8 in base 2 (probabilities then stay <= 2^8), so the O rescale is skipped
// for almost every tile. Expressed in raw-score units.
constexpr float FA_RESCALE_LOG2 = 8.0f;
constexpr float FA_RESCALE_RAW = FA_RESCALE_LOG2 / SCALE_LOG2;

// K tile [64 keys][128 d], 256-byte rows: 16-byte chunk c of key k at chunk
// c ^ (k & 15), so the 16 lanes of a fragment read (16 keys, one chunk) hit 16
// distinct slots.
__device__ __forceinline__ int k_off(int key, int c) { return key * D_HEAD + ((c ^ (key & 15)) << 3); }
// V tile [64 keys][128 d], row-major: chunk c of key k at chunk c ^ 4(k & 3).
// A transposed read covers 4 consecutive keys x 64 bytes per half-wave; the
// permutation spreads those 4 rows over all 16 slots of a 256-byte window.
__device__ __forceinline__ int v_off(int key, int c) { return key * D_HEAD + ((c ^ ((key & 3) << 2)) << 3); }

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_lds;

// ds_read_b64_tr_b16: within each 16-lane group, lane s supplies the address of
// 4 consecutive bf16 of row (s >> 2) of a 4-row block, columns 4(s & 3)..+3;
// lane i receives column i of the 4 rows (one value per row).
__device__ __forceinline__ u32x2 ld_tr(const uint16_t* p) {
  bf16x4_lds v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4_lds*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Causal launches with few query tiles run a host-made plan (flash_plan.h).

// Partial of one piece for one (sequence, KV head): O[4 heads][64 rows][128],
// then max[4][64] (base-2 units: the score times log2(e)/sqrt(128)), then
// sum[4][64], fp32.
constexpr int FA_PART = N_REP * FA_BQ * D_HEAD + 2 * N_REP * FA_BQ;
constexpr int FA_MERGE_ROWS = 8;   // (head, query) rows per merge workgroup

struct FlashArgs {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  long long kv_bstride;
  const float* mask;     // [T][kv_len] or null
  uint16_t* h;
  float* part;           // piece partials [slot][B][8][FA_PART] (planned launches)
  int B, T, kv_len, q_pos0, causal, n_qtiles;
  // the queries carry the factor log2(e)/sqrt(128) already (QKV epilogue of the
  // block paths), so a score MFMA yields the base-2 exponent directly
  // planned launch: workgroup i runs bin i / (8B) for (b, g) = split of i % (8B),
  // i.e. entries bin_start[bin] .. bin_start[bin + 1] - 1, each
  // qtile | first key tile << 8 | end key tile << 16 | slot << 24
  int n_bins;
  unsigned short bin_start[FA_MAX_BINS + 1];
  unsigned ent[FA_MAX_ENT];
  // explicit mask with its tile classes (flash_mask_classes_kernel): class of
  // (query tile qt, key tile t) at mcls[qt * nkp + t], rows padded to nkp (a
  // multiple of 4) bytes; null: every tile mixed
  const unsigned char* mcls;
  int nkp;
  // the mask rows are 16-byte aligned (aligned base, kv_len a multiple of 4):
  // a mixed tile's values are read four keys per load
  int mask_vec;
};

struct FlashMergeArgs {
  float* part; uint16_t* h;
  int B, T;
  unsigned mrg[FA_MAX_MERGE];   // qtile | first slot << 8 | pieces << 16
};

// Explicit additive masks (the M of "All 13 steps") are classified per 64x64
// tile before the attention launch: a tile whose in-range entries are all 0
// adds nothing to the scores, one whose entries are all -inf removes its keys,
// any other tile is added element by element. The attention then walks each
// query tile's key tiles only from the first to the last tile that is not all
// -inf (a causal or sliding-window mask passed explicitly costs what the
// causal flag costs), skips the mask for all-zero tiles and loads it only for
// mixed ones.
constexpr unsigned char FA_MASK_ZERO = 0, FA_MASK_NEG_INF = 1, FA_MASK_MIXED = 2;

// Workgroup (key tile t, query tile qt): 256 threads read the 64x64 tile and
// agree on its class. vec (a 16-byte aligned mask whose rows are a multiple
// of 4 floats): 16 bytes a lane (16 lanes per 256-byte row segment, 16 rows
// per load instruction, the four loads of a lane issued before the first is
// used); else one float a lane. Entries outside [T, kv_len] take part in
// neither test.
__global__ __launch_bounds__(256) void flash_mask_classes_kernel(const float* mask, int T,
                                                                 int kv_len, int nkp, int vec,
                                                                 unsigned char* cls) {
  const int t = blockIdx.x, qt = blockIdx.y;
  bool zero = true, ninf = true;
  if (vec) {
    const int col = t * FA_BN + 4 * (threadIdx.x & 15);
    const int r0 = qt * FA_BQ + (threadIdx.x >> 4);
    f32x4 x[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = r0 + 16 * i;
      ok[i] = q < T && col < kv_len;
      x[i] = ok[i] ? *reinterpret_cast<const f32x4*>(mask + (size_t)q * kv_len + col) : f32x4{};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (ok[i]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          zero = zero && x[i][j] == 0.f;
          ninf = ninf && x[i][j] == NEG_INF;
        }
      }
  } else {
    const int col = t * FA_BN + (threadIdx.x & 63);
    if (col < kv_len) {
#pragma unroll 4
      for (int r = threadIdx.x >> 6; r < FA_BQ; r += 4) {
        const int q = qt * FA_BQ + r;
        if (q >= T) break;
        const float x = mask[(size_t)q * kv_len + col];
        zero = zero && x == 0.f;
        ninf = ninf && x == NEG_INF;
      }
    }
  }
  const int all_zero = __syncthreads_and(zero);
  const int all_ninf = __syncthreads_and(ninf);
  if (threadIdx.x == 0)
    cls[(size_t)qt * nkp + t] = all_ninf ? FA_MASK_NEG_INF : all_zero ? FA_MASK_ZERO : FA_MASK_MIXED;
}

// One (query tile, key tiles kt0..kt1-1) entry for (sequence b, KV head g).
// QS: the queries are pre-scaled by log2(e)/sqrt(128) (see FlashArgs); the
// score MFMA chain then starts from minus the row's reference, so each
// accumulator is the exponent of its probability with no VALU work.
template <bool QS, bool MASK>
__device__ __forceinline__ void flash_entry(const FlashArgs& a, uint16_t* smem, int b, int g,
                                            int qt, int kt0, int kt1, int slot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lhalf = lane >> 5;
  // Waves w and w+4 share a SIMD. The first four run each tile as QK -> softmax
  // -> P·V; the other four run the softmax and P·V of the previous tile first
  // and the QK of this tile last, so on every SIMD one wave's softmax VALU
  // work overlaps the other's MFMAs for most of a trip.
  const bool lag = wave >= 4;
  const int q0 = qt * FA_BQ;
  const int h = g * N_REP + (wave & 3);
  const int qi = q0 + (wave >> 2) * 32 + lrow;        // this lane's query index
  const int qpos = a.q_pos0 + qi;

  const uint16_t* kbase = a.k + b * a.kv_bstride + g * D_HEAD;
  const uint16_t* vbase = a.v + b * a.kv_bstride + g * D_HEAD;

  u32x4 qf[8];

  // Direct-to-LDS loads of tile t: instruction i (0..31) covers rows 4(i&15)..+3
  // of K (i < 16) or V; lane l writes row 4(i&15) + (l >> 4), physical chunk
  // l & 15. Wave w issues instructions i = w + 8j, j = 0..3: K for j < 2, V
  // for j >= 2, and row rr + 32(j & 1) with rr = 4w + (lane >> 4), whose
  // chunk swizzle is the same for j and j + 1. So the lane's part of each
  // source address is one of two loop-invariant byte offsets, and a tile adds
  // only a wave-uniform base (scalar arithmetic). Keys past the end are
  // clamped to the last key (finite values; masked); only a tile reaching past
  // the last key takes that path.
  const int wave_u = wave_id();
  const uint32_t lds0 = lds_addr(smem);
  const int rr = 4 * wave_u + (lane >> 4);
  const uint32_t voffK = (uint32_t)(rr * (N_KV * D_HEAD) + (((lane & 15) ^ (rr & 15)) << 3)) * 2u;
  const uint32_t voffV = (uint32_t)(rr * (N_KV * D_HEAD) + (((lane & 15) ^ ((rr & 3) << 2)) << 3)) * 2u;
  auto issue = [&](int t) {
    const uint32_t st = lds0 + 2u * (uint32_t)((t % FA_STAGES) * 2 * FA_TILE);
    if (t * FA_BN + FA_BN <= a.kv_len) {
      const size_t toff = (size_t)t * FA_BN * (N_KV * D_HEAD);
#pragma unroll
      for (int j = 0; j < FA_NI_W; ++j) {
        const int i = wave_u + 8 * j;
        const uint16_t* sb = (j < 2 ? kbase : vbase) + toff + (size_t)(j & 1) * 32 * (N_KV * D_HEAD);
        dma16_sv(sb, j < 2 ? voffK : voffV, st + 2u * (uint32_t)((i >= 16 ? FA_TILE : 0) + (i & 15) * 512));
      }
    } else {
      const size_t toff = (size_t)t * FA_BN * (N_KV * D_HEAD);
#pragma unroll
      for (int j = 0; j < FA_NI_W; ++j) {
        const int i = wave_u + 8 * j;
        const int key = min(t * FA_BN + rr + 32 * (j & 1), a.kv_len - 1);
        // byte offset of (key, chunk) from the tile's first row: in [0, 128 KiB)
        // (the tile starts before the last key), whatever the sequence length
        const uint32_t vo = (j < 2 ? voffK : voffV) + (uint32_t)((key - t * FA_BN - rr) * (N_KV * D_HEAD)) * 2u;
        dma16_sv((j < 2 ? kbase : vbase) + toff, vo, st + 2u * (uint32_t)((i >= 16 ? FA_TILE : 0) + (i & 15) * 512));
      }
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_ref = NEG_INF;   // reference max of this lane's query row (raw-score units; base 2 if QS)
  float l_run = 0.f;       // this lane's share of the row sum (relative to m_ref)
  u32x4 pf[4];             // bf16 probabilities of the last softmax (P^T fragments)
  // QS: the score chain starts from -m_eff, m_eff = m_ref or 0 while the row has
  // no reference yet; thr is the rescale threshold on scores relative to m_eff
  float m_eff = 0.f, thr = NEG_INF;
  f32x16 negm = f32x16{};

  // MASK: an explicit additive mask (a kernel of its own: its loads need
  // registers the causal and unmasked launches keep for their loop)
  constexpr bool has_mask = MASK;
  const float* mrow = MASK ? a.mask + (size_t)(qi < a.T ? qi : 0) * a.kv_len : nullptr;

  // S^T = K·Q^T for tile t into s.
  auto qk = [&](int t, f32x16 (&s)[2]) {
    const uint16_t* sk = smem + (t % FA_STAGES) * 2 * FA_TILE;
    // One accumulation chain per 32-key block, the two blocks interleaved. The K
    // fragments of step st+2 are read while the MFMAs of step st run (a ring of
    // three register buffers; the scheduling fences keep the compiler from
    // sinking the reads next to their use).
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) s[kb2] = QS ? negm : f32x16{};
    u32x4 kf[3][2];
    auto read_k = [&](int st, u32x4 (&f)[2]) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) f[kb2] = ld16(sk + k_off(kb2 * 32 + lrow, 2 * st + lhalf));
    };
    read_k(0, kf[0]);
    read_k(1, kf[1]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 2 < 8) read_k(st + 2, kf[(st + 2) % 3]);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) s[kb2] = mfma_32x32x16(kf[st % 3][kb2], qf[st], s[kb2]);
    }
    // order: the first two steps' reads, then MFMA, read, MFMA, read, ...
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };

  // The online softmax of tile t from its raw scores s, leaving P^T in pf.
  // mc: the tile's mask class (wave-uniform; FA_MASK_ZERO without a mask)
  auto softmax = [&](int t, f32x16 (&s)[2], int mc) {
    // lane holds query lrow, keys 32kb + 8(i>>2) + 4*lhalf + (i&3)
    const int k0 = t * FA_BN;
    const bool edge = (a.causal && (k0 + FA_BN - 1 > a.q_pos0 + q0)) || (k0 + FA_BN > a.kv_len) ||
                      mc != FA_MASK_ZERO;
    if (edge) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        // a mixed tile's mask values, 16 at a time: every load of a block issued
        // before the first is used (indices clamped into the mask; the values
        // past its end are not used), then one wait for all of them. vmcnt
        // counts in order, so these loads complete only after the K/V tile
        // loads issued before them anyway; the explicit wait also tells the
        // compiler's wait-count pass that nothing is left in flight, so it
        // puts no vmcnt(0) on the path of tiles that load no mask
        float mv[16];
        if (mc == FA_MASK_MIXED) {
          if (a.mask_vec) {
            // the lane's keys come in runs of four (i & 3), 16-byte aligned; a
            // run past the last key is read from the mask's last four (unused)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int kg = k0 + kb2 * 32 + 8 * c + 4 * lhalf;
              const f32x4 m4 = *reinterpret_cast<const f32x4*>(mrow + (kg < a.kv_len ? kg : a.kv_len - 4));
#pragma unroll
              for (int e = 0; e < 4; ++e) mv[4 * c + e] = m4[e];
            }
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kg = k0 + kb2 * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
              mv[i] = mrow[kg < a.kv_len ? kg : a.kv_len - 1];
            }
          }
          wait_vmcnt<0>();
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kg = k0 + kb2 * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
          float x = s[kb2][i];
          if (mc == FA_MASK_MIXED) x += mv[i] * (QS ? LOG2E : SQRT_DH);
          if (mc == FA_MASK_NEG_INF || kg >= a.kv_len || (a.causal && kg > qpos)) x = NEG_INF;
          s[kb2][i] = x;
        }
      }
    }
    // Lanes l and l ^ 32 hold the two halves of a query row's keys and keep the
    // same reference max. Each half tests its own maximum; only when some half
    // exceeds the threshold (rare) are the halves combined and the row rescaled.
    float mx = NEG_INF;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb2][i]);
    float moff;
    if constexpr (QS) {
      // scores are relative to m_eff, in base-2 units
      if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool need = mx > thr;                     // false when mx = -inf
        const float m_new = need ? mx + m_eff : m_ref;
        // as below: a row that keeps its reference keeps its sums; a first finite
        // maximum gives alpha = 0 from m_ref = -inf
        const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        // this tile's scores move to the new reference, and so does the next chain
        const float m_eff_new = m_ref == NEG_INF ? 0.f : m_ref;
        const float shift = m_eff - m_eff_new;
        m_eff = m_eff_new;
        thr = m_ref == NEG_INF ? NEG_INF : FA_RESCALE_LOG2;
#pragma unroll
        for (int i = 0; i < 16; ++i) negm[i] = -m_eff;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kb2][i] += shift;
      }
      moff = 0.f;
    } else {
      if (__builtin_amdgcn_ballot_w64(mx > m_ref + FA_RESCALE_RAW) != 0) {
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool need = mx > m_ref + FA_RESCALE_RAW;   // false when mx = -inf
        const float m_new = need ? mx : m_ref;
        // lanes that keep their reference keep their sums (alpha 1: with m_ref = -inf,
        // a row that has seen no key yet, the difference would be -inf - -inf = NaN);
        // a first finite max gives alpha = 0 from m_ref = -inf
        const float alpha = need ? __builtin_amdgcn_exp2f((m_ref - m_new) * SCALE_LOG2) : 1.f;
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      }
      moff = (m_ref == NEG_INF) ? 0.f : -m_ref * SCALE_LOG2;
    }
    // The row sum adds the bf16 probabilities the P·V MFMA uses, two per dot2
    // instruction against (1, 1): half the VALU work of fp32 adds, and the
    // numerator and denominator then weight the same rounded values.
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x2 pb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2 pp =
              QS ? f32x2{__builtin_amdgcn_exp2f(s[kb2][8 * hf + 2 * e]),
                         __builtin_amdgcn_exp2f(s[kb2][8 * hf + 2 * e + 1])}
                 : f32x2{__builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][8 * hf + 2 * e], SCALE_LOG2, moff)),
                         __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][8 * hf + 2 * e + 1], SCALE_LOG2, moff))};
          pb[e] = __builtin_convertvector(pp, bf16x2);
        }
        ls0 = __builtin_amdgcn_fdot2_f32_bf16(pb[0], ones, ls0, false);
        ls1 = __builtin_amdgcn_fdot2_f32_bf16(pb[1], ones, ls1, false);
        ls0 = __builtin_amdgcn_fdot2_f32_bf16(pb[2], ones, ls0, false);
        ls1 = __builtin_amdgcn_fdot2_f32_bf16(pb[3], ones, ls1, false);
        pf[kb2 * 2 + hf] = u32x4{__builtin_bit_cast(uint32_t, pb[0]), __builtin_bit_cast(uint32_t, pb[1]),
                                 __builtin_bit_cast(uint32_t, pb[2]), __builtin_bit_cast(uint32_t, pb[3])};
      }
    l_run += ls0 + ls1;
  };

  // O^T[d][q] += V^T[d][keys] · P^T[keys][q] for tile t; group sg holds keys
  // 16sg..16sg+15. V^T fragments come from two transposed reads: lane group
  // (lane >> 4) = (key quad u = lane >> 5, d half); source lane s = lane & 15
  // points at key 4u + (s >> 2) (+8 for the second read), d = 32db + 16*dhalf + 4(s & 3).
  const int tr_key = 4 * lhalf + ((lane & 15) >> 2);
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto pv = [&](int t) {
    const uint16_t* sv = smem + (t % FA_STAGES) * 2 * FA_TILE + FA_TILE;
#pragma unroll
    for (int sg = 0; sg < 4; ++sg)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* p = sv + v_off(16 * sg + tr_key, (32 * db + tr_d) >> 3) + (tr_d & 7);
        const u32x2 r1 = ld_tr(p);
        const u32x2 r2 = ld_tr(p + 8 * D_HEAD);
        const u32x4 vf = {r1[0], r1[1], r2[0], r2[1]};
        o[db] = mfma_32x32x16(vf, pf[sg], o[db]);
      }
  };

  issue(kt0);
  if (kt0 + 1 < kt1) issue(kt0 + 1);
  // Mask classes of this query tile's key tiles, held in a register: lane l
  // has those of tiles cbase + 4l .. cbase + 4l + 3 (one dword of the class
  // row), a window of 256 tiles, moved on every 256 tiles. A class is then a
  // lane read with a uniform index, no memory access inside the loop.
  const uint32_t* crow =
      (MASK && a.mcls) ? reinterpret_cast<const uint32_t*>(a.mcls + (size_t)qt * a.nkp) : nullptr;
  int cbase = kt0 & ~3;
  uint32_t cwin = 0;
  auto load_classes = [&]() {
    const int wi = (cbase >> 2) + lane;
    cwin = wi < (a.nkp >> 2) ? crow[wi] : 0u;
  };
  if (MASK && a.mcls) load_classes();
  // Query fragments (MFMA B operand): k-step s covers d = 16s + 8*lhalf .. +7.
  {
    const bool ok = qi < a.T;
    const uint16_t* qrow = a.q + ((size_t)(b * a.T + (ok ? qi : 0)) * N_HEADS + h) * D_HEAD + 8 * lhalf;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[s] = ok ? ld16(qrow + 16 * s) : z;
    }
  }

  // Wait for the query loads (and the first tiles) before the loop: vmcnt is one
  // in-order counter, and with the query registers known complete here the
  // compiler adds no wait of its own inside the loop.
  wait_vmcnt<0>();
  // trip t: tile t is computed (the lagging waves finish tile t-1); one extra
  // trip lets the lagging waves do the last P·V.
  f32x16 s[2];
  int mc_prev = FA_MASK_ZERO;   // class of tile t - 1 (the lagging waves' softmax)
  for (int t = kt0; t <= kt1; ++t) {
    int mc = FA_MASK_ZERO;       // class of tile t
    if (MASK) {
      mc = FA_MASK_MIXED;
      if (a.mcls && t < kt1) {
        if (t - cbase >= 256) {
          // next window: waits for every load in flight, once per 256 tiles
          cbase += 256;
          load_classes();
          wait_vmcnt<0>();
        }
        const int d = t - cbase;
        mc = (int)(((uint32_t)__builtin_amdgcn_readlane((int)cwin, d >> 2) >> (8 * (d & 3))) & 255u);
      }
    }
    // tile t resident (tile t+1 may still be in flight); every wave is past
    // trip t-1, so stage (t+2)%4 — last read as tile t-2 — is free
    if (t + 1 < kt1) wait_vmcnt<FA_NI_W>(); else wait_vmcnt<0>();
    barrier_no_fence();
    if (t + 2 < kt1) issue(t + 2);
    if (!lag) {
      if (t < kt1) { qk(t, s); softmax(t, s, mc); pv(t); }
    } else {
      // softmax VALU work first, while the SIMD's leading wave runs its score MFMAs
      if (t > kt0) { softmax(t - 1, s, mc_prev); pv(t - 1); }
      if (t < kt1) qk(t, s);
    }
    mc_prev = mc;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (slot != FA_DIRECT) {
    // piece of a cut query tile: unnormalised partial, rows beyond T included
    // (the merge skips them)
    float* pp = a.part + ((size_t)(slot * a.B + b) * N_KV + g) * FA_PART;
    const int row = (wave & 3) * FA_BQ + (wave >> 2) * 32 + lrow;   // head h4, query qi - q0
    float* orow = pp + (size_t)row * D_HEAD + 4 * lhalf;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        *reinterpret_cast<f32x4*>(orow + db * 32 + gq * 8) =
            f32x4{o[db][4 * gq], o[db][4 * gq + 1], o[db][4 * gq + 2], o[db][4 * gq + 3]};
    if (lhalf == 0) {
      pp[N_REP * FA_BQ * D_HEAD + row] = QS ? m_ref : m_ref * SCALE_LOG2;   // base 2
      pp[N_REP * FA_BQ * D_HEAD + N_REP * FA_BQ + row] = l_tot;
    }
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qi < a.T) {
    uint16_t* hrow = a.h + ((size_t)(b * a.T + qi) * N_HEADS + h) * D_HEAD + 4 * lhalf;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 w = {pack_bf16x2(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv),
                   pack_bf16x2(o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv)};
        *reinterpret_cast<u32x2*>(hrow + db * 32 + gq * 8) = w;
      }
  }
}

template <bool QS, bool MASK>
__global__ __launch_bounds__(FA_THREADS) void flash_fwd_kernel(FlashArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[FA_STAGES * 2 * FA_TILE];
  const int g = blockIdx.x & (N_KV - 1);
  const int rest = blockIdx.x >> 3;
  const int b = rest % a.B;
  if (a.n_bins > 0) {
    const int bin = rest / a.B;
    const int e1 = a.bin_start[bin + 1];
    for (int i = a.bin_start[bin]; i < e1; ++i) {
      const unsigned e = a.ent[i];
      // every wave is done with the LDS ring of the previous entry
      if (i > a.bin_start[bin]) barrier_no_fence();
      flash_entry<QS, MASK>(a, smem, b, g, e & 255, (e >> 8) & 255, (e >> 16) & 255, e >> 24);
    }
    return;
  }
  // plain launch: one query tile per workgroup, last query tile first when
  // causal or masked (the longest first under a causal mask, a window over a
  // cache or a chunk's mask: the structured masks whose later rows see at
  // least as many keys; any order is correct)
  const int qt = (a.causal || MASK) ? (a.n_qtiles - 1 - rest / a.B) : (rest / a.B);
  int kv_end = a.kv_len;
  if (a.causal) kv_end = min(kv_end, a.q_pos0 + (qt + 1) * FA_BQ);
  int kt0 = 0, kt1 = (kv_end + FA_BN - 1) / FA_BN;
  if (MASK && a.mcls) {
    // key tiles from the first to the last that is not all -inf (each wave
    // scans the query tile's classes itself; none: the rows get H = 0)
    const int lane = threadIdx.x & 63;
    int lo = kt1, hi = -1;
    for (int t = lane; t < kt1; t += 64)
      if (a.mcls[(size_t)qt * a.nkp + t] != FA_MASK_NEG_INF) { lo = min(lo, t); hi = max(hi, t); }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      lo = min(lo, __shfl_xor(lo, off));
      hi = max(hi, __shfl_xor(hi, off));
    }
    lo = __builtin_amdgcn_readfirstlane(lo);
    hi = __builtin_amdgcn_readfirstlane(hi);
    if (hi < lo) { lo = 0; hi = -1; }
    kt0 = lo;
    kt1 = hi + 1;
  }
  flash_entry<QS, MASK>(a, smem, b, g, qt, kt0, kt1, FA_DIRECT);
}

// Combines the pieces of cut query tiles. Workgroup (r, t, b, g) takes rows
// 8r .. 8r+7 of (head, query) of cut tile t; each 32-lane half-wave takes one
// row, lane i holding d = 4i .. 4i+3. Pieces are rescaled to their common max
// and summed, then divided by the summed row sums (pieces in slot order). The
// pieces' maxima are in base-2 units.
__global__ __launch_bounds__(256) void flash_merge_kernel(FlashMergeArgs a) {
  constexpr int MAXP = FA_MERGE_MAXP;
  const int g = blockIdx.x & (N_KV - 1);
  int rest = blockIdx.x >> 3;
  const int b = rest % a.B;
  rest /= a.B;
  const int rblk = rest % (N_REP * FA_BQ / FA_MERGE_ROWS);
  const unsigned e = a.mrg[rest / (N_REP * FA_BQ / FA_MERGE_ROWS)];
  const int qt = e & 255, slot0 = (e >> 8) & 255, np = (e >> 16) & 255;
  const int li = threadIdx.x & 31;
  const int row = rblk * FA_MERGE_ROWS + (threadIdx.x >> 5);
  const int h4 = row / FA_BQ, qi = qt * FA_BQ + row % FA_BQ;
  if (qi >= a.T) return;
  const size_t piece_stride = (size_t)a.B * N_KV * FA_PART;
  const float* base = a.part + ((size_t)(slot0 * a.B + b) * N_KV + g) * FA_PART;
  float mp[MAXP], lp[MAXP];
  f32x4 op[MAXP];
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    if (p < np) {
      const float* pp = base + p * piece_stride;
      mp[p] = pp[N_REP * FA_BQ * D_HEAD + row];
      lp[p] = pp[N_REP * FA_BQ * D_HEAD + N_REP * FA_BQ + row];
      op[p] = *reinterpret_cast<const f32x4*>(pp + (size_t)row * D_HEAD + 4 * li);
    } else {
      mp[p] = NEG_INF; lp[p] = 0.f; op[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float M = mp[0];
#pragma unroll
  for (int p = 1; p < MAXP; ++p) M = fmaxf(M, mp[p]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const float f = mp[p] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(mp[p] - M);
    acc += op[p] * f;
    L += lp[p] * f;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int h = g * N_REP + h4;
  uint16_t* hrow = a.h + ((size_t)(b * a.T + qi) * N_HEADS + h) * D_HEAD + 4 * li;
  *reinterpret_cast<u32x2*>(hrow) = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                          pack_bf16x2(acc[2] * inv, acc[3] * inv)};
}

size_t flash_partials_bytes(int B, int T, int kv_len, int q_pos0, int causal) {
  if (!causal) {
    // a class byte per (query tile, key tile) for an explicit mask, rows padded
    // to a multiple of 4 bytes
    const size_t nq = (T + FA_BQ - 1) / FA_BQ;
    const size_t nkp = (((size_t)kv_len + FA_BN - 1) / FA_BN + 3) & ~(size_t)3;
    return (nq * nkp + 255) & ~(size_t)255;
  }
  FlashPlan p;
  if (!flash_plan(B, T, kv_len, q_pos0, causal, N_KV, p)) return 0;
  return (size_t)p.n_slots * B * N_KV * FA_PART * sizeof(float);
}

hipError_t launch_flash_attention(const uint16_t* q_r, const uint16_t* k, const uint16_t* v,
                                  long long kv_bstride, const float* mask, int causal, int B,
                                  int T, int kv_len, int q_pos0, uint16_t* h_out,
                                  float* partials, bool q_scaled, hipStream_t s) {
  FlashArgs a{};
  a.q = q_r; a.k = k; a.v = v; a.kv_bstride = kv_bstride; a.mask = mask; a.h = h_out;
  a.B = B; a.T = T; a.kv_len = kv_len; a.q_pos0 = q_pos0; a.causal = causal;
  a.n_qtiles = (T + FA_BQ - 1) / FA_BQ;
  a.mask_vec = mask && (kv_len & 3) == 0 && (reinterpret_cast<uintptr_t>(mask) & 15) == 0;
  if (mask && !causal && partials) {
    // the workspace holds the mask's tile classes (flash_partials_bytes, non-causal)
    const int nk = (kv_len + FA_BN - 1) / FA_BN;
    a.nkp = (nk + 3) & ~3;
    auto* cls = reinterpret_cast<unsigned char*>(partials);
    hipLaunchKernelGGL(flash_mask_classes_kernel, dim3((unsigned)nk, (unsigned)a.n_qtiles),
                       dim3(256), 0, s, mask, T, kv_len, a.nkp,
                       (int)((kv_len & 3) == 0 && (reinterpret_cast<uintptr_t>(mask) & 15) == 0), cls);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.mcls = cls;
  }
  FlashPlan plan;
  const bool planned = partials && flash_plan(B, T, kv_len, q_pos0, causal, N_KV, plan);
  long long grid = (long long)a.n_qtiles * B * N_KV;
  if (planned) {
    a.part = partials;
    a.n_bins = plan.n_bins;
    for (int i = 0; i <= plan.n_bins; ++i) a.bin_start[i] = plan.bin_start[i];
    for (int i = 0; i < plan.n_ent; ++i) a.ent[i] = plan.ent[i];
    grid = (long long)plan.n_bins * B * N_KV;
  }
  if (mask) {
    if (q_scaled)
      hipLaunchKernelGGL((flash_fwd_kernel<true, true>), dim3((unsigned)grid), dim3(FA_THREADS), 0, s, a);
    else
      hipLaunchKernelGGL((flash_fwd_kernel<false, true>), dim3((unsigned)grid), dim3(FA_THREADS), 0, s, a);
  } else {
    if (q_scaled)
      hipLaunchKernelGGL((flash_fwd_kernel<true, false>), dim3((unsigned)grid), dim3(FA_THREADS), 0, s, a);
    else
      hipLaunchKernelGGL((flash_fwd_kernel<false, false>), dim3((unsigned)grid), dim3(FA_THREADS), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !planned || plan.n_merge == 0) return e;
  FlashMergeArgs m{};
  m.part = partials; m.h = h_out; m.B = B; m.T = T;
  for (int i = 0; i < plan.n_merge; ++i) m.mrg[i] = plan.mrg[i];
  const long long mgrid = (long long)plan.n_merge * B * N_KV * (N_REP * FA_BQ / FA_MERGE_ROWS);
  hipLaunchKernelGGL(flash_merge_kernel, dim3((unsigned)mgrid), dim3(256), 0, s, m);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Decode
// ----------------------------------------------------------------------------

constexpr int DC_THREADS = 64 * DC_HG;   // wave w handles KV head DC_HG * slice + w
constexpr int DC_ROW = N_KV * D_HEAD;        // 1024 elements per cache row
constexpr int DC_TROW = DC_HG * D_HEAD;      // elements per tile row (the workgroup's heads)
constexpr int DC_TILE = DC_BN * DC_TROW;     // elements of one K or V tile (16 KiB)
constexpr int DC_NI = DC_TILE / 512;         // 1-KiB loads per K or V tile
constexpr int DC_NI_W = 2 * DC_NI / DC_HG;   // 1-KiB direct-to-LDS loads per wave per tile
constexpr int DC_PART = N_REP * D_HEAD + 2 * N_REP;   // floats per partial: O[4][128], m[4], l[4]
constexpr int DC_QSLOT = DC_HG * 512;        // elements of one query slot: [wave][4 heads][128]
static_assert((DC_STAGES * 2 * DC_TILE + DC_QSLOTS * DC_QSLOT) * 2 <= 160 * 1024, "LDS budget");

// Tile layout: [16 keys][4 heads][128 d]: each load reads 1 KiB of contiguous
// cache row (the workgroup's 4 heads). Inside each head's 256 bytes, K chunk c of
// key k sits at c ^ k (16 keys per fragment read hit 16 slots) and V chunk c
// at c ^ 2(k & 7) (a transposed read of 16 keys x 32 bytes covers each slot
// pair twice).
__device__ __forceinline__ int dk_off(int key, int w, int c) { return key * DC_TROW + w * D_HEAD + ((c ^ (key & 15)) << 3); }
__device__ __forceinline__ int dv_off(int key, int w, int c) { return key * DC_TROW + w * D_HEAD + ((c ^ ((key & 7) << 1)) << 3); }

struct DecodeArgs {
  const uint16_t* q; const uint16_t* kc; const uint16_t* vc;
  float* part; uint16_t* h;
  int B, S_max, kv_len, n_split, chunk;   // chunk: keys per item (multiple of DC_BN)
  int n_items;
};

// Merge of the split partials of (sequence b, KV head g), query head q = 4g + qq,
// dims d0 .. d0 + 7: rescale each chunk's O and sum by its running max, add,
// divide by the rescaled sum of the running sums; chunks in order. (Merging
// inside the split kernel, by the last chunk of a head to finish, would need a
// device-scope release/acquire per workgroup, which writes back and invalidates
// the whole L2 each time and costs far more than this kernel.)
__device__ __forceinline__ void decode_merge_dims(const DecodeArgs& a, int b, int g, int qq,
                                                  int d0) {
  constexpr int ND = 8;
  const float* base = a.part + (size_t)(b * N_KV + g) * a.n_split * DC_PART;
  float M = NEG_INF;
  // unrolled so that several chunks' loads are in flight at once
#pragma unroll 8
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, base[s * DC_PART + N_REP * D_HEAD + qq]);
  float acc[ND], L = 0.f;
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = 0.f;
#pragma unroll 4
  for (int s = 0; s < a.n_split; ++s) {
    const float* p = base + s * DC_PART;
    const float ms = p[N_REP * D_HEAD + qq];
    const float f = ms == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((ms - M) * SCALE_LOG2);
#pragma unroll
    for (int i = 0; i < ND; ++i) acc[i] += p[qq * D_HEAD + d0 + i] * f;
    L += p[N_REP * D_HEAD + N_REP + qq] * f;
  }
  const float r = L > 0.f ? 1.f / L : 0.f;
  uint16_t* hp = a.h + ((size_t)b * N_HEADS + g * N_REP + qq) * D_HEAD + d0;
  *reinterpret_cast<u32x4*>(hp) = u32x4{pack_bf16x2(acc[0] * r, acc[1] * r),
                                        pack_bf16x2(acc[2] * r, acc[3] * r),
                                        pack_bf16x2(acc[4] * r, acc[5] * r),
                                        pack_bf16x2(acc[6] * r, acc[7] * r)};
}

// Persistent split-KV decode. Item = (sequence b, head half hh, chunk sp)
// covers keys [sp*chunk, min(kv_len, (sp+1)*chunk)) of KV heads 4hh .. 4hh+3.
// Workgroup w takes items w, w+G, w+2G, ... and streams their 16-key tiles of
// those heads' cache-row slices HBM -> LDS as one continuous sequence (the
// next tiles always loading while one is computed, across item boundaries).
// Wave w owns KV head 4hh + w and its 4 query heads: scores S^T[16 keys][16
// columns] from 16x16x32 MFMAs whose columns are the 4 query heads (the other
// 12 are zero), so a lane of the accumulator holds 4 keys of one head —
// exactly the P^T operand of the 16x16x16 P·V MFMA, whose V^T operand is one
// transposed LDS read. Online softmax with a lazily moved reference max; each
// wave writes an unnormalised fp32 partial per item.
__global__ __launch_bounds__(DC_THREADS) void decode_splitkv_kernel(DecodeArgs a) {
  // K/V tile ring, then DC_QSLOTS query slots (item ordinal j uses slot j % DC_QSLOTS)
  __shared__ __attribute__((aligned(1024))) uint16_t smem[DC_STAGES * 2 * DC_TILE + DC_QSLOTS * DC_QSLOT];
  uint16_t* const qslots = smem + DC_STAGES * 2 * DC_TILE;
  const uint32_t lds0 = lds_addr(smem);

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int l16 = lane & 15, lg = lane >> 4;
  const int G = gridDim.x;
  // cache bases as values: selecting between fields of the argument struct per
  // lane makes the compiler load the pointer from memory with a vector load
  const uint16_t* const kcache = a.kc;
  const uint16_t* const vcache = a.vc;

  // item = (sequence b, head half hh, chunk sp) = ((b * 2 + hh) * n_split + sp)
  auto item_tiles = [&](int item) {
    const int k0 = (item % a.n_split) * a.chunk;
    return (min(a.kv_len - k0, a.chunk) + DC_BN - 1) / DC_BN;
  };
  const int my_items = (a.n_items - (int)blockIdx.x + G - 1) / G;

  // load cursor over this workgroup's tiles: (item index j, tile t)
  int ld_j = 0, ld_t = 0, ld_n = 0, stage_ld = 0;
  auto issue_next = [&]() {
    const int item = blockIdx.x + ld_j * G;
    const int bh = item / a.n_split;               // b * (8 / DC_HG) + head slice
    const int key_t = (item % a.n_split) * a.chunk + ld_t * DC_BN;
    const size_t seq = (size_t)(bh / (N_KV / DC_HG)) * a.S_max * DC_ROW + (bh % (N_KV / DC_HG)) * DC_TROW;
    const uint32_t st = lds0 + 2u * (uint32_t)(stage_ld * 2 * DC_TILE);
    if (ld_t == 0) {
      // first tile of an item: its queries go ahead of the tile, into slot
      // ld_j % DC_QSLOTS (lane l: query head 4g + l/16, dims 8(l%16) .. +7 of this
      // wave's KV head g); no later item can refill that slot before it is read
      // (decode_plan.h)
      const int b = bh / (N_KV / DC_HG), g = (bh % (N_KV / DC_HG)) * DC_HG + w;
      dma16((const void*)(a.q + ((size_t)b * N_HEADS + g * N_REP) * D_HEAD + lane * 8),
            lds0 + 2u * (uint32_t)(DC_STAGES * 2 * DC_TILE + (ld_j % DC_QSLOTS) * DC_QSLOT + w * 512));
    }
#pragma unroll
    for (int j = 0; j < DC_NI_W; ++j) {
      // instruction i: the 1-KiB piece ii of the K (i < DC_NI) or V tile; lane l
      // fills tile elements ii*512 + 8l .. +7: row r, head hg, physical chunk pc
      const int i = w + DC_HG * j;
      const bool isv = i >= DC_NI;
      const int ii = i % DC_NI;
      const int e = ii * 512 + lane * 8;
      const int r = e / DC_TROW, col = e % DC_TROW;
      const int hg = col >> 7, pc = (col >> 3) & 15;
      const int lc = isv ? (pc ^ ((r & 7) << 1)) : (pc ^ (r & 15));
      const int key = min(key_t + r, a.kv_len - 1);   // clamped keys are masked below
      const uint16_t* src = (isv ? vcache : kcache) + seq + (size_t)key * DC_ROW + hg * D_HEAD + lc * 8;
      dma16_nt((const void*)src, st + 2u * (uint32_t)((isv ? DC_TILE : 0) + ii * 512));
    }
    stage_ld = (stage_ld + 1) % DC_STAGES;
    if (++ld_t == ld_n) { ld_t = 0; ++ld_j; if (ld_j < my_items) ld_n = item_tiles(blockIdx.x + ld_j * G); }
  };
  int total_tiles = 0;
  for (int j = 0; j < my_items; ++j) total_tiles += item_tiles(blockIdx.x + j * G);
  if (my_items > 0) ld_n = item_tiles(blockIdx.x);
  int issued = 0;
#pragma unroll
  for (int s = 0; s < DC_STAGES - 1; ++s)
    if (issued < total_tiles) { issue_next(); ++issued; }

  int done = 0;
  for (int j = 0; j < my_items; ++j) {
    const int item = blockIdx.x + j * G;
    const int sp = item % a.n_split;
    const int bh = item / a.n_split;
    const int b = bh / (N_KV / DC_HG);
    const int g = (bh % (N_KV / DC_HG)) * DC_HG + w;   // this wave's KV head
    const int nt = item_tiles(item);

    // Query fragments (MFMA B operand, 16x16x32): column l16 = query head 4g + l16
    // (zero for l16 >= 4), k-step s covers d = 32s + 8*lg .. +7. Read from the
    // item's query slot once its first tile is resident (the query load went
    // ahead of that tile's loads, and loads complete in order).
    u32x4 qf[4];
    f32x4 o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f32x4{};
    float m_ref = NEG_INF, l_run = 0.f;

    for (int t = 0; t < nt; ++t, ++done) {
      // tile `done` resident (later issued tiles may still load); every wave is past
      // tile done-1, whose stage the next load reuses
      wait_keep<DC_NI_W, DC_STAGES - 2>(min(DC_STAGES - 2, issued - done - 1));
      barrier_no_fence();
      if (t == 0) {
        const uint16_t* qrow = qslots + (j % DC_QSLOTS) * DC_QSLOT + w * 512 + (l16 & 3) * D_HEAD + 8 * lg;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 v = ld16(qrow + 32 * s);
          qf[s] = l16 < N_REP ? v : z;
        }
      }
      if (issued < total_tiles) { issue_next(); ++issued; }

      const uint16_t* sk = smem + (done % DC_STAGES) * 2 * DC_TILE;
      const uint16_t* sv = sk + DC_TILE;
      // S^T: lane holds query l16, keys 4lg + i of this tile
      f32x4 sacc = f32x4{};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sacc = mfma_16x16x32(ld16(sk + dk_off(l16, w, 4 * s + lg)), qf[s], sacc);
      const int kb = sp * a.chunk + t * DC_BN + 4 * lg;
      float mx = NEG_INF;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (kb + i >= a.kv_len) sacc[i] = NEG_INF;
        mx = fmaxf(mx, sacc[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool need = mx > m_ref + FA_RESCALE_RAW;     // false when mx = -inf
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float m_new = need ? mx : m_ref;
        const float alpha = need ? __builtin_amdgcn_exp2f((m_ref - m_new) * SCALE_LOG2) : 1.f;
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] *= alpha;
      }
      const float moff = (m_ref == NEG_INF) ? 0.f : -m_ref * SCALE_LOG2;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], SCALE_LOG2, moff));
        l_run += p[i];
      }
      const u32x2 pf = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      // O^T[d][q] += V^T[d][keys] · P^T[keys][q] in 8 blocks of 16 d: a transposed
      // read gives lane l the values V[4lg + e][16db + l16], e = 0..3.
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int d = 16 * db + 4 * (l16 & 3);
        const u32x2 vf = ld_tr(sv + dv_off(4 * lg + (l16 >> 2), w, d >> 3) + (d & 7));
        o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, vf),
                                                           __builtin_bit_cast(i16x4, pf), o[db], 0, 0, 0);
      }
    }

    // this wave's partial for (b, g, sp): o[db][i] is query l16, d = 16db + 4lg + i
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    float* part = a.part + ((size_t)(b * N_KV + g) * a.n_split + sp) * DC_PART;
    if (l16 < N_REP) {
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *reinterpret_cast<f32x4*>(part + l16 * D_HEAD + 16 * db + 4 * lg) = o[db];
      if (lg == 0) { part[N_REP * D_HEAD + l16] = m_ref; part[N_REP * D_HEAD + N_REP + l16] = l_run; }
    }
  }
}

// One wave per (sequence, KV head): rescale and sum the split partials of its
// four query heads; lane l takes query head 4g + l/16, dims 8(l%16) .. +7.
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int b = blockIdx.x / N_KV, g = blockIdx.x % N_KV;
  decode_merge_dims(a, b, g, threadIdx.x >> 4, (threadIdx.x & 15) * 8);
}

size_t decode_partials_bytes(int B, int S_max) {
  return (size_t)B * N_KV * decode_n_split(B, S_max, N_KV) * DC_PART * sizeof(float);
}

hipError_t launch_decode_attention(const uint16_t* q_r, const uint16_t* k_cache,
                                   const uint16_t* v_cache, int B, int S_max, int kv_len,
                                   float* partials, uint16_t* h_out, hipStream_t s) {
  // CUs of the current device, asked on every call (no state kept between calls)
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu <= 0)
    return hipErrorInvalidDevice;
  const DecodePlan p = decode_plan(B, kv_len, N_KV, n_cu);
  DecodeArgs a{};
  a.q = q_r; a.kc = k_cache; a.vc = v_cache; a.part = partials; a.h = h_out;
  a.B = B; a.S_max = S_max; a.kv_len = kv_len;
  a.n_split = p.n_split; a.chunk = p.chunk; a.n_items = p.n_items;
  hipLaunchKernelGGL(decode_splitkv_kernel, dim3((unsigned)p.grid), dim3(DC_THREADS), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(B * N_KV)), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa

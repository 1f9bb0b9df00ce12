// Projection GEMMs of the GQA block on bf16 MFMA (gfx950).
//
//  * qkv_rope: [Q | K | V] = x · [W_Q; W_K; W_V]ᵀ over the fused 6144 output
//    columns (Grouped-query attention page, "All 13 steps", the three
//    projection equations; weights stored [out, in] per the Query projection
//    page), with the pair rotation of Q and K applied in the epilogue (the 2x2
//    rotation display) before the single rounding to bf16.
//  * out_proj: Δ = H · W_Oᵀ in fp32 (the last equation; Merge and project page),
//    optionally plus a bf16 residual (the block's handoff).
//  * The SwiGLU MLP ("Llama 3" page, SwiGLU MLP): gate and up as one product
//    whose epilogue forms silu(gate)·up, and the down product (K = 14336)
//    with the fp32 epilogue.
//
// All are "NT" products: each operand is contiguous along the reduction axis
// (K = 4096, or 14336 for the MLP's down product). A workgroup computes a
// TOK x FEAT tile with a K step of 64.
// Operand tiles go from HBM straight into LDS (global_load_lds_dwordx4, no
// register staging) through a ring of STAGES buffers, so STAGES-1 K steps of
// loads are in flight while one is computed; one barrier per K step. Where a
// weight tile lies inside one matrix the loads take a scalar tile base and a
// fixed per-lane offset, and the fragment reads a per-lane address plus
// immediate offsets, so the step loop has almost no VALU address arithmetic
// (6 VALU instructions per 64 MFMAs at 256x256 instead of 43: 1.5-5 % faster
// at M = 2048 to 131072). LDS rows
// are 128 bytes (64 bf16) with 16-byte chunk c of row r stored at c ^ rperm(r):
// the 16x16x32 MFMA fragment reads (each group of 16 lanes: one chunk of 16
// consecutive rows) are then conflict-free, and each 64-lane load instruction
// still writes one contiguous kilobyte of LDS as the direct-to-LDS path
// requires. Within a K step each slice's fragment reads are spread between the
// MFMAs of the slice before. The 16x16x32 shape runs the same tiles 5-10 %
// faster than 32x32x16 (same LDS traffic per flop, twice as many shorter
// MFMAs to interleave the reads with) and gives bit-identical fp32 sums.
//
// For qkv_rope (and the gate/up product) the MFMA "A" operand is the weight
// tile and "B" the token tile, so the accumulator holds features down its
// rows: a lane then owns 4 consecutive features of one token, i.e. both
// members of two rotation pairs, and the rotation needs no cross-lane
// traffic. Their bf16 results go through LDS (the idle load ring) so that the
// global stores are whole 16-byte chunks of token rows.
//
// Few tokens (decode, M <= 64) make both products weight streams: every
// weight is used by at most 64 tokens, so the time is HBM bytes, and a
// workgroup that walks all 64 K steps is bound by the latency of its own
// step loop, with too few workgroups to keep enough bytes in flight. There
// the reduction axis is split over SPLITK workgroups (grid y), each writing
// fp32 partial sums to a workspace, and a second kernel adds the partials in
// a fixed order (deterministic) and applies the epilogue (rotation + bf16,
// or fp32 store).

#include <type_traits>

#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {

constexpr int BK = 64;  // K step

enum Epilogue { EPI_QKV_ROPE = 0, EPI_OUT_F32 = 1, EPI_PARTIAL_F32 = 2, EPI_SWIGLU = 3 };

struct GemmArgs {
  const uint16_t* act;   // [M][K] bf16 activations
  const uint16_t* w0;    // weight rows [.][K] (W_Q, W_O, the MLP's gate w1 or down w2)
  const uint16_t* w1;    // fused QKV: W_K rows; gate/up product: up (w3) rows
  const uint16_t* w2;    // fused QKV: W_V rows
  int M;                 // tokens
  int N;                 // output features (6144, 4096, or 2 x 14336 gate/up)
  int K;                 // reduction length (4096, or 14336 for the MLP's down product)
  // rotation epilogue
  const float* rope;     // [T][64][2]
  int T;                 // tokens per sequence (rope row = token % T)
  float q_scale;         // factor on the rotated Q features before rounding (1: none)
  uint16_t* q_dst; long long q_bstride, q_rstride;     // elements
  uint16_t* k_dst; uint16_t* v_dst; long long kv_bstride, kv_rstride;
  // fp32 epilogue: out[M][N]; split-K partials: out + blockIdx.y*M*N
  float* out;
  // fp32 epilogue: optional bf16 residual [M][N] added to the product (null: none)
  const uint16_t* resid;
  // gate/up epilogue: silu(gate)·up as bf16 [M][N/2]
  uint16_t* glu_out;
  // this launch covers output features n_off .. n_off + n_len - 1 (n_len = 0: all N)
  int n_off, n_len;
};

// Chunk permutation of row r for LDS rows of KB bf16 (KB/8 chunks of 16 bytes).
// The 16 lanes of a fragment read take one chunk c of 16 consecutive rows.
//  * KB = 64 (128-byte rows): chunk c at c ^ (r & 7). Measured with the LDS
//    counters on the 16x16x32 fragment pattern (a probe reading every
//    candidate layout): 4 active LDS cycles per ds_read_b128 and no bank
//    conflicts, where c ^ (r & 7) ^ ((r >> 3) & 1) (conflict-free for the
//    32-row fragments of 32x32x16 MFMAs) took 8, half of them conflicts, and
//    no permutation 16.
//  * KB = 32 (64-byte rows, 4 per 256-byte window): rows r mod 4 fill the
//    window's four 64-byte quarters and (r >> 2) & 3 picks the chunk inside each.
template <int KB>
__device__ __forceinline__ int rperm(int r) {
  if constexpr (KB == 64) return r & 7;
  else return (r >> 2) & 3;
}
template <int KB>
__device__ __forceinline__ int swz(int r, int c) { return r * KB + ((c ^ rperm<KB>(r)) << 3); }

// Maps a linear workgroup id to (token tile, feature tile): workgroups are
// dealt round-robin to the 8 XCDs, so ids are first regrouped so that each
// XCD owns a contiguous run of tiles, and runs are walked in groups of
// GROUP token tiles so concurrently resident tiles share operand rows in
// that XCD's L2.
template <int GROUP>
__device__ __forceinline__ void tile_coords(int bid, int nwg, int tiles_tok, int tiles_feat,
                                            int& tt, int& tf) {
  int lin = bid;
  if ((nwg & 7) == 0) lin = (bid & 7) * (nwg >> 3) + (bid >> 3);
  int per_group = GROUP * tiles_feat;
  int g = lin / per_group;
  int first = g * GROUP;
  int gsz = min(tiles_tok - first, GROUP);
  int r = lin - g * per_group;
  tt = first + r % gsz;
  tf = r / gsz;
}

// silu(g)·u with silu(g) = g / (1 + e^-g) ("Llama 3" page, SwiGLU MLP), in
// fp32: e^-g as 2^(-g·log2 e) (v_exp_f32); for g below about -88 the power is
// +inf and the quotient -0, the limit.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g / (1.0f + e) * u;
}

// Rotation of pairs (v0, v1) and (v2, v3) by the angles whose (cos, sin) are
// (cs[0], cs[1]) and (cs[2], cs[3]) (Grouped-query attention page, "All 13
// steps", the 2x2 rotation display: first member c*z0 - s*z1, second
// s*z0 + c*z1).
__device__ __forceinline__ void rotate_pairs(float& v0, float& v1, float& v2, float& v3, f32x4 cs) {
  const float r0 = v0 * cs[0] - v1 * cs[1];
  const float r1 = v0 * cs[1] + v1 * cs[0];
  const float r2 = v2 * cs[2] - v3 * cs[3];
  const float r3 = v2 * cs[3] + v3 * cs[2];
  v0 = r0; v1 = r1; v2 = r2; v3 = r3;
}

// Row f of the weight operand.
//  * Fused QKV product (N = 6144): output columns [0,4096) are W_Q rows, then
//    W_K, then W_V.
//  * Gate/up product of the MLP: each wave's WPF feature rows are WPF/2 gate
//    (w1) rows followed by the up (w3) rows of the same hidden units, so that
//    a lane's accumulators hold both factors of silu(gate)·up. Wave block
//    starting at feature fb covers hidden units fb/2 .. fb/2 + WPF/2 - 1.
//  * Otherwise rows of w0.
template <int EPI, int WPF>
__device__ __forceinline__ const uint16_t* weight_row(const GemmArgs& a, int f) {
  if constexpr (EPI == EPI_SWIGLU) {
    const int w = f % WPF;
    const int unit = (f - w) / 2 + (w % (WPF / 2));
    return (w < WPF / 2 ? a.w0 : a.w1) + (size_t)unit * a.K;
  } else {
    if (a.N == N_QKV) {
      if (f >= D_MODEL + N_KV * D_HEAD) return a.w2 + (size_t)(f - D_MODEL - N_KV * D_HEAD) * a.K;
      if (f >= D_MODEL) return a.w1 + (size_t)(f - D_MODEL) * a.K;
    }
    return a.w0 + (size_t)f * a.K;
  }
}

template <int TOK, int FEAT, int WPN, int WQN, int STAGES, int EPI, int KB = BK>
struct GemmCfg {
  static_assert(KB == 64 || KB == 32, "K step");
  static constexpr int BK = KB;
  static constexpr int CPR = KB / 8;                   // 16-byte chunks per LDS row
  static constexpr int RPI = 512 / KB;                 // LDS rows per 1 KiB load instruction
  static constexpr bool SWAP = (EPI == EPI_QKV_ROPE || EPI == EPI_SWIGLU);
  static constexpr int PR = SWAP ? FEAT : TOK;   // MFMA A operand rows
  static constexpr int QR = SWAP ? TOK : FEAT;   // MFMA B operand rows
  static constexpr int NW = WPN * WQN;
  static constexpr int THREADS = 64 * NW;
  static constexpr int WP = PR / WPN, WQ = QR / WQN;   // wave tile
  static constexpr int NP = WP / 16, NQ = WQ / 16;   // 16x16 MFMA blocks per wave
  static constexpr int STAGE_ELEMS = (PR + QR) * BK;
  static constexpr int LDS_BYTES = STAGES * STAGE_ELEMS * 2;
  static constexpr int NI = (PR + QR) / RPI;           // 1 KiB load instructions per stage
  static constexpr int NI_W = NI / NW;                 // per wave
  static_assert(NI % NW == 0, "load instructions must split evenly across waves");
  static_assert(WP % 16 == 0 && WQ % 16 == 0, "wave tile must be whole 16x16 MFMA blocks");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 2 && NI_W * (STAGES - 2) < 64, "vmcnt range");
  static_assert(EPI != EPI_SWIGLU || NP % 2 == 0, "gate/up pairs need an even feature block count");
  // barrier before the last slice of a step; its register double-buffering
  // needs an even number of 32-wide slices per step (K step 64)
  static constexpr bool XSTAGE = NP * NQ >= 12 && KB == 64;
  // Waves per SIMD the workgroups that fit a CU's LDS can provide (at most 2):
  // the register budget is sized for it (256 per wave at 2).
  static constexpr int WG_PER_CU = (160 * 1024) / LDS_BYTES;
  static constexpr int MIN_WAVES_EU = (NW * WG_PER_CU + 3) / 4 >= 2 ? 2 : 1;
  // Token tiles per group of tile_coords: an XCD's run of 32 tiles is GROUP
  // token tiles x 32/GROUP feature tiles, and it fetches GROUP*TOK + (32/GROUP)*FEAT
  // operand rows past its L2; GROUP = 8 minimises that for FEAT >= 1.5 TOK
  // (128x256: W_O at M = 2048 fetches 134 instead of 168 MB), 4 otherwise
  // (256x192: QKV fetches 172 instead of 192 MB; 256x256 at M = 32768 1-2 %
  // faster than with 8).
  static constexpr int GROUP = 2 * FEAT >= 3 * TOK ? 8 : 4;
  static constexpr int RPM = NP * NQ / (NP + NQ) > 1 ? NP * NQ / (NP + NQ) : 1;   // MFMAs per spread read
  // Tiles of 64 tokens serve M <= 64 (decode), a single token tile: every weight
  // row is read by exactly one workgroup, once, so those loads stream past the
  // caches (non-temporal). Load instruction j of every wave fills P rows iff
  // j < NJ_P (P rows come first and split evenly over the waves).
  static constexpr bool NT_W = TOK == 64;
  // Scalar-base loads: where a weight tile lies inside one matrix (Q, K and V
  // bounds are multiples of 1024) and the P rows split evenly over the waves,
  // every load is a wave-uniform tile base (token or weight, plus the step's K
  // offset: scalar adds) and a loop-invariant per-lane byte offset.
  static constexpr bool SV = !NT_W && EPI != EPI_SWIGLU && 1024 % FEAT == 0 && (PR / RPI) % NW == 0;
  static constexpr int NJ_P = PR / RPI / NW;
  static_assert(!NT_W || (PR / RPI) % NW == 0, "weight loads must be whole instructions of every wave");
};

// Registers for two waves per SIMD where the LDS admits them: eight-wave
// workgroups need it, and four-wave ones then fit two workgroups per CU.
template <int TOK, int FEAT, int WPN, int WQN, int STAGES, int EPI, int KB = BK>
__global__ __launch_bounds__(64 * WPN * WQN)
__attribute__((amdgpu_waves_per_eu(GemmCfg<TOK, FEAT, WPN, WQN, STAGES, EPI, KB>::MIN_WAVES_EU)))
void gemm_nt_kernel(GemmArgs a) {
  using C = GemmCfg<TOK, FEAT, WPN, WQN, STAGES, EPI, KB>;
  constexpr int PR = C::PR, QR = C::QR, NP = C::NP, NQ = C::NQ;
  constexpr int BK = C::BK;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[STAGES * C::STAGE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int wp = wave / WQN, wq = wave % WQN;

  const int tiles_tok = (a.M + TOK - 1) / TOK;
  const int tiles_feat = (a.n_len > 0 ? a.n_len : a.N) / FEAT;
  int tt, tf;
  tile_coords<C::GROUP>(blockIdx.x, gridDim.x, tiles_tok, tiles_feat, tt, tf);
  const int m0 = tt * TOK;
  const int n0 = a.n_off + tf * FEAT;

  // K range of this workgroup: all of it, or slice blockIdx.y of gridDim.y (split K)
  const int NK = a.K / BK / (int)gridDim.y;
  const int k_first = (int)blockIdx.y * NK;
  const uint16_t* abase = a.act + (size_t)m0 * a.K;
  const int tok_last = a.M - m0 - 1;   // rows past it are clamped (their outputs are discarded)

  // This lane's source pointers for its NI_W load instructions (K offset added per step).
  // Instruction i covers LDS rows RPI*i .. RPI*i + RPI-1 of the stage (P rows first,
  // then Q rows); lane l writes row RPI*i + l / CPR, physical chunk l % CPR, which
  // holds logical chunk (l % CPR) ^ rperm(row).
  // SV: the lane's byte offset from its operand's tile base; otherwise its own
  // source pointer.
  const uint16_t* src[C::NI_W];
  uint32_t voff[C::NI_W];
  const char* tbase = nullptr;
  const char* wbase = nullptr;
  if constexpr (C::SV) {
    tbase = (const char*)(abase + (size_t)k_first * BK);
    wbase = (const char*)(weight_row<EPI, C::WP>(a, n0) + (size_t)k_first * BK);
  }
#pragma unroll
  for (int j = 0; j < C::NI_W; ++j) {
    const int i = wave + j * C::NW;
    int row = C::RPI * i + lane / C::CPR;
    const int lc = (lane % C::CPR) ^ rperm<BK>(row);
    const bool is_p = row < PR;
    const int r = is_p ? row : row - PR;
    const bool is_tok = C::SWAP ? !is_p : is_p;
    if constexpr (C::SV) {
      // < 256 rows of at most 14336 elements: well inside 32 bits
      voff[j] = (uint32_t)(((is_tok ? min(r, tok_last) : r) * a.K + lc * 8) * 2);
    } else {
      const uint16_t* rowp = is_tok ? abase + (size_t)min(r, tok_last) * a.K
                                    : weight_row<EPI, C::WP>(a, n0 + r);
      src[j] = rowp + (size_t)k_first * BK + lc * 8;
    }
  }
  const uint32_t lds0 = lds_addr(smem);
  // LDS ring, operand-major: the P rows of every stage, then the Q rows of
  // every stage (a stage's P and Q blocks then each sit within 16-bit
  // immediate offsets of a fragment read's lane address)
  auto pst = [&](int stage) { return stage * (PR * BK); };
  auto qst = [&](int stage) { return STAGES * PR * BK + stage * (QR * BK); };
  // load instruction j of this wave for step kt into ring stage `stage`
  auto issue_one = [&](int kt, int stage, int j) {
    const int i = wave + j * C::NW;
    // whether instruction i fills P rows: known at compile time when the P rows
    // split evenly over the waves (i < PR / RPI exactly when j < NJ_P)
    const bool in_p = (PR / C::RPI) % C::NW == 0 ? j < C::NJ_P : i < PR / C::RPI;
    const uint32_t dst =
        lds0 + 2u * (uint32_t)(in_p ? pst(stage) + i * 512 : qst(stage) + (i - PR / C::RPI) * 512);
    if constexpr (C::SV) {
      const bool is_tok = C::SWAP ? !(j < C::NJ_P) : (j < C::NJ_P);
      dma16_sv((is_tok ? tbase : wbase) + (size_t)kt * (BK * 2), voff[j], dst);
    } else if (C::NT_W && (j < C::NJ_P) == C::SWAP) {
      dma16_nt((const void*)(src[j] + kt * BK), dst);   // weight rows
    } else {
      dma16((const void*)(src[j] + kt * BK), dst);
    }
  };
  auto issue = [&](int kt, int stage) {
#pragma unroll
    for (int j = 0; j < C::NI_W; ++j) issue_one(kt, stage, j);
  };

  f32x4 acc[NP][NQ];
#pragma unroll
  for (int i = 0; i < NP; ++i)
#pragma unroll
    for (int j = 0; j < NQ; ++j) acc[i][j] = f32x4{};

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < NK) issue(s, s);

  const int l16 = lane & 15, lg = lane >> 4;
  // fragments double-buffered in registers: reads of slice kk+1 overlap the MFMAs
  // of kk (declared outside the step loop: the generated loop is faster)
  u32x4 af[2][NP], bf[2][NQ];
  // after_read(r) runs after fragment read r (0 .. NP+NQ-1) in program order
  // Rows wp*WP + 16i + l16 all take the chunk permutation of row l16 (WP and 16
  // are multiples of the permutation's period), so fragment i is the lane's
  // fragment 0 plus a constant: one address per operand and slice, the rest
  // immediate offsets.
  auto read_frags_then = [&](int stage, int kk, u32x4 (&fa)[NP], u32x4 (&fb)[NQ],
                             auto&& after_read) {
    const int ch = kk * 4 + lg;
    const uint16_t* sp = smem + pst(stage) + swz<BK>(wp * C::WP + l16, ch);
    const uint16_t* sq = smem + qst(stage) + swz<BK>(wq * C::WQ + l16, ch);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      fa[i] = ld16(sp + i * 16 * BK);
      after_read(i);
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      fb[j] = ld16(sq + j * 16 * BK);
      after_read(NP + j);
    }
  };
  auto read_frags = [&](int stage, int kk, u32x4 (&fa)[NP], u32x4 (&fb)[NQ]) {
    read_frags_then(stage, kk, fa, fb, [](int) {});
  };
  auto mfmas = [&](int kk) {
#pragma unroll
    for (int i = 0; i < NP; ++i)
#pragma unroll
      for (int j = 0; j < NQ; ++j) acc[i][j] = mfma_16x16x32(af[kk & 1][i], bf[kk & 1][j], acc[i][j]);
  };
  // The reads of the next slice go out one at a time between the MFMAs of this
  // one (scheduling groups: MFMA, read, MFMA, read, ...): a burst of reads from
  // all eight waves queues up in the LDS; spread out they return in time (QKV
  // at M = 2048: 8 % faster than issuing them as a block).
  auto spread = [&]() {
#pragma unroll
    for (int r = 0; r < NP + NQ; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, C::RPM, 0);   // RPM MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
  };
  constexpr int NS = BK / 32;   // MFMA slices per K step
  static_assert(!C::XSTAGE || NS % 2 == 0, "slice parity of the register buffers");
  if constexpr (C::XSTAGE) {
    // The step's barrier sits before its last slice: once every wave has its
    // last fragments in registers (lgkmcnt(0)) and the next step's loads have
    // landed, the next step's first reads go out between the last slice's
    // MFMAs instead of stalling the start of the next step. Used where a slice
    // has enough MFMAs (NP * NQ >= 6) to cover those reads.
    wait_keep<C::NI_W, STAGES - 2>(min(STAGES - 2, NK - 1));
    barrier_no_fence();
    read_frags(0, 0, af[0], bf[0]);
    if (STAGES - 1 < NK) issue(STAGES - 1, (STAGES - 1) % STAGES);
    auto body = [&](int sp) {
#pragma unroll
      for (int kk = 0; kk < NS - 1; ++kk) {
        read_frags(sp, kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
        mfmas(kk);
        spread();
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Step kt: slices 0 .. NS-2, the wait and barrier, then the last slice
    // with the next step's first fragment reads between its MFMAs. While
    // steps remain to be loaded, the refill of the stage just finished goes
    // out one load instruction after each of those reads rather than as a
    // block after the barrier, so no wave stalls on issuing its loads before
    // its first MFMA (QKV 2-3 % faster at M = 2048 and 32768). The two loops
    // keep the refill decision out of the loop body (a branch there splits
    // the scheduling region and the accumulators' registers).
    auto step = [&](int kt, auto refill) {
      body(kt % STAGES);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), other counters free (gfx9 encoding)
      wait_keep<C::NI_W, STAGES - 2>(min(STAGES - 2, NK - 2 - kt));
      barrier_no_fence();
      const int next = (kt + 1) % STAGES;
      if constexpr (decltype(refill)::value) {
        // every wave is done with stage kt % STAGES: refill it with step kt + STAGES
        read_frags_then(next, 0, af[NS & 1], bf[NS & 1], [&](int r) {
          if (r < C::NI_W) issue_one(kt + STAGES, kt % STAGES, r);
        });
#pragma unroll
        for (int j = NP + NQ; j < C::NI_W; ++j) issue_one(kt + STAGES, kt % STAGES, j);
      } else {
        read_frags(next, 0, af[NS & 1], bf[NS & 1]);
      }
      mfmas(NS - 1);
      spread();
      __builtin_amdgcn_sched_barrier(0);
    };
    int kt = 0;
    for (; kt < NK - STAGES; ++kt) step(kt, std::true_type{});
    for (; kt < NK - 1; ++kt) step(kt, std::false_type{});
    body((NK - 1) % STAGES);
    mfmas(NS - 1);
  } else {
    for (int kt = 0; kt < NK; ++kt) {
      // wait for this step's loads; keep the later steps' loads (at most STAGES-2) in flight
      wait_keep<C::NI_W, STAGES - 2>(min(STAGES - 2, NK - 1 - kt));
      barrier_no_fence();
      const int sp = kt % STAGES;
      read_frags(sp, 0, af[0], bf[0]);
      // the next stage's loads go out while the first fragment reads are in flight
      if (kt + STAGES - 1 < NK) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
#pragma unroll
      for (int kk = 0; kk < NS; ++kk) {
        if (kk + 1 < NS) read_frags(sp, kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
        mfmas(kk);
        if (kk + 1 < NS) spread();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  if constexpr (EPI == EPI_QKV_ROPE) {
    // Rotation in registers and one bf16 rounding; the rounded tile then goes
    // through LDS (the load ring is idle after the last K step) so that the
    // global stores are whole 16-byte chunks of token rows instead of 8-byte
    // pieces of 32 different rows per instruction.
    // acc[i][j][e]: feature n0 + wp*WP + 16i + 4*lg + e, token m0 + wq*WQ + 16j + l16.
    // A 16-feature block lies inside one of Q, K, V (their bounds are multiples of 1024).
    constexpr int CPT = FEAT / 8;                       // 16-byte chunks per tile row
    constexpr int SWZ = CPT >= 8 ? 7 : CPT - 1;         // chunk c of row r at c ^ (r & SWZ)
    static_assert(CPT % (SWZ + 1) == 0, "chunk swizzle stays inside the row");
    static_assert(TOK * FEAT * 2 <= C::LDS_BYTES, "bf16 tile fits the load ring");
    uint16_t* tile = smem;
    __syncthreads();   // every wave is done reading the last stage
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int tl = wq * C::WQ + j * 16 + l16;
      const int tok = min(m0 + tl, a.M - 1);
      const int t = tok - (tok / a.T) * a.T;
      const float* rrow = a.rope + (size_t)t * (2 * 64);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int fblk = n0 + wp * C::WP + i * 16;
        const bool rot = fblk < D_MODEL + N_KV * D_HEAD;   // Q and K rotate, V does not
        const int f = fblk + 4 * lg;
        float v0 = acc[i][j][0], v1 = acc[i][j][1], v2 = acc[i][j][2], v3 = acc[i][j][3];
        if (rot)
          rotate_pairs(v0, v1, v2, v3, *reinterpret_cast<const f32x4*>(rrow + (f & (D_HEAD - 1))));
        if (fblk < D_MODEL) {
          v0 *= a.q_scale; v1 *= a.q_scale; v2 *= a.q_scale; v3 *= a.q_scale;
        }
        const int c = (wp * C::WP + i * 16 + 4 * lg) >> 3;
        *reinterpret_cast<u32x2*>(tile + tl * FEAT + ((c ^ (tl & SWZ)) << 3) + 4 * (lg & 1)) =
            u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
      }
    }
    __syncthreads();
    for (int idx = tid; idx < TOK * CPT; idx += C::THREADS) {
      const int tl = idx / CPT, c = idx - tl * CPT;
      const int tok = m0 + tl;
      if (tok >= a.M) continue;
      const int b = tok / a.T;
      const int t = tok - b * a.T;
      const int f = n0 + 8 * c;
      uint16_t* dst;
      if (f < D_MODEL) {
        dst = a.q_dst + b * a.q_bstride + t * a.q_rstride + f;
      } else {
        const bool is_k = f < D_MODEL + N_KV * D_HEAD;
        dst = (is_k ? a.k_dst : a.v_dst) + b * a.kv_bstride + t * a.kv_rstride +
              (f - (is_k ? D_MODEL : D_MODEL + N_KV * D_HEAD));
      }
      st16(dst, ld16(tile + tl * FEAT + ((c ^ (tl & SWZ)) << 3)));
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // acc[i][j][e]: tile feature wp*WP + 16i + 4*lg + e, token
    // m0 + wq*WQ + 16j + l16. Blocks i < NP/2 are gate rows, block i + NP/2 the
    // up rows of the same hidden units (weight_row's order). silu(gate)·up is
    // rounded once to bf16 and, as for the rotation epilogue, the tile goes
    // through LDS to be stored as whole 16-byte chunks of token rows.
    constexpr int UNITS = FEAT / 2;                     // hidden units per tile
    constexpr int CPT = UNITS / 8;
    constexpr int SWZ = CPT >= 8 ? 7 : CPT - 1;
    static_assert(CPT % (SWZ + 1) == 0, "chunk swizzle stays inside the row");
    static_assert(TOK * UNITS * 2 <= C::LDS_BYTES, "bf16 tile fits the load ring");
    uint16_t* tile = smem;
    __syncthreads();   // every wave is done reading the last stage
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int tl = wq * C::WQ + j * 16 + l16;
#pragma unroll
      for (int i = 0; i < NP / 2; ++i) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = silu_mul(acc[i][j][e], acc[i + NP / 2][j][e]);
        const int c = (wp * C::WP / 2 + i * 16 + 4 * lg) >> 3;
        *reinterpret_cast<u32x2*>(tile + tl * UNITS + ((c ^ (tl & SWZ)) << 3) + 4 * (lg & 1)) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
    __syncthreads();
    const int ld = a.N / 2;
    for (int idx = tid; idx < TOK * CPT; idx += C::THREADS) {
      const int tl = idx / CPT, c = idx - tl * CPT;
      const int tok = m0 + tl;
      if (tok >= a.M) continue;
      st16(a.glu_out + (size_t)tok * ld + n0 / 2 + 8 * c,
           ld16(tile + tl * UNITS + ((c ^ (tl & SWZ)) << 3)));
    }
  } else {
    // acc[i][j][r]: token m0 + wp*WP + 16i + 4*lg + r, feature n0 + wq*WQ + 16j + l16.
    float* obase = a.out;
    if (EPI == EPI_PARTIAL_F32) obase += (size_t)blockIdx.y * a.M * a.N;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = m0 + wp * C::WP + i * 16 + 4 * lg + r;
        if (tok >= a.M) continue;
        const size_t off = (size_t)tok * a.N + n0 + wq * C::WQ + l16;
        float* orow = obase + off;
        if (EPI == EPI_OUT_F32 && a.resid) {
#pragma unroll
          for (int j = 0; j < NQ; ++j)
            orow[j * 16] = acc[i][j][r] + __builtin_bit_cast(float, (uint32_t)a.resid[off + j * 16] << 16);
        } else {
#pragma unroll
          for (int j = 0; j < NQ; ++j) orow[j * 16] = acc[i][j][r];
        }
      }
    }
  }
}

// Sum of the split-K partials (slices 0..KS-1 in order) of 4 consecutive
// columns of one token; all KS loads are issued before the adds.
template <int KS>
__device__ __forceinline__ f32x4 sum_partials(const GemmArgs& a, int tok, int col) {
  const size_t slice = (size_t)a.M * a.N;
  const float* p = a.out + (size_t)tok * a.N + col;
  f32x4 v[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) v[s] = *reinterpret_cast<const f32x4*>(p + s * slice);
  f32x4 acc = v[0];
#pragma unroll
  for (int s = 1; s < KS; ++s) acc += v[s];
  return acc;
}

// Split-K epilogue of the fused QKV product: one thread per 4 consecutive
// columns of one token; a.out holds the partials [KS][M][6144].
template <int KS>
__global__ __launch_bounds__(256) void splitk_qkv_rope_kernel(GemmArgs a) {
  constexpr int PER_TOK = N_QKV / 4;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.M * PER_TOK) return;
  const int tok = idx / PER_TOK;
  const int col = (idx - tok * PER_TOK) * 4;
  f32x4 v = sum_partials<KS>(a, tok, col);
  float v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
  const int b = tok / a.T;
  const int t = tok - b * a.T;
  uint16_t* dst;
  if (col < D_MODEL) {
    dst = a.q_dst + b * a.q_bstride + t * a.q_rstride + col;
  } else {
    const bool is_k = col < D_MODEL + N_KV * D_HEAD;
    const int f = col - (is_k ? D_MODEL : D_MODEL + N_KV * D_HEAD);
    dst = (is_k ? a.k_dst : a.v_dst) + b * a.kv_bstride + t * a.kv_rstride + f;
  }
  if (col < D_MODEL + N_KV * D_HEAD)
    rotate_pairs(v0, v1, v2, v3,
                 *reinterpret_cast<const f32x4*>(a.rope + (size_t)t * (2 * 64) + (col & (D_HEAD - 1))));
  if (col < D_MODEL) {
    v0 *= a.q_scale; v1 *= a.q_scale; v2 *= a.q_scale; v3 *= a.q_scale;
  }
  u32x2 w = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
  *reinterpret_cast<u32x2*>(dst) = w;
}

// Split-K epilogue of the output projection: out[M][4096] = sum of partials
// (+ the bf16 residual when a.resid is set).
template <int KS>
__global__ __launch_bounds__(256) void splitk_out_kernel(GemmArgs a, float* out) {
  constexpr int PER_TOK = D_MODEL / 4;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.M * PER_TOK) return;
  const int tok = idx / PER_TOK;
  const int col = (idx - tok * PER_TOK) * 4;
  const size_t off = (size_t)tok * D_MODEL + col;
  f32x4 v = sum_partials<KS>(a, tok, col);
  if (a.resid) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(a.resid + off);
    v += f32x4{bf16lo(x[0]), bf16hi(x[0]), bf16lo(x[1]), bf16hi(x[1])};
  }
  *reinterpret_cast<f32x4*>(out + off) = v;
}

template <int TOK, int FEAT, int WPN, int WQN, int STAGES, int EPI, int KB = BK>
static hipError_t launch_gemm(const GemmArgs& a, hipStream_t s, int ksplit = 1) {
  using C = GemmCfg<TOK, FEAT, WPN, WQN, STAGES, EPI, KB>;
  const int tiles = ((a.M + TOK - 1) / TOK) * ((a.n_len > 0 ? a.n_len : a.N) / FEAT);
  hipLaunchKernelGGL((gemm_nt_kernel<TOK, FEAT, WPN, WQN, STAGES, EPI, KB>), dim3(tiles, ksplit),
                     dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

// Split-K product into the partial buffer `part` ([KS][M][N] fp32), then the
// epilogue kernel. a.out is the final fp32 destination (out_proj) or unused.
template <int TOK, int FEAT, int WPN, int WQN, int STAGES, int KS>
static hipError_t launch_gemm_splitk(GemmArgs a, float* part, hipStream_t s) {
  if ((a.K / BK) % KS != 0) return hipErrorInvalidValue;   // K steps must split evenly
  float* final_out = a.out;
  a.out = part;
  hipError_t e = launch_gemm<TOK, FEAT, WPN, WQN, STAGES, EPI_PARTIAL_F32>(a, s, KS);
  if (e != hipSuccess) return e;
  const int threads = a.M * (a.N / 4);
  const dim3 grid((threads + 255) / 256);
  if (a.N == N_QKV)
    hipLaunchKernelGGL(splitk_qkv_rope_kernel<KS>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(splitk_out_kernel<KS>, grid, dim3(256), 0, s, a, final_out);
  return hipGetLastError();
}

// Split reduction for few tokens (with a workspace): M <= 64 takes one 64-token
// tile and 4 slices of K (weight streams, non-temporal); 64 < M <= 128 takes
// 128-token x 64-feature tiles and 4 slices (384 workgroups for the QKV
// product, 256 for W_O; the block step at M = 128 12 % faster than 128x128
// tiles in 8 slices, whose partials were twice as many); 128 < M <= 256 takes
// 128x128 tiles and 4 slices (the 64-feature tiles are 5-7 % slower there).
// Unsplit 128x128 tiles would give 48 workgroups for the QKV product at
// M = 128; the partials stay within 1024 rows of 6144 floats.
constexpr int SPLITK_MAX_M = 64;
constexpr int SPLITK = 4;
constexpr int SPLITK_MID_M = 256;
constexpr int GEMM_CUS = 256;   // CUs a launch is sized for (MI355X)

// K slices of the split reduction for M tokens (0: not split)
inline int splitk_slices(int M) {
  return M <= SPLITK_MID_M ? SPLITK : 0;
}

size_t gemm_splitk_bytes(int M) {
  return (size_t)splitk_slices(M) * M * N_QKV * sizeof(float);
}

// Products with 4096 fp32 output features (W_O, the MLP's down product), by M:
// split K with a workspace at M <= 64; 128x128 tiles to M = 1024; 128-token x
// 256-feature tiles of 8 waves below M = 4096 (one workgroup per CU at M = 2048;
// 3-10 % faster there than 128x128); 256x256 from M = 4096 (one per CU there:
// 1121 vs 960 TFLOP/s).
static hipError_t launch_fp32_out(GemmArgs a, float* splitk, hipStream_t s) {
  const int M = a.M;
  if (M <= SPLITK_MAX_M && splitk) return launch_gemm_splitk<64, 64, 2, 2, 4, SPLITK>(a, splitk, s);
  if (M <= 128 && splitk) return launch_gemm_splitk<128, 64, 2, 2, 4, SPLITK>(a, splitk, s);
  if (M <= SPLITK_MID_M && splitk) return launch_gemm_splitk<128, 128, 2, 2, 3, 4>(a, splitk, s);
  if (M <= 64) return launch_gemm<64, 32, 2, 1, 8, EPI_OUT_F32>(a, s);
  if (M <= 1024) return launch_gemm<128, 128, 2, 2, 2, EPI_OUT_F32>(a, s);
  if (M < 4096) return launch_gemm<128, 256, 2, 4, 2, EPI_OUT_F32>(a, s);
  return launch_gemm<256, 256, 2, 4, 2, EPI_OUT_F32>(a, s);
}

hipError_t launch_qkv_rope(const uint16_t* x, const uint16_t* wq, const uint16_t* wk,
                           const uint16_t* wv, const float* rope, int M, int T,
                           uint16_t* q_dst, long long q_bstride, long long q_rstride,
                           uint16_t* k_dst, uint16_t* v_dst, long long kv_bstride,
                           long long kv_rstride, float* splitk, float q_scale, hipStream_t s) {
  GemmArgs a{};
  a.act = x; a.w0 = wq; a.w1 = wk; a.w2 = wv; a.M = M; a.N = N_QKV; a.K = D_MODEL;
  a.rope = rope; a.T = T; a.q_scale = q_scale;
  a.q_dst = q_dst; a.q_bstride = q_bstride; a.q_rstride = q_rstride;
  a.k_dst = k_dst; a.v_dst = v_dst; a.kv_bstride = kv_bstride; a.kv_rstride = kv_rstride;
  // Few tokens (decode): split K with a workspace, else thin weight strips and a
  // deep load ring; otherwise the largest tile that still fills the chip.
  if (M <= SPLITK_MAX_M && splitk) return launch_gemm_splitk<64, 128, 2, 2, 4, SPLITK>(a, splitk, s);
  if (M <= 128 && splitk) return launch_gemm_splitk<128, 64, 2, 2, 4, SPLITK>(a, splitk, s);
  if (M <= SPLITK_MID_M && splitk) return launch_gemm_splitk<128, 128, 2, 2, 3, 4>(a, splitk, s);
  if (M <= 64) return launch_gemm<64, 32, 1, 2, 8, EPI_QKV_ROPE>(a, s);
  if (M <= 1024) return launch_gemm<128, 128, 2, 2, 2, EPI_QKV_ROPE>(a, s);
  // 192-wide feature tiles: 256 tokens x 192 features give exactly one
  // workgroup of 8 waves per CU at M = 2048 (4-5 % faster there and at M = 4096
  // than two workgroups of 128 x 192 per CU); 256x256 tiles would leave 192
  // workgroups at M = 2048. From M = 8192 on 256x256 tiles are faster (1170 vs
  // 1080 TFLOP/s at M = 32768).
  if (M < 2048) return launch_gemm<128, 192, 2, 2, 2, EPI_QKV_ROPE>(a, s);
  if (M <= 4096) return launch_gemm<256, 192, 2, 4, 2, EPI_QKV_ROPE>(a, s);
  return launch_gemm<256, 256, 4, 2, 2, EPI_QKV_ROPE>(a, s);
}

hipError_t launch_out_proj(const uint16_t* h, const uint16_t* wo, int M, float* out,
                           const uint16_t* resid, float* splitk, hipStream_t s) {
  GemmArgs a{};
  a.act = h; a.w0 = wo; a.M = M; a.N = D_MODEL; a.K = D_MODEL; a.out = out; a.T = 1;
  a.resid = resid;
  return launch_fp32_out(a, splitk, s);
}

size_t gemm_mlp_splitk_bytes(int M) {
  return M <= SPLITK_MAX_M ? (size_t)SPLITK * M * D_MODEL * sizeof(float) : 0;
}

hipError_t launch_mlp_gate_up(const uint16_t* x, const uint16_t* w1, const uint16_t* w3, int M,
                              uint16_t* a_out, hipStream_t s) {
  GemmArgs a{};
  a.act = x; a.w0 = w1; a.w1 = w3; a.M = M; a.N = 2 * D_FF; a.K = D_MODEL; a.glu_out = a_out;
  a.T = 1;
  // 2 x 14336 features give enough workgroups at any M without splitting K. At
  // M <= 64 the product streams weights: a 4-stage ring (48 KiB of LDS) lets
  // several workgroups share a CU, which moves them faster (35.7 us for the
  // 235 MB of w1 and w3) than a deeper ring at one workgroup per CU (57 us).
  if (M <= 64) return launch_gemm<64, 64, 1, 2, 4, EPI_SWIGLU>(a, s);
  if (M <= 1024) return launch_gemm<128, 128, 2, 2, 2, EPI_SWIGLU>(a, s);
  // 256x256 tiles (about a fifth faster than 128x256 at M = 2048). Their
  // 112 feature tiles per token tile would leave a last, partial round of
  // workgroups on the CUs (896 tiles at M = 2048: 3.5 rounds on 256 CUs, the
  // last one on half of them); the features that do not make whole rounds go
  // to a second launch of 256x128 tiles, twice as many workgroups of half
  // the work.
  const int tok_tiles = (M + 255) / 256;
  int full = 112;
  if (tok_tiles * 112 > GEMM_CUS) {
    full = (tok_tiles * 112 / GEMM_CUS) * GEMM_CUS / tok_tiles;
    if (full * tok_tiles % GEMM_CUS != 0) full = 112;   // whole rounds only
  }
  if (full == 112) return launch_gemm<256, 256, 4, 2, 2, EPI_SWIGLU>(a, s);
  a.n_off = 0; a.n_len = full * 256;
  hipError_t e = launch_gemm<256, 256, 4, 2, 2, EPI_SWIGLU>(a, s);
  if (e != hipSuccess) return e;
  a.n_off = full * 256; a.n_len = 2 * D_FF - full * 256;
  return launch_gemm<256, 128, 2, 4, 2, EPI_SWIGLU>(a, s);
}

hipError_t launch_mlp_down(const uint16_t* act, const uint16_t* w2, int M, float* out,
                           const uint16_t* resid, float* splitk, hipStream_t s) {
  GemmArgs a{};
  a.act = act; a.w0 = w2; a.M = M; a.N = D_MODEL; a.K = D_FF; a.out = out; a.T = 1;
  a.resid = resid;
  // K = 14336 makes every workgroup 3.5x longer than for W_O: at M = 2048 the
  // 512 workgroups of 128x128 beat 128x256 tiles (221 vs 240 us); from M = 8192
  // on, 256x256
  if (M > SPLITK_MAX_M && M <= 4096) return launch_gemm<128, 128, 2, 2, 2, EPI_OUT_F32>(a, s);
  return launch_fp32_out(a, splitk, s);
}

}  // namespace gqa

// Projection GEMMs of the GQA block on bf16 MFMA (gfx950).
//
//  * qkv_rope: [Q | K | V] = x · [W_Q; W_K; W_V]ᵀ over the fused 6144 output
//    columns (Grouped-query attention page, "All 13 steps", the three
//    projection equations; weights stored [out, in] per the Query projection
//    page), with the pair rotation of Q and K applied in the epilogue (the 2x2
//    rotation display) before the single rounding to bf16.
//  * out_proj: Δ = H · W_Oᵀ in fp32 (the last equation; Merge and project page).
//
// Both are "NT" products: each operand is contiguous along the 4096-long
// reduction axis. A workgroup of 4 waves computes a TOKxFEAT tile with a
// K step of 64; tiles of both operands are staged in LDS (double buffered,
// XOR-swizzled 16-byte chunks so fragment reads are bank-conflict free).
//
// For qkv_rope the MFMA "A" operand is the weight tile and "B" the token
// tile, so the accumulator holds features down its rows: a lane then owns 4
// consecutive features of one token, i.e. both members of two rotation
// pairs, and the rotation needs no cross-lane traffic.

#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {

constexpr int BK = 64;          // K step staged per iteration
constexpr int GEMM_THREADS = 256;

enum Epilogue { EPI_QKV_ROPE = 0, EPI_OUT_F32 = 1 };

struct GemmArgs {
  const uint16_t* act;   // [M][4096] bf16 activations
  const uint16_t* w0;    // weight rows [0, n0_rows)
  const uint16_t* w1;    // fused QKV: W_K rows; unused otherwise
  const uint16_t* w2;    // fused QKV: W_V rows
  int M;                 // tokens
  int N;                 // output features (6144 or 4096)
  // rotation epilogue
  const float* rope;     // [T][64][2]
  int T;                 // tokens per sequence (rope row = token % T)
  uint16_t* q_dst; long long q_bstride, q_rstride;     // elements
  uint16_t* k_dst; uint16_t* v_dst; long long kv_bstride, kv_rstride;
  // fp32 epilogue
  float* out;            // [M][4096]
};

// LDS tile of R rows x 64 bf16: row r, 16-byte chunk c is stored at chunk c ^ (r & 7).
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 3); }

template <int ROWS>
__device__ __forceinline__ void load_tile(u32x4 (&reg)[ROWS * 8 / GEMM_THREADS],
                                          const uint16_t* base, int rows_valid, int k0, int tid) {
#pragma unroll
  for (int c = 0; c < ROWS * 8 / GEMM_THREADS; ++c) {
    int idx = c * GEMM_THREADS + tid;
    int r = idx >> 3, ch = idx & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < rows_valid) v = ld16(base + (size_t)r * D_MODEL + k0 + ch * 8);
    reg[c] = v;
  }
}

template <int ROWS>
__device__ __forceinline__ void store_tile(uint16_t* lds, const u32x4 (&reg)[ROWS * 8 / GEMM_THREADS],
                                           int tid) {
#pragma unroll
  for (int c = 0; c < ROWS * 8 / GEMM_THREADS; ++c) {
    int idx = c * GEMM_THREADS + tid;
    int r = idx >> 3, ch = idx & 7;
    st16(lds + swz(r, ch), reg[c]);
  }
}

// Maps a linear workgroup id to (token tile, feature tile): workgroups are
// dealt round-robin to the 8 XCDs, so ids are first regrouped so that each
// XCD owns a contiguous run of tiles, and runs are walked in groups of
// GROUP token tiles so concurrently resident tiles share operand rows in
// that XCD's L2.
__device__ __forceinline__ void tile_coords(int bid, int nwg, int tiles_tok, int tiles_feat,
                                            int& tt, int& tf) {
  constexpr int GROUP = 8;
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

template <int TOK, int FEAT, int EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_nt_kernel(GemmArgs a) {
  // P: MFMA A operand rows, Q: MFMA B operand rows.
  constexpr bool SWAP = (EPI == EPI_QKV_ROPE);
  constexpr int PR = SWAP ? FEAT : TOK;
  constexpr int QR = SWAP ? TOK : FEAT;
  constexpr int WP = PR / 2, WQ = QR / 2;
  constexpr int NP = WP / 32, NQ = WQ / 32;
  constexpr int LP = PR * BK, LQ = QR * BK;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (LP + LQ)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wp = wave >> 1, wq = wave & 1;

  const int tiles_tok = (a.M + TOK - 1) / TOK;
  const int tiles_feat = a.N / FEAT;
  int tt, tf;
  tile_coords(blockIdx.x, gridDim.x, tiles_tok, tiles_feat, tt, tf);
  const int m0 = tt * TOK;
  const int n0 = tf * FEAT;

  const uint16_t* wbase;
  if (EPI == EPI_QKV_ROPE) {
    wbase = n0 < D_MODEL ? a.w0 + (size_t)n0 * D_MODEL
          : n0 < D_MODEL + N_KV * D_HEAD ? a.w1 + (size_t)(n0 - D_MODEL) * D_MODEL
          : a.w2 + (size_t)(n0 - D_MODEL - N_KV * D_HEAD) * D_MODEL;
  } else {
    wbase = a.w0 + (size_t)n0 * D_MODEL;
  }
  const uint16_t* abase = a.act + (size_t)m0 * D_MODEL;
  const int tok_valid = a.M - m0;
  const uint16_t* pbase = SWAP ? wbase : abase;
  const uint16_t* qbase = SWAP ? abase : wbase;
  const int p_valid = SWAP ? PR : tok_valid;
  const int q_valid = SWAP ? tok_valid : QR;

  f32x16 acc[NP][NQ];
#pragma unroll
  for (int i = 0; i < NP; ++i)
#pragma unroll
    for (int j = 0; j < NQ; ++j) acc[i][j] = f32x16{};

  u32x4 preg[PR * 8 / GEMM_THREADS];
  u32x4 qreg[QR * 8 / GEMM_THREADS];

  load_tile<PR>(preg, pbase, p_valid, 0, tid);
  load_tile<QR>(qreg, qbase, q_valid, 0, tid);
  store_tile<PR>(smem, preg, tid);
  store_tile<QR>(smem + LP, qreg, tid);
  __syncthreads();

  constexpr int NK = D_MODEL / BK;
  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < NK; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < NK) {
      load_tile<PR>(preg, pbase, p_valid, (kt + 1) * BK, tid);
      load_tile<QR>(qreg, qbase, q_valid, (kt + 1) * BK, tid);
    }
    const uint16_t* sp = smem + cur * (LP + LQ);
    const uint16_t* sq = sp + LP;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      u32x4 af[NP], bf[NQ];
      const int ch = kk * 2 + lhalf;
#pragma unroll
      for (int i = 0; i < NP; ++i) af[i] = ld16(sp + swz(wp * WP + i * 32 + lrow, ch));
#pragma unroll
      for (int j = 0; j < NQ; ++j) bf[j] = ld16(sq + swz(wq * WQ + j * 32 + lrow, ch));
#pragma unroll
      for (int i = 0; i < NP; ++i)
#pragma unroll
        for (int j = 0; j < NQ; ++j) acc[i][j] = mfma_32x32x16(af[i], bf[j], acc[i][j]);
    }
    if (kt + 1 < NK) {
      uint16_t* dp = smem + (cur ^ 1) * (LP + LQ);
      store_tile<PR>(dp, preg, tid);
      store_tile<QR>(dp + LP, qreg, tid);
    }
    __syncthreads();
  }

  if (EPI == EPI_QKV_ROPE) {
    // acc[i][j][4g + e]: feature n0 + wp*WP + 32i + 8g + 4*lhalf + e, token m0 + wq*WQ + 32j + lrow.
    const int region = n0 < D_MODEL ? 0 : (n0 < D_MODEL + N_KV * D_HEAD ? 1 : 2);
    const int fbase = region == 0 ? 0 : (region == 1 ? D_MODEL : D_MODEL + N_KV * D_HEAD);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int tok = m0 + wq * WQ + j * 32 + lrow;
      if (tok >= a.M) continue;
      const int b = tok / a.T;
      const int t = tok - b * a.T;
      uint16_t* drow;
      if (region == 0) drow = a.q_dst + b * a.q_bstride + t * a.q_rstride;
      else drow = (region == 1 ? a.k_dst : a.v_dst) + b * a.kv_bstride + t * a.kv_rstride;
      const float* rrow = a.rope + (size_t)t * (2 * 64);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int f = n0 + wp * WP + i * 32 + 8 * g + 4 * lhalf - fbase;
          float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
          float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
          if (region != 2) {
            // pairs (f, f+1) and (f+2, f+3) of head f/128: pair index (f % 128)/2
            const f32x4 cs = *reinterpret_cast<const f32x4*>(rrow + (f & (D_HEAD - 1)));
            const float r0 = v0 * cs[0] - v1 * cs[1];
            const float r1 = v0 * cs[1] + v1 * cs[0];
            const float r2 = v2 * cs[2] - v3 * cs[3];
            const float r3 = v2 * cs[3] + v3 * cs[2];
            v0 = r0; v1 = r1; v2 = r2; v3 = r3;
          }
          u32x2 w = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          *reinterpret_cast<u32x2*>(drow + f) = w;
        }
      }
    }
  } else {
    // acc[i][j][r]: token m0 + wp*WP + 32i + 8(r/4) + 4*lhalf + (r&3), feature n0 + wq*WQ + 32j + lrow.
#pragma unroll
    for (int i = 0; i < NP; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = m0 + wp * WP + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
        if (tok >= a.M) continue;
        float* orow = a.out + (size_t)tok * D_MODEL + n0 + wq * WQ + lrow;
#pragma unroll
        for (int j = 0; j < NQ; ++j) orow[j * 32] = acc[i][j][r];
      }
    }
  }
}

template <int TOK, int FEAT, int EPI>
static hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + TOK - 1) / TOK) * (a.N / FEAT);
  hipLaunchKernelGGL((gemm_nt_kernel<TOK, FEAT, EPI>), dim3(tiles), dim3(GEMM_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_qkv_rope(const uint16_t* x, const uint16_t* wq, const uint16_t* wk,
                           const uint16_t* wv, const float* rope, int M, int T,
                           uint16_t* q_dst, long long q_bstride, long long q_rstride,
                           uint16_t* k_dst, uint16_t* v_dst, long long kv_bstride,
                           long long kv_rstride, hipStream_t s) {
  GemmArgs a{};
  a.act = x; a.w0 = wq; a.w1 = wk; a.w2 = wv; a.M = M; a.N = N_QKV;
  a.rope = rope; a.T = T;
  a.q_dst = q_dst; a.q_bstride = q_bstride; a.q_rstride = q_rstride;
  a.k_dst = k_dst; a.v_dst = v_dst; a.kv_bstride = kv_bstride; a.kv_rstride = kv_rstride;
  return launch_gemm<128, 128, EPI_QKV_ROPE>(a, s);
}

hipError_t launch_out_proj(const uint16_t* h, const uint16_t* wo, int M, float* out,
                           hipStream_t s) {
  GemmArgs a{};
  a.act = h; a.w0 = wo; a.M = M; a.N = D_MODEL; a.out = out; a.T = 1;
  return launch_gemm<128, 128, EPI_OUT_F32>(a, s);
}

}  // namespace gqa

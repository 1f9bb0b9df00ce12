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
// 32 of the 64 positions. Every 64-key tile of K_r and V is staged in LDS
// once and used by all four heads of the group. Scores are computed
// transposed (keys down the MFMA rows, queries across the lanes), so each lane
// owns one query: the running max and sum need only in-lane work plus one
// swap with the lane 32 away, and the bf16 probabilities feed the P·V MFMA
// straight from the score accumulator. V is transposed into LDS while being
// staged, with the key order inside each 16-key group permuted to match the
// accumulator layout. The softmax is the online (running max / running sum)
// form in base 2 with log2(e)/sqrt(128) folded into one multiply-add; the
// division by the row sum happens once, at the end, in fp32.
//
// Decode (decode_splitkv_kernel + decode_merge_kernel): the key range of each
// (sequence, KV head) is split into chunks of 512 keys; a workgroup of 4 waves
// takes one chunk (128 keys per wave) for the 4 query heads of the group,
// combines its waves in LDS, and writes an unnormalised partial (max, sum,
// O[4][128]); the merge kernel rescales and sums the partials.

#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {

constexpr float LOG2E = 1.4426950408889634f;
// log2(e) / sqrt(128): one multiply turns a raw score into the base-2 exponent.
constexpr float SCALE_LOG2 = 0.12751743082459868f;
constexpr float SQRT_DH = 11.313708498984761f;
constexpr float NEG_INF = -__builtin_inff();

// ----------------------------------------------------------------------------
// Prefill
// ----------------------------------------------------------------------------

constexpr int FA_BQ = 64;       // query positions per workgroup
constexpr int FA_BN = 64;       // keys per staged tile
constexpr int FA_THREADS = 512;

// K tile: [64 keys][128 d]; 16-byte chunk c of key k at chunk c ^ (k & 15).
__device__ __forceinline__ int k_off(int key, int c) { return key * D_HEAD + ((c ^ (key & 15)) << 3); }
// V^T tile: [128 d][64 key slots]; chunk c (8 slots) of row d at c ^ vsw(d).
__device__ __forceinline__ int vsw(int d) { return (d & 7) ^ ((d >> 3) & 7); }
__device__ __forceinline__ int vt_off(int d, int c) { return d * FA_BN + ((c ^ vsw(d)) << 3); }
// Slot of key offset ko (0..15) inside its 16-key group: swaps keys 4..7 and 8..11
// so that slot 8u + e holds key 8(e>>2) + 4u + (e&3), the key a lane of the
// score accumulator holds in register e of that group.
__device__ __forceinline__ int vslot(int ko) { return (((ko >> 2) & 1) << 3) | ((ko >> 3) << 2) | (ko & 3); }

struct FlashArgs {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  long long kv_bstride;
  const float* mask;     // [T][kv_len] or null
  uint16_t* h;
  int B, T, kv_len, q_pos0, causal, n_qtiles;
};

__global__ __launch_bounds__(FA_THREADS) void flash_fwd_kernel(FlashArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][FA_BN * D_HEAD];
  __shared__ __attribute__((aligned(16))) uint16_t sv[2][D_HEAD * FA_BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int g = blockIdx.x & (N_KV - 1);
  const int rest = blockIdx.x >> 3;
  const int b = rest % a.B;
  const int qt = a.causal ? (a.n_qtiles - 1 - rest / a.B) : (rest / a.B);
  const int q0 = qt * FA_BQ;
  const int h = g * N_REP + (wave & 3);
  const int qi = q0 + (wave >> 2) * 32 + lrow;        // this lane's query index
  const int qpos = a.q_pos0 + qi;

  const uint16_t* kb = a.k + b * a.kv_bstride + g * D_HEAD;
  const uint16_t* vb = a.v + b * a.kv_bstride + g * D_HEAD;

  // Query fragments (MFMA B operand): k-step s covers d = 16s + 8*lhalf .. +7.
  u32x4 qf[8];
  {
    const bool ok = qi < a.T;
    const uint16_t* qrow = a.q + ((size_t)(b * a.T + (ok ? qi : 0)) * N_HEADS + h) * D_HEAD + 8 * lhalf;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[s] = ok ? ld16(qrow + 16 * s) : z;
    }
  }

  int kv_end = a.kv_len;
  if (a.causal) kv_end = min(kv_end, a.q_pos0 + q0 + FA_BQ);
  const int n_tiles = (kv_end + FA_BN - 1) / FA_BN;

  // staging: K chunk (key kk, chunk kc) and a V key pair (2*vp, 2*vp+1) x chunk vc
  u32x4 kr[2], vr[2];
  auto gload = [&](int t) {
    const int base = t * FA_BN;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = c * FA_THREADS + tid;
      const int key = idx >> 4, ch = idx & 15;
      u32x4 z = {0u, 0u, 0u, 0u};
      kr[c] = (base + key < a.kv_len) ? ld16(kb + (size_t)(base + key) * (N_KV * D_HEAD) + ch * 8) : z;
    }
    const int vp = tid >> 4, vc = tid & 15;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int key = base + 2 * vp + c;
      u32x4 z = {0u, 0u, 0u, 0u};
      vr[c] = (key < a.kv_len) ? ld16(vb + (size_t)key * (N_KV * D_HEAD) + vc * 8) : z;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = c * FA_THREADS + tid;
      const int key = idx >> 4, ch = idx & 15;
      st16(&sk[buf][k_off(key, ch)], kr[c]);
    }
    const int vp = tid >> 4, vc = tid & 15;
    const int key = 2 * vp;
    const int slot = (key & ~15) | vslot(key & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wa = vr[0][e >> 1];
      const uint32_t wb = vr[1][e >> 1];
      const uint32_t w = (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
      const int d = vc * 8 + e;
      *reinterpret_cast<uint32_t*>(&sv[buf][d * FA_BN + (((slot >> 3) ^ vsw(d)) << 3) + (slot & 7)]) = w;
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_run = NEG_INF;   // running max, raw-score units
  float l_run = 0.f;       // this lane's share of the running sum

  const bool has_mask = a.mask != nullptr;
  const float* mrow = has_mask ? a.mask + (size_t)(qi < a.T ? qi : 0) * a.kv_len : nullptr;

  gload(0);
  sstore(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < n_tiles) gload(t + 1);
    const int k0 = t * FA_BN;

    // S^T for two 32-key blocks: lane holds query lrow, keys 32kb + 8(i>>2) + 4*lhalf + (i&3)
    f32x16 s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      s[kb2] = f32x16{};
      const int key = kb2 * 32 + lrow;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 kf = ld16(&sk[cur][k_off(key, 2 * st + lhalf)]);
        s[kb2] = mfma_32x32x16(kf, qf[st], s[kb2]);
      }
    }

    const bool edge = (a.causal && (k0 + FA_BN - 1 > a.q_pos0 + q0)) || (k0 + FA_BN > a.kv_len) || has_mask;
    if (edge) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kg = k0 + kb2 * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
          float x = s[kb2][i];
          if (has_mask && kg < a.kv_len && qi < a.T) x += mrow[kg] * SQRT_DH;
          if (kg >= a.kv_len || (a.causal && kg > qpos)) x = NEG_INF;
          s[kb2][i] = x;
        }
    }

    float mx = NEG_INF;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb2][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * SCALE_LOG2);
    m_run = m_new;
    const float moff = -m_use * SCALE_LOG2;

    float lsum = 0.f;
    u32x4 pf[4];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][8 * hf + e], SCALE_LOG2, moff));
          lsum += p[e];
        }
        pf[kb2 * 2 + hf] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                 pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

    // O^T[d][q] += V^T[d][keys] · P^T[keys][q]; k-step sg covers slots 16sg .. 16sg+15
#pragma unroll
    for (int sg = 0; sg < 4; ++sg)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + lrow;
        const u32x4 vf = ld16(&sv[cur][vt_off(d, 2 * sg + lhalf)]);
        o[db] = mfma_32x32x16(vf, pf[sg], o[db]);
      }

    if (t + 1 < n_tiles) sstore(cur ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
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

hipError_t launch_flash_attention(const uint16_t* q_r, const uint16_t* k, const uint16_t* v,
                                  long long kv_bstride, const float* mask, int causal, int B,
                                  int T, int kv_len, int q_pos0, uint16_t* h_out,
                                  hipStream_t s) {
  FlashArgs a{};
  a.q = q_r; a.k = k; a.v = v; a.kv_bstride = kv_bstride; a.mask = mask; a.h = h_out;
  a.B = B; a.T = T; a.kv_len = kv_len; a.q_pos0 = q_pos0; a.causal = causal;
  a.n_qtiles = (T + FA_BQ - 1) / FA_BQ;
  const long long grid = (long long)a.n_qtiles * B * N_KV;
  hipLaunchKernelGGL(flash_fwd_kernel, dim3((unsigned)grid), dim3(FA_THREADS), 0, s, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Decode
// ----------------------------------------------------------------------------

constexpr int DC_CHUNK = 512;    // keys per workgroup
constexpr int DC_WKEYS = 128;    // keys per wave
constexpr int DC_THREADS = 256;
constexpr int DC_PART = N_REP * D_HEAD + 2 * N_REP;   // floats per partial: O[4][128], m[4], l[4]

// Per-wave V^T block: [128 d][32 slots]; 16-byte chunk u of row d at u ^ ((d >> 1) & 3).
__device__ __forceinline__ int dvt_off(int d, int u) { return d * 32 + ((u ^ ((d >> 1) & 3)) << 3); }

// Orders this wave's LDS writes before its later LDS reads (and vice versa)
// across lanes, without involving the other waves of the workgroup.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct DecodeArgs {
  const uint16_t* q; const uint16_t* kc; const uint16_t* vc;
  float* part; uint16_t* h;
  int B, S_max, kv_len, n_split;
};

__global__ __launch_bounds__(DC_THREADS) void decode_splitkv_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t svt[4][D_HEAD * 32];
  __shared__ float s_o[4][N_REP][D_HEAD];
  __shared__ float s_ml[4][2][N_REP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int g = blockIdx.x & (N_KV - 1);
  const int rest = blockIdx.x >> 3;
  const int sp = rest % a.n_split;
  const int b = rest / a.n_split;

  const size_t row_stride = N_KV * D_HEAD;
  const uint16_t* kbase = a.kc + (size_t)b * a.S_max * row_stride + g * D_HEAD;
  const uint16_t* vbase = a.vc + (size_t)b * a.S_max * row_stride + g * D_HEAD;

  // Query fragments (MFMA B operand, 16x16x32): column l16 = query head 4g + l16 (valid < 4),
  // k-step s covers d = 32s + 8*lg .. +7.
  u32x4 qf[4];
  {
    const bool ok = l16 < N_REP;
    const uint16_t* qrow = a.q + ((size_t)b * N_HEADS + g * N_REP + (ok ? l16 : 0)) * D_HEAD + 8 * lg;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[s] = ok ? ld16(qrow + 32 * s) : z;
    }
  }

  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{};
  float m_run = NEG_INF, l_run = 0.f;

  const int wk0 = sp * DC_CHUNK + wave * DC_WKEYS;
  uint16_t* vt = svt[wave];

  for (int blk = 0; blk < DC_WKEYS / 32; ++blk) {
    const int kbeg = wk0 + blk * 32;
    if (kbeg >= a.kv_len) break;                      // wave-uniform
    // K fragments: sub-block kb2 (16 keys), k-step s: key kbeg + 16kb2 + l16, chunk 4s + lg
    u32x4 kf[2][4];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int key = kbeg + 16 * kb2 + l16;
      const bool ok = key < a.kv_len;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 z = {0u, 0u, 0u, 0u};
        kf[kb2][s] = ok ? ld16(kbase + (size_t)key * row_stride + 32 * s + 8 * lg) : z;
      }
    }
    // V rows: load j = 4r + c covers key kbeg + 16r + 4lg + c, chunk l16
    u32x4 vr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = kbeg + 16 * (j >> 2) + 4 * lg + (j & 3);
      u32x4 z = {0u, 0u, 0u, 0u};
      vr[j] = key < a.kv_len ? ld16(vbase + (size_t)key * row_stride + 8 * l16) : z;
    }

    f32x4 sacc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sacc[kb2] = f32x4{};
#pragma unroll
      for (int s = 0; s < 4; ++s) sacc[kb2] = mfma_16x16x32(kf[kb2][s], qf[s], sacc[kb2]);
    }
    // lane holds query l16, keys kbeg + 16kb2 + 4lg + i
    float mx = NEG_INF;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kbeg + 16 * kb2 + 4 * lg + i;
        if (key >= a.kv_len) sacc[kb2][i] = NEG_INF;
        mx = fmaxf(mx, sacc[kb2][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);              // finite: key kbeg is valid
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * SCALE_LOG2);
    m_run = m_new;
    const float moff = -m_new * SCALE_LOG2;
    float p[8];
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e >> 2][e & 3], SCALE_LOG2, moff));
      lsum += p[e];
    }
    l_run = l_run * alpha + lsum;
    // P^T fragment: slot 8lg + e holds key 16(e>>2) + 4lg + (e&3)
    const u32x4 pf = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                      pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};

    // V^T into this wave's LDS block: key 16r + 4lg + c -> slot 8lg + 4r + c
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = vr[4 * r + 0][e >> 1], w1 = vr[4 * r + 1][e >> 1];
        const uint32_t w2 = vr[4 * r + 2][e >> 1], w3 = vr[4 * r + 3][e >> 1];
        u32x2 w;
        if (e & 1) {
          w[0] = (w0 >> 16) | (w1 & 0xffff0000u);
          w[1] = (w2 >> 16) | (w3 & 0xffff0000u);
        } else {
          w[0] = (w0 & 0xffffu) | (w1 << 16);
          w[1] = (w2 & 0xffffu) | (w3 << 16);
        }
        const int d = 8 * l16 + e;
        *reinterpret_cast<u32x2*>(vt + dvt_off(d, lg) + 4 * r) = w;
      }
    wave_lds_sync();   // the transposed block is written by other lanes of this wave

#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x4 vf = ld16(vt + dvt_off(16 * db + l16, lg));
      o[db] = mfma_16x16x32(vf, pf, o[db]);
    }
    wave_lds_sync();   // all reads of the block done before the next block overwrites it
  }

  // wave totals: sum over the 4 lane groups
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  // o[db][i]: query l16, d = 16db + 4lg + i
  if (l16 < N_REP) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[wave][l16][16 * db + 4 * lg + i] = o[db][i];
    if (lg == 0) { s_ml[wave][0][l16] = m_run; s_ml[wave][1][l16] = l_run; }
  }
  __syncthreads();

  float* part = a.part + ((size_t)(b * N_KV + g) * a.n_split + sp) * DC_PART;
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int idx = rep * DC_THREADS + tid;        // 0..511 = query * 128 + d
    const int q = idx >> 7, d = idx & 127;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_ml[w][0][q]);
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_ml[w][0][q];
      const float f = mw == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((mw - M) * SCALE_LOG2);
      acc += s_o[w][q][d] * f;
      L += s_ml[w][1][q] * f;
    }
    part[q * D_HEAD + d] = acc;
    if (d == 0) { part[N_REP * D_HEAD + q] = M; part[N_REP * D_HEAD + N_REP + q] = L; }
  }
}

// One workgroup per (sequence, query head): rescale and sum the split partials.
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeArgs a) {
  const int b = blockIdx.x / N_HEADS, h = blockIdx.x % N_HEADS;
  const int g = h / N_REP, q = h % N_REP;
  const int d = threadIdx.x;
  const float* base = a.part + (size_t)(b * N_KV + g) * a.n_split * DC_PART;
  float M = NEG_INF;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, base[s * DC_PART + N_REP * D_HEAD + q]);
  float acc = 0.f, L = 0.f;
  for (int s = 0; s < a.n_split; ++s) {
    const float* p = base + s * DC_PART;
    const float ms = p[N_REP * D_HEAD + q];
    const float f = ms == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((ms - M) * SCALE_LOG2);
    acc += p[q * D_HEAD + d] * f;
    L += p[N_REP * D_HEAD + N_REP + q] * f;
  }
  const float r = L > 0.f ? acc / L : 0.f;
  f32x2 v = {r, 0.f};
  bf16x2 bv = __builtin_convertvector(v, bf16x2);
  a.h[((size_t)b * N_HEADS + h) * D_HEAD + d] = (uint16_t)(__builtin_bit_cast(uint32_t, bv) & 0xffffu);
}

size_t decode_partials_bytes(int B, int S_max) {
  const size_t n_split = (size_t)(S_max + DC_CHUNK - 1) / DC_CHUNK;
  return (size_t)B * N_KV * n_split * DC_PART * sizeof(float);
}

hipError_t launch_decode_attention(const uint16_t* q_r, const uint16_t* k_cache,
                                   const uint16_t* v_cache, int B, int S_max, int kv_len,
                                   float* partials, uint16_t* h_out, hipStream_t s) {
  DecodeArgs a{};
  a.q = q_r; a.kc = k_cache; a.vc = v_cache; a.part = partials; a.h = h_out;
  a.B = B; a.S_max = S_max; a.kv_len = kv_len;
  a.n_split = (kv_len + DC_CHUNK - 1) / DC_CHUNK;
  const long long grid = (long long)B * N_KV * a.n_split;
  hipLaunchKernelGGL(decode_splitkv_kernel, dim3((unsigned)grid), dim3(DC_THREADS), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(B * N_HEADS)), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa

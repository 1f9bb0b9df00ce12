// C ABI of libgqa: argument validation (host only, before any HIP call),
// workspace carve-up, and the kernel sequence of each entry point.
// Semantics, layouts and error codes are documented in include/gqa.h.

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "gqa.h"
#include "gqa_device.h"
#include "gqa_launch.h"

namespace {

using gqa::D_HEAD;
using gqa::D_MODEL;
using gqa::N_HEADS;
using gqa::N_KV;

constexpr size_t KV_W = (size_t)N_KV * D_HEAD;  // 1024 features of K or V per token

inline size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }
inline bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// Prefill: Q_r, K_r, V, H (bf16), then one fp32 region shared, one kernel at a
// time, by the projections' split-reduction partials (M <= 64 tokens only) and
// the balanced causal attention's partials (few query tiles only).
struct PrefillWs {
  size_t q, k, v, h, part, total;
};

inline PrefillWs prefill_layout(int B, int T) {
  PrefillWs w{};
  const size_t m = (size_t)B * T;   // <= GQA_MAX_TOKENS
  w.q = 0;
  w.k = w.q + align_up(m * D_MODEL * 2);
  w.v = w.k + align_up(m * KV_W * 2);
  w.h = w.v + align_up(m * KV_W * 2);
  w.part = w.h + align_up(m * D_MODEL * 2);
  const size_t proj = gqa::gemm_splitk_bytes((int)m);
  // the causal plan's partials, or an explicit mask's tile classes
  const size_t plan = gqa::flash_partials_bytes(B, T, T, 0, 1);
  const size_t cls = gqa::flash_partials_bytes(B, T, T, 0, 0);
  const size_t attn = plan > cls ? plan : cls;
  w.total = w.part + align_up(proj > attn ? proj : attn);
  return w;
}

// Chunked prefill: Q_r, H (bf16; K_r and V go to the cache), then one fp32
// region for the split-K partials (M <= 64) or the balanced attention's partials.
struct ChunkWs {
  size_t q, h, part, total;
};

inline ChunkWs chunk_layout(int B, int T, int start_pos) {
  ChunkWs w{};
  const size_t m = (size_t)B * T;   // <= GQA_MAX_TOKENS
  w.q = 0;
  w.h = align_up(m * D_MODEL * 2);
  w.part = w.h + align_up(m * D_MODEL * 2);
  const size_t proj = gqa::gemm_splitk_bytes((int)m);
  const size_t attn = gqa::flash_partials_bytes(B, T, start_pos + T, start_pos, 1);
  w.total = w.part + align_up(proj > attn ? proj : attn);
  return w;
}

// Decode: Q_r, H (bf16), then one fp32 region shared, one kernel at a time, by
// the projections' split-reduction partials and the attention's split-KV partials.
struct DecodeWs {
  size_t q, h, part, total;
};

inline DecodeWs decode_layout(int B, int S_max) {
  DecodeWs w{};
  w.q = 0;
  w.h = align_up((size_t)B * D_MODEL * 2);
  w.part = w.h + align_up((size_t)B * D_MODEL * 2);
  const size_t attn = gqa::decode_partials_bytes(B, S_max);
  const size_t proj = gqa::gemm_splitk_bytes(B);
  w.total = w.part + align_up(attn > proj ? attn : proj);
  return w;
}

// SwiGLU MLP: x̂ (bf16, pre-norm form only), A = silu(gate)·up (bf16), then the
// down product's split-reduction partials (M <= 64 tokens only).
struct MlpWs {
  size_t xn, a, part, total;
};

inline MlpWs mlp_layout(int M) {
  MlpWs w{};
  w.xn = 0;
  w.a = align_up((size_t)M * D_MODEL * 2);
  w.part = w.a + align_up((size_t)M * gqa::D_FF * 2);
  w.total = w.part + align_up(gqa::gemm_mlp_splitk_bytes(M));
  return w;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ERR_HIP; }

inline bool tokens_ok(int B, int T) {
  return B >= 1 && T >= 1 && (long long)B * T <= GQA_MAX_TOKENS;
}

int check_weights(const gqa_bf16* wq, const gqa_bf16* wk, const gqa_bf16* wv,
                  const gqa_bf16* wo) {
  if (!wq || !wk || !wv || !wo) return GQA_ERR_NULL;
  if (misaligned(wq) || misaligned(wk) || misaligned(wv) || misaligned(wo)) return GQA_ERR_ALIGN;
  return GQA_OK;
}

// Pre-attention RMS normalisation and residual of the *_prenorm entries; a
// null gain means the plain block (no normalisation, out = Δ).
struct PreNorm {
  const gqa_bf16* gain;
  float eps;
};

int check_prenorm(const PreNorm& n) {
  if (!n.gain) return GQA_ERR_NULL;
  if (!(n.eps >= 0.f) || !std::isfinite(n.eps)) return GQA_ERR_ARG;
  if (misaligned(n.gain)) return GQA_ERR_ALIGN;
  return GQA_OK;
}

// With a gain: x̂ = RMSNorm(x) into `xn` (a workspace region the attention
// output overwrites later on the same stream) and the projections read x̂.
const gqa_bf16* norm_input(const PreNorm* n, const gqa_bf16* x, int M, gqa_bf16* xn,
                           hipStream_t s, hipError_t* e) {
  *e = hipSuccess;
  if (!n) return x;
  *e = gqa::launch_rmsnorm(x, n->gain, n->eps, M, xn, s);
  return xn;
}

int block_impl(const gqa_bf16* x, const PreNorm* norm, const gqa_bf16* w_q,
               const gqa_bf16* w_k, const gqa_bf16* w_v, const gqa_bf16* w_o,
               const float* rope, const float* mask, int causal, int B, int T, int kv_len,
               float* out, gqa_bf16* h_out, void* workspace, size_t workspace_bytes,
               void* stream) {
  if (!x || !rope || !out) return GQA_ERR_NULL;
  int st = check_weights(w_q, w_k, w_v, w_o);
  if (st == GQA_OK && norm) st = check_prenorm(*norm);
  if (st != GQA_OK) return st;
  if (causal != 0 && causal != 1) return GQA_ERR_ARG;
  if (causal && mask) return GQA_ERR_ARG;
  if (!tokens_ok(B, T) || kv_len < 1) return GQA_ERR_SHAPE;
  if (kv_len != T) return GQA_ERR_UNSUPPORTED;
  if (misaligned(x) || misaligned(rope) || misaligned(out) || (mask && misaligned(mask)) ||
      (h_out && misaligned(h_out)))
    return GQA_ERR_ALIGN;
  const long long M = (long long)B * T;
  const PrefillWs L = prefill_layout(B, T);
  if (!workspace || workspace_bytes < L.total) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;

  char* ws = static_cast<char*>(workspace);
  auto* q = reinterpret_cast<gqa_bf16*>(ws + L.q);
  auto* k = reinterpret_cast<gqa_bf16*>(ws + L.k);
  auto* v = reinterpret_cast<gqa_bf16*>(ws + L.v);
  gqa_bf16* h = h_out ? h_out : reinterpret_cast<gqa_bf16*>(ws + L.h);
  float* part = L.total > L.part ? reinterpret_cast<float*>(ws + L.part) : nullptr;
  hipStream_t s = (hipStream_t)stream;

  hipError_t e;
  const gqa_bf16* xin =
      norm_input(norm, x, (int)M, reinterpret_cast<gqa_bf16*>(ws + L.h), s, &e);
  if (e != hipSuccess) return GQA_ERR_HIP;
  // Q_r is stored pre-scaled by log2(e)/sqrt(128) for the attention (internal)
  e = gqa::launch_qkv_rope(xin, w_q, w_k, w_v, rope, (int)M, T, q,
                           (long long)T * D_MODEL, D_MODEL, k, v,
                           (long long)T * KV_W, KV_W, part, gqa::QK_SCALE_LOG2, s);
  if (e != hipSuccess) return GQA_ERR_HIP;
  e = gqa::launch_flash_attention(q, k, v, (long long)T * KV_W, mask, causal, B, T, kv_len, 0,
                                  h, part, true, s);
  if (e != hipSuccess) return GQA_ERR_HIP;
  return hip_status(gqa::launch_out_proj(h, w_o, (int)M, out, norm ? x : nullptr, part, s));
}

int chunk_impl(const gqa_bf16* x, const PreNorm* norm, const gqa_bf16* w_q,
               const gqa_bf16* w_k, const gqa_bf16* w_v, const gqa_bf16* w_o,
               const float* rope, gqa_bf16* k_cache, gqa_bf16* v_cache, int B, int T,
               int S_max, int start_pos, float* out, gqa_bf16* h_out, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (!x || !rope || !k_cache || !v_cache || !out) return GQA_ERR_NULL;
  int st = check_weights(w_q, w_k, w_v, w_o);
  if (st == GQA_OK && norm) st = check_prenorm(*norm);
  if (st != GQA_OK) return st;
  if (!tokens_ok(B, T) || S_max < 1 || start_pos < 0 || (long long)start_pos + T > S_max)
    return GQA_ERR_SHAPE;
  if (misaligned(x) || misaligned(rope) || misaligned(k_cache) || misaligned(v_cache) ||
      misaligned(out) || (h_out && misaligned(h_out)))
    return GQA_ERR_ALIGN;
  const ChunkWs L = chunk_layout(B, T, start_pos);
  if (!workspace || workspace_bytes < L.total) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;

  char* ws = static_cast<char*>(workspace);
  auto* q = reinterpret_cast<gqa_bf16*>(ws + L.q);
  gqa_bf16* h = h_out ? h_out : reinterpret_cast<gqa_bf16*>(ws + L.h);
  float* part = L.total > L.part ? reinterpret_cast<float*>(ws + L.part) : nullptr;
  hipStream_t s = (hipStream_t)stream;
  const long long M = (long long)B * T;
  const long long cache_bstride = (long long)S_max * KV_W;

  hipError_t e;
  const gqa_bf16* xin =
      norm_input(norm, x, (int)M, reinterpret_cast<gqa_bf16*>(ws + L.h), s, &e);
  if (e != hipSuccess) return GQA_ERR_HIP;
  // new keys and values go straight into cache slots start_pos .. start_pos+T-1
  e = gqa::launch_qkv_rope(xin, w_q, w_k, w_v, rope, (int)M, T, q,
                           (long long)T * D_MODEL, D_MODEL,
                           k_cache + (size_t)start_pos * KV_W,
                           v_cache + (size_t)start_pos * KV_W, cache_bstride, KV_W,
                           part, gqa::QK_SCALE_LOG2, s);
  if (e != hipSuccess) return GQA_ERR_HIP;
  e = gqa::launch_flash_attention(q, k_cache, v_cache, cache_bstride, nullptr, 1, B, T,
                                  start_pos + T, start_pos, h, part, true, s);
  if (e != hipSuccess) return GQA_ERR_HIP;
  return hip_status(gqa::launch_out_proj(h, w_o, (int)M, out, norm ? x : nullptr, part, s));
}

// Every argument check of a decode step except the workspace.
int decode_check(const gqa_bf16* x, const PreNorm* norm, const gqa_bf16* w_q,
                 const gqa_bf16* w_k, const gqa_bf16* w_v, const gqa_bf16* w_o,
                 const float* rope, const gqa_bf16* k_cache, const gqa_bf16* v_cache, int B,
                 int S_max, int start_pos, const float* out, const gqa_bf16* h_out) {
  if (!x || !rope || !k_cache || !v_cache || !out) return GQA_ERR_NULL;
  int st = check_weights(w_q, w_k, w_v, w_o);
  if (st == GQA_OK && norm) st = check_prenorm(*norm);
  if (st != GQA_OK) return st;
  if (B < 1 || B > GQA_MAX_TOKENS || S_max < 1 || start_pos < 0 || start_pos >= S_max)
    return GQA_ERR_SHAPE;
  if (misaligned(x) || misaligned(rope) || misaligned(k_cache) || misaligned(v_cache) ||
      misaligned(out) || (h_out && misaligned(h_out)))
    return GQA_ERR_ALIGN;
  return GQA_OK;
}

int decode_impl(const gqa_bf16* x, const PreNorm* norm, const gqa_bf16* w_q,
                const gqa_bf16* w_k, const gqa_bf16* w_v, const gqa_bf16* w_o,
                const float* rope, gqa_bf16* k_cache, gqa_bf16* v_cache, int B, int S_max,
                int start_pos, float* out, gqa_bf16* h_out, void* workspace,
                size_t workspace_bytes, void* stream) {
  const int st = decode_check(x, norm, w_q, w_k, w_v, w_o, rope, k_cache, v_cache, B, S_max,
                              start_pos, out, h_out);
  if (st != GQA_OK) return st;
  const DecodeWs L = decode_layout(B, S_max);
  if (!workspace || workspace_bytes < L.total) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;

  char* ws = static_cast<char*>(workspace);
  auto* q = reinterpret_cast<gqa_bf16*>(ws + L.q);
  gqa_bf16* h = h_out ? h_out : reinterpret_cast<gqa_bf16*>(ws + L.h);
  float* part = reinterpret_cast<float*>(ws + L.part);
  hipStream_t s = (hipStream_t)stream;
  const long long cache_bstride = (long long)S_max * KV_W;

  hipError_t e;
  const gqa_bf16* xin = norm_input(norm, x, B, reinterpret_cast<gqa_bf16*>(ws + L.h), s, &e);
  if (e != hipSuccess) return GQA_ERR_HIP;
  e = gqa::launch_qkv_rope(xin, w_q, w_k, w_v, rope, B, 1, q, D_MODEL, 0,
                           k_cache + (size_t)start_pos * KV_W,
                           v_cache + (size_t)start_pos * KV_W, cache_bstride, 0,
                           part, 1.0f, s);
  if (e != hipSuccess) return GQA_ERR_HIP;
  e = gqa::launch_decode_attention(q, k_cache, v_cache, B, S_max, start_pos + 1, part, h, s);
  if (e != hipSuccess) return GQA_ERR_HIP;
  return hip_status(gqa::launch_out_proj(h, w_o, B, out, norm ? x : nullptr, part, s));
}

int mlp_impl(const gqa_bf16* x, const PreNorm* norm, const gqa_bf16* w1, const gqa_bf16* w2,
             const gqa_bf16* w3, int M, float* out, gqa_bf16* a_out, void* workspace,
             size_t workspace_bytes, void* stream) {
  if (!x || !out || !w1 || !w2 || !w3) return GQA_ERR_NULL;
  if (norm) {
    const int st = check_prenorm(*norm);
    if (st != GQA_OK) return st;
  }
  if (M < 1 || M > GQA_MAX_TOKENS) return GQA_ERR_SHAPE;
  if (misaligned(x) || misaligned(out) || misaligned(w1) || misaligned(w2) || misaligned(w3) ||
      (a_out && misaligned(a_out)))
    return GQA_ERR_ALIGN;
  const MlpWs L = mlp_layout(M);
  if (!workspace || workspace_bytes < L.total) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;

  char* ws = static_cast<char*>(workspace);
  gqa_bf16* act = a_out ? a_out : reinterpret_cast<gqa_bf16*>(ws + L.a);
  float* part = L.total > L.part ? reinterpret_cast<float*>(ws + L.part) : nullptr;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  const gqa_bf16* xin = norm_input(norm, x, M, reinterpret_cast<gqa_bf16*>(ws + L.xn), s, &e);
  if (e != hipSuccess) return GQA_ERR_HIP;
  e = gqa::launch_mlp_gate_up(xin, w1, w3, M, act, s);
  if (e != hipSuccess) return GQA_ERR_HIP;
  return hip_status(gqa::launch_mlp_down(act, w2, M, out, norm ? x : nullptr, part, s));
}

// Device scratch of gqa_decode_forward_static: one array per GPU the library
// runs on, held until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device (with that device current), and only
// that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[GQA_STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void*> scratch_ptr[MAX_DEVICES];
std::mutex scratch_init;

// Device address of `scratch` on the current device, looked up on the first
// call for that device; null (with *err set) if the lookup fails.
void* scratch_address(hipError_t* err) {
  *err = hipSuccess;
  int dev = 0;
  if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= MAX_DEVICES) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(scratch_init);
  p = scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if ((*err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess || !p) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

const char* gqa_status_string(int s) {
  switch (s) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_NULL: return "GQA_ERR_NULL: a required pointer is NULL";
    case GQA_ERR_SHAPE: return "GQA_ERR_SHAPE: a size argument is out of range";
    case GQA_ERR_ALIGN: return "GQA_ERR_ALIGN: a device pointer is not 16-byte aligned";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace missing or too small";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED: request not implemented";
    case GQA_ERR_HIP: return "GQA_ERR_HIP: a HIP launch failed";
    case GQA_ERR_ARG: return "GQA_ERR_ARG: inconsistent arguments";
    case GQA_ERR_TOO_LARGE:
      return "GQA_ERR_TOO_LARGE: the request needs more scratch than the fixed device array of "
             "the no-allocation entry holds";
    default: return "GQA_ERR_UNKNOWN";
  }
}

void gqa_dims(int* d_model, int* n_heads, int* n_kv_heads, int* d_head) {
  if (d_model) *d_model = GQA_D_MODEL;
  if (n_heads) *n_heads = GQA_N_HEADS;
  if (n_kv_heads) *n_kv_heads = GQA_N_KV_HEADS;
  if (d_head) *d_head = GQA_D_HEAD;
}

int gqa_rope_table(const int32_t* positions, int n, double theta, float* table) {
  if (n < 0 || !(theta > 1.0)) return GQA_ERR_SHAPE;
  if (n == 0) return GQA_OK;
  if (!positions || !table) return GQA_ERR_NULL;
  double omega[GQA_N_PAIRS];
  for (int j = 0; j < GQA_N_PAIRS; ++j)
    omega[j] = std::exp(-(2.0 * j / (double)GQA_D_HEAD) * std::log(theta));
  return gqa_rope_table_freqs(positions, n, omega, table);
}

int gqa_rope_table_freqs(const int32_t* positions, int n, const double* omega, float* table) {
  if (n < 0) return GQA_ERR_SHAPE;
  if (!omega) return GQA_ERR_NULL;
  for (int j = 0; j < GQA_N_PAIRS; ++j)
    if (!std::isfinite(omega[j])) return GQA_ERR_ARG;
  if (n == 0) return GQA_OK;
  if (!positions || !table) return GQA_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    const double t = (double)positions[i];
    for (int j = 0; j < GQA_N_PAIRS; ++j) {
      const double ang = t * omega[j];
      table[(size_t)i * 2 * GQA_N_PAIRS + 2 * j] = (float)std::cos(ang);
      table[(size_t)i * 2 * GQA_N_PAIRS + 2 * j + 1] = (float)std::sin(ang);
    }
  }
  return GQA_OK;
}

size_t gqa_prefill_workspace_bytes(int B, int T) {
  if (!tokens_ok(B, T)) return 0;
  return prefill_layout(B, T).total;
}

size_t gqa_attention_workspace_bytes(int B, int T, int kv_len, int causal) {
  if (!tokens_ok(B, T) || kv_len != T || (causal != 0 && causal != 1)) return 0;
  return gqa::flash_partials_bytes(B, T, kv_len, 0, causal);
}

size_t gqa_chunk_workspace_bytes(int B, int T, int start_pos) {
  if (!tokens_ok(B, T) || start_pos < 0 || (long long)start_pos + T > (1LL << 30)) return 0;
  return chunk_layout(B, T, start_pos).total;
}

size_t gqa_decode_workspace_bytes(int B, int S_max) {
  if (B < 1 || S_max < 1) return 0;
  return decode_layout(B, S_max).total;
}

int gqa_qkv_rope(const gqa_bf16* x, const gqa_bf16* w_q, const gqa_bf16* w_k,
                 const gqa_bf16* w_v, const float* rope, int B, int T, gqa_bf16* q_r,
                 gqa_bf16* k_r, gqa_bf16* v, int q_scaled, void* stream) {
  if (!x || !rope || !q_r || !k_r || !v || !w_q || !w_k || !w_v) return GQA_ERR_NULL;
  if (q_scaled != 0 && q_scaled != 1) return GQA_ERR_ARG;
  if (!tokens_ok(B, T)) return GQA_ERR_SHAPE;
  if (misaligned(x) || misaligned(rope) || misaligned(q_r) || misaligned(k_r) ||
      misaligned(v) || misaligned(w_q) || misaligned(w_k) || misaligned(w_v))
    return GQA_ERR_ALIGN;
  const long long M = (long long)B * T;
  return hip_status(gqa::launch_qkv_rope(x, w_q, w_k, w_v, rope, (int)M, T, q_r,
                                         (long long)T * D_MODEL, D_MODEL, k_r, v,
                                         (long long)T * KV_W, KV_W, nullptr,
                                         q_scaled ? gqa::QK_SCALE_LOG2 : 1.0f,
                                         (hipStream_t)stream));
}

int gqa_attention(const gqa_bf16* q_r, const gqa_bf16* k_r, const gqa_bf16* v,
                  const float* mask, int causal, int B, int T, int kv_len, gqa_bf16* h_out,
                  void* workspace, size_t workspace_bytes, int q_scaled, void* stream) {
  if (!q_r || !k_r || !v || !h_out) return GQA_ERR_NULL;
  if (causal != 0 && causal != 1) return GQA_ERR_ARG;
  if (q_scaled != 0 && q_scaled != 1) return GQA_ERR_ARG;
  if (causal && mask) return GQA_ERR_ARG;
  if (!tokens_ok(B, T) || kv_len < 1) return GQA_ERR_SHAPE;
  if (kv_len != T) return GQA_ERR_UNSUPPORTED;
  if (misaligned(q_r) || misaligned(k_r) || misaligned(v) || misaligned(h_out) ||
      (mask && misaligned(mask)) || misaligned(workspace))
    return GQA_ERR_ALIGN;
  const size_t need = gqa::flash_partials_bytes(B, T, kv_len, 0, causal);
  if (workspace && workspace_bytes < need) return GQA_ERR_WORKSPACE;
  float* part = workspace && need ? static_cast<float*>(workspace) : nullptr;
  return hip_status(gqa::launch_flash_attention(q_r, k_r, v, (long long)kv_len * KV_W, mask,
                                                causal, B, T, kv_len, 0, h_out, part,
                                                q_scaled != 0, (hipStream_t)stream));
}

int gqa_output_projection(const gqa_bf16* h, const gqa_bf16* w_o, int M, float* out,
                          void* stream) {
  if (!h || !w_o || !out) return GQA_ERR_NULL;
  if (M < 1 || M > GQA_MAX_TOKENS) return GQA_ERR_SHAPE;
  if (misaligned(h) || misaligned(w_o) || misaligned(out)) return GQA_ERR_ALIGN;
  return hip_status(gqa::launch_out_proj(h, w_o, M, out, nullptr, nullptr, (hipStream_t)stream));
}

int gqa_decode_attention(const gqa_bf16* q_r, const gqa_bf16* k_cache,
                         const gqa_bf16* v_cache, int B, int S_max, int kv_len,
                         gqa_bf16* h_out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!q_r || !k_cache || !v_cache || !h_out) return GQA_ERR_NULL;
  if (B < 1 || B > GQA_MAX_TOKENS || S_max < 1 || kv_len < 1 || kv_len > S_max)
    return GQA_ERR_SHAPE;
  if (misaligned(q_r) || misaligned(k_cache) || misaligned(v_cache) || misaligned(h_out))
    return GQA_ERR_ALIGN;
  const DecodeWs L = decode_layout(B, S_max);
  if (!workspace || workspace_bytes < L.total) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GQA_ERR_ALIGN;
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.part);
  return hip_status(gqa::launch_decode_attention(q_r, k_cache, v_cache, B, S_max, kv_len, part,
                                                 h_out, (hipStream_t)stream));
}

int gqa_block_forward(const gqa_bf16* x, const gqa_bf16* w_q, const gqa_bf16* w_k,
                      const gqa_bf16* w_v, const gqa_bf16* w_o, const float* rope,
                      const float* mask, int causal, int B, int T, int kv_len, float* out,
                      gqa_bf16* h_out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return block_impl(x, nullptr, w_q, w_k, w_v, w_o, rope, mask, causal, B, T, kv_len, out,
                    h_out, workspace, workspace_bytes, stream);
}

int gqa_block_forward_prenorm(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                              const gqa_bf16* w_q, const gqa_bf16* w_k, const gqa_bf16* w_v,
                              const gqa_bf16* w_o, const float* rope, const float* mask,
                              int causal, int B, int T, int kv_len, float* out,
                              gqa_bf16* h_out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const PreNorm n{norm_w, eps};
  return block_impl(x, &n, w_q, w_k, w_v, w_o, rope, mask, causal, B, T, kv_len, out, h_out,
                    workspace, workspace_bytes, stream);
}

int gqa_chunk_forward(const gqa_bf16* x, const gqa_bf16* w_q, const gqa_bf16* w_k,
                      const gqa_bf16* w_v, const gqa_bf16* w_o, const float* rope,
                      gqa_bf16* k_cache, gqa_bf16* v_cache, int B, int T, int S_max,
                      int start_pos, float* out, gqa_bf16* h_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return chunk_impl(x, nullptr, w_q, w_k, w_v, w_o, rope, k_cache, v_cache, B, T, S_max,
                    start_pos, out, h_out, workspace, workspace_bytes, stream);
}

int gqa_chunk_forward_prenorm(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                              const gqa_bf16* w_q, const gqa_bf16* w_k, const gqa_bf16* w_v,
                              const gqa_bf16* w_o, const float* rope, gqa_bf16* k_cache,
                              gqa_bf16* v_cache, int B, int T, int S_max, int start_pos,
                              float* out, gqa_bf16* h_out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const PreNorm n{norm_w, eps};
  return chunk_impl(x, &n, w_q, w_k, w_v, w_o, rope, k_cache, v_cache, B, T, S_max, start_pos,
                    out, h_out, workspace, workspace_bytes, stream);
}

int gqa_decode_forward(const gqa_bf16* x, const gqa_bf16* w_q, const gqa_bf16* w_k,
                       const gqa_bf16* w_v, const gqa_bf16* w_o, const float* rope,
                       gqa_bf16* k_cache, gqa_bf16* v_cache, int B, int S_max, int start_pos,
                       float* out, gqa_bf16* h_out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return decode_impl(x, nullptr, w_q, w_k, w_v, w_o, rope, k_cache, v_cache, B, S_max,
                     start_pos, out, h_out, workspace, workspace_bytes, stream);
}

int gqa_decode_forward_static(const gqa_bf16* x, const gqa_bf16* w_q, const gqa_bf16* w_k,
                              const gqa_bf16* w_v, const gqa_bf16* w_o, const float* rope,
                              gqa_bf16* k_cache, gqa_bf16* v_cache, int B, int S_max,
                              int start_pos, float* out, gqa_bf16* h_out, void* stream) {
  // every argument is checked before the first HIP call (the scratch lookup)
  const int st = decode_check(x, nullptr, w_q, w_k, w_v, w_o, rope, k_cache, v_cache, B, S_max,
                              start_pos, out, h_out);
  if (st != GQA_OK) return st;
  const size_t need = decode_layout(B, S_max).total;
  if (need > (size_t)GQA_STATIC_SCRATCH_BYTES) return GQA_ERR_TOO_LARGE;
  hipError_t e;
  void* ws = scratch_address(&e);
  if (!ws) return GQA_ERR_HIP;
  return decode_impl(x, nullptr, w_q, w_k, w_v, w_o, rope, k_cache, v_cache, B, S_max,
                     start_pos, out, h_out, ws, (size_t)GQA_STATIC_SCRATCH_BYTES, stream);
}

int gqa_decode_forward_prenorm(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                               const gqa_bf16* w_q, const gqa_bf16* w_k, const gqa_bf16* w_v,
                               const gqa_bf16* w_o, const float* rope, gqa_bf16* k_cache,
                               gqa_bf16* v_cache, int B, int S_max, int start_pos, float* out,
                               gqa_bf16* h_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const PreNorm n{norm_w, eps};
  return decode_impl(x, &n, w_q, w_k, w_v, w_o, rope, k_cache, v_cache, B, S_max, start_pos,
                     out, h_out, workspace, workspace_bytes, stream);
}

int gqa_rmsnorm(const gqa_bf16* x, const gqa_bf16* norm_w, float eps, int M, gqa_bf16* y,
                void* stream) {
  if (!x || !y) return GQA_ERR_NULL;
  if (M < 1 || M > GQA_MAX_TOKENS) return GQA_ERR_SHAPE;
  const PreNorm n{norm_w, eps};
  const int st = check_prenorm(n);
  if (st != GQA_OK) return st;
  if (misaligned(x) || misaligned(y)) return GQA_ERR_ALIGN;
  return hip_status(gqa::launch_rmsnorm(x, norm_w, eps, M, y, (hipStream_t)stream));
}

size_t gqa_mlp_workspace_bytes(int M) {
  if (M < 1 || M > GQA_MAX_TOKENS) return 0;
  return mlp_layout(M).total;
}

int gqa_mlp_forward(const gqa_bf16* x, const gqa_bf16* w1, const gqa_bf16* w2,
                    const gqa_bf16* w3, int M, float* out, gqa_bf16* a_out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return mlp_impl(x, nullptr, w1, w2, w3, M, out, a_out, workspace, workspace_bytes, stream);
}

int gqa_mlp_forward_prenorm(const gqa_bf16* h, const gqa_bf16* norm_w, float eps,
                            const gqa_bf16* w1, const gqa_bf16* w2, const gqa_bf16* w3, int M,
                            float* out, gqa_bf16* a_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  const PreNorm n{norm_w, eps};
  return mlp_impl(h, &n, w1, w2, w3, M, out, a_out, workspace, workspace_bytes, stream);
}

}  // extern "C"

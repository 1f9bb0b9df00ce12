// Internal launchers of libgqa (host side). Arguments are validated by the
// C ABI layer before any of these is called; these only enqueue kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// Fused Q/K/V projection + pair rotation over M tokens (T tokens per sequence;
// rope row = token % T). Destination of token m = b*T + t:
//   Q row: q_dst + b*q_bstride + t*q_rstride           (4096 elements)
//   K/V row: k_dst/v_dst + b*kv_bstride + t*kv_rstride  (1024 elements)
// `splitk` (may be null) is fp32 scratch of gemm_splitk_bytes(M) bytes: with
// it, M <= 256 products split the reduction across workgroups. The rotated Q
// features are multiplied by q_scale before their rounding (1: plain Q_r;
// QK_SCALE_LOG2: the form launch_flash_attention takes with q_scaled).
hipError_t launch_qkv_rope(const uint16_t* x, const uint16_t* wq, const uint16_t* wk,
                           const uint16_t* wv, const float* rope, int M, int T,
                           uint16_t* q_dst, long long q_bstride, long long q_rstride,
                           uint16_t* k_dst, uint16_t* v_dst, long long kv_bstride,
                           long long kv_rstride, float* splitk, float q_scale, hipStream_t s);

// out[M][4096] (fp32) = h[M][4096] · w_oᵀ (+ resid[M][4096] bf16 when not null);
// `splitk` as for launch_qkv_rope.
hipError_t launch_out_proj(const uint16_t* h, const uint16_t* wo, int M, float* out,
                           const uint16_t* resid, float* splitk, hipStream_t s);

// SwiGLU MLP: a[M][14336] (bf16) = silu(x·w1ᵀ)·(x·w3ᵀ), one fused product of
// x[M][4096] with w1, w3 [14336][4096]; then out[M][4096] (fp32) = a·w2ᵀ
// (w2 [4096][14336]) + resid (bf16, when not null). `splitk` (may be null) is
// fp32 scratch of gemm_mlp_splitk_bytes(M) bytes for M <= 64 (decode).
hipError_t launch_mlp_gate_up(const uint16_t* x, const uint16_t* w1, const uint16_t* w3, int M,
                              uint16_t* a_out, hipStream_t s);
hipError_t launch_mlp_down(const uint16_t* act, const uint16_t* w2, int M, float* out,
                           const uint16_t* resid, float* splitk, hipStream_t s);
size_t gemm_mlp_splitk_bytes(int M);

// y[M][4096] (bf16) = RMS normalisation of x[M][4096] rows with gain w[4096].
hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* w, float eps, int M, uint16_t* y,
                          hipStream_t s);

// Scratch bytes of the split-reduction path for M tokens (0 when M > 64).
size_t gemm_splitk_bytes(int M);

// Prefill grouped flash attention. q_r/h_out [B][T][32][128]; k/v rows of
// sequence b start at k + b*kv_bstride (row stride 1024 elements); query i is
// at position q_pos0 + i; keys 0..kv_len-1. `partials` (may be null: plain
// launch, every explicit-mask tile added element by element) is scratch of
// flash_partials_bytes(B, T, kv_len, q_pos0, causal) bytes: fp32 piece partials
// for the balanced causal launch of few query tiles, or (non-causal) a class
// byte per 64x64 tile of an explicit mask (rows of tiles padded to 4 bytes). q_scaled: the queries carry the
// factor QK_SCALE_LOG2 already (launch_qkv_rope's q_scale).
size_t flash_partials_bytes(int B, int T, int kv_len, int q_pos0, int causal);
hipError_t launch_flash_attention(const uint16_t* q_r, const uint16_t* k, const uint16_t* v,
                                  long long kv_bstride, const float* mask, int causal, int B,
                                  int T, int kv_len, int q_pos0, uint16_t* h_out,
                                  float* partials, bool q_scaled, hipStream_t s);

// Split-KV decode attention: q_r [B][32][128]; caches [B][S_max][8][128];
// keys 0..kv_len-1; h_out [B][32][128]. `partials` needs decode_partials_bytes.
size_t decode_partials_bytes(int B, int S_max);
hipError_t launch_decode_attention(const uint16_t* q_r, const uint16_t* k_cache,
                                   const uint16_t* v_cache, int B, int S_max, int kv_len,
                                   float* partials, uint16_t* h_out, hipStream_t s);

}  // namespace gqa

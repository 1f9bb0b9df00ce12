/*
 * gqa.h — C ABI of libgqa: forward pass of one Llama-3/3.1-8B grouped-query
 * attention block on an AMD Instinct MI355X (gfx950).
 *
 * The operation is the one on the OpenModelAtlas page "Llama 3.1 8B ·
 * Grouped-query attention", section "All 13 steps":
 *     Q = x·W_Q, K = x·W_K, V = x·W_V                (no bias; weights [out, in])
 *     Q_r, K_r = pair rotation of Q, K by the table R (adjacent pairs 2j, 2j+1)
 *     K_G[h] = K_r[floor(h/4)], V_G[h] = V[floor(h/4)]
 *     A = softmax(Q_r·K_Gᵀ / sqrt(128) + M)   over keys
 *     H = A·V_G, merged to [.., 32*128] with feature 128*h + d
 *     Δ = H·W_O
 * Dimensions are those of the page's header and parameter table and are fixed:
 * d = 4096, 32 query heads, 8 KV heads, head width 128, 64 rotation pairs.
 *
 * Conventions for every entry point below:
 *  - Device pointers point to HBM buffers the caller allocated and owns; they
 *    must be 16-byte aligned and hold contiguous row-major data in the stated
 *    layout. Host pointers are marked (host). The library never allocates,
 *    frees or synchronises; it enqueues kernels on `stream` (a hipStream_t;
 *    NULL is the default stream) and returns.
 *  - Outputs must not alias inputs.
 *  - bf16 values are passed as raw 16-bit patterns (gqa_bf16).
 *  - The return value is a gqa_status. Arguments are validated on the host
 *    before any HIP call; a rejected call launches nothing and writes
 *    nothing. GQA_ERR_HIP reports a failed launch. Faults inside a kernel
 *    surface at the caller's next synchronisation, not here.
 *  - Calls on one stream are ordered; apart from gqa_decode_forward_static
 *    (which holds one fixed device array per GPU, see there) the library
 *    keeps no mutable state, so calls on different streams with disjoint
 *    outputs and workspaces may run concurrently.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t gqa_bf16;

typedef enum {
  GQA_OK = 0,
  GQA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  GQA_ERR_SHAPE = 2,       /* B, T, kv_len, S_max or start_pos out of range      */
  GQA_ERR_ALIGN = 3,       /* a device pointer is not 16-byte aligned            */
  GQA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required          */
  GQA_ERR_UNSUPPORTED = 5, /* a valid request this build does not implement      */
  GQA_ERR_HIP = 6,         /* a HIP launch failed                                 */
  GQA_ERR_ARG = 7,         /* inconsistent flags (e.g. causal with a mask)       */
  GQA_ERR_TOO_LARGE = 8    /* more scratch than gqa_decode_forward_static holds   */
} gqa_status;

#define GQA_D_MODEL 4096
#define GQA_N_HEADS 32
#define GQA_N_KV_HEADS 8
#define GQA_D_HEAD 128
#define GQA_N_PAIRS 64
#define GQA_MAX_TOKENS (1 << 24) /* B*T limit of one call */
#define GQA_STATIC_SCRATCH_BYTES (32u << 20) /* device array of gqa_decode_forward_static */

/* Human-readable name of a status code. Never NULL. */
const char* gqa_status_string(int status);

/* Fills d_model, n_heads, n_kv_heads, d_head (any may be NULL). */
void gqa_dims(int* d_model, int* n_heads, int* n_kv_heads, int* d_head);

/*
 * Rotation table R for the given positions (host-side helper, no GPU call).
 * Grouped-query attention page, "All 13 steps", the pair rotation by the
 * angle t·ω_j; ω_j = theta^(-2j/128), theta = rope_theta of the catalogue
 * entry (500000 for Llama 3 / 3.1 8B).
 *   positions (host) [n]         position t of each row
 *   table     (host) [n][64][2]  out: (cos(t·ω_j), sin(t·ω_j)), computed in
 *                                double precision and stored as float
 * Returns GQA_ERR_NULL / GQA_ERR_SHAPE (n < 0, theta <= 1) or GQA_OK.
 */
int gqa_rope_table(const int32_t* positions, int n, double theta, float* table);

/*
 * Rotation table R from explicit per-pair frequencies (host-side helper, no
 * GPU call). The block takes R as an input (Grouped-query attention page,
 * in/out header) and the rotation in "All 13 steps" uses frequencies ω'_j:
 * callers whose frequencies are not theta^(-2j/128) (rescaled ones for long
 * contexts, as the 3.1 catalogue entry's use_scaled_rope flag asks for; the
 * rescaling rule itself is not on the pages) build their table here. The
 * kernels apply whatever table they are given.
 *   positions (host) [n], omega (host) [64] finite frequencies (rad/position)
 *   table     (host) [n][64][2]  out: (cos(t·omega_j), sin(t·omega_j)),
 *                                double precision, stored as float
 * Returns GQA_ERR_NULL / GQA_ERR_SHAPE (n < 0) / GQA_ERR_ARG (a non-finite
 * omega) or GQA_OK.
 */
int gqa_rope_table_freqs(const int32_t* positions, int n, const double* omega, float* table);

/* Workspace bytes gqa_block_forward needs for B sequences of T positions
 * (the bf16 Q_r, K_r, V and H of the step, plus the larger of the projections'
 * split-reduction partials and the attention stage's own workspace: the
 * causal plan's partials, or an explicit mask's tile classes). */
size_t gqa_prefill_workspace_bytes(int B, int T);

/*
 * Prefill: Δ for B sequences of T new positions each.
 * Grouped-query attention page, "All 13 steps" (all of them) and the in/out
 * header (x [B,T,4096], R [T,64], M [T,T] -> Δ [B,T,4096]).
 *   x      [B][T][4096]   bf16  block input (the normalised activations)
 *   w_q    [4096][4096]   bf16  query projection, [out][in]
 *   w_k    [1024][4096]   bf16  key projection (8 heads x 128), [out][in]
 *   w_v    [1024][4096]   bf16  value projection, [out][in]
 *   w_o    [4096][4096]   bf16  output projection, [out][in]
 *   rope   [T][64][2]     f32   (cos, sin) of row t's angle per pair; shared by
 *                               all B sequences (gqa_rope_table makes it)
 *   mask   [T][kv_len]    f32   additive mask, or NULL; must be NULL if causal
 *   causal                      1: key j is masked for query i when j > i
 *                               0: `mask` (or no mask when NULL)
 *   B, T                        B >= 1, T >= 1, B*T <= GQA_MAX_TOKENS
 *   kv_len                      must equal T (keys are the same T positions)
 *   out    [B][T][4096]   f32   Δ (written; fp32 so the result carries no
 *                               bf16 output rounding)
 *   h_out  [B][T][32][128] bf16 merged head outputs H, or NULL
 *   workspace                   >= gqa_prefill_workspace_bytes(B, T) bytes
 * Kernels: fused QKV projection + rotation, grouped flash attention, output
 * projection. A row whose every key is masked by `mask` yields H = 0. An
 * explicit mask is first classified per 64x64 tile (all 0 / all -inf / mixed),
 * so key tiles it removes whole are never loaded; the result is the one of
 * adding it element by element, bit for bit.
 */
int gqa_block_forward(const gqa_bf16* x, const gqa_bf16* w_q, const gqa_bf16* w_k,
                      const gqa_bf16* w_v, const gqa_bf16* w_o, const float* rope,
                      const float* mask, int causal, int B, int T, int kv_len,
                      float* out, gqa_bf16* h_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace bytes gqa_chunk_forward needs for B sequences of T new positions
 * starting at start_pos. */
size_t gqa_chunk_workspace_bytes(int B, int T, int start_pos);

/*
 * Chunked prefill into a KV cache: T new positions per sequence, at positions
 * start_pos .. start_pos+T-1, after a cache that already holds positions
 * 0 .. start_pos-1. Grouped-query attention page, "All 13 steps" with the
 * model.py excerpt's cache semantics: row i of the new block is token
 * start_pos + i and sees keys 0 .. start_pos + i (the excerpt's mask: zeros
 * for the cached columns, then the causal triangle).
 *   x       [B][T][4096]           bf16  block input of the new positions
 *   w_q, w_k, w_v, w_o                   as for gqa_block_forward
 *   rope    [T][64][2]             f32   (cos, sin) at positions start_pos + t
 *   k_cache [B][S_max][8][128]     bf16  rotated keys of positions 0..start_pos-1;
 *                                        slots start_pos..start_pos+T-1 are
 *                                        overwritten with the new rotated keys
 *   v_cache [B][S_max][8][128]     bf16  values, same slots
 *   B, T, S_max, start_pos               B >= 1, T >= 1, start_pos >= 0,
 *                                        start_pos + T <= S_max, B*T <= GQA_MAX_TOKENS
 *   out     [B][T][4096]           f32   Δ
 *   h_out   [B][T][32][128]        bf16  merged head outputs, or NULL
 *   workspace                            >= gqa_chunk_workspace_bytes(B, T, start_pos)
 * start_pos = 0 is an ordinary causal prefill that also fills the cache.
 */
int gqa_chunk_forward(const gqa_bf16* x, const gqa_bf16* w_q, const gqa_bf16* w_k,
                      const gqa_bf16* w_v, const gqa_bf16* w_o, const float* rope,
                      gqa_bf16* k_cache, gqa_bf16* v_cache, int B, int T, int S_max,
                      int start_pos, float* out, gqa_bf16* h_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace bytes gqa_decode_forward needs for B sequences and a cache of S_max rows. */
size_t gqa_decode_workspace_bytes(int B, int S_max);

/*
 * Decode: one new position per sequence, at position start_pos, over a KV
 * cache. Grouped-query attention page, "All 13 steps" at T = 1 with the
 * model.py excerpt's cache semantics: row i of the new block is token
 * cache_len + i, and a single position needs no mask.
 *   x       [B][4096]              bf16  block input of the new token
 *   w_q, w_k, w_v, w_o                   as for gqa_block_forward
 *   rope    [64][2]                f32   (cos, sin) at position start_pos
 *   k_cache [B][S_max][8][128]     bf16  rotated keys of positions 0..start_pos-1;
 *                                        slot start_pos is overwritten with the
 *                                        new token's rotated key
 *   v_cache [B][S_max][8][128]     bf16  values; slot start_pos is overwritten
 *   B, S_max, start_pos                  B >= 1, 0 <= start_pos < S_max;
 *                                        the new token attends to keys 0..start_pos
 *   out     [B][4096]              f32   Δ
 *   h_out   [B][32][128]           bf16  merged head outputs, or NULL
 *   workspace                            >= gqa_decode_workspace_bytes(B, S_max)
 */
int gqa_decode_forward(const gqa_bf16* x, const gqa_bf16* w_q, const gqa_bf16* w_k,
                       const gqa_bf16* w_v, const gqa_bf16* w_o, const float* rope,
                       gqa_bf16* k_cache, gqa_bf16* v_cache, int B, int S_max,
                       int start_pos, float* out, gqa_bf16* h_out, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * gqa_decode_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, kernels and results as
 * gqa_decode_forward, minus workspace / workspace_bytes: the scratch those
 * kernels need (Q_r, H and the split partials) lives in a fixed device array
 * of GQA_STATIC_SCRATCH_BYTES (32 MiB) that the library holds on each GPU it
 * runs on until the process ends. The call allocates and frees nothing.
 *  - Accepted when gqa_decode_workspace_bytes(B, S_max) <= 32 MiB, which holds
 *    for every B <= 256 at any S_max; larger requests return
 *    GQA_ERR_TOO_LARGE and launch nothing.
 *  - The first call on a device looks up the array's device address there
 *    (hipGetSymbolAddress, not a stream operation; GQA_ERR_HIP if it fails).
 *    This per-device address is the only state the library keeps.
 *  - Every call on one GPU uses that GPU's one array: calls that overlap in
 *    time on the same GPU (different streams, or several host threads) race
 *    and give undefined results. Calls on one stream are ordered and safe.
 *    The array keeps the last call's contents; nothing in it needs to start
 *    at zero.
 */
int gqa_decode_forward_static(const gqa_bf16* x, const gqa_bf16* w_q, const gqa_bf16* w_k,
                              const gqa_bf16* w_v, const gqa_bf16* w_o, const float* rope,
                              gqa_bf16* k_cache, gqa_bf16* v_cache, int B, int S_max,
                              int start_pos, float* out, gqa_bf16* h_out, void* stream);

/*
 * The attention half of the decoder block with its handoff ("Llama 3.1 8B ·
 * Merge and project", section "Contextual evidence from Output projection",
 * the model.py handoff excerpt): the block reads the RMS-normalised input and
 * its update is added to the input,
 *     x̂ = RMSNorm(x),  out = x + Δ(x̂),
 *     RMSNorm(x)[t][i] = norm_w[i] · x[t][i] / sqrt(mean over j of x[t][j]^2 + eps)
 * (the pages name RMSNorm and norm_eps = 1e-5 but not its formula; this is
 * root-mean-square layer normalisation with eps under the root). x̂ is rounded
 * to bf16 once before the projections; the residual adds the bf16 input x to
 * the fp32 Δ. Each variant takes the arguments, workspace and errors of the
 * entry point it extends, plus
 *   norm_w  [4096]   bf16   per-feature gain (device)
 *   eps     >= 0, finite   (else GQA_ERR_ARG; with eps = 0 an all-zero row
 *                           gives non-finite output)
 * and returns out = x + Δ instead of Δ. h_out, when given, is still H of the
 * normalised input. x̂ lives in the workspace region H uses later.
 */
int gqa_block_forward_prenorm(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                              const gqa_bf16* w_q, const gqa_bf16* w_k, const gqa_bf16* w_v,
                              const gqa_bf16* w_o, const float* rope, const float* mask,
                              int causal, int B, int T, int kv_len, float* out,
                              gqa_bf16* h_out, void* workspace, size_t workspace_bytes,
                              void* stream);
int gqa_chunk_forward_prenorm(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                              const gqa_bf16* w_q, const gqa_bf16* w_k, const gqa_bf16* w_v,
                              const gqa_bf16* w_o, const float* rope, gqa_bf16* k_cache,
                              gqa_bf16* v_cache, int B, int T, int S_max, int start_pos,
                              float* out, gqa_bf16* h_out, void* workspace,
                              size_t workspace_bytes, void* stream);
int gqa_decode_forward_prenorm(const gqa_bf16* x, const gqa_bf16* norm_w, float eps,
                               const gqa_bf16* w_q, const gqa_bf16* w_k, const gqa_bf16* w_v,
                               const gqa_bf16* w_o, const float* rope, gqa_bf16* k_cache,
                               gqa_bf16* v_cache, int B, int S_max, int start_pos, float* out,
                               gqa_bf16* h_out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * The normalisation alone (same definition as above):
 *   x [M][4096] bf16, norm_w [4096] bf16, y [M][4096] bf16 out; 1 <= M
 */
int gqa_rmsnorm(const gqa_bf16* x, const gqa_bf16* norm_w, float eps, int M, gqa_bf16* y,
                void* stream);

/*
 * SwiGLU MLP, the other half of the decoder block ("Llama 3" page, section
 * "SwiGLU MLP"): three bias-free projections,
 *     out = w2( silu(x·w1ᵀ) ⊙ (x·w3ᵀ) ),  silu(g) = g / (1 + e^-g),
 * d_ff = 14336 (the SiLU panel's shapes). Gate and up are one product whose
 * epilogue forms silu(gate)·up in fp32 and rounds it once to bf16 (A); the
 * down product accumulates in fp32.
 *   x      [M][4096]    bf16   input rows (tokens)
 *   w1, w3 [14336][4096] bf16  gate and up projections, [out][in]
 *   w2     [4096][14336] bf16  down projection, [out][in]
 *   out    [M][4096]    f32    result
 *   a_out  [M][14336]   bf16   A = silu(gate)·up, or NULL (then it stays in
 *                              the workspace)
 *   workspace  >= gqa_mlp_workspace_bytes(M) bytes (device)
 * 1 <= M <= GQA_MAX_TOKENS. The _prenorm form reads RMSNorm(x) (gain norm_w
 * [4096] bf16, eps as for gqa_block_forward_prenorm; the block's ffn_norm)
 * and returns out = x + MLP(x̂) (Merge and project page, handoff excerpt).
 */
size_t gqa_mlp_workspace_bytes(int M);
int gqa_mlp_forward(const gqa_bf16* x, const gqa_bf16* w1, const gqa_bf16* w2,
                    const gqa_bf16* w3, int M, float* out, gqa_bf16* a_out, void* workspace,
                    size_t workspace_bytes, void* stream);
int gqa_mlp_forward_prenorm(const gqa_bf16* h, const gqa_bf16* norm_w, float eps,
                            const gqa_bf16* w1, const gqa_bf16* w2, const gqa_bf16* w3, int M,
                            float* out, gqa_bf16* a_out, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Stage 1 alone: Q, K, V projections with the pair rotation applied to Q and K
 * ("All 13 steps": the three projections and the rotation). Each output is
 * rounded to bf16 once, after the rotation.
 *   x [B][T][4096], w_q, w_k, w_v, rope [T][64][2] as above
 *   q_r [B][T][32][128], k_r [B][T][8][128], v [B][T][8][128]   bf16 out
 *   q_scaled   0: q_r holds Q_r; 1: q_r holds Q_r times log2(e)/sqrt(128) (the
 *              softmax's score scale in base 2, rounded once with it), the form
 *              the block and chunk entries hand to their attention stage
 */
int gqa_qkv_rope(const gqa_bf16* x, const gqa_bf16* w_q, const gqa_bf16* w_k,
                 const gqa_bf16* w_v, const float* rope, int B, int T,
                 gqa_bf16* q_r, gqa_bf16* k_r, gqa_bf16* v, int q_scaled, void* stream);

/*
 * Workspace bytes gqa_attention uses: for a causal launch with few query tiles,
 * the balanced plan's partials (the last query tile attends to every key tile,
 * so with fewer than two 64-row tiles per CU the longest workgroup would set
 * the time; 0 with enough query tiles); for a non-causal launch, one byte per
 * 64x64 tile of the mask (its class: all 0, all -inf or mixed; each row of
 * tiles padded to a multiple of 4 bytes, the total to a multiple of 256), so
 * that an explicit mask costs about what the same mask given as a flag costs.
 */
size_t gqa_attention_workspace_bytes(int B, int T, int kv_len, int causal);

/*
 * Stage 2 alone: grouped attention over already rotated queries and keys
 * ("All 13 steps": group map, scores, scale, mask, softmax, A·V_G, merge).
 *   q_r [B][T][32][128], k_r and v [B][kv_len][8][128]   bf16
 *   mask / causal as for gqa_block_forward (kv_len must equal T)
 *   h_out [B][T][32][128]   bf16 out
 *   workspace   NULL (plain launch; an explicit mask is then added tile by
 *               tile everywhere), or >= gqa_attention_workspace_bytes(B, T,
 *               kv_len, causal) bytes of device memory (balanced causal launch,
 *               the same result up to fp32 summation order; or the mask's tile
 *               classes, the same result bit for bit)
 *   q_scaled    0: q_r is Q_r; 1: q_r is Q_r times log2(e)/sqrt(128), as
 *               gqa_qkv_rope writes it with q_scaled = 1 (the kernel the block
 *               and chunk entries run: it spends no instruction on the scale)
 * Returns GQA_ERR_ARG for q_scaled other than 0 or 1.
 */
int gqa_attention(const gqa_bf16* q_r, const gqa_bf16* k_r, const gqa_bf16* v,
                  const float* mask, int causal, int B, int T, int kv_len,
                  gqa_bf16* h_out, void* workspace, size_t workspace_bytes, int q_scaled,
                  void* stream);

/*
 * Stage 3 alone: Δ = H·W_O (Merge and project page, Explanation; "All 13
 * steps", last equation).
 *   h [M][4096] bf16, w_o [4096][4096] bf16, out [M][4096] f32; 1 <= M
 */
int gqa_output_projection(const gqa_bf16* h, const gqa_bf16* w_o, int M, float* out,
                          void* stream);

/*
 * Decode attention alone: the split-KV grouped attention of gqa_decode_forward
 * for already rotated queries over a cache that already holds keys 0..kv_len-1.
 *   q_r [B][32][128] bf16, k_cache/v_cache [B][S_max][8][128] bf16,
 *   1 <= kv_len <= S_max, h_out [B][32][128] bf16 out,
 *   workspace >= gqa_decode_workspace_bytes(B, S_max)
 */
int gqa_decode_attention(const gqa_bf16* q_r, const gqa_bf16* k_cache,
                         const gqa_bf16* v_cache, int B, int S_max, int kv_len,
                         gqa_bf16* h_out, void* workspace, size_t workspace_bytes,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */

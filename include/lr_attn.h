/* lr_attn.h -- C ABI of the MI355X (gfx950) library for the decode step of
 * per-head low-rank attention over a quantised latent KV cache.
 *
 * The operation (WSVD page, "Fine-grained per-head SVD" and "System
 * implementation (fused kernel)"; LASER page, "Hybrid SVD-quantisation" and
 * "Loss-aware cross-layer rank allocation"): for layer l and head h the K and
 * V projections are factorised per head, W^K_h ~ A^K_h B^K_h and
 * W^V_h ~ A^V_h B^V_h, with A (E x r) and B (r x d).  The cache keeps only the
 * per-head latents c^K_t = x_t A^K_h and c^V_t = x_t A^V_h, quantised
 * round-to-nearest to int8 or int4.  A decode step rebuilds
 * k_t = c~^K_t B^K_h, v_t = c~^V_t B^V_h and returns
 *     o = softmax_t(scale * q . k_t) v_t
 * over the cached tokens.  Ranks may differ per (layer, head) and between K
 * and V (LASER's non-uniform rank allocation).
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises, and never keeps a pointer.
 *   - Every argument error is detected on the host before any launch and is
 *     returned as a status; nothing is launched in that case.
 *   - Launches are asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream).  A failed launch returns LR_EHIP; the HIP error code
 *     is then available from lr_attn_last_hip_error() on the same thread.
 *   - A plan is immutable after creation and may be shared between threads.
 *   - head_dim must be 128; 1 <= n_heads <= 128; every rank r satisfies
 *     8 <= r <= 128 and r % 8 == 0.
 */
#ifndef LR_ATTN_H
#define LR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LR_OK = 0,
  LR_EINVAL = 1,        /* bad argument: null pointer, bad size, misalignment */
  LR_EUNSUPPORTED = 2,  /* valid but unsupported: head_dim != 128, rank rules */
  LR_ERANGE = 3,        /* index or length out of range (layer, head, max_len) */
  LR_EWORKSPACE = 4,    /* workspace missing or smaller than required */
  LR_EHIP = 5           /* a HIP launch failed */
} lr_status;

/* Latent quantisation formats (LASER page, round-to-nearest quantisation;
 * WSVD page, W8A8 / W8A4 activations).  Both are symmetric:
 *   LR_Q_INT8_TOKEN: one fp32 scale s = max|c| / 127 per (token, head, K or V);
 *                    codes clamp(rne(c / s), -127, 127), 0 when s == 0.
 *   LR_Q_INT4_G32:   one fp16 scale s_g = fp16(max|c| / 7) per group of 32
 *                    consecutive ranks (the last group may be 8, 16 or 24);
 *                    codes clamp(rne(c / s_g), -7, 7), 0 when s_g == 0. */
typedef enum { LR_Q_INT8_TOKEN = 0, LR_Q_INT4_G32 = 1 } lr_qfmt;

/* Element type of q, the B factors and the output. */
typedef enum { LR_DT_BF16 = 0, LR_DT_F32 = 1 } lr_dtype;

#define LR_HEAD_DIM 128
#define LR_MAX_HEADS 128
#define LR_MAX_RANK 128
#define LR_TILE_TOKENS 64

typedef struct lr_attn_desc {
  int32_t n_layers;      /* >= 1 */
  int32_t batch;         /* B >= 1 */
  int32_t n_heads;       /* H, 1..128 */
  int32_t head_dim;      /* d, must be 128 */
  int32_t capacity;      /* token slots per sequence, 1..16777216 */
  int32_t qfmt;          /* lr_qfmt */
  int32_t io_dtype;      /* lr_dtype of q, B^K, B^V and out */
  int32_t max_splits;    /* 0 = automatic; n >= 1 caps the context splits per (b, h) */
  int32_t wg_waves;      /* 0 = automatic; 4, 8 or 16 forces the wavefronts per work-group
                            (16 is lowered to 8 for layers whose largest rank is an
                            int8 rank of 33-64 or 97-128, or an int4 rank above 64).
                            Automatic picks 3 for those int8 layers when B x H is
                            769..1024, so that every (b, h) work-group is resident.
                            The explicit form takes 4 or 8, and 8 only in layers whose
                            largest rank is at most 32 (4 otherwise) */
  int32_t reserved;      /* must be 0 */
  const int32_t* rank_k; /* HOST [n_layers * n_heads], row-major (layer, head) */
  const int32_t* rank_v; /* HOST [n_layers * n_heads] */
} lr_attn_desc;

typedef struct lr_attn_plan lr_attn_plan; /* opaque */

/* Byte layout of one head's latent planes inside a layer's cache buffer.
 * For head h and sequence b the K plane starts at
 *     k_offset + b * plane_bytes_k
 * and holds ceil(capacity / 64) tiles of tile_bytes_k bytes; token slot t
 * lives in tile t / 64 at lane i = t % 64.  Inside a tile the row bytes come
 * first, split in chunks of 16 bytes (the last chunk may be shorter, width
 * w = row_bytes - 16 * c): chunk c of lane i is at 1024 * c + w_c * i.  int8
 * codes are two's-complement bytes, rank index = 16 * c + byte.  int4 codes are
 * two's-complement nibbles, rank index = 32 * c + 2 * byte (low nibble) or
 * + 1 (high nibble).  The scales follow the rows at 64 * row_bytes: int8 one
 * fp32 at + 4 * i; int4 fp16 per group g at + 2 * (64 * g + i).  V is the same
 * with the _v fields. */
typedef struct lr_attn_head_layout {
  uint64_t k_offset, v_offset;         /* bytes from the cache base, 256-aligned */
  uint64_t plane_bytes_k, plane_bytes_v;
  int32_t rank_k, rank_v;
  int32_t row_bytes_k, row_bytes_v;    /* code bytes per token */
  int32_t scale_bytes_k, scale_bytes_v;/* scale bytes per token */
  int32_t tile_bytes_k, tile_bytes_v;  /* 64 * (row_bytes + scale_bytes) */
  int32_t latent_offset_k;             /* first element of head h in a token's K latent vector */
  int32_t latent_offset_v;             /* ... and in a token's V latent vector */
  int64_t factor_offset_k;             /* first element of B^K_h (r_k x d, row-major) in the K factor tensor */
  int64_t factor_offset_v;
} lr_attn_head_layout;

/* Validate `desc` and build a host-only plan (no device memory is touched).
 * max_splits and wg_waves only shape the decode launch; results agree to
 * rounding whatever their values.
 * Errors: LR_EINVAL (null desc/out/rank pointers, non-positive sizes, bad
 * enum, wg_waves not in {0, 4, 8, 16}, reserved != 0), LR_EUNSUPPORTED (head_dim != 128, n_heads > 128, rank not in
 * {8, 16, ..., 128}), LR_ERANGE (capacity beyond 2^24). */
lr_status lr_attn_plan_create(const lr_attn_desc* desc, lr_attn_plan** out);
void lr_attn_plan_destroy(lr_attn_plan* plan);

/* Bytes of one layer's cache buffer (0 on a bad plan or layer).  The caller
 * allocates it with 256-byte alignment; its contents are only read at slots
 * below len[b]. */
size_t lr_attn_cache_bytes(const lr_attn_plan* plan, int32_t layer);
/* Elements per token of the K (kv = 0) or V (kv = 1) latent vector of a
 * layer: sum over heads of r_h (0 on bad arguments). */
size_t lr_attn_latent_elems(const lr_attn_plan* plan, int32_t layer, int32_t kv);
/* Elements of the K or V factor tensor of a layer: sum_h r_h * d.  Head h's
 * B_h is the row-major r_h x d block at factor_offset (0 on bad arguments). */
size_t lr_attn_factor_elems(const lr_attn_plan* plan, int32_t layer, int32_t kv);
/* Layout of head `head` of layer `layer`.  Errors: LR_EINVAL, LR_ERANGE. */
lr_status lr_attn_head_layout_get(const lr_attn_plan* plan, int32_t layer, int32_t head,
                                  lr_attn_head_layout* out);

/* Workspace bytes needed by lr_attn_decode for any layer when called with
 * this max_len (0 means none is needed; the size is a multiple of 256).  It
 * holds the per-split partials (m, l, u) when a launch splits the context of
 * each (b, h) Flash-Decoding style (few sequences and heads, long contexts).
 * Its contents need no initialisation and are scratch between calls. */
size_t lr_attn_workspace_bytes(const lr_attn_plan* plan, int32_t max_len);

/* Quantise fp32 latents and write them at token slots pos[b] .. pos[b]+n_new-1
 * of every head of layer `layer` (LASER page, "System implementation": fused
 * quantisation of the latent activations; WSVD page, per-head latents).
 *   cache   device, lr_attn_cache_bytes(layer) bytes, 256-aligned
 *   ck, cv  device fp32 [batch][n_new][latent_elems(kv)], 16-aligned; head h's
 *           latent of a token is the r_h elements at latent_offset(h)
 *   pos     device int32 [batch]; slots outside [0, capacity) are skipped
 *   n_new   tokens per sequence, 0..capacity (0 is a no-op), with
 *           batch x n_heads x n_new <= 2^26
 * The cache is only written; lengths are not tracked by the library.  The
 * quantised codes and scales are bit-exact with the definition given at
 * lr_qfmt (correctly rounded fp32 division, round-half-even, fp16 RNE).
 * Errors: LR_EINVAL, LR_ERANGE (layer, n_new), LR_EHIP. */
lr_status lr_attn_append_latent(const lr_attn_plan* plan, int32_t layer, void* cache,
                                const float* ck, const float* cv, const int32_t* pos,
                                int32_t n_new, void* stream);

/* One decode step of layer `layer` for every (b, h):
 *     out[b][h][:] = sum_t p_t v_t,  p = softmax_t(softmax_scale * q[b][h] . k_t),
 * over token slots t < len[b], with k_t = c~^K_t B^K_h and v_t = c~^V_t B^V_h
 * rebuilt from the cache (WSVD page, "System implementation": reconstruction
 * plus Flash-Decoding QK^T, softmax and PV in one kernel, with nothing rebuilt
 * written to memory).  This entry point uses the absorbed form
 * q' = softmax_scale * q B^K_h^T scored against the latents and applies B^V_h
 * once to the accumulated latent, which is algebraically identical.
 *   cache       device, written by lr_attn_append_latent
 *   len         device int32 [batch]; values are clamped to [0, max_len]; a
 *               sequence with len 0 gets a zero output
 *   max_len     host upper bound of len[], 1..capacity; sizes the launch
 *   q           device [batch][n_heads][128] io_dtype
 *   bk, bv      device factor tensors (lr_attn_factor_elems) io_dtype
 *   out         device [batch][n_heads][128] io_dtype
 *   workspace   device, >= lr_attn_workspace_bytes(max_len) bytes; may be
 *               NULL when that is 0.  Concurrent calls must not share one.
 * All pointers 16-aligned.  Errors: LR_EINVAL, LR_ERANGE, LR_EWORKSPACE, LR_EHIP. */
lr_status lr_attn_decode(const lr_attn_plan* plan, int32_t layer, const void* cache,
                         const int32_t* len, int32_t max_len, const void* q, const void* bk,
                         const void* bv, float softmax_scale, void* out, void* workspace,
                         size_t ws_bytes, void* stream);

/* lr_attn_append_latent with n_new = 1 followed by lr_attn_decode, in one
 * launch (two when the context is split): for every sequence b the new
 * token's latents are quantised and written at slot pos[b], then every (b, h)
 * attends over slots t < len[b], the new one included when pos[b] < len[b]
 * (LASER page, "System implementation": quantisation fused into the kernel).
 * The cache bytes written and the output are bit-identical to the two calls.
 *   cache       device, as for both calls; written at slot pos[b] only
 *   ck, cv      device fp32 [batch][latent_elems(kv)], 16-aligned
 *   pos         device int32 [batch]; a slot outside [0, capacity) is neither
 *               written nor substituted (the decode then reads the cache as is)
 *   len ... ws  as for lr_attn_decode
 * Errors: LR_EINVAL, LR_ERANGE, LR_EWORKSPACE, LR_EHIP. */
lr_status lr_attn_append_decode(const lr_attn_plan* plan, int32_t layer, void* cache,
                                const float* ck, const float* cv, const int32_t* pos,
                                const int32_t* len, int32_t max_len, const void* q,
                                const void* bk, const void* bv, float softmax_scale, void* out,
                                void* workspace, size_t ws_bytes, void* stream);

/* lr_attn_append_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same launches and the same results, bit for bit, with the
 * context-split partials kept in a device array that the library holds, one
 * per GPU, from the first call on that GPU until the process ends.  The
 * array holds LR_NOALLOC_SCRATCH_BYTES (2 MiB); the partials of any plan fit
 * in it (at most 1.06 MB), and a call whose lr_attn_workspace_bytes(max_len)
 * would exceed it returns LR_EWORKSPACE before any launch.  No call allocates
 * or frees memory.  Every call on one GPU uses that GPU's one array, which
 * keeps the last call's contents (each launch writes every partial it later
 * reads, so nothing needs clearing): calls that may run at the same time on
 * one GPU (different streams or threads) race on it and must be serialised by
 * the caller.  Arguments and errors as lr_attn_append_decode, without the
 * workspace; LR_EHIP also when the array's address cannot be obtained. */
#define LR_NOALLOC_SCRATCH_BYTES (2u << 20)
lr_status lr_attn_append_decode_noalloc(const lr_attn_plan* plan, int32_t layer, void* cache,
                                        const float* ck, const float* cv, const int32_t* pos,
                                        const int32_t* len, int32_t max_len, const void* q,
                                        const void* bk, const void* bv, float softmax_scale,
                                        void* out, void* stream);

/* The same result through explicit per-token reconstruction: every k_t and
 * v_t (d = 128 values) is rebuilt on chip with matrix-core products of the
 * dequantised latents and B_h, then scored and accumulated (WSVD page,
 * "System implementation": K_h rebuilt in an on-chip buffer).  Same arguments,
 * rules and errors as lr_attn_decode; it needs no workspace beyond what
 * lr_attn_workspace_bytes reports. */
lr_status lr_attn_decode_explicit(const lr_attn_plan* plan, int32_t layer, const void* cache,
                                  const int32_t* len, int32_t max_len, const void* q,
                                  const void* bk, const void* bv, float softmax_scale, void* out,
                                  void* workspace, size_t ws_bytes, void* stream);

/* Latent generation for every head of layer `layer` at once (WSVD page,
 * "Fine-grained per-head SVD": the cached latent of a token is c_t = x_t A_h;
 * LASER page, "System implementation": the latent activations are generated
 * in a GPU kernel ahead of the fused quantisation):
 *     ck[t][:] = x[t] A^K,   cv[t][:] = x[t] A^V,   t < n_tokens,
 * where A^K (E x latent_elems(0)) is A^K_h of every head side by side, head
 * h's r_h columns at its latent_offset_k, and A^V likewise.
 *
 * The factors are given once, TRANSPOSED (one row of E values per latent
 * dimension: the layout of a linear layer's weight) and packed by
 * lr_attn_pack_projection into matrix-core operand blocks; the packed buffer
 * depends only on the factors, so it is made once per layer and reused.
 * Packed layout (bf16 elements): tiles r = 0 .. k_tiles + v_tiles - 1 of 16
 * latent rows (k_tiles = ceil(latent_elems(0) / 16), K tiles first), each of
 * E / 32 steps of 512 elements; element 8 l + i of step c of tile r is row
 * 16 r' + (l % 16) of W^K (r' = r) or W^V (r' = r - k_tiles), column
 * 32 c + 8 (l / 16) + i (l < 64, i < 8); rows past the last are zero. */

/* Elements of the packed factor buffer of a layer for this embed (0 on bad
 * arguments: embed must be a positive multiple of 32). */
size_t lr_attn_packed_projection_elems(const lr_attn_plan* plan, int32_t layer, int32_t embed);

/* Pack the row-major factors of layer `layer`:
 *   wk, wv   device bf16 [latent_elems(kv)][embed] (W^K = A^K transposed), 16-aligned
 *   packed   device bf16, lr_attn_packed_projection_elems elements, 16-aligned
 * Errors: LR_EINVAL (null or misaligned pointer, bad embed), LR_ERANGE
 * (layer), LR_EHIP. */
lr_status lr_attn_pack_projection(const lr_attn_plan* plan, int32_t layer, int32_t embed,
                                  const void* wk, const void* wv, void* packed, void* stream);

/* The latents of n_tokens tokens, on the matrix cores: bf16 inputs, exact
 * products, fp32 sums in a fixed order for a given n_tokens (results are
 * deterministic; the work-group shape, and with it the summation order,
 * depends on the token count, so a token's latents may differ in the last
 * bits between calls with different n_tokens).  The plan's io_dtype does not
 * apply.
 *   x         device bf16 [n_tokens][embed], 16-aligned
 *   n_tokens  0 (no-op) or more; rows of x are tokens in any order
 *   embed     E: a multiple of 32, >= 32, the value the factors were packed with
 *   packed    device, from lr_attn_pack_projection
 *   ck, cv    device fp32 [n_tokens][latent_elems(kv)], 16-aligned, written
 * Errors: LR_EINVAL (null or misaligned pointer, bad embed, n_tokens < 0),
 * LR_ERANGE (layer), LR_EHIP. */
lr_status lr_attn_project_latent(const lr_attn_plan* plan, int32_t layer, const void* x,
                                 int32_t n_tokens, int32_t embed, const void* packed, float* ck,
                                 float* cv, void* stream);

/* The latents of n_tokens tokens as n_parts partial sums: E is split into
 * n_parts ranges of consecutive 32-element steps, part q covering steps
 * [q S / n_parts, (q + 1) S / n_parts) of S = embed / 32, and part q's sums
 * are written to block q of ck and cv:
 *     ck[q][t][:] = sum over e in part q of x[t][e] A^K[e][:]   (cv likewise)
 * Adding the blocks in order q = 0, 1, .. gives the latents; the one-step
 * entry point lr_attn_project_append_decode does exactly that inside its
 * decode launch.  More parts give more work-groups: a decode-sized product
 * (a few dozen tokens) then uses the whole GPU.
 *   n_parts   1 .. 8 and at most embed / 32 (lr_attn_project_parts gives the
 *             count the one-step entry point uses)
 *   ck, cv    device fp32 [n_parts][n_tokens][latent_elems(kv)], 16-aligned
 * Other arguments and errors as lr_attn_project_latent; n_parts out of range
 * is LR_EINVAL.  With n_parts = 1 the result equals lr_attn_project_latent's
 * bit for bit. */
lr_status lr_attn_project_latent_parts(const lr_attn_plan* plan, int32_t layer, const void* x,
                                       int32_t n_tokens, int32_t embed, const void* packed,
                                       int32_t n_parts, float* ck, float* cv, void* stream);

/* The part count lr_attn_project_append_decode uses for a call of n_tokens
 * tokens (its batch) at this embed; 0 on bad arguments. */
int32_t lr_attn_project_parts(const lr_attn_plan* plan, int32_t layer, int32_t n_tokens,
                              int32_t embed);

/* Workspace bytes of lr_attn_project_append for any layer with this n_new
 * (the fp32 latents of batch * n_new tokens, K and V); 0 on bad arguments. */
size_t lr_attn_project_workspace_bytes(const lr_attn_plan* plan, int32_t n_new);

/* lr_attn_project_latent followed by lr_attn_append_latent, on the same
 * stream: the new tokens' latents are generated from x into the workspace,
 * then quantised and written at slots pos[b] .. pos[b] + n_new - 1.  The
 * cache bytes are identical to those two calls.
 *   x          device bf16 [batch][n_new][embed]
 *   embed, packed  as for lr_attn_project_latent
 *   pos, n_new as for lr_attn_append_latent (n_new = 0 is a no-op)
 *   workspace  device, >= lr_attn_project_workspace_bytes(n_new) bytes,
 *              256-aligned, scratch; concurrent calls must not share one
 * Errors: LR_EINVAL, LR_ERANGE, LR_EWORKSPACE, LR_EHIP. */
lr_status lr_attn_project_append(const lr_attn_plan* plan, int32_t layer, void* cache,
                                 const void* x, int32_t embed, const void* packed,
                                 const int32_t* pos, int32_t n_new, void* workspace,
                                 size_t ws_bytes, void* stream);

/* Workspace bytes of lr_attn_project_append_decode for any layer of the plan
 * at this max_len and embed: the projection's partial sums, then what
 * lr_attn_decode needs; 0 on bad arguments. */
size_t lr_attn_project_decode_workspace_bytes(const lr_attn_plan* plan, int32_t max_len,
                                              int32_t embed);

/* One whole decode step of a layer from activations: the new token of every
 * sequence is projected to its latents (c = x A_h, every head; WSVD page,
 * "Fine-grained per-head SVD"), quantised and written at slot pos[b], and
 * every (b, h) attends over slots t < len[b] (LASER page, "System
 * implementation": latent generation and quantisation fused ahead of the
 * attention kernel).  Two launches on the stream: the projection, with E
 * split into parts so that a decode-sized product fills the GPU, writes fp32
 * partial sums to the workspace; the fused append + decode adds each
 * latent's parts in a fixed order, then proceeds as lr_attn_append_decode.
 * Results are deterministic; a latent equals lr_attn_project_latent's up to
 * the order of its fp32 sums (exactly equal where those sums are exact).
 *   x          device bf16 [batch][embed], 16-aligned: one token per sequence
 *   embed      E, a multiple of 32, the value the factors were packed with
 *   packed     device, from lr_attn_pack_projection
 *   pos        device int32 [batch], as for lr_attn_append_decode
 *   len ... out  as for lr_attn_decode
 *   workspace  device, >= lr_attn_project_decode_workspace_bytes(max_len,
 *              embed) bytes, 256-aligned; concurrent calls must not share one
 * Errors: LR_EINVAL, LR_ERANGE, LR_EWORKSPACE, LR_EHIP; every argument error
 * is reported before the first launch. */
lr_status lr_attn_project_append_decode(const lr_attn_plan* plan, int32_t layer, void* cache,
                                        const void* x, int32_t embed, const void* packed,
                                        const int32_t* pos, const int32_t* len, int32_t max_len,
                                        const void* q, const void* bk, const void* bv,
                                        float softmax_scale, void* out, void* workspace,
                                        size_t ws_bytes, void* stream);

/* Outlier smoothing by a rotation between the factors (WSVD page,
 * "Quantisation": orthogonal S_1, S_2, S_1 a Hadamard matrix, smooth channel
 * outliers of the latent; LASER page, "Hybrid SVD-quantisation": a rotation
 * inserted between the SVD factors before RTN).  For an orthogonal S,
 * A B = (A S)(S^T B): folded into the factors once, the cached latent becomes
 * c S and no kernel changes.  S is block-diagonal per head with normalised
 * Sylvester-Hadamard blocks H_g (entries +-1/sqrt(g), H_g = H_g^T), g the
 * largest power of two that divides the head's rank and is <= block.  Host
 * functions (no device memory, no stream); they are meant for the offline
 * factors, before conversion to bf16. */

/* g for head `head` of layer `layer`, K (kv = 0) or V (kv = 1); 0 on bad
 * arguments (block must be a power of two in [8, 128]). */
int32_t lr_attn_hadamard_block(const lr_attn_plan* plan, int32_t layer, int32_t kv, int32_t head,
                               int32_t block);

/* Replace every head's rows of `rows` (HOST fp32, [latent_elems(kv)][cols]
 * row-major, head h's r_h rows at its latent offset) by S_h^T times them, in
 * fp64, rounded once to fp32.  Applied to A^T ([latent_elems][E], the layout
 * lr_attn_pack_projection takes) and to B ([latent_elems][128], the decode
 * factors) it folds the rotation: latents c S, product unchanged.  Applying
 * it twice restores the rows (S^2 = I) up to rounding.
 * Errors: LR_EINVAL (null pointer, kv, block, cols < 1), LR_ERANGE (layer). */
lr_status lr_attn_hadamard_rotate_rows(const lr_attn_plan* plan, int32_t layer, int32_t kv,
                                       int32_t block, float* rows, int64_t cols);

/* Greedy global rank allocation (LASER page, "Loss-aware cross-layer rank
 * allocation": singular components are taken greedily by importance score
 * per parameter cost until a parameter budget is met).  Host function; its
 * output is the rank table of lr_attn_desc.
 *   scores   HOST fp32 [n_layers][n_heads][2][max_rank]: the importance of
 *            component j (in singular-value order) of K (index 0) or V (1) of
 *            each head; finite
 *   max_rank 8..128, a multiple of 8: components available per head
 *   cost_per_rank  parameters one component costs (E + head_dim: a column of
 *            A and a row of B), >= 1
 *   budget   parameters for all K and V factors of all layers
 *   rank_k, rank_v  HOST int32 [n_layers * n_heads], written
 * Ranks are multiples of 8 (the kernels' granularity) and prefixes of the
 * components: every head starts at 8; then, while the next block fits the
 * budget, the block of 8 components with the highest summed score per
 * parameter over all heads is added (ties: the lower (layer, head, K/V)
 * index).  Allocation stops at the first best block that does not fit.
 * Errors: LR_EINVAL (null pointer, non-finite score, sizes, cost < 1),
 * LR_EUNSUPPORTED (max_rank), LR_ERANGE (budget below 8 components per head
 * and K/V; more than 2^24 heads). */
lr_status lr_attn_allocate_ranks(int32_t n_layers, int32_t n_heads, int32_t max_rank,
                                 const float* scores, int64_t cost_per_rank, int64_t budget,
                                 int32_t* rank_k, int32_t* rank_v);

/* Hybrid low-rank / dense SwiGLU FFN with W8A8 round-to-nearest
 * quantisation, decode step (LASER page, "Hybrid SVD-quantisation for FFNs":
 * SVD-friendly hidden channels of the gate and up projections are kept as
 * low-rank factors, the others dense, both branches RTN-quantised; "System
 * implementation": fused kernels for the input projection, latent
 * activations, SwiGLU and quantisation).  For each token t:
 *     g_c = (B_g A_g x_t)_c, u_c = (B_u A_u x_t)_c   for hidden channels c < S
 *     g_c = (W_g x_t)_c,     u_c = (W_u x_t)_c       for S <= c < F
 *     h = silu(g) * u,       y_t = W_d h
 * Weights are int8 with one fp32 scale per row (s = max|w| / 127, codes
 * clamp(rne(w / s), -127, 127)); the activations x, z = A x (per gate/up) and
 * h are int8 with one fp32 scale per token and per group of 64 consecutive
 * elements along the reduction dimension (the last group may be shorter),
 * by the same rule; dot products are exact integer sums per group, scaled in
 * fp32 by the group's activation scale and the row's weight scale. */
typedef struct {
  int32_t embed;      /* E: multiple of 64, 64..8192 */
  int32_t hidden;     /* F: multiple of 16 */
  int32_t n_lowrank;  /* S: hidden channels [0, S) are low-rank; multiple of 16, 0..F */
  int32_t rank;       /* r of both gate and up factors: multiple of 64, 64..4096 (0 when S == 0) */
  int32_t reserved;   /* 0 */
} lr_ffn_desc;

/* Bytes of the packed weights (0 on a bad description). */
size_t lr_ffn_weight_bytes(const lr_ffn_desc* desc);

/* Quantise and pack the weights on the host, from fp32 row-major HOST arrays
 * (rows = outputs): wg, wu [F - S][E] (dense gate / up rows of channels
 * S .. F - 1), ag, au [r][E], bg, bu [S][r], wd [E][F] (unused inputs may be
 * NULL).  out: HOST buffer of lr_ffn_weight_bytes bytes, to be copied to
 * device memory (256-aligned) as is.
 * Errors: LR_EINVAL (null pointer, non-finite weight, reserved != 0),
 * LR_EUNSUPPORTED (sizes outside the ranges above). */
lr_status lr_ffn_prepare_weights(const lr_ffn_desc* desc, const float* wg, const float* wu,
                                 const float* ag, const float* au, const float* bg, const float* bu,
                                 const float* wd, void* out);

/* Workspace bytes of lr_ffn_decode for n_tokens tokens (0 on bad arguments,
 * n_tokens < 1 or > 2^20).  Calls run the tokens in passes of at most 16 x
 * floor(2^16 / u) tokens, u the largest work-group count per 16 tokens among
 * the launches (max of E/16 x chunks, r/8, Fp/16, (F-S)/16 + r/16, S/16; Fp
 * = F rounded up to 64, chunks = 1 if Fp <= 2048 else ceil(Fp / 4096)), and
 * the workspace holds one pass. */
size_t lr_ffn_workspace_bytes(const lr_ffn_desc* desc, int32_t n_tokens);

/* One FFN evaluation for n_tokens tokens (four launches per pass of
 * tokens, in order on `stream`):
 *   weights    device, the packed weights, 256-aligned
 *   x          device bf16 [n_tokens][E], 16-aligned
 *   y          device fp32 [n_tokens][E], 16-aligned, written
 *   workspace  device, >= lr_ffn_workspace_bytes(n_tokens), 256-aligned, scratch
 * Results are deterministic.  n_tokens = 0 is a no-op.
 * Errors: LR_EINVAL, LR_EUNSUPPORTED, LR_ERANGE (n_tokens > 2^20),
 * LR_EWORKSPACE, LR_EHIP. */
lr_status lr_ffn_decode(const lr_ffn_desc* desc, const void* weights, const void* x, int32_t n_tokens,
                        float* y, void* workspace, size_t ws_bytes, void* stream);

/* Measurement aid, not part of the decode path: streams bytes / 16 16-byte
 * words from device memory src (16-byte aligned, bytes >= 16; a trailing
 * partial word is not read) with a plain grid-stride read kernel, the
 * practical HBM read roof that the decode kernels' achieved bandwidth is set
 * against.  sink: device pointer to one uint32_t, written only in a case that
 * does not occur in practice (it keeps the reads from being optimised away).
 * Asynchronous on stream.  Errors: LR_EINVAL (null pointer, bytes < 16,
 * misaligned src or sink), LR_EHIP (launch failed). */
lr_status lr_attn_probe_read(const void* src, size_t bytes, void* sink, void* stream);

/* Debugging aid, not part of the decode path: the checked build of this
 * library (liblr_attn_check.so, built with LR_ATTN_CHECK=1) tests every cache
 * access of its kernels (appends, decodes, the explicit form) against the
 * extent of the cache buffer the plan describes; an access outside it is
 * counted and redirected to the buffer's first bytes, so the launch completes
 * instead of faulting.  lr_attn_check_count stores the count of the current
 * device and resets it to 0; it synchronises with the device (two copies of
 * one counter), unlike every other call.  lr_attn_check_shrink sets how many
 * bytes later launches take off each cache's extent (0 by default), which
 * makes accesses near the end count as outside -- the hook a test uses to show
 * that the check fires.  In the release library both return LR_EUNSUPPORTED.
 * Errors: LR_EINVAL (count NULL), LR_EHIP (the copy failed). */
lr_status lr_attn_check_count(uint64_t* count);
lr_status lr_attn_check_shrink(uint64_t bytes);

/* Static description of a status. */
const char* lr_attn_strerror(lr_status status);
/* hipError_t of the last call on this thread that returned LR_EHIP (0 if none). */
int32_t lr_attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LR_ATTN_H */

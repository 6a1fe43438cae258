/*
 * kvlr.h -- C ABI of libkvlr.so: decode attention over a key/value cache
 * stored as rank-r latents, for AMD Instinct MI355X (gfx950).
 *
 * The method (StiefAttention technical summary, "Metodologia:
 * StiefAttention" > "Mecanismo Central", item 5 "Inferência"; the German
 * page "Don't be so Stief!", "Technisches Resümee" > "Kernmechanismus" >
 * "Inferenz"): keys are kept in compressed form K_lat = K P_K and
 * reconstructed as K_lat P_K^T before attention; values likewise with P_V.
 * P_K and P_V have orthonormal columns (same section, item 2; item 3: the Q
 * factor of a QR factorisation). STAR-KV ("Metodologia" section 1,
 * "Inferenza") truncates the projections per attention head, so every KV
 * head h carries its own ranks r_k[h], r_v[h].
 *
 * The library computes the same quantity in latent order:
 *   q~ = q P_K[h],  s_t = (K_lat[t] . q~) * scale,  p = softmax(s),
 *   o  = (sum_t p_t V_lat[t]) P_V[h]^T
 * which equals softmax(K~ q * scale) V~ by associativity.
 *
 * Conventions for every entry point:
 *  - Every function returns 0 (KVLR_OK) or a negative kvlr_status.
 *    Argument checks run on the host before any work is enqueued; on failure
 *    nothing is launched and no buffer is touched.
 *  - The caller owns every buffer. The library allocates nothing, keeps no
 *    pointer after returning and never synchronises: work is enqueued on
 *    `stream` (a hipStream_t passed as void*; NULL is the null stream) and
 *    is complete when that stream is.
 *  - Pointers named "device" must be device memory (or memory the device
 *    can read/write); descriptor rank arrays are host memory.
 *  - Buffers the kernels access with 16-byte vector loads or stores must
 *    start on a 16-byte boundary: K, V, the latent caches, the bases, the
 *    workspace and q_lat (KVLR_ERR_ARG otherwise). q, out, o_lat, k_new,
 *    v_new, pos and seq_lens need only their element alignment.
 *  - Calls are re-entrant and thread-safe on disjoint output buffers.
 *  - Device-resident indices (seq_lens, pos) are trusted preconditions;
 *    kernels clamp them to [0, capacity] and never access memory out of
 *    bounds.
 *  - The library never prints.
 *  - Tuning overrides are read from the environment once, the first time the
 *    library plans a call; later changes to the environment have no effect.
 *    They exist for measurement; every setting keeps results within the same
 *    bounds. Values outside the listed ones are ignored.
 *      KVLR_SPLIT_TOKENS   tokens per split when the library's choice is the
 *                          fixed plan (a positive multiple of 64)
 *      KVLR_TILE=64        64-token wave steps in the bf16 split kernel
 *                          (default 32)
 *      KVLR_BALANCE_FIXED  fixed work per token in the balanced plan, 0..4096
 *                          (default 512; the latent elements are added to it)
 *  - Plans size one round of workgroups over the compute units of the
 *    current device (queried once per device; 256, the MI355X count, when no
 *    device is visible), so the workspace size and the plan queries belong
 *    to the device that is current when they are made.
 */
#ifndef KVLR_H
#define KVLR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVLR_API __attribute__((visibility("default")))

/* Status codes. */
typedef enum kvlr_status {
  KVLR_OK = 0,
  KVLR_ERR_NULL = -1,      /* a required pointer is NULL */
  KVLR_ERR_SHAPE = -2,     /* inconsistent shape: Hq % Hkv, head_dim, start + n_tok > capacity ... */
  KVLR_ERR_RANK = -3,      /* rank outside [1, min(head_dim, 128)] or not a multiple of the
                              storage granule (16 for bf16 and 4/3-bit latents, 4 for fp32 latents) */
  KVLR_ERR_DTYPE = -4,     /* unsupported dtype code */
  KVLR_ERR_WORKSPACE = -5, /* workspace NULL or smaller than kvlr_decode_workspace_bytes() */
  KVLR_ERR_HIP = -6,       /* a kernel launch, stream or event operation failed */
  KVLR_ERR_ARG = -7,       /* other invalid argument (split_tokens, scale, start, a buffer not
                              16-byte aligned) */
  KVLR_ERR_SCRATCH = -8    /* kvlr_decode_attn_noalloc: the call needs more decode workspace than
                              KVLR_STATIC_SCRATCH_BYTES */
} kvlr_status;

/* Size of the library's static decode scratch (kvlr_decode_attn_noalloc). */
#define KVLR_STATIC_SCRATCH_BYTES (16u << 20)

/* split_tokens value that asks kvlr_decode_attn for the balanced plan. */
#define KVLR_SPLIT_BALANCED (-1)

/* Element types. */
typedef enum kvlr_dtype {
  KVLR_F32 = 0,  /* IEEE binary32 */
  KVLR_BF16 = 1, /* bfloat16, stored as the upper 16 bits of binary32; fp32 -> bf16 rounds to nearest even */
  KVLR_Q43 = 2   /* latent caches only: mixed-precision rows, 4-bit outlier block and 3-bit inlier
                    block per token (layout below) */
} kvlr_dtype;

/* How values are decomposed (STAR-KV technical summary, "Metodologia" section 2:
 * joint decomposition factorises the concatenated heads, per-head decomposition
 * each head on its own; STAR-KV keeps keys per head and decomposes values
 * jointly). Keys are always per head. */
typedef enum kvlr_value_mode {
  KVLR_VALUES_PER_HEAD = 0, /* V_lat[h] = V_h P_V[h] */
  KVLR_VALUES_JOINT = 1     /* one latent per token shared by every head:
                               V_lat = [V_0 ... V_{Hkv-1}] P_J, P_J of shape [Hkv d][r];
                               head h reconstructs with rows h d .. (h+1) d - 1 of P_J */
} kvlr_value_mode;

/* Shape of one layer's cache.
 *   batch       B   >= 1
 *   n_q_heads   Hq  >= 1, a multiple of n_kv_heads, with G = Hq / Hkv <= 16
 *               (joint values with bf16 latents: Hq <= 32 and Hkv <= 8)
 *   n_kv_heads  Hkv in [1, 64]; query head i reads KV head i / G
 *   head_dim    d   in [32, 256], a multiple of 32
 *   capacity    T_cap in [1, 2^30]: usable rows per (batch row, KV head); with
 *               4/3-bit latents at most 35791392 (a block stays below 2^31 bytes)
 *   r_k, r_v    host arrays [Hkv]: ranks of each KV head (uniform per-layer
 *               ranks repeat one value); 1 <= r <= min(d, 128), a multiple of 16
 *               for bf16 and 4/3-bit latents and of 4 for fp32 latents
 *   in_dtype    dtype of the full-width K/V rows given to compression and append
 *   latent_dtype dtype of the latent cache
 *   value_mode  KVLR_VALUES_PER_HEAD or KVLR_VALUES_JOINT. Joint values: every
 *               r_v[h] holds the joint rank r (1 <= r <= min(Hkv d, 128), same
 *               granule), the value bases argument is P_J row-major [Hkv d][r]
 *               (which is the per-head packing of its d-row slices), and the
 *               value cache holds one block per batch row (below)
 *
 * Latent cache layout (lat_k; lat_v likewise with r_v): with
 * R = sum_h r_k[h], R_pre(h) = sum_{h' < h} r_k[h'] and
 * C16 = T_cap rounded up to a multiple of 16, the block of (b, h) starts at
 * element C16 * (b * R + R_pre(h)) and holds C16 rows of r_k[h] elements.
 * Inside a block:
 *  - fp32 latents: row-major, (t, j) at t * r + j;
 *  - bf16 key latents: MFMA operand order, so that the decode kernel's
 *    64-lane loads read 1 KiB contiguously. With n = t % 16 and
 *    np = r / 32, 16-row group t / 16 starts at (t / 16) * 16 * r and holds,
 *    for j < 32 np: (j / 32) * 512 + ((j % 32) / 8) * 128 + n * 8 + j % 8;
 *    for the 16-channel tail jj = j - 32 np: np * 512 + (jj / 4) * 64 + n * 4 + jj % 4.
 * Blocks are contiguous, so a split of a sequence streams one byte range.
 *  - bf16 value latents: the operand order of the decode kernel's value
 *    product (tokens as the reduction dimension), below.
 * Joint values: the value cache holds one block of C16 rows of r elements per
 * batch row, at element C16 * b * r, read by every head of that batch row.
 * bf16 value latents (per head and joint) are in the operand order of the
 * decode kernels' value product: with q = (t % 16) / 4,
 * e = t % 4 and np = r / 32, 16-row group t / 16 starts at (t / 16) * 16 * r
 * and holds, for j < 32 np:
 *   (j / 32) * 512 + q * 128 + (j % 16) * 8 + ((j % 32) / 16) * 4 + e;
 * for the 16-channel tail jj = j - 32 np: np * 512 + q * 64 + jj * 4 + e.
 * (A 64-lane load then reads 1 KiB contiguously: lane 16 q + n gets tokens
 * 4 q .. 4 q + 3 of channels n and n + 16 of a pair.)
 *
 * Mixed-precision latents (latent_dtype KVLR_Q43; STAR-KV technical summary,
 * "Metodologia" section 3): the leading n_o(r) = 16 * max(1, (r + 40) / 80)
 * latent channels form the outlier block (20% of the channels, in whole
 * 16-channel Hadamard blocks), the rest (n_i = r - n_o) the inlier block. Each
 * block of each token is quantised on its own: asymmetric round-to-nearest
 * between its minimum and maximum, 15 steps (4 bits) for the outlier block, 7
 * steps (3 bits) for the inlier block, with the step and the minimum kept as
 * IEEE half floats; the stored value is step * code + minimum. In fp32 the code is
 *   step = half((max - min) / (2^bits - 1)), base = half(min),
 *   code = clamp(rint((x - base) * (1 / step)), 0, 2^bits - 1)   (0 if step == 0).
 * The caches are byte arrays. A token of rank r takes
 *   rb(r) = 8 + n_o / 2 + 3 n_i / 8 bytes
 * and tokens are stored in tiles of 32: with RB = sum_h rb(r_k[h]), RB_pre(h)
 * its prefix sum and C32 = T_cap rounded up to a multiple of 32, the block of
 * (b, h) starts at byte C32 * (b * RB + RB_pre(h)) and tile k (rows 32 k ..
 * 32 k + 31) at 32 k rb(r) inside it. Token u of a tile sits in slot
 * s(u) = 8 ((u % 16) / 4) + 4 (u / 16) + u % 4. Inside a tile:
 *   [0, 256)  block parameters as half floats: parameter P of the token in slot
 *             s at byte 64 (s / 8) + 16 P + 2 (s % 8), with P = 0 outlier step,
 *             1 outlier minimum, 2 inlier step, 3 inlier minimum;
 *   then n_o / 16 groups of 16 outlier channels, 256 bytes each: 64 words,
 *             word w = n + 16 kq (n < 16, kq < 4), byte i of word w holds code
 *             (block 0, i) in its low nibble and (block 1, i) in its high nibble;
 *   then n_i / 16 groups of 16 inlier channels, 192 bytes each: bytes 3 w ..
 *             3 w + 2 form a little-endian 24-bit field of eight 3-bit codes,
 *             bits 3 e .. 3 e + 2 holding (block, i) = (0,0) (0,2) (1,0) (1,2)
 *             (0,1) (0,3) (1,1) (1,3) for e = 0 .. 7.
 * (block, n, kq, i) names token 16 block + n, channel 4 kq + i of the group in
 * the key cache, and token 16 block + 4 kq + i, channel n of the group in the
 * value cache: every word or field is what one lane of the decode kernel feeds
 * to the score product (keys) or the value product (values), so no code is
 * moved before use. Rows past a sequence's length may hold any bits. Joint
 * values: one block of C32 rows per batch row, at byte C32 * b * rb(r).
 * The bases used with such a cache must have the block-wise Hadamard folded
 * in (kvlr_hadamard_bases); compression, append and decode all take those
 * folded bases.
 *
 * Basis layout: P_K is fp32, heads packed back to back, head h a row-major
 * [d][r_k[h]] block starting at element d * R_pre(h); P_V likewise. */
typedef struct kvlr_desc {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t capacity;
  const int32_t* r_k;
  const int32_t* r_v;
  int32_t in_dtype;
  int32_t latent_dtype;
  int32_t value_mode;
} kvlr_desc;

/* Library version as 10000 * major + 100 * minor + patch. */
KVLR_API int kvlr_version(void);

/* Static message for a status code (never NULL). */
KVLR_API const char* kvlr_status_string(int status);

/* Validates `desc` and returns, through k_elems / v_elems, the number of
 * latent elements of lat_k and lat_v: B * C16 * sum_h r(h), C16 = T_cap
 * rounded up to a multiple of 16 (bytes, B * C32 * sum_h rb(r(h)), for
 * KVLR_Q43 latents, C32 = T_cap rounded up to a multiple of 32). */
KVLR_API int kvlr_cache_elems(const kvlr_desc* desc, size_t* k_elems, size_t* v_elems);

/* Bytes of decode workspace that kvlr_decode_attn needs for this
 * descriptor and split length (split_tokens as in kvlr_decode_attn; 0 picks
 * the library's choice, the same one kvlr_decode_attn makes for 0).
 * Layout: int32 arrival counters (kvlr_decode_counter_bytes bytes), then the
 * fp32 split records of round_up(max_h r_v[h] + 2, 4) floats each:
 * [B][Hq][n_splits] for a fixed split length; with split_tokens 0 or -1 on
 * caches that allow the balanced plan, the region also fits that plan's
 * (n_wg + B Hkv ceil(G / 4)) slots of 4 records (n_wg = its workgroups), so one
 * workspace serves both plans; then (joint values with bf16 latents only) the
 * projected queries, fp32 [B][Hq][max_h r_k[h]]. */
KVLR_API int kvlr_decode_workspace_bytes(const kvlr_desc* desc, int32_t split_tokens, size_t* bytes);

/* Size of the counter region at the start of a decode workspace:
 * 4 * B * Hkv * ceil(G / 4) bytes rounded up to a multiple of 256. */
KVLR_API int kvlr_decode_counter_bytes(const kvlr_desc* desc, size_t* bytes);

/* Splits that kvlr_decode_attn uses per (batch row, KV head) for
 * split_tokens (0 = library choice: one round of workgroups over the
 * device), and the tokens per split. For the balanced plan: n_splits is its
 * number of workgroups (one round over the device) and tokens_per_split 0. */
KVLR_API int kvlr_decode_plan(const kvlr_desc* desc, int32_t split_tokens, int32_t* n_splits,
                              int32_t* tokens_per_split);

/* Fold the block-wise Hadamard rotation into bases (STAR-KV technical
 * summary, "Metodologia" section 3: every block of latent channels gets its own
 * Hadamard transform, and the factors are fused into the projection matrices,
 * so the rotation costs nothing when the cache is written or read):
 *   out[h] = P[h] R,  R = diag(H16 / 4, ..., H16 / 4) of order r(h),
 * H16 the Sylvester Hadamard matrix (entries +-1). R is orthogonal, so the
 * folded bases stay orthonormal and span the same space. Required before
 * using a KVLR_Q43 cache.
 *   P_K, P_V     device fp32 packed bases (layout above)
 *   out_K, out_V device fp32 packed bases of the same size; each may alias its
 *                input (the transform works in place) */
KVLR_API int kvlr_hadamard_bases(const kvlr_desc* desc, const float* P_K, const float* P_V, float* out_K,
                                 float* out_V, void* stream);

/* Prefill compression: store the latents of n_tok consecutive tokens.
 * (StiefAttention technical summary, "Mecanismo Central" item 5: keys are
 * stored as K P_K; values likewise as V P_V.)
 *   K, V      device, in_dtype, [B][n_tok][Hkv][d] (the layout a fused k/v
 *             projection produces), token n of the call is cache row start + n
 *   start     first cache row written, >= 0, start + n_tok <= capacity
 *   n_tok     >= 0 (0 is a no-op)
 *   P_K, P_V  device fp32 packed bases (see kvlr_desc)
 *   lat_k, lat_v device latent caches (latent_dtype, layout in kvlr_desc);
 *             rows start .. start+n_tok-1 of every (b, h) are overwritten,
 *             nothing else is written.
 * Products accumulate in fp32 (bf16 inputs: MFMA with the basis split into a
 * high and a low bf16 part); results are rounded to the latent dtype
 * (KVLR_Q43: quantised as described above, from the fp32 latents; the
 * bases must be the Hadamard-folded ones). */
KVLR_API int kvlr_prefill_compress(const kvlr_desc* desc, const void* K, const void* V, int32_t start,
                                   int32_t n_tok, const float* P_K, const float* P_V, void* lat_k,
                                   void* lat_v, void* stream);

/* Append one token per batch row: lat_k[b, h, pos[b], :] = k_new[b, h, :] P_K[h],
 * the same with v (autoregressive growth of the cache; StiefAttention
 * technical summary, "Definição do Problema"; storage rule of
 * "Mecanismo Central" item 5).
 *   k_new, v_new device, in_dtype, [B][Hkv][d]
 *   pos       device int32 [B]: row written for batch row b; a row outside
 *             [0, capacity) is not written. The library never increments it
 *             and never changes seq_lens: the caller advances both.
 * fp32 accumulation, rounded to the latent dtype. */
KVLR_API int kvlr_append(const kvlr_desc* desc, const void* k_new, const void* v_new, const int32_t* pos,
                         const float* P_K, const float* P_V, void* lat_k, void* lat_v, void* stream);

/* Decode attention over the latent cache for one new query per (batch row,
 * query head) (StiefAttention technical summary, "Mecanismo Central" item 5;
 * evaluated in the latent order given at the top of this file).
 *   q         device fp32 [B][Hq][d]
 *   P_K, P_V  device fp32 packed bases
 *   lat_k, lat_v device latent caches
 *   seq_lens  device int32 [B]: batch row b attends to rows t < seq_lens[b]
 *             (clamped to [0, capacity]); 0 gives a zero output row
 *   scale     finite score scale (1/sqrt(d) for standard attention)
 *   out       device fp32 [B][Hq][d], fully overwritten
 *   workspace device scratch of at least kvlr_decode_workspace_bytes(desc,
 *             split_tokens) bytes. Its counter region (the first
 *             kvlr_decode_counter_bytes bytes) must be all zero before the
 *             first kvlr_decode_attn call that uses it; every completed call
 *             leaves it zero again. The records need no initialisation.
 *             Calls sharing one workspace must be ordered on one stream.
 *   split_tokens 0 for the library's choice (see kvlr_decode_plan), a
 *             multiple of 64: tokens per split of the sequence (every split
 *             yields a partial softmax state; the workgroup that finishes
 *             last for a group of query heads merges the states and
 *             back-projects with P_V^T, all in one kernel launch), or
 *             KVLR_SPLIT_BALANCED (-1): the balanced plan (bf16 latents with
 *             per-head values; other caches take the library's choice). The
 *             kernel reads seq_lens and gives every workgroup an equal share
 *             of the work, each token counting a fixed part plus its latent
 *             elements, cut across (batch row, KV head) units where needed;
 *             the last workgroup to finish a unit merges it. The plan depends
 *             only on seq_lens, so results are reproducible. The library's
 *             choice is the balanced plan when the KV heads' ranks differ
 *             (batches of 4096 rows at most), the fixed one otherwise.
 * Scores and the softmax are computed in fp32; bf16 latents are read as
 * stored and multiplied in fp32 (the key side on MFMA with the query split
 * into a high and a low bf16 part).
 * Joint values with bf16 latents take three launches instead: the query
 * projection (q~ into the workspace), one workgroup per (split, batch row)
 * that streams every head's keys and the shared value latent once (the value
 * product on MFMA too, with the softmax weights split into a high and a low
 * bf16 part), and a merge per (query head, batch row); the counter region is
 * not used. */
KVLR_API int kvlr_decode_attn(const kvlr_desc* desc, const float* q, const float* P_K, const float* P_V,
                              const void* lat_k, const void* lat_v, const int32_t* seq_lens, float scale,
                              float* out, void* workspace, size_t workspace_bytes, int32_t split_tokens,
                              void* stream);

/* Folded decode: the bases are folded into the attention projections
 * (StiefAttention technical summary, "Mecanismo Central" item 5: the
 * projection bases can be incorporated into the attention linear weights;
 * STAR-KV "Metodologia" section 2: reconstruction absorbed into the output
 * projection). The caller supplies the query already in key latent space and
 * receives the normalised latent output, to be multiplied by its output
 * projection with P_V folded in:
 *   o_lat[b, i, :] = softmax_t(K_lat[b, h, t] . q_lat[b, i] * scale) V_lat[b, h, t]
 *   q_lat     device fp32 [B][Hq][rk_max], rk_max = max_h r_k[h]; row i reads
 *             its first r_k[i / G] entries
 *   o_lat     device fp32 [B][Hq][rv_max], rv_max = max_h r_v[h]; entries
 *             j >= r_v[i / G] are written as zero; empty caches give zero rows
 * Other arguments as in kvlr_decode_attn (one launch, two for joint bf16
 * values; same workspace rules). */
KVLR_API int kvlr_decode_attn_latent(const kvlr_desc* desc, const float* q_lat, const void* lat_k,
                                     const void* lat_v, const int32_t* seq_lens, float scale, float* o_lat,
                                     void* workspace, size_t workspace_bytes, int32_t split_tokens,
                                     void* stream);

/* One autoregressive decode step with its append fused in (StiefAttention
 * technical summary, "Definição do Problema": the cache grows by one row per
 * generated token, and the new token attends to itself): the result, in out
 * and in the caches, is that of
 *   kvlr_append(desc, k_new, v_new, pos, P_K, P_V, lat_k, lat_v, stream);
 *   kvlr_decode_attn(desc, q, P_K, P_V, lat_k, lat_v, seq_lens, scale, out,
 *                    workspace, workspace_bytes, split_tokens, stream);
 * bit for bit. For bf16 latents with per-head values it is one launch: the
 * workgroups whose split holds row pos[b] form the new latent rows, store
 * them and read them back once the stores are acknowledged (no other
 * workgroup reads that row). Other caches take the two launches above.
 * Arguments as in kvlr_append and kvlr_decode_attn; the caller sets
 * seq_lens[b] = pos[b] + 1 to attend to the new row. */
KVLR_API int kvlr_append_decode_attn(const kvlr_desc* desc, const void* k_new, const void* v_new,
                                     const int32_t* pos, const float* q, const float* P_K, const float* P_V,
                                     void* lat_k, void* lat_v, const int32_t* seq_lens, float scale, float* out,
                                     void* workspace, size_t workspace_bytes, int32_t split_tokens, void* stream);

/* Decode attention of several independent layers in one call. Each layer has
 * its own bases and ranks (StiefAttention technical summary, "Mecanismo
 * Central" item 4: ranks are allocated layer by layer under one cache budget),
 * so a model step is one kvlr_decode_attn per layer. The result is that of
 *   for l in 0 .. n_layers-1: kvlr_decode_attn(layers[l]..., stream);
 * bit for bit, but the kernels of different layers may run at the same time,
 * so that one layer's last workgroups overlap the next layers' streaming:
 * the call forks `lanes` internal streams of the library (created once per
 * device, default priority) from `stream` with an event, issues layer l on
 * lane l mod lanes, and joins every lane back into `stream` with events.
 * Work enqueued on `stream` after the call sees every layer's output; the
 * pattern can be captured into a HIP graph.
 *   layers    host array of n_layers kvlr_layer (read during the call only);
 *             each entry holds the arguments of kvlr_decode_attn for its layer
 *   n_layers  >= 0; 0 does nothing
 *   lanes     1 .. KVLR_MAX_LANES; 1 issues every layer on `stream` itself
 * With lanes > 1 the layers' workspaces must not overlap (KVLR_ERR_ARG
 * otherwise), and no layer's output may overlap another layer's inputs or
 * output. Every layer is checked before anything is enqueued: on an error
 * nothing is launched and the first failing layer's status is returned.
 * Calls on one device from several host threads take turns to enqueue; while
 * a call is being captured into a graph, make no other call of this entry
 * point on that device until the capture ends (the lanes are then part of the
 * capture). */
#define KVLR_MAX_LANES 4

typedef struct kvlr_layer {
  const kvlr_desc* desc;
  const float* q;
  const float* P_K;
  const float* P_V;
  const void* lat_k;
  const void* lat_v;
  const int32_t* seq_lens;
  float scale;
  float* out;
  void* workspace;
  size_t workspace_bytes;
  int32_t split_tokens;
} kvlr_layer;

KVLR_API int kvlr_decode_attn_layers(const kvlr_layer* layers, int32_t n_layers, int32_t lanes, void* stream);

/* kvlr_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments and result are those of kvlr_decode_attn without the workspace:
 * the workspace is a static device array owned by the library,
 * KVLR_STATIC_SCRATCH_BYTES (16 MiB) per device, held until the process ends.
 * A call whose kvlr_decode_workspace_bytes(desc, split_tokens) exceeds that
 * returns KVLR_ERR_SCRATCH and launches nothing. The call allocates nothing.
 * The first call on a device does a one-time set-up with that device current
 * (looks up the array's device address, and zeroes the array on `stream`);
 * make that first call outside graph capture. Every call on a device shares
 * that device's array and leaves its counters zero: calls that overlap on one
 * device (concurrent streams or threads) race and must not be made; calls
 * ordered on one stream are safe. */
KVLR_API int kvlr_decode_attn_noalloc(const kvlr_desc* desc, const float* q, const float* P_K, const float* P_V,
                                      const void* lat_k, const void* lat_v, const int32_t* seq_lens, float scale,
                                      float* out, int32_t split_tokens, void* stream);

/* The two stages of kvlr_decode_attn, for callers that schedule them
 * separately (e.g. to time or overlap them). kvlr_decode_partials(...)
 * followed by kvlr_decode_combine(...) on the same stream with the same
 * workspace and split_tokens gives kvlr_decode_attn's result: with a fixed
 * split length the same split records, merged in another order (per-head
 * values: fp32 rounding of the merge may differ; joint bf16 values: bit for
 * bit, the launches are the same); where kvlr_decode_attn takes the balanced
 * plan, other cuts of the sequences, so the softmax weights round differently
 * (about 1e-5 relative).
 *
 * The two stages always take a fixed split length (split_tokens -1 means the
 * library's fixed choice here).
 *
 * kvlr_decode_partials: query projection q~ = q P_K, latent scores, online
 * softmax and the p-weighted sum of value latents for every split of every
 * (batch row, query head). Writes one record (running max in log2 units,
 * softmax denominator, unnormalised latent sum of r_v(h) channels) per
 * split into the record region of `workspace`; arguments as in
 * kvlr_decode_attn. Neither stage reads or writes the counter region. */
KVLR_API int kvlr_decode_partials(const kvlr_desc* desc, const float* q, const float* P_K, const void* lat_k,
                                  const void* lat_v, const int32_t* seq_lens, float scale, void* workspace,
                                  size_t workspace_bytes, int32_t split_tokens, void* stream);

/* kvlr_decode_combine: log-sum-exp merge of the split records written by
 * kvlr_decode_partials with the same desc and split_tokens, normalisation,
 * and back-projection o = o_lat P_V[h]^T (the value reconstruction of
 * "Mecanismo Central" item 5, applied once per query head). Writes
 * out [B][Hq][d] fp32; rows with an empty cache are zero. */
KVLR_API int kvlr_decode_combine(const kvlr_desc* desc, const float* P_V, const void* workspace,
                                 size_t workspace_bytes, int32_t split_tokens, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVLR_H */

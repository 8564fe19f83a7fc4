/*
 * qsparse.h -- C ABI of the decode-time sparse top-k KV-block attention library
 * (libqsparse.so, HIP kernels for CDNA4 / gfx950).
 *
 * The operations, in the order a serving loop uses them:
 *   at prefill
 *     qs_build_metadata      per-block, per-channel max/min of K;
 *     qs_prefill_importance  page 1's per-token importance (for qs_probe_select);
 *   every BS decoded tokens
 *     qs_update_metadata     max/min of only the blocks completed since the last refresh;
 *   every decode step
 *     qs_block_select        Quest top-k block selection on the grouped query, optional
 *                            sink / local-window forcing;   (or)
 *     qs_probe_select        probe + prefill-importance + recency block selection;
 *     qs_sparse_attn_decode  exact softmax attention over the selected blocks only;
 *     qs_select_attn_decode  qs_block_select then qs_sparse_attn_decode in one call;
 *     qs_probe_attn_decode   qs_probe_select then qs_sparse_attn_decode (one selection row
 *                            per query head) in one call.
 *
 * Sources, cited by page title and section:
 *   [P1] "0.8MB 跑通 Qwen | 第 10-2 篇: 推理引擎的 sparse top-k 块选择"
 *        (developer.aliyun.com/article/1767763).
 *   [P3] "ops-transformer select_attention_operators: 基于 Quest 在 Ascend 910B 上实现
 *        稀疏注意力块预测的加速内核" (bjdmk.com.cn/news/4805529).
 *
 * Conventions shared by every call
 *   - Sizes: B requests, H query heads, N KV heads (H % N == 0, G = H / N query heads
 *     per KV head, grouped contiguously: KV head n serves heads n*G .. n*G+G-1),
 *     D = 128 head dimension, BS = block_size tokens per KV block (16, 32, 64 or 128).
 *     A request with L tokens has nb = ceil(L / BS) blocks, numbered 0 .. nb-1 in
 *     sequence order ("sequence-relative" indices).
 *   - Pointers: every array argument is a device pointer to caller-owned, contiguous,
 *     row-major memory in the layout stated next to it. The library never allocates,
 *     frees or keeps a pointer after the call returns.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream). Every call only
 *     enqueues work on it and returns without synchronising.
 *   - Errors: arguments the host can see are checked before any HIP call; a failed
 *     check returns QS_ERR_INVALID (inconsistent or null arguments) or
 *     QS_ERR_UNSUPPORTED (valid but not implemented: D != 128, other block sizes or
 *     dtypes) and enqueues nothing. A failed launch returns QS_ERR_HIP. qs_last_error()
 *     gives a message for the calling thread's last failure. Nothing aborts or prints.
 *   - Device-resident data (seq_lens, tables, selections) is read by the kernels. Table
 *     entries out of range are never dereferenced: the block they name is skipped.
 *     Negative seq_lens count as 0.
 *   - Checked build (libqsparse_checked.so, same kernels and signatures; qs_checked_build()
 *     returns 1): before its own kernels, every call checks on its stream the device-resident
 *     entries it will use, waits for that check, and returns QS_ERR_INVALID, with a message
 *     naming the first bad entry (lowest request first), if any is out of range:
 *       qs_build_metadata, qs_update_metadata: ceil(L / BS) <= max_kv_blocks_per_req,
 *         its metadata blocks <= max_meta_blocks_per_req, and the block_tables and
 *         metadata_block_tables entries of every block the call reduces (all blocks, or
 *         the refreshed range) in [0, num_kv_blocks) and [0, num_meta_blocks);
 *       qs_block_select: ceil(L / BS) <= max_meta_blocks_per_req * BS and the
 *         metadata_block_tables entry of every block of the request (forced ones too);
 *       qs_probe_select, qs_probe_attn_decode: ceil(L / BS) <= max_kv_blocks_per_req and
 *         every block's block_tables entry;
 *       qs_sparse_attn_decode: the block_tables entry of every selected entry it attends
 *         (slots below the clamped n_selected that name a block < min(nb, width));
 *       qs_select_attn_decode: the qs_block_select rules and the block_tables entry of
 *         every block < min(nb, max_kv_blocks_per_req);
 *       qs_prefill_importance: L <= max_len, ceil(L / BS) <= max_kv_blocks_per_req and
 *         every block's block_tables entry.
 *     The check allocates and frees one 8-byte device word and synchronises the stream, so
 *     the checked build is for debugging; a call under stream capture returns
 *     QS_ERR_UNSUPPORTED.
 *   - Determinism: identical inputs give bit-identical outputs ([P1] section 1: same
 *     query and same KV must select the same blocks; ties go to the lower index).
 *   - Workspaces: calls that take `workspace` use it as scratch for scores and partial
 *     results; its contents on entry are ignored. It must be 256-byte aligned, at least
 *     the size the matching *_workspace_bytes() returns, and not used by calls that may
 *     run concurrently (calls on one stream are ordered). Kernels never synchronise
 *     across workgroups; a call may run as several stream-ordered kernels.
 *   - Placement (speed only; any 16-byte aligned base is accepted and results do not
 *     depend on it): the kernels read a head's K and V rows together, and a block's max
 *     and min rows together, at the same offset inside their pools. When the two pools'
 *     base addresses also agree modulo 1 KiB (as separate allocations, or the two halves
 *     of one [2, ...] pool, usually do), each such pair falls in one 256-byte address
 *     class, which MI355X's memory serves more slowly. Start the V pool 256 bytes past a
 *     1 KiB multiple from the K pool, and the min pool likewise from the max pool: the
 *     serving-size fused step (128 requests, 1.21 GB) measured 195 -> 187 us with that.
 */
#ifndef QSPARSE_H
#define QSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QS_OK = 0,
    QS_ERR_INVALID = 1,
    QS_ERR_UNSUPPORTED = 2,
    QS_ERR_HIP = 3
} qs_status;

typedef enum {
    QS_F32 = 0,  /* IEEE binary32 */
    QS_BF16 = 1, /* bfloat16 (upper half of a binary32) */
    QS_I8 = 2,   /* int8 codes with fp32 per-row scales (KV caches only) */
    QS_F16 = 3   /* IEEE binary16 */
} qs_dtype;

/* flag bits of the selection calls */
enum {
    QS_FORCE_SINK = 1u,   /* qs_block_select: always include block 0 */
    QS_FORCE_WINDOW = 2u, /* qs_block_select: always include the local-window blocks */
    QS_RECENCY = 4u       /* qs_probe_select: recency insurance for the last block */
};

/*
 * qs_build_metadata -- Quest block metadata.
 * [P3] "quest_prefill_metadata: 元数据构建原理": for every KV block of every request and
 * every KV head, the per-channel max and min of K over the block's tokens (the last
 * block of a request over its valid tokens only). The BS vectors of BS consecutive
 * blocks of a request fill one metadata block (same shape as a KV block), placed by
 * metadata_block_tables; the unused rows of a request's last metadata block are set
 * to +0.0 ([P3] "三个核心算子": absent blocks' metadata must be 0).
 *
 *   k_cache                [num_kv_blocks, BS, N, D], kv_dtype QS_F32, QS_BF16 or QS_F16
 *   block_tables           [B, max_kv_blocks_per_req] int32, physical KV block of
 *                          sequence block i of request b
 *   seq_lens               [B] int32, tokens the metadata covers for each request
 *   metadata_block_tables  [B, max_meta_blocks_per_req] int32, physical metadata block
 *                          holding blocks j*BS .. j*BS+BS-1 of request b
 *   maxblocks, minblocks   [num_meta_blocks, BS, N, D], same dtype as k_cache (outputs)
 * Results are bit-exact: max/min use the IEEE total order (-0 < +0). Metadata blocks
 * and rows beyond a request's last used metadata block are left untouched.
 */
qs_status qs_build_metadata(int32_t B, int32_t N, int32_t D, int32_t block_size, qs_dtype kv_dtype,
                            const void* k_cache, int32_t num_kv_blocks,
                            const int32_t* block_tables, int32_t max_kv_blocks_per_req,
                            const int32_t* seq_lens,
                            const int32_t* metadata_block_tables, int32_t max_meta_blocks_per_req,
                            void* maxblocks, void* minblocks, int32_t num_meta_blocks,
                            void* stream);

/*
 * qs_update_metadata -- refresh the Quest metadata of the newest blocks only.
 * [P3] "生产实践建议": the metadata is built once after prefill and then refreshed every
 * 128 decoded tokens. A refresh needs only the blocks whose tokens changed since the
 * last one, so this call recomputes, for each request b, the sequence blocks
 *     i = first_block[b] ... min(nb_b, first_block[b] + max_new_blocks) - 1
 * (negative first_block entries count as 0; nb_b = ceil(seq_lens[b] / BS)) with exactly
 * the per-channel max/min qs_build_metadata writes for them, bit for bit. No other row is
 * written: rows past nb_b are not zero-filled, so metadata blocks must start zeroed
 * (as from a zero-filled pool) where a consumer needs the +0.0 rows of absent blocks.
 * A refresh after the last one covered L_old tokens passes first_block = floor(L_old / BS)
 * (the block that was partial then) and max_new_blocks >= the blocks added since.
 *
 *   arguments as qs_build_metadata, plus
 *   first_block     [B] int32 (device), first sequence block to recompute per request
 *   max_new_blocks  host bound on the blocks recomputed per request (>= 1)
 */
qs_status qs_update_metadata(int32_t B, int32_t N, int32_t D, int32_t block_size, qs_dtype kv_dtype,
                             const void* k_cache, int32_t num_kv_blocks,
                             const int32_t* block_tables, int32_t max_kv_blocks_per_req,
                             const int32_t* seq_lens, const int32_t* first_block,
                             int32_t max_new_blocks,
                             const int32_t* metadata_block_tables, int32_t max_meta_blocks_per_req,
                             void* maxblocks, void* minblocks, int32_t num_meta_blocks,
                             void* stream);

/* bytes of workspace qs_block_select needs for these sizes */
size_t qs_block_select_workspace_bytes(int32_t B, int32_t N, int32_t block_size,
                                       int32_t max_meta_blocks_per_req);

/*
 * qs_block_select -- Quest top-k block selection.
 * [P3] "quest_block_select_paged: 解码期 top-k 预测算法": the grouped query of KV head n
 * is the mean of its G query heads; the score of block i is
 *     sum_d max(gq_d * kmax_d, gq_d * kmin_d),
 * an upper bound of gq . k for every key k of the block; the k best blocks are returned
 * as sequence-relative indices. [P3] "三个核心算子", variant _w: the sink block and the
 * local-window blocks can be forced in; [P1] section 1: ties go to the lower index.
 *
 *   query                  [B, H, D], dtype QS_F32, QS_BF16 or QS_F16 (metadata has the same dtype)
 *   maxblocks, minblocks   [num_meta_blocks, BS, N, D] (as written by qs_build_metadata)
 *   metadata_block_tables  [B, max_meta_blocks_per_req] int32
 *   seq_lens               [B] int32, tokens in each request (blocks 0..nb-1 are candidates)
 *   tokens_since_update    [B] int32 or NULL (= all 0): tokens decoded since the metadata
 *                          was built; blocks from floor((L - u) / BS) on have no metadata.
 *                          A negative entry turns forcing off for that request.
 *   flags                  QS_FORCE_SINK | QS_FORCE_WINDOW (other bits invalid)
 *   k                      >= 1 blocks per (request, KV head)
 *   selected               [B, N, k] int32 output: ascending block indices, then -1s
 *   n_selected             [B, N] int32 output: min(k, nb)
 *   block_scores           [B, N, max_meta_blocks_per_req * BS] fp32 output or NULL: the
 *                          score of every non-forced block i < nb (NaN for forced blocks;
 *                          entries i >= nb are not written)
 * Forcing: with QS_FORCE_WINDOW the last block and every block without metadata are
 * forced, the most recent first; with QS_FORCE_SINK block 0 is forced after them; at
 * most k blocks are forced. The other min(k, nb) - forced picks are the best-scoring
 * remaining blocks (higher score first, lower index on ties).
 */
qs_status qs_block_select(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size, qs_dtype dtype,
                          const void* query, const void* maxblocks, const void* minblocks,
                          int32_t num_meta_blocks,
                          const int32_t* metadata_block_tables, int32_t max_meta_blocks_per_req,
                          const int32_t* seq_lens, const int32_t* tokens_since_update,
                          uint32_t flags, int32_t k,
                          int32_t* selected, int32_t* n_selected, float* block_scores,
                          void* workspace, size_t workspace_bytes, void* stream);

/* bytes of workspace qs_probe_select needs for these sizes (B * H *
 * max_kv_blocks_per_req probe keys, rounded up to 256) */
size_t qs_probe_select_workspace_bytes(int32_t B, int32_t H, int32_t max_kv_blocks_per_req);

/*
 * qs_probe_select -- page 1's probe + importance + recency selection, per query head.
 * [P1] sections 1 and 2 (sparse_attn_head): for query head h (KV head h / G) the probe
 * score of a block is the max of the unscaled q_h . K over the positions p0, p0+step, ...
 * inside the block, step = max(1, block_tokens / n_probe); (k+1)/2 picks go first to the
 * blocks with the largest summed prefill importance (fp32 sum in token order), the rest
 * to the best probe scores (ties: lower index); with QS_RECENCY, if the last block is
 * not picked it replaces the lowest-scoring probe pick (never an importance pick).
 *
 *   query          [B, H, D], q_dtype QS_F32, QS_BF16 or QS_F16
 *   k_cache        [num_kv_blocks, BS, N, D], kv_dtype QS_F32, QS_BF16 or QS_F16
 *   block_tables   [B, max_kv_blocks_per_req] int32 (max_kv_blocks_per_req <= 4096)
 *   seq_lens       [B] int32
 *   importance     [B, importance_stride] fp32 per-token prefill importance, or NULL
 *                  (then every pick is a probe pick); tokens at or past importance_stride
 *                  contribute nothing
 *   n_probe        probes per block (values < 1 act as 1)
 *   flags          0 or QS_RECENCY
 *   selected       [B, H, k] int32 output (ascending, -1 padded); n_selected [B, H] int32
 *   probe_scores   [B, H, max_kv_blocks_per_req] fp32 output or NULL (entries i >= nb
 *                  are not written)
 *   workspace      device scratch of at least qs_probe_select_workspace_bytes(), 256-byte
 *                  aligned, contents ignored
 */
qs_status qs_probe_select(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size,
                          qs_dtype q_dtype, qs_dtype kv_dtype,
                          const void* query, const void* k_cache, int32_t num_kv_blocks,
                          const int32_t* block_tables, int32_t max_kv_blocks_per_req,
                          const int32_t* seq_lens,
                          const float* importance, int32_t importance_stride,
                          int32_t n_probe, int32_t k, uint32_t flags,
                          int32_t* selected, int32_t* n_selected, float* probe_scores,
                          void* workspace, size_t workspace_bytes, void* stream);

/* bytes of workspace qs_sparse_attn_decode needs for these sizes */
size_t qs_sparse_attn_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D, int32_t sel_heads,
                                      int32_t k);

/*
 * qs_sparse_attn_decode -- exact attention over the selected blocks.
 * [P1] section 2: per-token scores only on the selected blocks (fp32 / bf16 K: float
 * dot; int8 K: int8 x int8 dot times the scales), softmax renormalised over the
 * selected tokens only, then the weighted sum of V. [P3] "quest_block_select_paged"
 * notes: selected indices are sequence-relative and go through block_tables.
 *
 *   query          [B, H, D], q_dtype QS_F32, QS_BF16 or QS_F16; out [B, H, D] in q_dtype
 *   k_cache/v_cache[num_kv_blocks, BS, N, D], kv_dtype QS_F32, QS_BF16, QS_F16 or QS_I8
 *                  (bf16 and f16 with a query of the same dtype run on the matrix cores,
 *                  with P rounded to that format; other pairs on the vector ALU in fp32)
 *   k_scale/v_scale[num_kv_blocks, BS, N] fp32 per-row scales (QS_I8 only, else ignored)
 *   block_tables   [B, max_kv_blocks_per_req] int32; seq_lens [B] int32
 *   selected       [B, sel_heads, k] int32; n_selected [B, sel_heads] int32 (entries
 *                  past n_selected, negative ones and ones >= nb are skipped; every other
 *                  entry is attended once per occurrence)
 *   sel_heads      selection rows per request: N (one per KV head, qs_block_select) or H
 *                  (one per query head, qs_probe_select); any value with
 *                  N | sel_heads | H. Query head h uses row h / (H / sel_heads).
 *   softmax_scale  logit = softmax_scale * q . k; <= 0 selects 1/sqrt(D)
 * int8: the query row of each head is quantised with s_q = absmax / 127 and codes
 * clamp(rint(q / s_q), -127, 127) (fp32, half to even); logit =
 * softmax_scale * float(int32 dot) * s_q * k_scale[t]; V[t] = v_code * v_scale[t].
 * An empty selection writes zeros.
 */
qs_status qs_sparse_attn_decode(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size,
                                qs_dtype q_dtype, qs_dtype kv_dtype,
                                const void* query, const void* k_cache, const void* v_cache,
                                const float* k_scale, const float* v_scale, int32_t num_kv_blocks,
                                const int32_t* block_tables, int32_t max_kv_blocks_per_req,
                                const int32_t* seq_lens,
                                const int32_t* selected, const int32_t* n_selected,
                                int32_t sel_heads, int32_t k, float softmax_scale,
                                void* out, void* workspace, size_t workspace_bytes, void* stream);

/* bytes of workspace qs_select_attn_decode needs for these sizes (0 for invalid sizes) */
size_t qs_select_attn_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t block_size,
                                      int32_t max_meta_blocks_per_req, int32_t k, qs_dtype dtype);

/*
 * qs_select_attn_decode -- Quest selection and the attention over the selected blocks in
 * one call. [P3] "quest_block_select_paged: 解码期 top-k 预测算法" and "三个核心算子", [P1]
 * section 2 (the attention loop runs over the blocks the selection points to). The
 * result is, by definition, qs_block_select (flags, tokens_since_update and k as there)
 * followed by qs_sparse_attn_decode with sel_heads = N on that selection: the same
 * output and, when selected / n_selected are given, the same selection. Rows of up to 64
 * selected blocks and 4096 candidate blocks run as one kernel that keeps the selection
 * on chip; other sizes run the two operations' kernels back to back.
 *
 *   dtype          QS_BF16, QS_F16 or QS_F32, for query, metadata and K/V alike
 *   query ... tokens_since_update, flags, k   as qs_block_select
 *   k_cache ... max_kv_blocks_per_req, softmax_scale   as qs_sparse_attn_decode
 *   out            [B, H, D] in dtype
 *   selected       [B, N, k] int32 and n_selected [B, N] int32 outputs, or both NULL
 *   workspace      at least qs_select_attn_workspace_bytes(); 256-byte aligned
 */
qs_status qs_select_attn_decode(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size,
                                qs_dtype dtype, const void* query,
                                const void* maxblocks, const void* minblocks, int32_t num_meta_blocks,
                                const int32_t* metadata_block_tables, int32_t max_meta_blocks_per_req,
                                const void* k_cache, const void* v_cache, int32_t num_kv_blocks,
                                const int32_t* block_tables, int32_t max_kv_blocks_per_req,
                                const int32_t* seq_lens, const int32_t* tokens_since_update,
                                uint32_t flags, int32_t k, float softmax_scale, void* out,
                                int32_t* selected, int32_t* n_selected,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * qs_select_attn_decode_static -- qs_select_attn_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same kernels and results.
 * Its scratch is a static device array of the library (QS_STATIC_SCRATCH_BYTES of
 * workspace plus 256 bytes), one per GPU, held from the device's first call until the
 * process ends; the call allocates and frees nothing (the checked build's verdict word is
 * in that array too). Sizes whose workspace (qs_select_attn_workspace_bytes()) exceeds
 * QS_STATIC_SCRATCH_BYTES return QS_ERR_INVALID before any HIP call. The array belongs
 * to the current device, which must be the stream's. Every call on one GPU shares it and
 * it keeps the last call's contents (no kernel needs it cleared): calls that may overlap
 * on one GPU (other streams, other threads, concurrent graph replays) race and must be
 * ordered by the caller. The device's first call looks up the array's address; make it
 * before a graph capture.
 */
#define QS_STATIC_SCRATCH_BYTES (32u << 20)
qs_status qs_select_attn_decode_static(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size,
                                       qs_dtype dtype, const void* query,
                                       const void* maxblocks, const void* minblocks, int32_t num_meta_blocks,
                                       const int32_t* metadata_block_tables, int32_t max_meta_blocks_per_req,
                                       const void* k_cache, const void* v_cache, int32_t num_kv_blocks,
                                       const int32_t* block_tables, int32_t max_kv_blocks_per_req,
                                       const int32_t* seq_lens, const int32_t* tokens_since_update,
                                       uint32_t flags, int32_t k, float softmax_scale, void* out,
                                       int32_t* selected, int32_t* n_selected, void* stream);

/* bytes of workspace qs_probe_attn_decode needs for these sizes (the probe keys, then the
 * attention partials; 0 for invalid sizes) */
size_t qs_probe_attn_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t max_kv_blocks_per_req, int32_t k);

/*
 * qs_probe_attn_decode -- page 1's probe selection and exact attention over it, in one
 * call. [P1] section 2 (sparse_attn_head): the selection of each query head feeds that
 * head's attention loop directly, over a float KV cache or a q8 one (int8 x int8 dot plus
 * the scales). The result is defined as qs_probe_select (on the float K the probes read)
 * followed by qs_sparse_attn_decode with sel_heads = H and the same k: the selection is
 * bitwise the one qs_probe_select returns, the output matches the two calls within the
 * attention's rounding (the pick is recomputed by each slot split of a row; it is
 * deterministic, so every split sees the same selection).
 *
 *   query          [B, H, D], q_dtype QS_F32, QS_BF16 or QS_F16; out [B, H, D] in q_dtype
 *   k_cache/v_cache[num_kv_blocks, BS, N, D], kv_dtype QS_F32, QS_BF16, QS_F16 or QS_I8
 *   k_scale/v_scale[num_kv_blocks, BS, N] fp32 per-row scales: required for QS_I8, NULL
 *                  otherwise
 *   probe_k_cache  the float K the probe scores read, [num_kv_blocks, BS, N, D] in
 *                  probe_k_dtype (QS_F32, QS_BF16 or QS_F16), paged like k_cache: required
 *                  for QS_I8 (the same call as qs_probe_select on it); NULL for a float
 *                  cache, whose k_cache the probes read (probe_k_dtype is then ignored)
 *   block_tables   [B, max_kv_blocks_per_req] int32 (max_kv_blocks_per_req <= 4096);
 *                  seq_lens [B] int32
 *   importance, importance_stride, n_probe, flags   as for qs_probe_select
 *   k              1 .. 4096 blocks per query head
 *   softmax_scale  logit = softmax_scale * q . k; <= 0 selects 1/sqrt(D)
 *   selected       [B, H, k] int32 output (ascending, -1 padded) and n_selected [B, H],
 *                  or both NULL
 *   workspace      device scratch of at least qs_probe_attn_workspace_bytes(), 256-byte
 *                  aligned, contents ignored
 * Attention runs on the vector ALU in fp32 for every dtype pair (QS_I8: the query is
 * quantised per head as in qs_sparse_attn_decode). An empty selection writes zeros.
 */
qs_status qs_probe_attn_decode(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size,
                               qs_dtype q_dtype, qs_dtype kv_dtype,
                               const void* query, const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale,
                               const void* probe_k_cache, qs_dtype probe_k_dtype,
                               int32_t num_kv_blocks, const int32_t* block_tables,
                               int32_t max_kv_blocks_per_req, const int32_t* seq_lens,
                               const float* importance, int32_t importance_stride,
                               int32_t n_probe, int32_t k, uint32_t flags, float softmax_scale,
                               void* out, int32_t* selected, int32_t* n_selected,
                               void* workspace, size_t workspace_bytes, void* stream);

/* bytes of workspace qs_prefill_importance can use (0 for invalid sizes): B * H * max_len
 * floats of row normalisers plus, per chunk of the causal work, three more (a job of fewer
 * than 8192 tiles of 64 rows x heads x requests is cut into up to 8 chunks) -- the minimum
 * the call accepts -- then, when the causal score matrices of all heads and requests take
 * at most 2 GiB in fp32 (B * H * T (T + 1) / 2 blocks of 16 x 16, T = ceil(max_len / 16)),
 * room for them: an fp32 call given that much stores its scores in the first pass and reads
 * them back in the second instead of computing them again (same results up to the order of
 * the fp32 column sums) */
size_t qs_prefill_importance_workspace_bytes(int32_t B, int32_t H, int32_t max_len);

/*
 * qs_prefill_importance -- the prefill importance that qs_probe_select consumes.
 * [P1] section 1, signal 2 (how much attention the prefill really gave each token,
 * recorded per head, reduced over heads) and section 2's closing note (each head's record
 * is added into prefill_importance[s] when the prefill ends). With exact causal prefill
 * attention, head h (KV head h / (H / N)) gives key s the weight
 *     p_h[t][s] = exp(c q_{t,h} . k_s) / sum_{s' <= t} exp(c q_{t,h} . k_{s'})   (s <= t < L)
 * in query row t; head_importance[b][h][s] = sum over t of p_h[t][s] and
 * importance[b][s] = sum over h of head_importance[b][h][s], for s < L = seq_lens[b];
 * entries s >= L (up to importance_stride) are written as 0.
 *
 *   query              [B, max_len, H, D] prefill query rows, dtype QS_F32, QS_BF16 or QS_F16
 *   k_cache            [num_kv_blocks, BS, N, D] in the same dtype, the prompt's keys through
 *                      block_tables [B, max_kv_blocks_per_req]; seq_lens [B] prompt lengths
 *                      (clamped to max_len and to the table's capacity)
 *   softmax_scale      c; <= 0 selects 1/sqrt(D)
 *   importance         [B, importance_stride] fp32 output, or NULL
 *   head_importance    [B, H, importance_stride] fp32 output, or NULL (not both NULL)
 *   workspace          256-byte aligned; the minimum of qs_prefill_importance_workspace_bytes()
 *                      (its size without the stored scores) is accepted, the full size lets
 *                      fp32 inputs skip the recomputation
 * Dot products run on the matrix cores in fp32 accumulation from exactly widened inputs;
 * chunk partials and heads are summed in a fixed order, so results are deterministic.
 */
qs_status qs_prefill_importance(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size,
                                qs_dtype dtype, const void* query, int32_t max_len,
                                const void* k_cache, int32_t num_kv_blocks,
                                const int32_t* block_tables, int32_t max_kv_blocks_per_req,
                                const int32_t* seq_lens, float softmax_scale,
                                float* importance, int32_t importance_stride,
                                float* head_importance,
                                void* workspace, size_t workspace_bytes, void* stream);

/* message for the calling thread's last failed call ("" if none) */
const char* qs_last_error(void);

/* library version string */
const char* qs_version(void);

/* 1 in the checked build (libqsparse_checked.so), 0 in libqsparse.so */
int32_t qs_checked_build(void);

#ifdef __cplusplus
}
#endif

#endif /* QSPARSE_H */

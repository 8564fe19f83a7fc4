/*
 * qs_oracle.c -- plain, slow, single-threaded CPU statement of the decode-time sparse
 * attention path (Quest block metadata, top-k block selection, page 1's probe
 * selection, exact attention over the selected blocks).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls this
 * file: only the tests, the smoke check and the benchmark's CPU-baseline leg do. It
 * shares no code, header, table or helper with the HIP library.
 *
 * Sources (cited by page title and section):
 *   [P1] "0.8MB 跑通 Qwen | 第 10-2 篇: 推理引擎的 sparse top-k 块选择"
 *        (developer.aliyun.com/article/1767763) -- sections 1 "知识点" and 2 "对应代码".
 *   [P3] "ops-transformer select_attention_operators: 基于 Quest 在 Ascend 910B 上实现
 *        稀疏注意力块预测的加速内核" (bjdmk.com.cn/news/4805529) -- sections
 *        "三个核心算子", "quest_prefill_metadata: 元数据构建原理",
 *        "quest_block_select_paged: 解码期 top-k 预测算法", "使用示例".
 *
 * Arithmetic: dot products, means and softmax accumulate in double. Quantities that
 * the path must reproduce bit for bit are computed in the precision the path uses:
 * max/min of stored keys (exact), the fp32 running sum of prefill importance per block
 * ([P1] section 2 probe loop accumulates a float per block), and the fp32 int8
 * quantiser of the query. bf16 values are widened exactly (bits << 16); IEEE binary16
 * values are decoded exactly from their sign, exponent and fraction fields.
 *
 * Readings where the pages are silent or ambiguous are marked "reading:" below.
 *
 * Parity pins: every function here is pinned by tests against library routines,
 * closed forms, invariants and brute force (see the oracle tests); none is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { QSO_F32 = 0, QSO_BF16 = 1, QSO_I8 = 2, QSO_F16 = 3 };
enum { QSO_FORCE_SINK = 1u, QSO_FORCE_WINDOW = 2u, QSO_RECENCY = 4u };
enum { QSO_OK = 0, QSO_BAD = -1 };

/* ------------------------------------------------------------------------------------ */
/* element access                                                                        */
/* ------------------------------------------------------------------------------------ */

static float bf16_bits_to_float(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0
 * holds zeros and subnormals (fraction * 2^-24), exponent 31 infinities and NaNs. Every
 * binary16 value is exactly representable as a float. */
static float f16_bits_to_float(uint16_t h) {
    const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    float v;
    if (e == 0) v = ldexpf((float)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexpf((float)(1024 + m), e - 25);
    return sign ? -v : v;
}

static int is_half(int dtype) { return dtype == QSO_BF16 || dtype == QSO_F16; }
static int is_float(int dtype) { return dtype == QSO_F32 || is_half(dtype); }

/* value of element idx of an array of the given dtype, as float (exact widening) */
static float elem_f(const void* base, int dtype, size_t idx) {
    if (dtype == QSO_F32) return ((const float*)base)[idx];
    if (dtype == QSO_BF16) return bf16_bits_to_float(((const uint16_t*)base)[idx]);
    if (dtype == QSO_F16) return f16_bits_to_float(((const uint16_t*)base)[idx]);
    return (float)((const int8_t*)base)[idx];
}

/* the element widening above, exported so that tests can pin it against a library decoder */
void qso_widen(int dtype, const void* in, int n, double* out) {
    for (int i = 0; i < n; ++i) out[i] = (double)elem_f(in, dtype, (size_t)i);
}

static int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int64_t floor_div64(int64_t a, int64_t b) {
    int64_t q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
    return q;
}

/* number of blocks of a request: every block holding at least one of its L tokens */
static int32_t n_blocks_of(int32_t L, int32_t BS) {
    if (L <= 0) return 0;
    return (int32_t)ceil_div64(L, BS);
}

/* reading: inputs are finite; max/min follow the IEEE total order, in which -0 < +0,
 * so the stored extreme does not depend on how an instruction treats signed zeros. */
static int total_greater(float a, float b) {
    if (a > b) return 1;
    if (a < b) return 0;
    return (!signbit(a)) && signbit(b); /* a == b: only +0 beats -0 */
}

/* ------------------------------------------------------------------------------------ */
/* O1: block metadata                                                                    */
/* ------------------------------------------------------------------------------------ */
/*
 * [P3] "quest_prefill_metadata: 元数据构建原理": for every KV block and KV head, reduce K
 * over the block's tokens channel by channel to a max vector and a min vector; the last
 * block of a request only covers its valid tokens. BLOCK_SIZE such vectors (one per KV
 * block of the request, in sequence order) fill one metadata block, which has a KV
 * block's shape [BS, N, D] and is placed by metadata_block_tables. Unused rows of the
 * request's last metadata block are set to 0 (the "Duplicate(0.0f)" tail fill), which
 * the select side relies on ([P3] "三个核心算子": absent blocks' metadata must be 0).
 *
 * reading: metadata blocks past the request's last used one are not touched.
 * Layouts: k_cache [num_kv_blocks, BS, N, D]; maxb/minb [num_meta_blocks, BS, N, D] in
 * the same dtype as k_cache (f32 or bf16), written bit-exactly from the winning key.
 */
/* max/min of one sequence block i of request b into its metadata row (O1's inner step) */
static int reduce_block(int N, int D, int BS, int dtype, const void* k_cache, int num_kv_blocks,
                        const int32_t* block_tables, int mkbpr, const int32_t* meta_tables, int mmbpr,
                        void* maxb, void* minb, int num_meta_blocks, int b, int32_t L, int32_t i) {
    const size_t row = (size_t)N * D;
    const int32_t phys = block_tables[(size_t)b * mkbpr + i];
    const int32_t m = meta_tables[(size_t)b * mmbpr + i / BS];
    if (phys < 0 || phys >= num_kv_blocks || m < 0 || m >= num_meta_blocks) return QSO_BAD;
    const int32_t r = i % BS;
    int32_t nt = L - i * BS;
    if (nt > BS) nt = BS;
    for (int n = 0; n < N; ++n) {
        for (int d = 0; d < D; ++d) {
            size_t best_hi = ((size_t)phys * BS + 0) * row + (size_t)n * D + d;
            size_t best_lo = best_hi;
            for (int32_t t = 1; t < nt; ++t) {
                const size_t idx = ((size_t)phys * BS + t) * row + (size_t)n * D + d;
                const float x = elem_f(k_cache, dtype, idx);
                if (total_greater(x, elem_f(k_cache, dtype, best_hi))) best_hi = idx;
                if (total_greater(elem_f(k_cache, dtype, best_lo), x)) best_lo = idx;
            }
            const size_t o = ((size_t)m * BS + r) * row + (size_t)n * D + d;
            if (dtype == QSO_F32) {
                ((float*)maxb)[o] = ((const float*)k_cache)[best_hi];
                ((float*)minb)[o] = ((const float*)k_cache)[best_lo];
            } else {
                ((uint16_t*)maxb)[o] = ((const uint16_t*)k_cache)[best_hi];
                ((uint16_t*)minb)[o] = ((const uint16_t*)k_cache)[best_lo];
            }
        }
    }
    return QSO_OK;
}

int qso_build_metadata(int B, int N, int D, int BS, int dtype,
                       const void* k_cache, int num_kv_blocks,
                       const int32_t* block_tables, int mkbpr,
                       const int32_t* seq_lens,
                       const int32_t* meta_tables, int mmbpr,
                       void* maxb, void* minb, int num_meta_blocks) {
    if (!is_float(dtype)) return QSO_BAD;
    const size_t row = (size_t)N * D;
    for (int b = 0; b < B; ++b) {
        const int32_t L = seq_lens[b];
        const int32_t nb = n_blocks_of(L, BS);
        if (nb > mkbpr || ceil_div64(nb, BS) > mmbpr) return QSO_BAD;
        for (int32_t i = 0; i < nb; ++i) {
            const int rc = reduce_block(N, D, BS, dtype, k_cache, num_kv_blocks, block_tables, mkbpr, meta_tables,
                                        mmbpr, maxb, minb, num_meta_blocks, b, L, i);
            if (rc != QSO_OK) return rc;
        }
        if (nb % BS != 0) {
            const int32_t m = meta_tables[(size_t)b * mmbpr + (nb - 1) / BS];
            if (m < 0 || m >= num_meta_blocks) return QSO_BAD;
            for (int32_t r = nb % BS; r < BS; ++r) {
                const size_t o = ((size_t)m * BS + r) * row;
                const size_t bytes = row * (dtype == QSO_F32 ? 4 : 2);
                memset((char*)maxb + o * (dtype == QSO_F32 ? 4 : 2), 0, bytes);
                memset((char*)minb + o * (dtype == QSO_F32 ? 4 : 2), 0, bytes);
            }
        }
    }
    return QSO_OK;
}

/*
 * O1': refresh of the newest blocks.
 * [P3] "生产实践建议": after prefill the metadata is built once, then refreshed every 128
 * decoded tokens. reading: a refresh recomputes, with O1's own per-block step, only
 * sequence blocks first_block[b] .. min(nb, first_block[b] + max_new) - 1 (negative
 * first_block counts as 0) and writes nothing else (no tail fill: rows past nb keep what
 * they held).
 */
int qso_update_metadata(int B, int N, int D, int BS, int dtype,
                        const void* k_cache, int num_kv_blocks,
                        const int32_t* block_tables, int mkbpr,
                        const int32_t* seq_lens, const int32_t* first_block, int max_new,
                        const int32_t* meta_tables, int mmbpr,
                        void* maxb, void* minb, int num_meta_blocks) {
    if (!is_float(dtype)) return QSO_BAD;
    if (max_new < 1) return QSO_BAD;
    for (int b = 0; b < B; ++b) {
        const int32_t L = seq_lens[b];
        const int32_t nb = n_blocks_of(L, BS);
        if (nb > mkbpr || ceil_div64(nb, BS) > mmbpr) return QSO_BAD;
        const int32_t i0 = first_block[b] > 0 ? first_block[b] : 0;
        for (int64_t i = i0; i < nb && i < (int64_t)i0 + max_new; ++i) {
            const int rc = reduce_block(N, D, BS, dtype, k_cache, num_kv_blocks, block_tables, mkbpr, meta_tables,
                                        mmbpr, maxb, minb, num_meta_blocks, b, L, (int32_t)i);
            if (rc != QSO_OK) return rc;
        }
    }
    return QSO_OK;
}

/* ------------------------------------------------------------------------------------ */
/* shared by the selections: ordering "higher value first, lower index on ties"         */
/* ------------------------------------------------------------------------------------ */

typedef struct { double v; int32_t i; } scored_t;

static int cmp_desc_then_index(const void* pa, const void* pb) {
    const scored_t* a = (const scored_t*)pa;
    const scored_t* b = (const scored_t*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->i < b->i) ? -1 : (a->i > b->i);
}

static int cmp_int(const void* pa, const void* pb) {
    const int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

static void write_sorted(int32_t* out, int k, int32_t* picks, int n) {
    qsort(picks, (size_t)n, sizeof(int32_t), cmp_int);
    for (int j = 0; j < k; ++j) out[j] = (j < n) ? picks[j] : -1;
}

/* ------------------------------------------------------------------------------------ */
/* O2: Quest block selection with optional sink / window forcing                         */
/* ------------------------------------------------------------------------------------ */
/*
 * [P3] "quest_block_select_paged: 解码期 top-k 预测算法":
 *   1. per batch, the H query heads are reduced by a mean over every group of H/N heads
 *      to one vector per KV head ("grouped_query[b, n]");
 *   2. for each (b, n), for each metadata row reached through metadata_block_tables:
 *      multiply grouped_query elementwise with the max row and with the min row, take
 *      the elementwise max of the two products and sum over D -> the block score, an
 *      upper bound of grouped_query . k for every key k of the block;
 *   3. top-k block indices over all the request's blocks; indices are sequence-relative
 *      (0 .. blocks-1), not physical.
 * [P3] "三个核心算子", variant _w: the sink block (block 0) and the local-window blocks
 * are forced into the result, decided from tokens_since_metadata_update and seq_len;
 * metadata updates happen only at BLOCK_SIZE multiples; -1 disables the feature.
 * [P1] section 1: equal scores are decided by the lower block index (determinism).
 *
 * readings:
 *  - groups are contiguous: KV head n owns query heads n*G .. n*G+G-1;
 *  - candidates are blocks 0 .. ceil(L/BS)-1 (a partial last block has metadata over its
 *    valid tokens); when k exceeds the block count every block is returned, then -1s;
 *  - window: with u = tsmu[b] (0 when tsmu is NULL), the metadata covers the first
 *    floor((L-u)/BS) blocks; the last block and every block from there on is forced.
 *    Priority when the forced set exceeds k: last block, then the others in descending
 *    order, then the sink. A negative tsmu[b] turns forcing off for request b;
 *  - output ascending by block index, padded with -1; n_selected = number of indices.
 * scores (optional, [B, N, mmbpr*BS]): the fill-stage score of each candidate; NaN for
 * forced blocks and for indices past the request's blocks.
 */
int qso_block_select(int B, int H, int N, int D, int BS, int dtype,
                     const void* query, const void* maxb, const void* minb,
                     const int32_t* meta_tables, int mmbpr, int num_meta_blocks,
                     const int32_t* seq_lens, const int32_t* tsmu,
                     unsigned flags, int k,
                     int32_t* selected, int32_t* n_selected, double* scores) {
    if (!is_float(dtype)) return QSO_BAD;
    if (N <= 0 || H % N != 0 || k < 1) return QSO_BAD;
    const int G = H / N;
    const int cap = mmbpr * BS;
    const size_t row = (size_t)N * D;
    double* gq = (double*)malloc(sizeof(double) * (size_t)D);
    scored_t* cand = (scored_t*)malloc(sizeof(scored_t) * (size_t)(cap > 0 ? cap : 1));
    int32_t* picks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(cap + 1 > k ? cap + 1 : k));
    char* forced = (char*)malloc((size_t)(cap > 0 ? cap : 1));
    int rc = QSO_OK;
    for (int b = 0; b < B && rc == QSO_OK; ++b) {
        const int32_t L = seq_lens[b];
        const int32_t nb = n_blocks_of(L, BS);
        if (nb > cap) { rc = QSO_BAD; break; }
        for (int n = 0; n < N; ++n) {
            /* step 1: grouped query (mean over the group's heads), double */
            for (int d = 0; d < D; ++d) {
                double s = 0.0;
                for (int g = 0; g < G; ++g)
                    s += (double)elem_f(query, dtype, ((size_t)b * H + (size_t)n * G + g) * D + d);
                gq[d] = s / (double)G;
            }
            /* forced set, in priority order */
            int nf = 0;
            memset(forced, 0, (size_t)(cap > 0 ? cap : 1));
            const int active = (tsmu == NULL) || (tsmu[b] >= 0);
            if (active && (flags & QSO_FORCE_WINDOW) && nb > 0) {
                const int64_t u = (tsmu == NULL) ? 0 : tsmu[b];
                int64_t n_meta = floor_div64((int64_t)L - u, BS);
                if (n_meta < 0) n_meta = 0;
                if (n_meta > nb) n_meta = nb;
                if (nf < k && !forced[nb - 1]) { forced[nb - 1] = 1; picks[nf++] = nb - 1; }
                for (int64_t i = nb - 2; i >= n_meta && nf < k; --i)
                    if (!forced[i]) { forced[i] = 1; picks[nf++] = (int32_t)i; }
            }
            if (active && (flags & QSO_FORCE_SINK) && nb > 0 && nf < k && !forced[0]) {
                forced[0] = 1;
                picks[nf++] = 0;
            }
            /* step 2: scores of the remaining candidates */
            int nc = 0;
            for (int32_t i = 0; i < nb; ++i) {
                if (forced[i]) continue;
                const int32_t m = meta_tables[(size_t)b * mmbpr + i / BS];
                if (m < 0 || m >= num_meta_blocks) { rc = QSO_BAD; break; }
                const size_t base = ((size_t)m * BS + (size_t)(i % BS)) * row + (size_t)n * D;
                double s = 0.0;
                for (int d = 0; d < D; ++d) {
                    const double pmax = gq[d] * (double)elem_f(maxb, dtype, base + d);
                    const double pmin = gq[d] * (double)elem_f(minb, dtype, base + d);
                    s += (pmax > pmin) ? pmax : pmin;
                }
                cand[nc].v = s;
                cand[nc].i = i;
                ++nc;
            }
            if (rc != QSO_OK) break;
            if (scores) {
                double* srow = scores + ((size_t)b * N + n) * (size_t)cap;
                for (int i = 0; i < cap; ++i) srow[i] = NAN;
                for (int c = 0; c < nc; ++c) srow[cand[c].i] = cand[c].v;
            }
            /* step 3: top-(k - forced) by (score desc, index asc) */
            int want = (k < nb ? k : nb) - nf;
            if (want < 0) want = 0;
            qsort(cand, (size_t)nc, sizeof(scored_t), cmp_desc_then_index);
            int np = nf;
            for (int c = 0; c < want && c < nc; ++c) picks[np++] = cand[c].i;
            write_sorted(selected + ((size_t)b * N + n) * (size_t)k, k, picks, np);
            n_selected[(size_t)b * N + n] = np;
        }
    }
    free(gq);
    free(cand);
    free(picks);
    free(forced);
    return rc;
}

/* ------------------------------------------------------------------------------------ */
/* O3: page 1's probe + importance + recency selection                                   */
/* ------------------------------------------------------------------------------------ */
/*
 * [P1] section 1 "知识点" (the two signals and the insurance) and section 2 "对应代码"
 * (sparse_attn_head), stated as sets and rankings. Per query head h (KV head kh = h / G):
 *
 *   probe offsets of block i, with nt = min(BS, L - i*BS) valid tokens: the stride is
 *     floor(nt / n_probe), at least 1, and the offsets are 0, stride, 2*stride, ... below
 *     nt (so a short last block can take more than n_probe offsets; n_probe < 1 counts
 *     as 1). The probe score is the largest unscaled dot q_h . K[i*BS + offset][kh] over
 *     that (never empty) set;
 *   importance sum of block i: the prefill importance of its tokens added in token order
 *     in float (a running fp32 sum, which the path reproduces bit for bit);
 *   ranking: blocks ordered by value, higher first, the lower index first among equal
 *     values (section 1: ties go to the lower index);
 *   importance picks (only with importance): the first ceil(k / 2) = (k + 1) / 2 blocks
 *     of the ranking by importance sum (fewer if the request has fewer blocks);
 *   probe picks: the first k - (importance picks) blocks, among those not yet picked, of
 *     the ranking by probe score;
 *   recency (QS_RECENCY): if the last block nb-1 is not picked and there is a probe pick,
 *     the probe pick that ranks last (lowest probe score; of equal ones the higher index)
 *     gives its place to nb-1; importance picks are never given up.
 *
 * readings: no threshold in the importance stage (page 1 elides a line there), so blocks
 *   of zero importance can fill the budget; importance is read as importance[b * stride +
 *   token] and tokens at or past the stride add nothing; output ascending, -1 padded.
 * Outputs besides the selection (all optional): probe [B, H, mkbpr] (double),
 *   imp_sum [B, mkbpr] (float), n_imp [B, H], kind [B, H, mkbpr] (int8: 0 not picked,
 *   1 importance pick, 2 probe pick, 3 added by recency, 4 probe pick given up for it).
 */

/* the probe score of one block: the largest dot over its probe offsets */
static double probe_score(const void* query, int q_dtype, size_t q_off, const void* k_cache, int kv_dtype,
                          size_t first_token_off, size_t token_pitch, int32_t nt, int n_probe, int D) {
    const int32_t stride = (nt / n_probe) > 1 ? (nt / n_probe) : 1;
    double top = 0.0;
    int have = 0;
    for (int32_t off = 0; off < nt; off += stride) {
        double dot = 0.0;
        const size_t kb = first_token_off + (size_t)off * token_pitch;
        for (int d = 0; d < D; ++d)
            dot += (double)elem_f(query, q_dtype, q_off + d) * (double)elem_f(k_cache, kv_dtype, kb + d);
        if (!have || dot > top) top = dot;
        have = 1;
    }
    return top;
}

int qso_probe_select(int B, int H, int N, int D, int BS, int q_dtype, int kv_dtype,
                     const void* query, const void* k_cache, int num_kv_blocks,
                     const int32_t* block_tables, int mkbpr,
                     const int32_t* seq_lens,
                     const float* importance, int imp_stride,
                     int n_probe, int k, unsigned flags,
                     int32_t* selected, int32_t* n_selected,
                     double* probe_out, float* imp_out, int32_t* n_imp_out, int8_t* kind_out) {
    if (!is_float(q_dtype) || !is_float(kv_dtype))
        return QSO_BAD;
    if (N <= 0 || H % N != 0 || k < 1) return QSO_BAD;
    const int G = H / N;
    const size_t pitch = (size_t)N * D;                 /* elements between tokens of one KV head */
    const int cap = mkbpr > 0 ? mkbpr : 1;
    const int np = n_probe < 1 ? 1 : n_probe;
    double* probe = (double*)malloc(sizeof(double) * (size_t)cap);
    float* imp = (float*)malloc(sizeof(float) * (size_t)cap);
    scored_t* rank = (scored_t*)malloc(sizeof(scored_t) * (size_t)cap);
    int8_t* role = (int8_t*)malloc((size_t)cap);        /* this head's kind of each block */
    int32_t* picks = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
    int rc = QSO_OK;
    for (int b = 0; b < B && rc == QSO_OK; ++b) {
        const int32_t L = seq_lens[b];
        const int32_t nb = n_blocks_of(L, BS);
        if (nb > mkbpr) { rc = QSO_BAD; break; }
        for (int32_t i = 0; i < nb; ++i) {
            const int32_t phys = block_tables[(size_t)b * mkbpr + i];
            if (phys < 0 || phys >= num_kv_blocks) { rc = QSO_BAD; break; }
        }
        if (rc != QSO_OK) break;
        /* per-request importance sums (every head of the request reads the same ones) */
        for (int32_t i = 0; i < nb; ++i) {
            const int32_t nt = (L - i * BS) < BS ? (L - i * BS) : BS;
            float sum = 0.0f;
            for (int32_t t = i * BS; importance && t < i * BS + nt && t < imp_stride; ++t)
                sum += importance[(size_t)b * imp_stride + t];
            imp[i] = sum;
            if (imp_out) imp_out[(size_t)b * mkbpr + i] = sum;
        }
        for (int h = 0; h < H; ++h) {
            const int kh = h / G;
            for (int32_t i = 0; i < nb; ++i) {
                const int32_t nt = (L - i * BS) < BS ? (L - i * BS) : BS;
                const size_t first = (size_t)block_tables[(size_t)b * mkbpr + i] * BS * pitch + (size_t)kh * D;
                probe[i] = probe_score(query, q_dtype, ((size_t)b * H + h) * D, k_cache, kv_dtype, first, pitch, nt,
                                       np, D);
                if (probe_out) probe_out[((size_t)b * H + h) * mkbpr + i] = probe[i];
            }
            for (int32_t i = 0; i < cap; ++i) role[i] = 0;
            int n_imp = 0, n_pick = 0;
            /* importance picks: a prefix of the importance ranking */
            if (importance) {
                for (int32_t i = 0; i < nb; ++i) { rank[i].v = (double)imp[i]; rank[i].i = i; }
                qsort(rank, (size_t)nb, sizeof(scored_t), cmp_desc_then_index);
                const int budget = (k + 1) / 2;
                for (int32_t r = 0; r < nb && n_imp < budget; ++r) { role[rank[r].i] = 1; picks[n_pick++] = rank[r].i; ++n_imp; }
            }
            /* probe picks: a prefix of the probe ranking of the remaining blocks */
            int nr = 0;
            for (int32_t i = 0; i < nb; ++i)
                if (!role[i]) { rank[nr].v = probe[i]; rank[nr].i = i; ++nr; }
            qsort(rank, (size_t)nr, sizeof(scored_t), cmp_desc_then_index);
            int n_probe_picks = 0;
            for (int r = 0; r < nr && n_pick < k; ++r) { role[rank[r].i] = 2; picks[n_pick++] = rank[r].i; ++n_probe_picks; }
            /* recency: the last-ranked probe pick gives its place to the last block */
            if ((flags & QSO_RECENCY) && nb > 0 && role[nb - 1] == 0 && n_probe_picks > 0) {
                const int32_t victim = rank[n_probe_picks - 1].i;
                role[victim] = 4;
                role[nb - 1] = 3;
                for (int j = 0; j < n_pick; ++j)
                    if (picks[j] == victim) picks[j] = nb - 1;
            }
            if (kind_out) {
                int8_t* kind = kind_out + ((size_t)b * H + h) * mkbpr;
                for (int32_t i = 0; i < mkbpr; ++i) kind[i] = i < cap ? role[i] : 0;
            }
            write_sorted(selected + ((size_t)b * H + h) * (size_t)k, k, picks, n_pick);
            n_selected[(size_t)b * H + h] = n_pick;
            if (n_imp_out) n_imp_out[(size_t)b * H + h] = n_imp;
        }
    }
    free(probe);
    free(imp);
    free(rank);
    free(role);
    free(picks);
    return rc;
}

/* ------------------------------------------------------------------------------------ */
/* O4: exact attention over the selected blocks                                          */
/* ------------------------------------------------------------------------------------ */
/*
 * reading of the int8 query quantiser (the pages name only "int8 x int8 dot + scale"):
 * one fp32 scale per query head, s = absmax / 127; code = clamp(rint(q / s), -127, 127)
 * in fp32 with round-half-to-even; s == 0 gives all-zero codes.
 */
void qso_quantize_row_i8(const float* x, int D, int8_t* codes, float* scale) {
    float amax = 0.0f;
    for (int d = 0; d < D; ++d) {
        const float a = fabsf(x[d]);
        if (a > amax) amax = a;
    }
    const float s = amax / 127.0f;
    *scale = s;
    for (int d = 0; d < D; ++d) {
        if (s == 0.0f) { codes[d] = 0; continue; }
        float r = rintf(x[d] / s);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        codes[d] = (int8_t)r;
    }
}

/*
 * [P1] section 2 "对应代码", the three passes after selection: per-token scores on the
 * selected blocks only (f32 KV: float dot; q8 KV: int8 x int8 dot times scales), then
 * subtract the max over the selected tokens, exponentiate and renormalise over the
 * selection ([P1] section 1: the softmax is renormalised on the selected blocks only),
 * then accumulate V with those weights -- the same loops as dense attention with the
 * token range replaced by the blocks sel[] points to.
 * [P3] "quest_block_select_paged" notes: the selected indices are sequence-relative and
 * go through block_tables before the paged KV cache is read.
 *
 * readings: logits are scale * q.k with scale = 1/sqrt(D) unless softmax_scale > 0;
 *   selection row of head h is h / (H / sel_heads); KV head is h / (H / N); entries that
 *   are negative or past the request's blocks are skipped; every other entry is
 *   attended once per occurrence, over its tokens t < seq_len; an empty selection gives
 *   an all-zero output. int8: logit = scale * float(int dot) * s_q * s_k[t],
 *   V[t] = v8[t] * s_v[t]. Output in double [B, H, D].
 */
int qso_sparse_attn_decode(int B, int H, int N, int D, int BS, int q_dtype, int kv_dtype,
                           const void* query, const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale, int num_kv_blocks,
                           const int32_t* block_tables, int mkbpr,
                           const int32_t* seq_lens,
                           const int32_t* selected, const int32_t* n_selected,
                           int sel_heads, int k, double softmax_scale, double* out) {
    if (!is_float(q_dtype)) return QSO_BAD;
    if (!is_float(kv_dtype) && kv_dtype != QSO_I8) return QSO_BAD;
    if (N <= 0 || H % N != 0 || sel_heads <= 0 || H % sel_heads != 0 || sel_heads % N != 0) return QSO_BAD;
    if (kv_dtype == QSO_I8 && (k_scale == NULL || v_scale == NULL)) return QSO_BAD;
    const int G = H / N;
    const int hpr = H / sel_heads;
    const size_t row = (size_t)N * D;
    const double scale = softmax_scale > 0.0 ? softmax_scale : 1.0 / sqrt((double)D);
    const size_t max_tok = (size_t)k * BS;
    double* logit = (double*)malloc(sizeof(double) * (max_tok > 0 ? max_tok : 1));
    size_t* trow = (size_t*)malloc(sizeof(size_t) * (max_tok > 0 ? max_tok : 1));
    float* qf = (float*)malloc(sizeof(float) * (size_t)D);
    int8_t* q8 = (int8_t*)malloc((size_t)D);
    int rc = QSO_OK;
    for (int b = 0; b < B && rc == QSO_OK; ++b) {
        const int32_t L = seq_lens[b];
        const int32_t nb = n_blocks_of(L, BS);
        for (int h = 0; h < H; ++h) {
            const int kh = h / G;
            const int srow = h / hpr;
            const int32_t* sel = selected + ((size_t)b * sel_heads + srow) * (size_t)k;
            int ns = n_selected ? n_selected[(size_t)b * sel_heads + srow] : k;
            if (ns > k) ns = k;
            if (ns < 0) ns = 0;
            for (int d = 0; d < D; ++d) qf[d] = elem_f(query, q_dtype, ((size_t)b * H + h) * D + d);
            float sq = 0.0f;
            if (kv_dtype == QSO_I8) qso_quantize_row_i8(qf, D, q8, &sq);
            /* gather the selected tokens (one entry = one block of tokens) */
            size_t nt = 0;
            for (int j = 0; j < ns; ++j) {
                const int32_t blk = sel[j];
                if (blk < 0 || blk >= nb || blk >= mkbpr) continue;
                const int32_t phys = block_tables[(size_t)b * mkbpr + blk];
                if (phys < 0 || phys >= num_kv_blocks) { rc = QSO_BAD; break; }
                for (int32_t t = blk * BS; t < L && t < (blk + 1) * BS; ++t)
                    trow[nt++] = (size_t)phys * BS + (size_t)(t % BS);
            }
            if (rc != QSO_OK) break;
            double* o = out + ((size_t)b * H + h) * D;
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            if (nt == 0) continue;
            /* scores */
            double mx = -INFINITY;
            for (size_t j = 0; j < nt; ++j) {
                const size_t kb = trow[j] * row + (size_t)kh * D;
                double lg;
                if (kv_dtype == QSO_I8) {
                    int64_t acc = 0;
                    for (int d = 0; d < D; ++d) acc += (int64_t)q8[d] * (int64_t)((const int8_t*)k_cache)[kb + d];
                    lg = scale * (double)acc * (double)sq * (double)k_scale[trow[j] * N + kh];
                } else {
                    double acc = 0.0;
                    for (int d = 0; d < D; ++d) acc += (double)qf[d] * (double)elem_f(k_cache, kv_dtype, kb + d);
                    lg = scale * acc;
                }
                logit[j] = lg;
                if (lg > mx) mx = lg;
            }
            /* softmax over the selection, then V */
            double z = 0.0;
            for (size_t j = 0; j < nt; ++j) {
                logit[j] = exp(logit[j] - mx);
                z += logit[j];
            }
            for (size_t j = 0; j < nt; ++j) {
                const size_t vb = trow[j] * row + (size_t)kh * D;
                const double w = logit[j] / z;
                const double vs = (kv_dtype == QSO_I8) ? (double)v_scale[trow[j] * N + kh] : 1.0;
                for (int d = 0; d < D; ++d) o[d] += w * (double)elem_f(v_cache, kv_dtype, vb + d) * vs;
            }
        }
    }
    free(logit);
    free(trow);
    free(qf);
    free(q8);
    return rc;
}

/* ------------------------------------------------------------------------------------ */
/* O5: prefill importance                                                                */
/* ------------------------------------------------------------------------------------ */
/*
 * [P1] section 1 "知识点", signal 2: the prefill importance of a token is how much
 * attention the prefill actually gave it, recorded per head (imp_head) and reduced over
 * heads into prefill_importance[s] when the prefill ends ([P1] section 2, closing
 * paragraph: every head's imp_head is added into prefill_importance[s]); with exact
 * prefill attention it is exact.
 *
 * reading: causal prefill of L = seq_lens[b] tokens; head h (KV head h / (H / N)) gives
 * token s the weight p_h[t][s] = exp(c q_{t,h}.k_s) / sum_{s' <= t} exp(c q_{t,h}.k_{s'})
 * in query row t >= s, c = softmax_scale (1/sqrt(D) when <= 0); imp_head[h][s] is the sum
 * of p_h[t][s] over the rows t = s .. L-1, and prefill_importance[s] the sum of
 * imp_head[h][s] over all heads. Entries s >= L are 0.
 * Layouts: query [B, max_len, H, D] (row t of request b, head h); K through the paged
 * cache [num_kv_blocks, BS, N, D] and block_tables. Heads h_lo .. h_hi-1 are computed
 * (the others are left 0 in head_imp and not added): a range lets a test evaluate a few
 * heads of a long prefill. Outputs in double: importance [B, stride] (may be NULL),
 * head_imp [B, H, stride] (may be NULL).
 */
int qso_prefill_importance(int B, int H, int N, int D, int BS, int dtype, const void* query, int max_len,
                           const void* k_cache, int num_kv_blocks, const int32_t* block_tables, int mkbpr,
                           const int32_t* seq_lens, double softmax_scale, int h_lo, int h_hi,
                           double* importance, double* head_imp, int stride) {
    if (!is_float(dtype) || H % N != 0 || h_lo < 0 || h_hi > H || h_lo > h_hi) return QSO_BAD;
    const int G = H / N;
    const double c = softmax_scale > 0.0 ? softmax_scale : 1.0 / sqrt((double)D);
    const size_t row = (size_t)N * D;
    if (importance) memset(importance, 0, sizeof(double) * (size_t)B * stride);
    if (head_imp) memset(head_imp, 0, sizeof(double) * (size_t)B * H * stride);
    double* x = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    size_t* krow = (size_t*)malloc(sizeof(size_t) * (size_t)(max_len > 0 ? max_len : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    int rc = QSO_OK;
    for (int b = 0; b < B && rc == QSO_OK; ++b) {
        const int L = seq_lens[b] > 0 ? seq_lens[b] : 0;
        if (L > max_len || ceil_div64(L, BS) > mkbpr) { rc = QSO_BAD; break; }
        for (int s = 0; s < L; ++s) {
            const int32_t phys = block_tables[(size_t)b * mkbpr + s / BS];
            if (phys < 0 || phys >= num_kv_blocks) { rc = QSO_BAD; break; }
            krow[s] = ((size_t)phys * BS + (size_t)(s % BS)) * row;
        }
        if (rc != QSO_OK) break;
        for (int h = h_lo; h < h_hi; ++h) {
            const int kh = h / G;
            for (int s = 0; s < L; ++s) acc[s] = 0.0;
            for (int t = 0; t < L; ++t) {
                const size_t qb = (((size_t)b * max_len + t) * H + h) * D;
                double m = -INFINITY;
                for (int s = 0; s <= t; ++s) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += (double)elem_f(query, dtype, qb + d) * (double)elem_f(k_cache, dtype, krow[s] + (size_t)kh * D + d);
                    x[s] = c * dot;
                    if (x[s] > m) m = x[s];
                }
                double z = 0.0;
                for (int s = 0; s <= t; ++s) {
                    x[s] = exp(x[s] - m);
                    z += x[s];
                }
                for (int s = 0; s <= t; ++s) acc[s] += x[s] / z;
            }
            for (int s = 0; s < L && s < stride; ++s) {
                if (head_imp) head_imp[((size_t)b * H + h) * stride + s] = acc[s];
                if (importance) importance[(size_t)b * stride + s] += acc[s];
            }
        }
    }
    free(x);
    free(krow);
    free(acc);
    return rc;
}

// select.hip -- Quest top-k block selection with sink / local-window forcing.
//
// Source: "ops-transformer select_attention_operators" (page 3), section
// "quest_block_select_paged: 解码期 top-k 预测算法" (grouped-query mean, per-channel
// max(gq*kmax, gq*kmin) summed over D, top-k over the request's blocks, sequence-relative
// indices) and section "三个核心算子" (the _w variant forces the sink block and the local
// window). Ties go to the lower block index ("0.8MB 跑通 Qwen 10-2" (page 1), section 1).
//
// Design (CDNA4): the score stream is HBM-bound (about 1 flop per metadata byte). A
// block's max row and min row are 256 B each in bf16; 16 lanes take 16 B apiece (one
// global_load_dwordx4), multiply by the grouped query held in registers, and a 16-lane
// shuffle reduction yields the score; four passes of 16 rows are in flight per
// workgroup. Two launch shapes, neither with any cross-workgroup synchronisation
// inside a kernel (a device-scope fence costs an L2 write-back on this chip):
//   row mode   one workgroup per (request, KV head) scores the whole row into LDS and
//              selects from there -- used when there are enough rows to fill the GPU;
//   split mode a scoring grid (chunk, KV head, request) writes the scores to the
//              workspace, then a second kernel selects per row -- used for few, long rows.
// The top-k is exact: a 4-pass, 8-bit radix select on an order-preserving integer image
// of the scores finds the k-th best value T, then one ordered pass keeps every block
// above T and the lowest-index blocks equal to T ("higher score first, lower index on
// ties"). Output is written in ascending block order.
#include <math.h>

#include <type_traits>

#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace {

constexpr int kChunk = 64;             // blocks per scoring workgroup in split mode
constexpr int kRowModeRows = 512;      // rows at which one workgroup per row fills the chip
constexpr int kRowModeMaxCap = 256;    // rows this short always use row mode
constexpr int kLdsScoreCap = 8192;     // row mode keeps up to this many scores in LDS
constexpr int kMtStageCap = 256;       // metadata-table rows up to this long are staged in LDS
static_assert(kMtStageCap <= kThreads, "one staging load per thread");
static_assert(kChunk / 16 + 2 <= kMtStageCap, "a split-mode chunk's table entries fit the stage");

struct Forced {
    int w_lo;   // blocks >= w_lo are forced (window); nb when none
    bool sink;  // block 0 forced
    int count;
    __device__ bool has(int i) const { return i >= w_lo || (sink && i == 0); }
};

__device__ __forceinline__ Forced forced_set(int L, int nb, int BS, int k, const int32_t* tsmu, int b,
                                             uint32_t flags) {
    Forced f{nb, false, 0};
    const bool active = (tsmu == nullptr) || (tsmu[b] >= 0);
    if (!active || nb <= 0) return f;
    if (flags & 2u) {  // window: the last block and every block without metadata
        const long long u = tsmu ? tsmu[b] : 0;
        const long long num = (long long)L - u;
        long long n_meta = (num >= 0) ? num / BS : -((-num + BS - 1) / BS);
        if (n_meta < 0) n_meta = 0;
        if (n_meta > nb - 1) n_meta = nb - 1;
        int lo = int(n_meta);
        if (lo < nb - k) lo = nb - k;
        f.w_lo = lo;
        f.count = nb - lo;
    }
    if ((flags & 1u) && f.count < k && f.w_lo > 0) {
        f.sink = true;
        f.count += 1;
    }
    return f;
}

struct RowInfo {
    int L, nb;
    Forced F;
};

__device__ __forceinline__ RowInfo row_info(const int32_t* sl, const int32_t* tsmu, uint32_t flags, int k, int b,
                                            int BS, int cap) {
    RowInfo r;
    r.L = max(sl[b], 0);
    r.nb = min((r.L + BS - 1) / BS, cap);
    r.F = forced_set(r.L, r.nb, BS, k, tsmu, b, flags);
    return r;
}

// Scores blocks [i0, i_end) of row (b, n) into dst[i] (LDS or global). Forced blocks are
// skipped (NaN written when nan_forced); an out-of-range metadata entry scores -inf.
// qstage: kThreads 16-byte LDS slots used to stage the group's query rows; mt_stage:
// kMtStageCap ints of LDS for the metadata-table entries of [i0, i_end) (MT_LDS: the
// caller guarantees they fit). Contains a barrier: every thread of the workgroup must
// call it.
template <bool BF16, bool MT_LDS>
__device__ __forceinline__ void score_range(const uint8_t* __restrict__ query, const uint8_t* __restrict__ maxb,
                                            const uint8_t* __restrict__ minb, int num_meta,
                                            const int32_t* __restrict__ mt, int mmbpr, int H, int N, int BS, int b,
                                            int n, const Forced& F, int i0, int i_end, float* dst, bool nan_forced,
                                            u32x4* qstage, int32_t* mt_stage) {
    constexpr int esize = BF16 ? 2 : 4;
    constexpr int D = 128;
    constexpr int LPR = D * esize / 16;  // lanes per metadata row
    constexpr int EPL = 16 / esize;      // channels per lane
    constexpr int RPP = kThreads / LPR;  // rows per pass
    constexpr int U = 4;                 // passes per batch
    const int tid = threadIdx.x;
    const int lr = tid % LPR, slot = tid / LPR;
    const int G = H / N;
    const size_t row_bytes = size_t(N) * D * esize;

    // One batch = U passes of RPP rows; the next batch's loads are issued before the
    // current batch is consumed. With MT_LDS the range's metadata-table entries are
    // staged in LDS so that the lookups of later batches are LDS reads (a global lookup
    // would have to wait for every load in flight before it); batch 0 looks up in global
    // memory while the staging loads are in flight.
    const int mbase = i0 / BS;
    auto issue = [&](int base, u32x4 (&vmx)[U], u32x4 (&vmn)[U], bool (&ok)[U], auto from_lds) {
        int mrow[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * RPP + slot;
            ok[u] = i < i_end && !F.has(i);
            if constexpr (decltype(from_lds)::value)
                mrow[u] = ok[u] ? mt_stage[i / BS - mbase] : 0;
            else
                mrow[u] = ok[u] ? mt[size_t(b) * mmbpr + i / BS] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * RPP + slot;
            ok[u] = ok[u] && mrow[u] >= 0 && mrow[u] < num_meta;
            // rows that are not scored read the first row (always valid) and are masked
            const size_t off = ok[u] ? (size_t(mrow[u]) * BS + (i % BS)) * row_bytes + size_t(n) * D * esize + lr * 16
                                     : size_t(lr) * 16;
            vmx[u] = ld16(maxb + off);
            vmn[u] = ld16(minb + off);
        }
    };

    // the group's query rows: one 16-byte piece per thread, loaded ahead of batch 0
    const int npieces = G * LPR;
    const bool staged = npieces <= kThreads;
    u32x4 qpiece{0u, 0u, 0u, 0u};
    if (staged && tid < npieces)
        qpiece = ld16(query + ((size_t(b) * H + size_t(n) * G + tid / LPR) * D + (tid % LPR) * EPL) * esize);
    const int n_ent = i0 < i_end ? (i_end - 1) / BS - mbase + 1 : 0;  // table entries of the range
    int32_t mt_piece = 0;
    if (MT_LDS && tid < n_ent) mt_piece = mt[size_t(b) * mmbpr + mbase + tid];
    u32x4 vmx[U], vmn[U];
    bool ok[U];
    if (i0 < i_end) issue(i0, vmx, vmn, ok, std::false_type{});
    if (MT_LDS && tid < n_ent) mt_stage[tid] = mt_piece;

    // grouped query for this lane's channels: mean over the group's G heads
    float gq[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) gq[e] = 0.f;
    auto add_piece = [&](const u32x4& v) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) { gq[2 * j] += bf_lo(w[j]); gq[2 * j + 1] += bf_hi(w[j]); }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) gq[j] += __uint_as_float(w[j]);
        }
    };
    if (staged && tid < npieces) qstage[tid] = qpiece;
    __syncthreads();  // query pieces and the table row are in LDS
    if (staged) {
        for (int g = 0; g < G; ++g) add_piece(qstage[g * LPR + lr]);
    } else {
        for (int g = 0; g < G; ++g)
            add_piece(ld16(query + ((size_t(b) * H + size_t(n) * G + g) * D + lr * EPL) * esize));
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) gq[e] = gq[e] / float(G);

    auto consume = [&](int base, const u32x4 (&vmx)[U], const u32x4 (&vmn)[U], const bool (&ok)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t a[4] = {vmx[u].x, vmx[u].y, vmx[u].z, vmx[u].w};
            const uint32_t z[4] = {vmn[u].x, vmn[u].y, vmn[u].z, vmn[u].w};
            float part = 0.f;
            if constexpr (BF16) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    part += fmaxf(gq[2 * j] * bf_lo(a[j]), gq[2 * j] * bf_lo(z[j]));
                    part += fmaxf(gq[2 * j + 1] * bf_hi(a[j]), gq[2 * j + 1] * bf_hi(z[j]));
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    part += fmaxf(gq[j] * __uint_as_float(a[j]), gq[j] * __uint_as_float(z[j]));
            }
            const float s = group_sum<LPR>(part);
            const int i = base + u * RPP + slot;
            if (lr == 0 && i < i_end) {
                if (ok[u])
                    dst[i] = s;
                else if (!F.has(i))
                    dst[i] = -INFINITY;
                else if (nan_forced)
                    dst[i] = __builtin_nanf("");
            }
        }
    };

    // ping-pong over two register sets, so a batch's loads are in flight while the other
    // batch is consumed, with no register copies between them
    constexpr int STEP = RPP * U;
    u32x4 wmx[U], wmn[U];
    bool wok[U];
    for (int base = i0; base < i_end; base += 2 * STEP) {
        const bool more1 = base + STEP < i_end;
        if (more1) issue(base + STEP, wmx, wmn, wok, std::integral_constant<bool, MT_LDS>{});
        consume(base, vmx, vmn, ok);
        if (base + 2 * STEP < i_end) issue(base + 2 * STEP, vmx, vmn, ok, std::integral_constant<bool, MT_LDS>{});
        if (more1) consume(base + STEP, wmx, wmn, wok);
    }
}

// Exact top-k of a row from its scores (LDS or global); writes selected / n_selected.
// The radix select finds the k-th best key T; then each thread takes a contiguous run of
// blocks, and two block-wide scans (equal-to-T ranks, then output positions) keep every
// block above T and the lowest-index blocks equal to T, written in ascending order.
__device__ __forceinline__ void topk_emit(const float* scores, int nb, const Forced& F, int k, int32_t* out,
                                          int32_t* n_out, uint32_t* hist, int* sh, int* wsum) {
    const int tid = threadIdx.x;
    const int R = max(0, min(k, nb) - F.count);  // fill picks
    const int nc = nb - F.count;                   // fill candidates
    const bool take_all = R >= nc;
    const bool radix = R > 0 && !take_all;
    uint32_t T = 0;
    int need_eq = 0;
    if (radix) {
        auto kf = [&](int i, uint32_t& key) -> bool {
            if (F.has(i)) return false;
            key = f2key(scores[i]);
            return true;
        };
        T = block_radix_select(nb, R, kf, hist, sh, need_eq);
    }
    const int E = (nb + kThreads - 1) / kThreads;  // blocks per thread, contiguous
    const int i0 = min(nb, tid * E), i1 = min(nb, i0 + E);
    int eq_off = 0, tot;
    if (radix) {
        int eq_local = 0;
        for (int i = i0; i < i1; ++i) eq_local += (!F.has(i) && f2key(scores[i]) == T) ? 1 : 0;
        eq_off = block_excl_scan(eq_local, wsum, tot);
    }
    int pick_local = 0;
    for (int i = i0, eq_seen = eq_off; i < i1; ++i) {
        bool pick = F.has(i);
        if (!pick && R > 0) {
            if (take_all) {
                pick = true;
            } else {
                const uint32_t key = f2key(scores[i]);
                pick = key > T || (key == T && eq_seen < need_eq);
                eq_seen += key == T ? 1 : 0;
            }
        }
        pick_local += pick ? 1 : 0;
    }
    int npick;
    int pos = block_excl_scan(pick_local, wsum, npick);
    for (int i = i0, eq_seen = eq_off; i < i1; ++i) {
        bool pick = F.has(i);
        if (!pick && R > 0) {
            if (take_all) {
                pick = true;
            } else {
                const uint32_t key = f2key(scores[i]);
                pick = key > T || (key == T && eq_seen < need_eq);
                eq_seen += key == T ? 1 : 0;
            }
        }
        if (pick) {
            if (pos < k) out[pos] = i;
            ++pos;
        }
    }
    for (int j = npick + tid; j < k; j += kThreads) out[j] = -1;
    if (tid == 0) *n_out = min(npick, k);
}

struct SelParams {
    const uint8_t* query;
    const uint8_t* maxb;
    const uint8_t* minb;
    int num_meta;
    const int32_t* mt;
    int mmbpr;
    const int32_t* sl;
    const int32_t* tsmu;
    uint32_t flags;
    int k, H, N, BS;
    int32_t* selected;
    int32_t* n_selected;
    float* dbg_scores;
    float* ws_scores;
};

// row mode: one workgroup per (KV head, request); MT_LDS when the request's metadata
// table row fits in LDS
template <bool BF16, bool MT_LDS>
__global__ __launch_bounds__(kThreads) void select_row_kernel(SelParams p) {
    extern __shared__ __attribute__((aligned(16))) float lds_scores[];
    __shared__ uint32_t hist[512];
    __shared__ int sh[4];
    __shared__ int wsum[kWaves];
    __shared__ u32x4 qstage[kThreads];
    __shared__ int32_t mt_stage[kMtStageCap];
    const int n = blockIdx.x, b = blockIdx.y;
    const int cap = p.mmbpr * p.BS;
    const RowInfo r = row_info(p.sl, p.tsmu, p.flags, p.k, b, p.BS, cap);
    float* gscores = (p.dbg_scores ? p.dbg_scores : p.ws_scores) + (size_t(b) * p.N + n) * cap;
    int32_t* out = p.selected + (size_t(b) * p.N + n) * p.k;
    int32_t* n_out = p.n_selected + size_t(b) * p.N + n;
    if (cap <= kLdsScoreCap) {  // scores on chip (LDS accesses resolved at compile time)
        score_range<BF16, MT_LDS>(p.query, p.maxb, p.minb, p.num_meta, p.mt, p.mmbpr, p.H, p.N, p.BS, b, n, r.F,
                                  0, r.nb, lds_scores, false, qstage, mt_stage);
        __syncthreads();
        if (p.dbg_scores)
            for (int i = threadIdx.x; i < r.nb; i += kThreads)
                gscores[i] = r.F.has(i) ? __builtin_nanf("") : lds_scores[i];
        topk_emit(lds_scores, r.nb, r.F, p.k, out, n_out, hist, sh, wsum);
    } else {
        score_range<BF16, MT_LDS>(p.query, p.maxb, p.minb, p.num_meta, p.mt, p.mmbpr, p.H, p.N, p.BS, b, n, r.F,
                                  0, r.nb, gscores, p.dbg_scores != nullptr, qstage, mt_stage);
        __syncthreads();
        topk_emit(gscores, r.nb, r.F, p.k, out, n_out, hist, sh, wsum);
    }
}

// split mode, step 1: scoring grid (chunk, KV head, request)
template <bool BF16>
__global__ __launch_bounds__(kThreads) void select_score_kernel(SelParams p, int chunk) {
    __shared__ u32x4 qstage[kThreads];
    __shared__ int32_t mt_stage[kMtStageCap];
    const int c = blockIdx.x, n = blockIdx.y, b = blockIdx.z;
    const int cap = p.mmbpr * p.BS;
    const RowInfo r = row_info(p.sl, p.tsmu, p.flags, p.k, b, p.BS, cap);
    const int i0 = c * chunk;
    if (i0 >= r.nb) return;
    float* scores = (p.dbg_scores ? p.dbg_scores : p.ws_scores) + (size_t(b) * p.N + n) * cap;
    // a chunk spans at most chunk / BS + 2 table entries, always within kMtStageCap
    score_range<BF16, true>(p.query, p.maxb, p.minb, p.num_meta, p.mt, p.mmbpr, p.H, p.N, p.BS, b, n, r.F, i0,
                            min(r.nb, i0 + chunk), scores, p.dbg_scores != nullptr, qstage, mt_stage);
}

// split mode, step 2: top-k per (KV head, request); the row's scores are first copied
// into LDS (all loads in flight together) when they fit
__global__ __launch_bounds__(kThreads) void select_topk_kernel(SelParams p) {
    extern __shared__ __attribute__((aligned(16))) float lds_scores[];
    __shared__ uint32_t hist[512];
    __shared__ int sh[4];
    __shared__ int wsum[kWaves];
    const int n = blockIdx.x, b = blockIdx.y;
    const int cap = p.mmbpr * p.BS;
    const RowInfo r = row_info(p.sl, p.tsmu, p.flags, p.k, b, p.BS, cap);
    const float* scores = (p.dbg_scores ? p.dbg_scores : p.ws_scores) + (size_t(b) * p.N + n) * cap;
    int32_t* out = p.selected + (size_t(b) * p.N + n) * p.k;
    int32_t* n_out = p.n_selected + size_t(b) * p.N + n;
    if (cap <= kLdsScoreCap) {
        for (int i0 = 0; i0 < r.nb; i0 += 4 * kThreads) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kThreads + threadIdx.x;
                v[u] = i < r.nb ? scores[i] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kThreads + threadIdx.x;
                if (i < r.nb) lds_scores[i] = v[u];
            }
        }
        __syncthreads();
        topk_emit(lds_scores, r.nb, r.F, p.k, out, n_out, hist, sh, wsum);
    } else {
        topk_emit(scores, r.nb, r.F, p.k, out, n_out, hist, sh, wsum);
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

SelectPlan plan_block_select(int B, int N, int BS, int mmbpr) {
    SelectPlan p;
    const size_t cap = size_t(mmbpr) * BS;
    const long long rows = (long long)B * N;
    p.row_mode = rows >= kRowModeRows || cap <= size_t(kRowModeMaxCap);
    p.chunk = kChunk;
    p.n_chunks = int((cap + kChunk - 1) / kChunk);
    p.lds_bytes = cap <= size_t(kLdsScoreCap) ? cap * sizeof(float) : 0;  // row / top-k kernel
    p.scores_off = 0;
    p.bytes = align256(size_t(B) * N * cap * sizeof(float));
    if (p.bytes < 256) p.bytes = 256;
    return p;
}

hipError_t launch_block_select(const SelectArgs& a, const SelectPlan& pl, hipStream_t s) {
    SelParams p{(const uint8_t*)a.query, (const uint8_t*)a.maxb, (const uint8_t*)a.minb, a.num_meta, a.meta_tables,
                a.mmbpr, a.seq_lens, a.tsmu, a.flags, a.k, a.H, a.N, a.BS, a.selected, a.n_selected,
                a.block_scores, (float*)((uint8_t*)a.workspace + pl.scores_off)};
    if (pl.row_mode) {
        dim3 grid(unsigned(a.N), unsigned(a.B));
        const bool mt_lds = a.mmbpr <= kMtStageCap;
        if (a.bf16) {
            if (mt_lds) hipLaunchKernelGGL((select_row_kernel<true, true>), grid, dim3(kThreads), pl.lds_bytes, s, p);
            else hipLaunchKernelGGL((select_row_kernel<true, false>), grid, dim3(kThreads), pl.lds_bytes, s, p);
        } else {
            if (mt_lds) hipLaunchKernelGGL((select_row_kernel<false, true>), grid, dim3(kThreads), pl.lds_bytes, s, p);
            else hipLaunchKernelGGL((select_row_kernel<false, false>), grid, dim3(kThreads), pl.lds_bytes, s, p);
        }
    } else {
        dim3 g1(unsigned(pl.n_chunks), unsigned(a.N), unsigned(a.B));
        if (a.bf16)
            hipLaunchKernelGGL(select_score_kernel<true>, g1, dim3(kThreads), 0, s, p, pl.chunk);
        else
            hipLaunchKernelGGL(select_score_kernel<false>, g1, dim3(kThreads), 0, s, p, pl.chunk);
        hipLaunchKernelGGL(select_topk_kernel, dim3(unsigned(a.N), unsigned(a.B)), dim3(kThreads), pl.lds_bytes, s, p);
    }
    return hipGetLastError();
}

}  // namespace qs

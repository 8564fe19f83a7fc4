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
// The top-k is exact. On an order-preserving integer image of the scores, one 256-bin
// histogram over the row's key range finds the bin holding the k-th best key, and the
// keys of that bin alone are searched to give the k-th best value T (an 8-bit radix
// select takes over when the bin is crowded); then one ordered pass keeps every block
// above T and the lowest-index blocks equal to T ("higher score first, lower index on
// ties"). Output is written in ascending block order. Rows of up to 256 blocks run it
// with one workgroup barrier (the histogram), every wave finishing the selection on its
// own from keys held in registers (sel::topk_waves); longer rows use the workgroup form
// (sel::topk_emit), cheaper there when many waves of a CU select at once.
#include <math.h>

#include <type_traits>

#include "qs_device.h"
#include "qs_internal.h"
#include "select_dev.h"

namespace qs {
namespace {

using namespace sel;

constexpr int kChunk = 64;             // blocks per scoring workgroup in split mode
constexpr int kRowModeRows = 512;      // rows at which one workgroup per row fills the chip
constexpr int kRowModeMaxCap = 256;    // rows this short always use row mode
static_assert(kChunk / 16 + 2 <= sel::kMtStageCap, "a split-mode chunk's table entries fit the stage");

// row mode: one workgroup per (KV head, request); MT_LDS when the request's metadata
// table row fits in LDS
template <int DT, bool MT_LDS>
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
        for (int j = threadIdx.x; j < 256; j += kThreads) hist[j] = 0u;  // ordered by score_range's barrier
        score_range<DT, MT_LDS>(p.query, p.maxb, p.minb, p.num_meta, p.mt, p.mmbpr, p.H, p.N, p.BS, b, n, r.F,
                                  0, r.nb, cap, lds_scores, false, qstage, mt_stage);
        __syncthreads();
        if (p.dbg_scores)
            for (int i = threadIdx.x; i < r.nb; i += kThreads)
                gscores[i] = r.F.has(i) ? __builtin_nanf("") : lds_scores[i];
        // the query stage is dead: it holds the waves' boundary lists (256 keys each)
        const int ns = topk_dispatch(lds_scores, r.nb, cap, r.F, p.k, out, n_out, hist,
                                     reinterpret_cast<uint32_t*>(qstage) + wave_id() * 256, sh, wsum);
        if (ns >= 0 && threadIdx.x == 0) *n_out = ns;
    } else {
        score_range<DT, MT_LDS>(p.query, p.maxb, p.minb, p.num_meta, p.mt, p.mmbpr, p.H, p.N, p.BS, b, n, r.F,
                                  0, r.nb, cap, gscores, p.dbg_scores != nullptr, qstage, mt_stage);
        __syncthreads();
        topk_emit(gscores, r.nb, r.F, p.k, out, n_out, hist, sh, wsum);
    }
}

// split mode, step 1: scoring grid (chunk, KV head, request)
template <int DT>
__global__ __launch_bounds__(kThreads) void select_score_kernel(SelParams p, int chunk) {
    __shared__ u32x4 qstage[kThreads];
    __shared__ int32_t mt_stage[kMtStageCap];
    const int c = blockIdx.x, n = blockIdx.y, b = blockIdx.z;
    const int cap = p.mmbpr * p.BS;
    const RowInfo r = row_info(p.sl, p.tsmu, p.flags, p.k, b, p.BS, cap);
    const int i0 = c * chunk;  // < cap: the grid has ceil(cap / chunk) chunks
    float* scores = (p.dbg_scores ? p.dbg_scores : p.ws_scores) + (size_t(b) * p.N + n) * cap;
    // a chunk spans at most chunk / BS + 2 table entries, always within kMtStageCap. A
    // chunk past the row's blocks scores nothing; it is not cut short before the call, so
    // that the table lookups of the others do not wait for the row length.
    score_range<DT, true>(p.query, p.maxb, p.minb, p.num_meta, p.mt, p.mmbpr, p.H, p.N, p.BS, b, n, r.F, i0,
                            min(r.nb, i0 + chunk), min(cap, i0 + chunk), scores, p.dbg_scores != nullptr, qstage,
                            mt_stage);
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
        topk_emit(lds_scores, r.nb, r.F, p.k, out, n_out, hist, sh, wsum);  // split mode: rows beyond 256 blocks
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

hipError_t launch_select_scores(const SelectArgs& a, const SelectPlan& pl, float* scores, hipStream_t s) {
    SelParams p{(const uint8_t*)a.query, (const uint8_t*)a.maxb, (const uint8_t*)a.minb, a.num_meta, a.meta_tables,
                a.mmbpr, a.seq_lens, a.tsmu, a.flags, a.k, a.H, a.N, a.BS, nullptr, nullptr, nullptr, scores};
    dim3 g1(unsigned(pl.n_chunks), unsigned(a.N), unsigned(a.B));
    if (a.dtype == kBF16)
        hipLaunchKernelGGL(select_score_kernel<kBF16>, g1, dim3(kThreads), 0, s, p, pl.chunk);
    else if (a.dtype == kF16)
        hipLaunchKernelGGL(select_score_kernel<kF16>, g1, dim3(kThreads), 0, s, p, pl.chunk);
    else
        hipLaunchKernelGGL(select_score_kernel<kF32>, g1, dim3(kThreads), 0, s, p, pl.chunk);
    return hipGetLastError();
}

hipError_t launch_block_select(const SelectArgs& a, const SelectPlan& pl, hipStream_t s) {
    SelParams p{(const uint8_t*)a.query, (const uint8_t*)a.maxb, (const uint8_t*)a.minb, a.num_meta, a.meta_tables,
                a.mmbpr, a.seq_lens, a.tsmu, a.flags, a.k, a.H, a.N, a.BS, a.selected, a.n_selected,
                a.block_scores, (float*)((uint8_t*)a.workspace + pl.scores_off)};
    if (pl.row_mode) {
        dim3 grid(unsigned(a.N), unsigned(a.B));
        const bool mt_lds = a.mmbpr <= kMtStageCap;
        auto row = [&](auto dt) {
            constexpr int DT = decltype(dt)::value;
            if (mt_lds) hipLaunchKernelGGL((select_row_kernel<DT, true>), grid, dim3(kThreads), pl.lds_bytes, s, p);
            else hipLaunchKernelGGL((select_row_kernel<DT, false>), grid, dim3(kThreads), pl.lds_bytes, s, p);
        };
        if (a.dtype == kBF16) row(std::integral_constant<int, kBF16>{});
        else if (a.dtype == kF16) row(std::integral_constant<int, kF16>{});
        else row(std::integral_constant<int, kF32>{});
    } else {
        dim3 g1(unsigned(pl.n_chunks), unsigned(a.N), unsigned(a.B));
        if (a.dtype == kBF16)
            hipLaunchKernelGGL(select_score_kernel<kBF16>, g1, dim3(kThreads), 0, s, p, pl.chunk);
        else if (a.dtype == kF16)
            hipLaunchKernelGGL(select_score_kernel<kF16>, g1, dim3(kThreads), 0, s, p, pl.chunk);
        else
            hipLaunchKernelGGL(select_score_kernel<kF32>, g1, dim3(kThreads), 0, s, p, pl.chunk);
        hipLaunchKernelGGL(select_topk_kernel, dim3(unsigned(a.N), unsigned(a.B)), dim3(kThreads), pl.lds_bytes, s, p);
    }
    return hipGetLastError();
}

}  // namespace qs

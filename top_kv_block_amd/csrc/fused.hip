// fused.hip -- Quest block selection and exact attention over the selected blocks in one
// kernel launch.
//
// Source: "ops-transformer select_attention_operators" (page 3), section
// "quest_block_select_paged: 解码期 top-k 预测算法" (grouped-query scoring and top-k per
// (request, KV head); sequence-relative indices mapped through block_tables) and section
// "三个核心算子" (sink / window forcing); "0.8MB 跑通 Qwen | 第 10-2 篇" (page 1), section 2
// (the selection feeds the attention loop directly: the loop runs over the blocks sel[]
// points to). The result is defined as qs_block_select followed by
// qs_sparse_attn_decode with one selection row per KV head.
//
// Design (CDNA4). Selection and attention are both per (request, KV head), so one
// workgroup can do both: it scores the row's blocks into LDS, runs the exact top-k there,
// and attends over the selection without writing it to HBM and without a second launch.
// The selection scratch (scores, histograms, staged query and table row, the selection)
// shares the attention kernels' LDS work area: the matrix-core body copies the selection
// into a per-wave register slot table and synchronises before its V^T tiles overwrite the
// area; the vector body keeps the selection in front of its merge buffer. When there are
// too few rows to fill the chip and the rows are short, each of a row's slot splits
// recomputes the (deterministic, hence identical) selection from L2-resident metadata and
// the splits' partials are merged by the attention combine pass. Long rows with few
// requests are scored first by the selection's wide scoring grid (the scores go to the
// workspace); each attention workgroup then stages its row's scores in LDS and runs the
// top-k itself, so the separate top-k launch and the selection's round trip through HBM
// disappear. Rows with more than 64 selected blocks use the two operations' kernels.
#include <math.h>

#include <type_traits>

#include "attn_dev.h"
#include "qs_device.h"
#include "qs_internal.h"
#include "select_dev.h"

namespace qs {
namespace {

constexpr int kFusedMaxK = 64;          // selection entries kept in LDS (and in one slot table)
constexpr int kFusedMaxCap = 4096;      // blocks per row scored into LDS
constexpr int kFusedSplitMaxCap = 256;  // rows at most this long may be recomputed per split
constexpr int kFusedRows = 1024;        // rows at which each row gets one workgroup
constexpr int kFusedTargetWg = 1024;

// LDS work area: [selection | count | scores | histograms | query stage | table stage | sh, wsum]
constexpr int kOffSel = 0;
constexpr int kOffNsel = kOffSel + kFusedMaxK * 4;
constexpr int kOffScores = kOffNsel + 16;
constexpr int kOffHist = kOffScores + kFusedMaxCap * 4;
constexpr int kOffQstage = kOffHist + 512 * 4;
constexpr int kOffMt = kOffQstage + kThreads * 16;
constexpr int kOffSh = kOffMt + sel::kMtStageCap * 4;
constexpr int kOffWsum = kOffSh + 16;
constexpr int kSelectLds = kOffWsum + 16;
static_assert(kSelectLds <= attn::kMfmaLdsBytes, "the selection scratch fits the attention work area");
static_assert(kOffQstage % 16 == 0, "16-byte query stage");
static_assert(kFusedMaxK <= kWave, "the selection fits one slot table");
static_assert(kFusedMaxCap <= sel::kLdsScoreCap, "scores stay on chip");

// Selection of row (b, n) into LDS (every thread must call it). Returns n_selected; the
// entries are at lds + kOffSel. With PRESCORED the row's scores come from the scoring
// grid's output (p.ws_scores) instead of being computed here. Split 0 of head chunk 0
// also writes the selection to the caller's selected / n_selected when those are given.
template <int DT, bool PRESCORED, int KPL, bool NT = false>
__device__ __forceinline__ int select_phase(const sel::SelParams& p, int b, int n, uint8_t* lds, bool publish) {
    float* scores = (float*)(lds + kOffScores);
    uint32_t* hist = (uint32_t*)(lds + kOffHist);
    u32x4* qstage = (u32x4*)(lds + kOffQstage);
    int32_t* mt_stage = (int32_t*)(lds + kOffMt);
    int* sh = (int*)(lds + kOffSh);
    int* wsum = (int*)(lds + kOffWsum);
    int32_t* selv = (int32_t*)(lds + kOffSel);
    int32_t* nsel = (int32_t*)(lds + kOffNsel);
    const int cap = p.mmbpr * p.BS;
    const sel::RowInfo r = sel::row_info(p.sl, p.tsmu, p.flags, p.k, b, p.BS, cap);
    for (int j = threadIdx.x; j < 256; j += kThreads) hist[j] = 0u;  // ordered by the barrier below
    if constexpr (PRESCORED) {
        // the whole workspace row (cap <= kFusedMaxCap entries) into LDS, all loads of a
        // thread in flight together and issued without waiting for the row length; entries
        // at or past the row's block count are never read
        const float* src = p.ws_scores + (size_t(b) * p.N + n) * cap;
        for (int i0 = 0; i0 < cap; i0 += 4 * kThreads) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kThreads + threadIdx.x;
                v[u] = i < cap ? src[i] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kThreads + threadIdx.x;
                if (i < cap) scores[i] = v[u];
            }
        }
    } else {
        sel::score_range<DT, true, NT>(p.query, p.maxb, p.minb, p.num_meta, p.mt, p.mmbpr, p.H, p.N, p.BS, b, n, r.F,
                                   0, r.nb, cap, scores, false, qstage, mt_stage);
    }
    __syncthreads();
    // the query stage is dead: it holds the waves' boundary lists (256 keys each)
    const int c = sel::topk_dispatch<KPL>(scores, r.nb, cap, r.F, p.k, selv, nsel, hist,
                                     reinterpret_cast<uint32_t*>(qstage) + (threadIdx.x / kWave) * 256, sh, wsum);
    __syncthreads();
    const int ns = c >= 0 ? c : *nsel;
    if (publish && p.selected) {
        int32_t* out = p.selected + (size_t(b) * p.N + n) * p.k;
        for (int j = threadIdx.x; j < p.k; j += kThreads) out[j] = selv[j];
        if (threadIdx.x == 0) p.n_selected[size_t(b) * p.N + n] = ns;
    }
    return ns;
}

// bf16 / f16: grid (splits x head chunks, KV head, request); KPL: the top-k variant for
// the row capacity (sel::topk_kpl); NT: metadata and K/V through non-temporal loads
template <int DT, bool PRESCORED, int KPL, bool NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void select_attn_mfma_kernel(sel::SelParams sp, attn::AttnParams ap) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[attn::kMfmaLdsBytes];
    const uint3 w = xcd_block_index(ap.splits > 1);
    const int split = int(w.x) % ap.splits, hcix = int(w.x) / ap.splits;
    const int n = int(w.y), b = int(w.z);
    const int ns = select_phase<DT, PRESCORED, KPL, NT>(sp, b, n, lds, split == 0 && hcix == 0);
    attn::mfma_body<DT, NT>(ap, split, hcix, n, b, (const int32_t*)(lds + kOffSel), ns, lds, true);
}

// f32: the vector-ALU attention; its merge buffer overlays the dead scoring scratch
template <int HC, bool PRESCORED>
__global__ __launch_bounds__(kThreads) void select_attn_vec_kernel(sel::SelParams sp, attn::AttnParams ap) {
    constexpr int kRedBytes = attn::vec_red_floats<HC>() * 4;
    constexpr int kLds = kSelectLds > kOffScores + kRedBytes ? kSelectLds : kOffScores + kRedBytes;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
    const int split = blockIdx.x % ap.splits, hcix = blockIdx.x / ap.splits;
    const int n = blockIdx.y, b = blockIdx.z;
    const int ns = select_phase<kF32, PRESCORED, 0>(sp, b, n, lds, split == 0 && hcix == 0);
    attn::vec_body<kF32, kF32, HC>(ap, split, hcix, n, b, (const int32_t*)(lds + kOffSel), ns,
                                   (float*)(lds + kOffScores));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

FusedPlan plan_select_attn(int B, int H, int N, int BS, int mmbpr, int k, int dtype) {
    FusedPlan f{};
    const long long cap = (long long)mmbpr * BS;
    f.attn = plan_sparse_attn(B, H, N, 128, N, k, dtype, dtype);
    f.sel = plan_block_select(B, N, BS, mmbpr);
    const long long rows = (long long)B * N * f.attn.hchunks;
    const bool fits = k <= kFusedMaxK && cap <= kFusedMaxCap && mmbpr <= sel::kMtStageCap;
    if (fits && (rows >= kFusedRows || cap <= kFusedSplitMaxCap)) f.mode = FusedPlan::kOneKernel;
    else if (fits) f.mode = FusedPlan::kPrescored;
    else f.mode = FusedPlan::kSeparate;
    if (f.mode != FusedPlan::kSeparate) {
        long long splits = 1;
        if (rows < kFusedRows) {
            const long long rows1 = rows > 0 ? rows : 1;
            splits = (kFusedTargetWg + rows1 - 1) / rows1;
            if (splits > k) splits = k;
            if (splits < 1) splits = 1;
        }
        f.attn.spb = int((k + splits - 1) / splits);
        f.attn.splits = (k + f.attn.spb - 1) / f.attn.spb;
        const size_t part = f.attn.splits > 1 ? size_t(rows) * f.attn.splits * f.attn.hc * attn::PSTRIDE * 4 : 0;
        const size_t scores = f.mode == FusedPlan::kPrescored ? size_t(B) * N * cap * 4 : 0;
        f.sel_off = 0;                      // prescored: the scores
        f.attn.part_off = align256(scores);  // the attention partials
        f.attn.bytes = align256(part);
        f.bytes = f.attn.part_off + f.attn.bytes;
        f.attn_off = f.idx_off = f.nidx_off = 0;
    } else {
        // separate kernels: select into workspace-held (or the caller's) selection, then attend
        f.sel_off = 0;
        f.attn.part_off = 0;
        f.attn_off = align256(f.sel.bytes);
        f.idx_off = f.attn_off + align256(f.attn.bytes);
        f.nidx_off = f.idx_off + align256(size_t(B) * N * k * 4);
        f.bytes = f.nidx_off + align256(size_t(B) * N * 4);
    }
    if (f.bytes < 256) f.bytes = 256;
    return f;
}

hipError_t launch_select_attn(const SelectArgs& s, const AttnArgs& a, const FusedPlan& pl, hipStream_t st) {
    uint8_t* ws = (uint8_t*)a.workspace;
    if (pl.mode == FusedPlan::kSeparate) {
        SelectArgs s2 = s;
        AttnArgs a2 = a;
        if (!s2.selected) {
            s2.selected = (int32_t*)(ws + pl.idx_off);
            s2.n_selected = (int32_t*)(ws + pl.nidx_off);
        }
        s2.workspace = ws + pl.sel_off;
        a2.selected = s2.selected;
        a2.n_selected = s2.n_selected;
        a2.workspace = ws + pl.attn_off;
        hipError_t e = launch_block_select(s2, pl.sel, st);
        if (e != hipSuccess) return e;
        return launch_sparse_attn(a2, pl.attn, st);
    }
    const bool pre = pl.mode == FusedPlan::kPrescored;
    float* scores = (float*)(ws + pl.sel_off);
    if (pre) {
        hipError_t e = launch_select_scores(s, pl.sel, scores, st);
        if (e != hipSuccess) return e;
    }
    const AttnPlan& ap = pl.attn;
    sel::SelParams sp{(const uint8_t*)s.query, (const uint8_t*)s.maxb, (const uint8_t*)s.minb, s.num_meta,
                      s.meta_tables, s.mmbpr, s.seq_lens, s.tsmu, s.flags, s.k, s.H, s.N, s.BS, s.selected,
                      s.n_selected, nullptr, pre ? scores : nullptr};
    attn::AttnParams prm{(const uint8_t*)a.query, (const uint8_t*)a.k_cache, (const uint8_t*)a.v_cache, nullptr,
                         nullptr, a.num_kv_blocks, a.block_tables, a.mkbpr, a.seq_lens, nullptr, nullptr, a.H, a.N,
                         a.BS, a.N, a.k, ap.hpr, ap.hchunks, ap.splits, ap.spb, a.scale * attn::kLog2e,
                         (uint8_t*)a.out, (float*)(ws + ap.part_off)};
    dim3 grid(unsigned(ap.splits * ap.hchunks), unsigned(a.N), unsigned(a.B));
    const int kpl = sel::topk_kpl(s.mmbpr * s.BS);
    auto launch = [&](auto pre_c) {
        constexpr bool P = decltype(pre_c)::value;
        if (ap.mfma) {
            // the call's streamed bytes (upper bounds: every row at capacity): metadata rows
            // (max and min) when scored here, K/V rows of the k selected blocks
            const size_t esz = 2, rows_kv = size_t(a.B) * a.N;  // 16-bit query, metadata and K/V here
            const size_t meta = P ? 0 : rows_kv * size_t(s.mmbpr) * s.BS * 2 * a.D * esz;
            const size_t kv = rows_kv * size_t(a.k) * a.BS * 2 * a.D * esz;
            const bool nt = meta + kv > attn::kNtStreamBytes;
            auto by_kpl = [&](auto dt) {
                constexpr int DT = decltype(dt)::value;
                auto go = [&](auto ntc) {
                    constexpr bool NT = decltype(ntc)::value;
                    switch (kpl) {
                        case 2: hipLaunchKernelGGL((select_attn_mfma_kernel<DT, P, 2, NT>), grid, dim3(kThreads), 0, st, sp, prm); break;
                        case 4: hipLaunchKernelGGL((select_attn_mfma_kernel<DT, P, 4, NT>), grid, dim3(kThreads), 0, st, sp, prm); break;
                        default: hipLaunchKernelGGL((select_attn_mfma_kernel<DT, P, -1, NT>), grid, dim3(kThreads), 0, st, sp, prm); break;
                    }
                };
                if (nt) go(std::true_type{});
                else go(std::false_type{});
            };
            if (a.q_dtype == kF16) by_kpl(std::integral_constant<int, kF16>{});
            else by_kpl(std::integral_constant<int, kBF16>{});
        } else {
            switch (ap.hc) {
                case 1: hipLaunchKernelGGL((select_attn_vec_kernel<1, P>), grid, dim3(kThreads), 0, st, sp, prm); break;
                case 2: hipLaunchKernelGGL((select_attn_vec_kernel<2, P>), grid, dim3(kThreads), 0, st, sp, prm); break;
                case 4: hipLaunchKernelGGL((select_attn_vec_kernel<4, P>), grid, dim3(kThreads), 0, st, sp, prm); break;
                default: hipLaunchKernelGGL((select_attn_vec_kernel<8, P>), grid, dim3(kThreads), 0, st, sp, prm); break;
            }
        }
    };
    if (pre) launch(std::true_type{});
    else launch(std::false_type{});
    if (ap.splits > 1) return attn::launch_combine(prm, a.B, ap.hc, a.q_dtype, st);
    return hipGetLastError();
}

}  // namespace qs

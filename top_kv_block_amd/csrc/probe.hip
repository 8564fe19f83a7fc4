// probe.hip -- page 1's block selection: probe scores, prefill-importance budget,
// probe fill and recency insurance, per query head; and the same selection fused with
// exact attention over it.
//
// Source: "0.8MB 跑通 Qwen | 第 10-2 篇: 推理引擎的 sparse top-k 块选择" (page 1),
// section 1 "知识点" (three signals + recency, lower-index ties, determinism) and
// section 2 "对应代码" (probe loop, importance preselect with budget (k+1)/2, greedy fill,
// recency replacing the lowest probe pick only; the selection feeds the attention loop
// directly).
//
// Design (CDNA4). The probe samples are independent dot products of the query with
// sampled key rows: a scoring grid (chunk of blocks, KV head, request) loads each sampled
// row once for all query heads of its group; a group of LPR lanes (16-byte loads, the
// whole 128-channel row) computes one dot, reduces it with shuffles and folds it into the
// block's probe score with an LDS atomic max on the score's order-preserving integer
// image (max is order-independent, so the result is exact and deterministic). The pick
// (probe_dev.h) then runs on one workgroup per (request, query head). The fused call
// runs the pick in every attention workgroup of the row (slot split, query head,
// request) and attends over the selection straight from LDS with the vector-ALU
// attention body: the pick's round trip through HBM and the attention launch's wait for
// it disappear; the splits recompute the same deterministic pick from L2-resident probe
// keys and the attention combine pass merges them.
#include <math.h>

#include <type_traits>

#include "attn_dev.h"
#include "probe_dev.h"
#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace {

constexpr int kProbeChunk = 8;   // blocks per probe-scoring workgroup
constexpr int kProbeHeads = 8;   // query heads scored per pass over the sampled rows

// Step 1: probe scores. Workgroup (chunk, kv head kh, request b) loads each sampled key
// row of its blocks once and scores it against every query head of the group (so each
// key row is read once for all of them), folding the dot into the block's probe score
// with an LDS atomic max on the order-preserving key. Results go to keys[b][h][block].
template <int QDT, int KDT>
__global__ __launch_bounds__(kThreads) void probe_score_kernel(
    const uint8_t* __restrict__ query, const uint8_t* __restrict__ kc, int num_kv_blocks,
    const int32_t* __restrict__ bt, int mkbpr, const int32_t* __restrict__ sl, int n_probe, int H, int N, int BS,
    uint32_t* __restrict__ keys) {
    constexpr int D = 128;
    constexpr int ke = elem_bytes(KDT);
    constexpr int qe = elem_bytes(QDT);
    constexpr int LPR = D * ke / 16;  // lanes per key row
    constexpr int EPL = 16 / ke;      // channels per lane
    constexpr int GRP = kThreads / LPR;
    constexpr int U = 8;              // sampled rows in flight per lane group

    __shared__ uint32_t pk[kProbeHeads][kProbeChunk];

    const int c = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
    const int G = H / N;
    const int tid = threadIdx.x, lr = tid % LPR, grp = tid / LPR;
    const int L = max(sl[b], 0);
    const int nb = min((L + BS - 1) / BS, mkbpr);
    const int i0 = c * kProbeChunk;
    if (i0 >= nb) return;
    const int nblk = min(kProbeChunk, nb - i0);
    const int np = max(1, n_probe);
    // samples per block: ceil(len / step), step = max(1, len / n_probe)
    int smax = 1;
    for (int t = 0; t < nblk; ++t) {
        const int len = min(BS, L - (i0 + t) * BS), step = max(1, len / np);
        smax = max(smax, (len + step - 1) / step);
    }
    const int items = nblk * smax;
    const size_t row_bytes = size_t(N) * D * ke;
    const uint32_t init_key = f2key(-1e30f);

    for (int g0 = 0; g0 < G; g0 += kProbeHeads) {
        const int gn = min(kProbeHeads, G - g0);
        for (int t = tid; t < kProbeHeads * kProbeChunk; t += kThreads) pk[t / kProbeChunk][t % kProbeChunk] = init_key;
        float q[kProbeHeads][EPL];
#pragma unroll
        for (int g = 0; g < kProbeHeads; ++g) {
            const int h = kh * G + g0 + (g < gn ? g : 0);
            const uint8_t* qp = query + (size_t(b) * H + h) * D * qe;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int d = lr * EPL + e;
                q[g][e] = load_elem<QDT>(qp, d);
            }
        }
        __syncthreads();
        for (int base = 0; base < items; base += GRP * U) {
            // table lookups of all items first, then the key loads back to back
            int blk[U], row[U], phys[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int it = base + u * GRP + grp;
                blk[u] = -1;
                row[u] = 0;
                phys[u] = 0;
                if (it < items) {
                    const int t = it / smax, j = it % smax;
                    const int i = i0 + t, p0 = i * BS, len = min(BS, L - p0);
                    const int step = max(1, len / np);
                    if (j * step < len) {
                        blk[u] = t;
                        row[u] = j * step;
                        phys[u] = bt[size_t(b) * mkbpr + i];
                    }
                }
            }
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (phys[u] < 0 || phys[u] >= num_kv_blocks) {
                    blk[u] = -1;
                    phys[u] = 0;
                }
                // items without a sample read row 0 of block 0 (always valid) and are masked
                const size_t off = blk[u] >= 0 ? (size_t(phys[u]) * BS + row[u]) * row_bytes + size_t(kh) * D * ke : 0;
                v[u] = ld16(kc + off + lr * 16);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                float kf[EPL];
                if constexpr (KDT != kF32) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) { kf[2 * jj] = lo16<KDT>(w[jj]); kf[2 * jj + 1] = hi16<KDT>(w[jj]); }
                } else {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) kf[jj] = __uint_as_float(w[jj]);
                }
#pragma unroll
                for (int g = 0; g < kProbeHeads; ++g) {
                    if (g >= gn) break;
                    float part = 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) part += q[g][e] * kf[e];
                    const float dot = group_sum<LPR>(part);
                    if (lr == 0 && blk[u] >= 0) atomicMax(&pk[g][blk[u]], f2key(dot));
                }
            }
        }
        __syncthreads();
        for (int t = tid; t < gn * kProbeChunk; t += kThreads) {
            const int g = t / kProbeChunk, bi = t % kProbeChunk;
            if (bi < nblk) keys[(size_t(b) * H + kh * G + g0 + g) * mkbpr + i0 + bi] = pk[g][bi];
        }
        __syncthreads();
    }
}

// Step 2: per (request, query head): the pick (importance budget, probe fill, recency),
// written out ascending and -1 padded.
__global__ __launch_bounds__(kThreads) void probe_pick_kernel(
    const uint32_t* __restrict__ keys, int mkbpr, const int32_t* __restrict__ sl, const float* __restrict__ importance,
    int imp_stride, int k, uint32_t flags, int H, int BS, int32_t* __restrict__ selected,
    int32_t* __restrict__ n_selected, float* __restrict__ probe_scores) {
    __shared__ probe::PickLds s;
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    const int L = max(sl[b], 0);
    const int nb = min((L + BS - 1) / BS, mkbpr);
    const int ns = probe::pick_row(keys + (size_t(b) * H + h) * mkbpr, nb, L,
                                   importance ? importance + size_t(b) * imp_stride : nullptr, imp_stride, BS, k,
                                   flags, s);
    int32_t* out = selected + (size_t(b) * H + h) * k;
    for (int j = tid; j < k; j += kThreads) out[j] = j < ns ? s.sel[j] : -1;
    if (tid == 0) n_selected[size_t(b) * H + h] = ns;
    if (probe_scores)
        for (int i = tid; i < nb; i += kThreads) probe_scores[(size_t(b) * H + h) * mkbpr + i] = key2f(s.pkey[i]);
}

// Fused: grid (slot split, query head, request). Each workgroup picks its row into LDS,
// split 0 publishes the selection when the caller asked for it, then the vector-ALU
// attention body attends over the split's slots of the selection (a float cache, or the
// int8 copy with its scales while the probes read the float K); its merge buffer
// overlays the probe keys, dead after the pick.
struct PickParams {
    const uint32_t* keys;
    int mkbpr;
    const float* importance;
    int imp_stride;
    uint32_t flags;
    int32_t* selected;
    int32_t* n_selected;
};
static_assert(attn::vec_red_floats<1>() <= kProbeMaxBlocks, "the merge buffer fits the probe keys' LDS");

template <int KV, int QDT>
__global__ __launch_bounds__(kThreads) void probe_attn_vec_kernel(PickParams pp, attn::AttnParams ap) {
    __shared__ probe::PickLds s;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int L = max(ap.sl[b], 0);
    const int nb = min((L + ap.BS - 1) / ap.BS, pp.mkbpr);
    const int ns = probe::pick_row(pp.keys + (size_t(b) * ap.H + h) * pp.mkbpr, nb, L,
                                   pp.importance ? pp.importance + size_t(b) * pp.imp_stride : nullptr,
                                   pp.imp_stride, ap.BS, ap.k, pp.flags, s);
    if (split == 0 && pp.selected) {
        int32_t* out = pp.selected + (size_t(b) * ap.H + h) * ap.k;
        for (int j = threadIdx.x; j < ap.k; j += kThreads) out[j] = j < ns ? s.sel[j] : -1;
        if (threadIdx.x == 0) pp.n_selected[size_t(b) * ap.H + h] = ns;
    }
    attn::vec_body<KV, QDT, 1>(ap, split, 0, h, b, s.sel, ns, reinterpret_cast<float*>(s.pkey));
}

template <int QB, int KB>
void launch_score(const ProbeArgs& a, uint32_t* keys, hipStream_t s) {
    const unsigned chunks = unsigned((a.mkbpr + kProbeChunk - 1) / kProbeChunk);
    hipLaunchKernelGGL((probe_score_kernel<QB, KB>), dim3(chunks, unsigned(a.N), unsigned(a.B)), dim3(kThreads), 0, s,
                       (const uint8_t*)a.query, (const uint8_t*)a.k_cache, a.num_kv_blocks, a.block_tables, a.mkbpr,
                       a.seq_lens, a.n_probe, a.H, a.N, a.BS, keys);
}

}  // namespace

size_t probe_workspace_bytes(int B, int H, int mkbpr) {
    size_t bytes = size_t(B) * H * mkbpr * sizeof(uint32_t);
    bytes = (bytes + 255) & ~size_t(255);
    return bytes < 256 ? 256 : bytes;
}

namespace {
void launch_scores(const ProbeArgs& a, uint32_t* keys, hipStream_t s) {
    auto by_k = [&](auto q) {
        constexpr int QD = decltype(q)::value;
        if (a.kv_dtype == kBF16) launch_score<QD, kBF16>(a, keys, s);
        else if (a.kv_dtype == kF16) launch_score<QD, kF16>(a, keys, s);
        else launch_score<QD, kF32>(a, keys, s);
    };
    if (a.q_dtype == kBF16) by_k(std::integral_constant<int, kBF16>{});
    else if (a.q_dtype == kF16) by_k(std::integral_constant<int, kF16>{});
    else by_k(std::integral_constant<int, kF32>{});
}
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

hipError_t launch_probe_select(const ProbeArgs& a, hipStream_t s) {
    uint32_t* keys = (uint32_t*)a.workspace;
    launch_scores(a, keys, s);
    hipLaunchKernelGGL(probe_pick_kernel, dim3(unsigned(a.H), unsigned(a.B)), dim3(kThreads), 0, s, keys, a.mkbpr,
                       a.seq_lens, a.importance, a.imp_stride, a.k, a.flags, a.H, a.BS, a.selected, a.n_selected,
                       a.probe_scores);
    return hipGetLastError();
}

// fused probe selection + attention: the probe keys, then the attention partials
AttnPlan plan_probe_attn(int B, int H, int N, int mkbpr, int k) {
    AttnPlan p = plan_sparse_attn(B, H, N, 128, H, k, kF32, kF32);  // one row per query head, vector ALU
    p.part_off = align256(size_t(B) * H * mkbpr * sizeof(uint32_t));
    p.bytes = p.part_off + (p.splits > 1 ? align256(size_t(B) * H * p.splits * p.hc * attn::PSTRIDE * 4) : 0);
    if (p.bytes < 256) p.bytes = 256;
    return p;
}

hipError_t launch_probe_attn(const ProbeArgs& a, const AttnArgs& t, const AttnPlan& pl, hipStream_t s) {
    uint8_t* ws = (uint8_t*)a.workspace;
    uint32_t* keys = (uint32_t*)ws;
    launch_scores(a, keys, s);
    PickParams pp{keys, a.mkbpr, a.importance, a.imp_stride, a.flags, a.selected, a.n_selected};
    attn::AttnParams prm{(const uint8_t*)t.query, (const uint8_t*)t.k_cache, (const uint8_t*)t.v_cache, t.k_scale,
                         t.v_scale, t.num_kv_blocks, t.block_tables, t.mkbpr, t.seq_lens, nullptr, nullptr, t.H, t.N,
                         t.BS, t.H, t.k, 1, 1, pl.splits, pl.spb, t.scale * attn::kLog2e, (uint8_t*)t.out,
                         (float*)(ws + pl.part_off)};
    const dim3 grid(unsigned(pl.splits), unsigned(t.H), unsigned(t.B));
    auto by_q = [&](auto kv) {
        constexpr int KV = decltype(kv)::value;
        if (t.q_dtype == kBF16) hipLaunchKernelGGL((probe_attn_vec_kernel<KV, kBF16>), grid, dim3(kThreads), 0, s, pp, prm);
        else if (t.q_dtype == kF16) hipLaunchKernelGGL((probe_attn_vec_kernel<KV, kF16>), grid, dim3(kThreads), 0, s, pp, prm);
        else hipLaunchKernelGGL((probe_attn_vec_kernel<KV, kF32>), grid, dim3(kThreads), 0, s, pp, prm);
    };
    if (t.kv_dtype == kBF16) by_q(std::integral_constant<int, kBF16>{});
    else if (t.kv_dtype == kF16) by_q(std::integral_constant<int, kF16>{});
    else if (t.kv_dtype == kI8) by_q(std::integral_constant<int, kI8>{});
    else by_q(std::integral_constant<int, kF32>{});
    if (pl.splits > 1) return attn::launch_combine(prm, t.B, 1, t.q_dtype, s);
    return hipGetLastError();
}

}  // namespace qs

// probe.hip -- page 1's block selection: probe scores, prefill-importance budget,
// probe fill and recency insurance, per query head.
//
// Source: "0.8MB 跑通 Qwen | 第 10-2 篇: 推理引擎的 sparse top-k 块选择" (page 1),
// section 1 "知识点" (three signals + recency, lower-index ties, determinism) and
// section 2 "对应代码" (probe loop, importance preselect with budget (k+1)/2, greedy fill,
// recency replacing the lowest probe pick only).
//
// Design (CDNA4): one workgroup per (request, query head). The probe samples are
// independent dot products of the query with sampled key rows; a group of LPR lanes
// (16-byte loads, the whole 128-channel row) computes one, reduces it with shuffles and
// folds it into the block's probe score with an LDS atomic max on the score's
// order-preserving integer image (max is order-independent, so the result is exact and
// deterministic). Importance sums are accumulated per block by one thread in token order
// in fp32, exactly as the page's loop does, so the importance stage is bit-exact. Each
// greedy stage ("repeatedly take the best unused block, lower index on ties") selects
// the same set as taking the top-r keys under (value desc, index asc); that is computed
// with the block-wide threshold select plus one ordered pass.
#include <math.h>

#include <type_traits>

#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace {

constexpr uint8_t kImp = 1, kProbe = 2;

// Marks the r best candidates (value desc, index asc), r >= 1: a threshold select finds
// the r-th best key T, then each thread takes a contiguous run of blocks and one block-wide
// scan ranks the candidates equal to T by index. Every thread must call it.
template <class Pred, class KeyOf>
__device__ void mark_top(int nb, int r, Pred cand, KeyOf key_of, uint8_t* flag, uint8_t mark, uint32_t* hist,
                         int* sh, int* wsum) {
    const int E = (nb + kThreads - 1) / kThreads;
    const int i0 = min(nb, int(threadIdx.x) * E), i1 = min(nb, i0 + E);
    int nc_local = 0;
    for (int i = i0; i < i1; ++i) nc_local += cand(i) ? 1 : 0;
    int ncand;
    block_excl_scan(nc_local, wsum, ncand);
    if (r >= ncand) {
        for (int i = i0; i < i1; ++i)
            if (cand(i)) flag[i] = mark;
        __syncthreads();
        return;
    }
    int need_eq = 0;
    auto kf = [&](int i, uint32_t& key) -> bool {
        if (!cand(i)) return false;
        key = key_of(i);
        return true;
    };
    const uint32_t T = block_topk_threshold(nb, r, kf, hist, sh, need_eq);
    int eq_local = 0;
    for (int i = i0; i < i1; ++i) eq_local += (cand(i) && key_of(i) == T) ? 1 : 0;
    int eq_tot;
    int eq_seen = block_excl_scan(eq_local, wsum, eq_tot);
    for (int i = i0; i < i1; ++i) {
        if (!cand(i)) continue;
        const uint32_t key = key_of(i);
        bool pick = key > T;
        if (key == T) {
            pick = eq_seen < need_eq;
            ++eq_seen;
        }
        if (pick) flag[i] = mark;
    }
    __syncthreads();
}

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

// Step 2: per (request, query head): importance sums, the two greedy stages, recency,
// ascending output.
__global__ __launch_bounds__(kThreads) void probe_pick_kernel(
    const uint32_t* __restrict__ keys, int mkbpr, const int32_t* __restrict__ sl, const float* __restrict__ importance,
    int imp_stride, int k, uint32_t flags, int H, int BS, int32_t* __restrict__ selected,
    int32_t* __restrict__ n_selected, float* __restrict__ probe_scores) {
    __shared__ uint32_t pkey[kProbeMaxBlocks];
    __shared__ uint32_t ikey[kProbeMaxBlocks];
    __shared__ uint8_t flag[kProbeMaxBlocks];
    __shared__ uint32_t hist[512];
    __shared__ int sh[4];
    __shared__ int wsum[kWaves];
    __shared__ uint32_t red_hi[kWaves], red_lo[kWaves];

    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    const int L = max(sl[b], 0);
    const int nb = min((L + BS - 1) / BS, mkbpr);
    const uint32_t* krow = keys + (size_t(b) * H + h) * mkbpr;
    for (int i = tid; i < nb; i += kThreads) {
        pkey[i] = krow[i];
        flag[i] = 0;
    }
    // importance sums: fp32, token order, one thread per block (page 1's running sum)
    if (importance) {
        const float* ip = importance + size_t(b) * imp_stride;
        for (int i = tid; i < nb; i += kThreads) {
            const int p0 = i * BS, pe = min(min(p0 + BS, L), imp_stride);  // tokens past the row count 0
            float s = 0.f;
            int ps = p0;
            for (; ps + 8 <= pe; ps += 8) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = ip[ps + u];
#pragma unroll
                for (int u = 0; u < 8; ++u) s += v[u];
            }
            for (; ps < pe; ++ps) s += ip[ps];
            ikey[i] = f2key(s);
        }
    }
    __syncthreads();

    // importance preselect
    const int budget = importance ? min((k + 1) / 2, nb) : 0;
    if (budget > 0)
        mark_top(nb, budget, [&](int i) { return true; }, [&](int i) { return ikey[i]; }, flag, kImp, hist, sh,
                 wsum);
    // probe fill
    const int r = min(k, nb) - budget;
    if (r > 0)
        mark_top(nb, r, [&](int i) { return flag[i] == 0; }, [&](int i) { return pkey[i]; }, flag, kProbe, hist,
                 sh, wsum);
    // recency insurance: the last block replaces the lowest probe pick
    if ((flags & 4u) && nb > 0 && r > 0 && flag[nb - 1] == 0) {
        uint64_t best = ~0ull;  // min over probe picks of (probe key, then higher index is lower)
        for (int i = tid; i < nb; i += kThreads) {
            if (flag[i] == kProbe) {
                const uint64_t cc = (uint64_t(pkey[i]) << 32) | uint64_t(0xffffffffu - uint32_t(i));
                best = cc < best ? cc : best;
            }
        }
        uint32_t hi = uint32_t(best >> 32), lo = uint32_t(best);
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
            const uint32_t h2 = __shfl_xor(hi, o, kWave), l2 = __shfl_xor(lo, o, kWave);
            if (h2 < hi || (h2 == hi && l2 < lo)) { hi = h2; lo = l2; }
        }
        if (lane_id() == 0) { red_hi[wave_id()] = hi; red_lo[wave_id()] = lo; }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < kWaves; ++w)
                if (red_hi[w] < hi || (red_hi[w] == hi && red_lo[w] < lo)) { hi = red_hi[w]; lo = red_lo[w]; }
            const int victim = int(0xffffffffu - lo);
            flag[victim] = 0;
            flag[nb - 1] = kProbe;
        }
        __syncthreads();
    }

    // ascending output: contiguous runs per thread, one block-wide scan for positions
    int32_t* out = selected + (size_t(b) * H + h) * k;
    const int E = (nb + kThreads - 1) / kThreads;
    const int j0 = min(nb, tid * E), j1 = min(nb, j0 + E);
    int pick_local = 0;
    for (int i = j0; i < j1; ++i) pick_local += flag[i] != 0 ? 1 : 0;
    int npick;
    int pos = block_excl_scan(pick_local, wsum, npick);
    for (int i = j0; i < j1; ++i) {
        if (flag[i] != 0) {
            if (pos < k) out[pos] = i;
            ++pos;
        }
    }
    for (int j = npick + tid; j < k; j += kThreads) out[j] = -1;
    if (tid == 0) n_selected[size_t(b) * H + h] = min(npick, k);
    if (probe_scores)
        for (int i = tid; i < nb; i += kThreads) probe_scores[(size_t(b) * H + h) * mkbpr + i] = key2f(pkey[i]);
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

hipError_t launch_probe_select(const ProbeArgs& a, hipStream_t s) {
    uint32_t* keys = (uint32_t*)a.workspace;
    auto by_k = [&](auto q) {
        constexpr int QD = decltype(q)::value;
        if (a.kv_dtype == kBF16) launch_score<QD, kBF16>(a, keys, s);
        else if (a.kv_dtype == kF16) launch_score<QD, kF16>(a, keys, s);
        else launch_score<QD, kF32>(a, keys, s);
    };
    if (a.q_dtype == kBF16) by_k(std::integral_constant<int, kBF16>{});
    else if (a.q_dtype == kF16) by_k(std::integral_constant<int, kF16>{});
    else by_k(std::integral_constant<int, kF32>{});
    hipLaunchKernelGGL(probe_pick_kernel, dim3(unsigned(a.H), unsigned(a.B)), dim3(kThreads), 0, s, keys, a.mkbpr,
                       a.seq_lens, a.importance, a.imp_stride, a.k, a.flags, a.H, a.BS, a.selected, a.n_selected,
                       a.probe_scores);
    return hipGetLastError();
}

}  // namespace qs

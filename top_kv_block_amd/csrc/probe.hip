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
// with the block-wide radix select plus one ordered pass.
#include <math.h>

#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace {

constexpr uint8_t kImp = 1, kProbe = 2;

template <class Pred, class KeyOf>
__device__ void mark_top(int nb, int r, Pred cand, KeyOf key_of, uint8_t* flag, uint8_t mark, uint32_t* hist,
                         int* sh, int* wsum) {
    // marks the r best candidates (value desc, index asc); r >= 1
    int ncand = 0;
    {
        int tot = 0;
        for (int ib = 0; ib < nb; ib += kThreads) {
            const int i = ib + threadIdx.x;
            int t;
            block_excl_count(i < nb && cand(i), wsum, t);
            tot += t;
        }
        ncand = tot;
    }
    if (r >= ncand) {
        for (int i = threadIdx.x; i < nb; i += kThreads)
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
    const uint32_t T = block_radix_select(nb, r, kf, hist, sh, need_eq);
    int eq_seen = 0;
    for (int ib = 0; ib < nb; ib += kThreads) {
        const int i = ib + threadIdx.x;
        const bool c = i < nb && cand(i);
        const uint32_t key = c ? key_of(i) : 0u;
        const bool eq = c && key == T;
        int eq_tot;
        const int rank = block_excl_count(eq, wsum, eq_tot) + eq_seen;
        if (c && (key > T || (eq && rank < need_eq))) flag[i] = mark;
        eq_seen += eq_tot;
    }
    __syncthreads();
}

template <bool QBF16, bool KBF16>
__global__ __launch_bounds__(kThreads) void probe_kernel(
    const uint8_t* __restrict__ query, const uint8_t* __restrict__ kc, int num_kv_blocks,
    const int32_t* __restrict__ bt, int mkbpr, const int32_t* __restrict__ sl,
    const float* __restrict__ importance, int imp_stride, int n_probe, int k, uint32_t flags,
    int H, int N, int BS, int32_t* __restrict__ selected, int32_t* __restrict__ n_selected,
    float* __restrict__ probe_scores) {
    constexpr int D = 128;
    constexpr int ke = KBF16 ? 2 : 4;
    constexpr int qe = QBF16 ? 2 : 4;
    constexpr int LPR = D * ke / 16;  // lanes per key row
    constexpr int EPL = 16 / ke;      // channels per lane
    constexpr int GRP = kThreads / LPR;
    constexpr int U = 4;

    __shared__ uint32_t pkey[kProbeMaxBlocks];
    __shared__ uint32_t ikey[kProbeMaxBlocks];
    __shared__ uint8_t flag[kProbeMaxBlocks];
    __shared__ uint32_t hist[256];
    __shared__ int sh[4];
    __shared__ int wsum[kWaves];
    __shared__ uint32_t red_hi[kWaves], red_lo[kWaves];

    const int h = blockIdx.x, b = blockIdx.y;
    const int G = H / N;
    const int kh = h / G;
    const int tid = threadIdx.x;
    const int L = max(sl[b], 0);
    const int nb = min((L + BS - 1) / BS, mkbpr);
    const int np = max(1, n_probe);
    const uint32_t init_key = f2key(-1e30f);

    for (int i = tid; i < nb; i += kThreads) {
        pkey[i] = init_key;
        flag[i] = 0;
    }
    // importance sums: fp32, token order, one thread per block
    if (importance) {
        for (int i = tid; i < nb; i += kThreads) {
            const int p0 = i * BS, pe = min(min(p0 + BS, L), imp_stride);  // tokens past the row count 0
            float s = 0.f;
            const float* ip = importance + size_t(b) * imp_stride;
            for (int ps = p0; ps < pe; ++ps) s += ip[ps];
            ikey[i] = f2key(s);
        }
    }
    __syncthreads();

    // query channels of this lane (fp32)
    const int lr = tid % LPR, grp = tid / LPR;
    float q[EPL];
    {
        const uint8_t* qp = query + (size_t(b) * H + h) * D * qe;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int d = lr * EPL + e;
            q[e] = QBF16 ? bf16_to_f32(((const uint16_t*)qp)[d]) : ((const float*)qp)[d];
        }
    }

    // probe dots: item = (block i, sample j); a block has ceil(len / step) samples
    const int smax = min(BS, 2 * np);
    const int items = nb * smax;
    const size_t row_bytes = size_t(N) * D * ke;
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
                const int i = it / smax, j = it % smax;
                const int p0 = i * BS, len = min(BS, L - p0);
                const int step = max(1, len / np);
                const int ps = p0 + j * step;
                if (ps < p0 + len) {
                    blk[u] = i;
                    row[u] = ps - p0;
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
            float part = 0.f;
            if constexpr (KBF16) {
#pragma unroll
                for (int j = 0; j < 4; ++j) part += q[2 * j] * bf_lo(w[j]) + q[2 * j + 1] * bf_hi(w[j]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) part += q[j] * __uint_as_float(w[j]);
            }
            const float dot = group_sum<LPR>(part);
            if (lr == 0 && blk[u] >= 0) atomicMax(&pkey[blk[u]], f2key(dot));
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
                const uint64_t c = (uint64_t(pkey[i]) << 32) | uint64_t(0xffffffffu - uint32_t(i));
                best = c < best ? c : best;
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

    // ascending output
    int32_t* out = selected + (size_t(b) * H + h) * k;
    int pos0 = 0;
    for (int ib = 0; ib < nb; ib += kThreads) {
        const int i = ib + tid;
        const bool pick = i < nb && flag[i] != 0;
        int tot;
        const int pos = block_excl_count(pick, wsum, tot) + pos0;
        if (pick && pos < k) out[pos] = i;
        pos0 += tot;
    }
    for (int j = pos0 + tid; j < k; j += kThreads) out[j] = -1;
    if (tid == 0) n_selected[size_t(b) * H + h] = min(pos0, k);
    if (probe_scores)
        for (int i = tid; i < nb; i += kThreads) probe_scores[(size_t(b) * H + h) * mkbpr + i] = key2f(pkey[i]);
}

template <bool QB, bool KB>
void launch_t(const ProbeArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((probe_kernel<QB, KB>), dim3(unsigned(a.H), unsigned(a.B)), dim3(kThreads), 0, s,
                       (const uint8_t*)a.query, (const uint8_t*)a.k_cache, a.num_kv_blocks, a.block_tables,
                       a.mkbpr, a.seq_lens, a.importance, a.imp_stride, a.n_probe, a.k, a.flags, a.H, a.N, a.BS,
                       a.selected, a.n_selected, a.probe_scores);
}

}  // namespace

hipError_t launch_probe_select(const ProbeArgs& a, hipStream_t s) {
    if (a.q_bf16) {
        if (a.kv_bf16) launch_t<true, true>(a, s); else launch_t<true, false>(a, s);
    } else {
        if (a.kv_bf16) launch_t<false, true>(a, s); else launch_t<false, false>(a, s);
    }
    return hipGetLastError();
}

}  // namespace qs

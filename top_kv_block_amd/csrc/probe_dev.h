// probe_dev.h -- page 1's pick for one (request, query head) row on one workgroup: the
// prefill-importance budget, the probe fill and the recency insurance, leaving the
// ascending selection in LDS. Shared by the selection kernel and the fused probe-select +
// attention kernel.
//
// Source: "0.8MB 跑通 Qwen | 第 10-2 篇: 推理引擎的 sparse top-k 块选择" (page 1),
// section 1 "知识点" (three signals + recency, lower-index ties, determinism) and
// section 2 "对应代码" (importance preselect with budget (k+1)/2, greedy probe fill,
// recency replacing the lowest probe pick only).
//
// Each greedy stage ("repeatedly take the best unused block, lower index on ties")
// selects the same set as taking the top-r keys under (value desc, index asc); that is
// computed with the block-wide threshold select plus one ordered pass. Importance sums
// are accumulated per block by one thread in token order in fp32, exactly as the page's
// loop does, so the importance stage is bit-exact.
#pragma once

#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace probe {

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

// LDS of one pick. After pick_row returns, sel holds the selection (it overlays the
// importance keys, dead by then) and pkey still holds the probe keys.
struct PickLds {
    uint32_t pkey[kProbeMaxBlocks];
    union {
        uint32_t ikey[kProbeMaxBlocks];
        int32_t sel[kProbeMaxBlocks];
    };
    uint8_t flag[kProbeMaxBlocks];
    uint32_t hist[512];
    int sh[4];
    int wsum[kWaves];
    uint32_t red_hi[kWaves], red_lo[kWaves];
};

// Picks row (b, h): krow = its nb probe keys (order-preserving images of the probe
// scores), imp_row = the request's importance row or nullptr. Leaves the min(k, nb)
// picks in s.sel in ascending block order and returns their count. Every thread must
// call it; s.sel and s.pkey are visible to all threads on return.
__device__ __forceinline__ int pick_row(const uint32_t* __restrict__ krow, int nb, int L,
                                        const float* __restrict__ imp_row, int imp_stride, int BS, int k,
                                        uint32_t flags, PickLds& s) {
    const int tid = threadIdx.x;
    for (int i = tid; i < nb; i += kThreads) {
        s.pkey[i] = krow[i];
        s.flag[i] = 0;
    }
    // importance sums: fp32, token order, one thread per block (page 1's running sum)
    if (imp_row) {
        for (int i = tid; i < nb; i += kThreads) {
            const int p0 = i * BS, pe = min(min(p0 + BS, L), imp_stride);  // tokens past the row count 0
            float sum = 0.f;
            int ps = p0;
            for (; ps + 8 <= pe; ps += 8) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = imp_row[ps + u];
#pragma unroll
                for (int u = 0; u < 8; ++u) sum += v[u];
            }
            for (; ps < pe; ++ps) sum += imp_row[ps];
            s.ikey[i] = f2key(sum);
        }
    }
    __syncthreads();

    // importance preselect
    const int budget = imp_row ? min((k + 1) / 2, nb) : 0;
    if (budget > 0)
        mark_top(nb, budget, [&](int i) { return true; }, [&](int i) { return s.ikey[i]; }, s.flag, kImp, s.hist,
                 s.sh, s.wsum);
    // probe fill
    const int r = min(k, nb) - budget;
    if (r > 0)
        mark_top(nb, r, [&](int i) { return s.flag[i] == 0; }, [&](int i) { return s.pkey[i]; }, s.flag, kProbe,
                 s.hist, s.sh, s.wsum);
    // recency insurance: the last block replaces the lowest probe pick
    if ((flags & 4u) && nb > 0 && r > 0 && s.flag[nb - 1] == 0) {
        uint64_t best = ~0ull;  // min over probe picks of (probe key, then higher index is lower)
        for (int i = tid; i < nb; i += kThreads) {
            if (s.flag[i] == kProbe) {
                const uint64_t cc = (uint64_t(s.pkey[i]) << 32) | uint64_t(0xffffffffu - uint32_t(i));
                best = cc < best ? cc : best;
            }
        }
        uint32_t hi = uint32_t(best >> 32), lo = uint32_t(best);
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
            const uint32_t h2 = __shfl_xor(hi, o, kWave), l2 = __shfl_xor(lo, o, kWave);
            if (h2 < hi || (h2 == hi && l2 < lo)) { hi = h2; lo = l2; }
        }
        if (lane_id() == 0) { s.red_hi[wave_id()] = hi; s.red_lo[wave_id()] = lo; }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < kWaves; ++w)
                if (s.red_hi[w] < hi || (s.red_hi[w] == hi && s.red_lo[w] < lo)) { hi = s.red_hi[w]; lo = s.red_lo[w]; }
            const int victim = int(0xffffffffu - lo);
            s.flag[victim] = 0;
            s.flag[nb - 1] = kProbe;
        }
        __syncthreads();
    }

    // ascending output: contiguous runs per thread, one block-wide scan for positions (the
    // scan's barrier also retires every read of the importance keys that sel overlays)
    const int E = (nb + kThreads - 1) / kThreads;
    const int j0 = min(nb, tid * E), j1 = min(nb, j0 + E);
    int pick_local = 0;
    for (int i = j0; i < j1; ++i) pick_local += s.flag[i] != 0 ? 1 : 0;
    int npick;
    int pos = block_excl_scan(pick_local, s.wsum, npick);
    for (int i = j0; i < j1; ++i) {
        if (s.flag[i] != 0) {
            s.sel[pos] = i;
            ++pos;
        }
    }
    __syncthreads();
    return min(npick, k);
}

}  // namespace probe
}  // namespace qs

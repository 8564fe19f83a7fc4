// select.hip -- Quest top-k block selection with sink / local-window forcing.
//
// Source: "ops-transformer select_attention_operators" (page 3), section
// "quest_block_select_paged: 解码期 top-k 预测算法" (grouped-query mean, per-channel
// max(gq*kmax, gq*kmin) summed over D, top-k over the request's blocks, sequence-relative
// indices) and section "三个核心算子" (the _w variant forces the sink block and the local
// window). Ties go to the lower block index ("0.8MB 跑通 Qwen 10-2" (page 1), section 1).
//
// Design (CDNA4): the score stream is HBM-bound (about 1 flop per metadata byte), so the
// grid spreads it wide: workgroup (chunk, n, b) scores up to `chunk` blocks of one
// (request, KV head). A block's max row and min row are 256 B each in bf16; 16 lanes
// take 16 B apiece (one global_load_dwordx4), multiply by the grouped query held in
// registers, and a 16-lane shuffle reduction yields the score. Scores go to a per-row
// fp32 array; the workgroup that finishes a row last (device-scope arrival counter,
// release/acquire fences) runs the exact top-k: a 4-pass, 8-bit radix select on an
// order-preserving integer image of the scores finds the k-th best value T, then one
// ordered pass keeps every block above T and the lowest-index blocks equal to T. That
// reproduces "higher score first, lower index on ties" exactly, independent of the
// order in which workgroups finish. Output is written in ascending block order.
#include <math.h>

#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace {

constexpr int kChunk = 64;

struct Forced {
    int w_lo;   // blocks >= w_lo are forced (window), nb when none
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
        long long num = (long long)L - u;
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

template <bool BF16>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const uint8_t* __restrict__ query, const uint8_t* __restrict__ maxb, const uint8_t* __restrict__ minb,
    int num_meta, const int32_t* __restrict__ mt, int mmbpr, const int32_t* __restrict__ sl,
    const int32_t* __restrict__ tsmu, uint32_t flags, int k, int H, int N, int BS, int chunk,
    int32_t* __restrict__ selected, int32_t* __restrict__ n_selected, float* __restrict__ dbg_scores,
    float* __restrict__ ws_scores, uint32_t* __restrict__ counters) {
    constexpr int esize = BF16 ? 2 : 4;
    constexpr int D = 128;
    constexpr int LPR = D * esize / 16;  // lanes per metadata row
    constexpr int EPL = 16 / esize;      // channels per lane
    constexpr int RPP = kThreads / LPR;  // rows per pass
    constexpr int U = 4;                 // passes in flight

    __shared__ uint32_t hist[256];
    __shared__ int sh[4];
    __shared__ int wsum[kWaves];
    __shared__ int is_last;

    const int c = blockIdx.x, n = blockIdx.y, b = blockIdx.z;
    const int cap = mmbpr * BS;
    const int L = max(sl[b], 0);
    const int nb = min((L + BS - 1) / BS, cap);
    const int n_chunks_b = max(1, (nb + chunk - 1) / chunk);
    if (c >= n_chunks_b) return;
    const Forced F = forced_set(L, nb, BS, k, tsmu, b, flags);
    const int tid = threadIdx.x;
    const int lr = tid % LPR;    // lane within the row
    const int slot = tid / LPR;  // row slot within a pass
    const int G = H / N;
    float* scores = (dbg_scores ? dbg_scores : ws_scores) + (size_t(b) * N + n) * cap;

    // grouped query for this lane's channels: mean over the group's G heads
    float gq[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) gq[e] = 0.f;
    for (int g = 0; g < G; ++g) {
        const u32x4 v = ld16(query + ((size_t(b) * H + size_t(n) * G + g) * D + lr * EPL) * esize);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) { gq[2 * j] += bf_lo(w[j]); gq[2 * j + 1] += bf_hi(w[j]); }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) gq[j] += __uint_as_float(w[j]);
        }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) gq[e] = gq[e] / float(G);

    // ---- scores of this chunk ----
    const int i0 = c * chunk;
    const int i_end = min(nb, i0 + chunk);
    const size_t row_bytes = size_t(N) * D * esize;
    for (int base = i0; base < i_end; base += RPP * U) {
        u32x4 vmx[U], vmn[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * RPP + slot;
            ok[u] = false;
            vmx[u] = u32x4{0u, 0u, 0u, 0u};
            vmn[u] = vmx[u];
            if (i < i_end && !F.has(i)) {
                const int m = mt[size_t(b) * mmbpr + i / BS];
                if (m >= 0 && m < num_meta) {
                    const size_t off = (size_t(m) * BS + (i % BS)) * row_bytes + size_t(n) * D * esize + lr * 16;
                    vmx[u] = ld16(maxb + off);
                    vmn[u] = ld16(minb + off);
                    ok[u] = true;
                }
            }
        }
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
                    scores[i] = s;
                else if (!F.has(i))
                    scores[i] = -INFINITY;  // metadata table entry out of range
                else if (dbg_scores)
                    scores[i] = __builtin_nanf("");
            }
        }
    }

    // ---- the workgroup that completes the row selects ----
    if (n_chunks_b > 1) {
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const uint32_t prev = atomicAdd(&counters[size_t(b) * N + n], 1u);
            is_last = (prev == uint32_t(n_chunks_b - 1));
        }
        __syncthreads();
        if (!is_last) return;
        __threadfence();
    } else {
        __syncthreads();
    }

    const int R = max(0, min(k, nb) - F.count);  // fill picks
    const int nc = nb - F.count;                   // fill candidates
    const bool take_all = R >= nc;
    uint32_t T = 0;
    int need_eq = 0;
    if (R > 0 && !take_all) {
        auto kf = [&](int i, uint32_t& key) -> bool {
            if (F.has(i)) return false;
            key = f2key(scores[i]);
            return true;
        };
        T = block_radix_select(nb, R, kf, hist, sh, need_eq);
    }
    int32_t* out = selected + (size_t(b) * N + n) * k;
    int pos0 = 0, eq_seen = 0;
    for (int ib = 0; ib < nb; ib += kThreads) {
        const int i = ib + tid;
        const bool valid = i < nb;
        const bool frc = valid && F.has(i);
        const bool cand = valid && !frc && R > 0;
        const uint32_t key = cand ? f2key(scores[i]) : 0u;
        const bool eq = cand && !take_all && key == T;
        int eq_tot;
        const int eq_rank = block_excl_count(eq, wsum, eq_tot) + eq_seen;
        const bool pick = frc || (cand && (take_all || key > T || (eq && eq_rank < need_eq)));
        int tot;
        const int pos = block_excl_count(pick, wsum, tot) + pos0;
        if (pick && pos < k) out[pos] = i;
        pos0 += tot;
        eq_seen += eq_tot;
    }
    for (int j = pos0 + tid; j < k; j += kThreads) out[j] = -1;
    if (tid == 0) {
        n_selected[size_t(b) * N + n] = min(pos0, k);
        if (n_chunks_b > 1) counters[size_t(b) * N + n] = 0u;
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

SelectPlan plan_block_select(int B, int N, int BS, int mmbpr) {
    SelectPlan p;
    const size_t cap = size_t(mmbpr) * BS;
    // rows beyond the counter area are scored by one workgroup each (no counters)
    p.chunk = ((long long)B * N <= kMaxCounters) ? kChunk : int(cap);
    p.n_chunks = int((cap + p.chunk - 1) / p.chunk);
    p.counters_off = 0;
    p.scores_off = kCounterBytes;
    p.bytes = p.scores_off + align256(size_t(B) * N * cap * sizeof(float));
    return p;
}

hipError_t launch_block_select(const SelectArgs& a, const SelectPlan& p, hipStream_t s) {
    dim3 grid(unsigned(p.n_chunks), unsigned(a.N), unsigned(a.B));
    float* ws_scores = (float*)((uint8_t*)a.workspace + p.scores_off);
    uint32_t* counters = (uint32_t*)((uint8_t*)a.workspace + p.counters_off);
    if (a.bf16)
        hipLaunchKernelGGL(select_kernel<true>, grid, dim3(kThreads), 0, s, (const uint8_t*)a.query,
                           (const uint8_t*)a.maxb, (const uint8_t*)a.minb, a.num_meta, a.meta_tables, a.mmbpr,
                           a.seq_lens, a.tsmu, a.flags, a.k, a.H, a.N, a.BS, p.chunk, a.selected, a.n_selected,
                           a.block_scores, ws_scores, counters);
    else
        hipLaunchKernelGGL(select_kernel<false>, grid, dim3(kThreads), 0, s, (const uint8_t*)a.query,
                           (const uint8_t*)a.maxb, (const uint8_t*)a.minb, a.num_meta, a.meta_tables, a.mmbpr,
                           a.seq_lens, a.tsmu, a.flags, a.k, a.H, a.N, a.BS, p.chunk, a.selected, a.n_selected,
                           a.block_scores, ws_scores, counters);
    return hipGetLastError();
}

}  // namespace qs

// attn.hip -- exact decode attention over the selected KV blocks only.
//
// Source: "0.8MB 跑通 Qwen | 第 10-2 篇" (page 1), section 2 "对应代码": per-token scores
// on the selected blocks (fp32 KV: float dot; q8 KV: int8 x int8 dot plus scale), max
// subtraction and softmax over the selected tokens only, weighted sum of V; section 1:
// the softmax is renormalised over the selection. "ops-transformer
// select_attention_operators" (page 3), section "quest_block_select_paged": selected
// indices are sequence-relative and are mapped through block_tables.
//
// Design (CDNA4): single-query decode attention reads each selected K/V row once and
// does O(G) flops per byte, so it is bound by the paged K/V gather. Workgroup
// (split, row, request) takes a contiguous range of the row's selection slots; all
// query heads that share the row (and the KV head) are processed together (up to 8 per
// workgroup), so every K/V row is fetched once for all of them. A token row of one KV
// head (128 channels) is read by LPR lanes with one 16-byte load each; the partial dot
// is reduced with shuffles inside that lane group; each lane group is an independent
// online-softmax worker (running max, sum and its slice of the output accumulator).
// Groups merge through shuffles and LDS at the end; splits write (max, sum, acc)
// partials and the workgroup that completes a row (device-scope arrival counter)
// combines them in split order, so the result does not depend on scheduling.
// int8 KV: the query row is quantised in fp32 (absmax / 127, half-to-even, clamp
// +-127) and dots run on v_dot4_i32_i8 with exact int32 accumulation.
#include <math.h>

#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace {

constexpr int kTargetWorkgroups = 2048;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void merge_state(float& m, float& l, float* a, int n, float m2, float l2,
                                            const float* a2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    const float c1 = exp2f(m - M), c2 = exp2f(m2 - M);
    l = l * c1 + l2 * c2;
    for (int e = 0; e < n; ++e) a[e] = a[e] * c1 + a2[e] * c2;
    m = M;
}

template <int KV, bool QBF16, int HC>
__global__ __launch_bounds__(kThreads) void attn_kernel(
    const uint8_t* __restrict__ query, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const float* __restrict__ ksc, const float* __restrict__ vsc, int num_kv_blocks,
    const int32_t* __restrict__ bt, int mkbpr, const int32_t* __restrict__ sl,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ nsel, int H, int N, int BS, int sel_heads, int k,
    int hpr, int hchunks, int splits, int spb, float scale_log2, uint8_t* __restrict__ out,
    float* __restrict__ part, uint32_t* __restrict__ counters) {
    constexpr int D = 128;
    constexpr int ke = KV == 0 ? 4 : (KV == 1 ? 2 : 1);
    constexpr int qe = QBF16 ? 2 : 4;
    constexpr int LPR = D * ke / 16;  // lanes per K/V row
    constexpr int EPL = 16 / ke;      // channels per lane
    constexpr int NG = kThreads / LPR;  // independent lane groups per workgroup
    constexpr int U = 2;              // tokens in flight per group

    __shared__ float red_m[kWaves][HC];
    __shared__ float red_l[kWaves][HC];
    __shared__ float red_a[kWaves][HC][D];
    __shared__ int is_last;

    const int split = blockIdx.x % splits, hcix = blockIdx.x / splits;
    const int s = blockIdx.y, b = blockIdx.z;
    const int h0 = s * hpr + hcix * HC;
    const int nh = min(HC, hpr - hcix * HC);
    const int G = H / N;
    const int kh = (s * hpr) / G;
    const int tid = threadIdx.x, lr = tid % LPR, grp = tid / LPR;

    // ---- query: fp32 (pre-scaled by softmax_scale * log2 e) or int8 codes ----
    float qf[HC][EPL];
    int32_t q8[HC][EPL / 4 > 0 ? EPL / 4 : 1];
    float qscale[HC];
#pragma unroll
    for (int g = 0; g < HC; ++g) {
        const int hh = h0 + (g < nh ? g : 0);
        const uint8_t* qp = query + (size_t(b) * H + hh) * D * qe;
        float x[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int d = lr * EPL + e;
            x[e] = QBF16 ? bf16_to_f32(((const uint16_t*)qp)[d]) : ((const float*)qp)[d];
        }
        if constexpr (KV == 2) {
            float amax = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
            amax = group_max<LPR>(amax);
            const float sq = amax / 127.0f;
            qscale[g] = sq * scale_log2;
#pragma unroll
            for (int w = 0; w < EPL / 4; ++w) {
                uint32_t packed = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float r = 0.f;
                    if (sq != 0.f) r = fminf(fmaxf(rintf(x[4 * w + j] / sq), -127.f), 127.f);
                    packed |= (uint32_t(int32_t(r)) & 0xffu) << (8 * j);
                }
                q8[g][w] = int32_t(packed);
            }
        } else {
            qscale[g] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) qf[g][e] = x[e] * scale_log2;
        }
    }

    // ---- this split's selection slots ----
    const int L = max(sl[b], 0);
    const int nb = (L + BS - 1) / BS;
    const int row = b * sel_heads + s;
    const int ns = min(max(nsel[row], 0), k);
    const int slot0 = split * spb, slot1 = min(ns, slot0 + spb);
    const int32_t* srow = sel + size_t(row) * k;
    const size_t tok_bytes = size_t(N) * D * ke;  // stride between tokens of one KV head

    float m[HC], l[HC], acc[HC][EPL];
#pragma unroll
    for (int g = 0; g < HC; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }

    for (int slot = slot0; slot < slot1; ++slot) {
        const int blk = srow[slot];
        if (blk < 0 || blk >= nb || blk >= mkbpr) continue;
        const int phys = bt[size_t(b) * mkbpr + blk];
        if (phys < 0 || phys >= num_kv_blocks) continue;
        const int nt = min(BS, L - blk * BS);
        const size_t tok0 = size_t(phys) * BS;
        const uint8_t* kb = kc + (tok0 * N + kh) * D * ke + lr * 16;
        const uint8_t* vb = vc + (tok0 * N + kh) * D * ke + lr * 16;
        for (int t0 = 0; t0 < nt; t0 += NG * U) {
            u32x4 kv[U], vv[U];
            float ks[U], vs[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int t = t0 + u * NG + grp;
                ok[u] = t < nt;
                const int tt = ok[u] ? t : 0;
                kv[u] = ld16(kb + size_t(tt) * tok_bytes);
                vv[u] = ld16(vb + size_t(tt) * tok_bytes);
                if constexpr (KV == 2) {
                    ks[u] = ksc[(tok0 + tt) * N + kh];
                    vs[u] = vsc[(tok0 + tt) * N + kh];
                } else {
                    ks[u] = vs[u] = 1.f;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t kw[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
                const uint32_t vw[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
                float vf[EPL];
                if constexpr (KV == 0) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) vf[j] = __uint_as_float(vw[j]);
                } else if constexpr (KV == 1) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) { vf[2 * j] = bf_lo(vw[j]); vf[2 * j + 1] = bf_hi(vw[j]); }
                } else {
#pragma unroll
                    for (int j = 0; j < 16; ++j) vf[j] = float(int8_t(vw[j / 4] >> (8 * (j % 4)))) * vs[u];
                }
#pragma unroll
                for (int g = 0; g < HC; ++g) {
                    float sc;
                    if constexpr (KV == 2) {
                        int dot = 0;
#pragma unroll
                        for (int j = 0; j < 4; ++j) dot = __builtin_amdgcn_sdot4(q8[g][j], int32_t(kw[j]), dot, false);
                        dot = group_sum_i<LPR>(dot);
                        sc = float(dot) * (qscale[g] * ks[u]);
                    } else {
                        float p = 0.f;
                        if constexpr (KV == 0) {
#pragma unroll
                            for (int j = 0; j < 4; ++j) p += qf[g][j] * __uint_as_float(kw[j]);
                        } else {
#pragma unroll
                            for (int j = 0; j < 4; ++j) p += qf[g][2 * j] * bf_lo(kw[j]) + qf[g][2 * j + 1] * bf_hi(kw[j]);
                        }
                        sc = group_sum<LPR>(p);
                    }
                    if (ok[u]) {
                        const float mn = fmaxf(m[g], sc);
                        const float cf = exp2f(m[g] - mn);
                        const float pw = exp2f(sc - mn);
                        l[g] = l[g] * cf + pw;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * cf + pw * vf[e];
                        m[g] = mn;
                    }
                }
            }
        }
    }

    // ---- merge the lane groups of each wave (same lr = same channels) ----
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
        for (int g = 0; g < HC; ++g) {
            const float m2 = __shfl_xor(m[g], o, kWave);
            const float l2 = __shfl_xor(l[g], o, kWave);
            float a2[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) a2[e] = __shfl_xor(acc[g][e], o, kWave);
            merge_state(m[g], l[g], acc[g], EPL, m2, l2, a2);
        }
    }
    const int w = wave_id();
    if (lane_id() < LPR) {
#pragma unroll
        for (int g = 0; g < HC; ++g) {
            if (lr == 0) { red_m[w][g] = m[g]; red_l[w][g] = l[g]; }
#pragma unroll
            for (int e = 0; e < EPL; ++e) red_a[w][g][lr * EPL + e] = acc[g][e];
        }
    }
    __syncthreads();

    // ---- workgroup result per (head, channel) ----
    const int qe_out = qe;
    constexpr int PER = (HC * D + kThreads - 1) / kThreads;
    float rm[PER], rl[PER], ra[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int idx = tid + r * kThreads;
        rm[r] = -INFINITY; rl[r] = 0.f; ra[r] = 0.f;
        if (idx < HC * D) {
            const int g = idx / D, d = idx % D;
            for (int ww = 0; ww < kWaves; ++ww) merge_state(rm[r], rl[r], &ra[r], 1, red_m[ww][g], red_l[ww][g], &red_a[ww][g][d]);
        }
    }

    auto emit = [&](int g, int d, float M, float Ls, float A) {
        if (g >= nh) return;
        const float v = (Ls > 0.f) ? A / Ls : 0.f;
        const size_t o = (size_t(b) * H + h0 + g) * D + d;
        if (QBF16) ((uint16_t*)out)[o] = f32_to_bf16_rne(v);
        else ((float*)out)[o] = v;
    };

    if (splits == 1) {
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int idx = tid + r * kThreads;
            if (idx < HC * D) emit(idx / D, idx % D, rm[r], rl[r], ra[r]);
        }
        return;
    }

    // partials: [row][hchunk][split][HC][D + 2] = acc[0..D-1], max, sum
    const size_t crow = size_t(row) * hchunks + hcix;
    float* pbase = part + crow * size_t(splits) * HC * (D + 2);
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int idx = tid + r * kThreads;
        if (idx < HC * D) {
            const int g = idx / D, d = idx % D;
            float* p = pbase + (size_t(split) * HC + g) * (D + 2);
            p[d] = ra[r];
            if (d == 0) { p[D] = rm[r]; p[D + 1] = rl[r]; }
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&counters[crow], 1u);
        is_last = (prev == uint32_t(splits - 1));
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int idx = tid + r * kThreads;
        if (idx < HC * D) {
            const int g = idx / D, d = idx % D;
            float M = -INFINITY, Ls = 0.f, A = 0.f;
            for (int j = 0; j < splits; ++j) {
                const float* p = pbase + (size_t(j) * HC + g) * (D + 2);
                merge_state(M, Ls, &A, 1, p[D], p[D + 1], &p[d]);
            }
            emit(g, d, M, Ls, A);
        }
    }
    if (tid == 0) counters[crow] = 0u;
    (void)qe_out;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

template <int KV, bool QB, int HC>
void launch_t(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
    float* part = (float*)((uint8_t*)a.workspace + p.part_off);
    uint32_t* counters = (uint32_t*)((uint8_t*)a.workspace + p.counters_off);
    dim3 grid(unsigned(p.splits * p.hchunks), unsigned(a.sel_heads), unsigned(a.B));
    hipLaunchKernelGGL((attn_kernel<KV, QB, HC>), grid, dim3(kThreads), 0, s, (const uint8_t*)a.query,
                       (const uint8_t*)a.k_cache, (const uint8_t*)a.v_cache, a.k_scale, a.v_scale, a.num_kv_blocks,
                       a.block_tables, a.mkbpr, a.seq_lens, a.selected, a.n_selected, a.H, a.N, a.BS, a.sel_heads,
                       a.k, p.hpr, p.hchunks, p.splits, p.spb, a.scale * kLog2e, (uint8_t*)a.out, part, counters);
}

template <int KV, bool QB>
void launch_hc(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
    switch (p.hc) {
        case 1: launch_t<KV, QB, 1>(a, p, s); break;
        case 2: launch_t<KV, QB, 2>(a, p, s); break;
        case 4: launch_t<KV, QB, 4>(a, p, s); break;
        default: launch_t<KV, QB, 8>(a, p, s); break;
    }
}

}  // namespace

AttnPlan plan_sparse_attn(int B, int H, int N, int D, int sel_heads, int k) {
    AttnPlan p;
    p.hpr = H / sel_heads;
    p.hc = p.hpr >= 8 ? 8 : (p.hpr >= 4 ? (p.hpr == 4 ? 4 : 8) : (p.hpr == 1 ? 1 : (p.hpr == 2 ? 2 : 4)));
    p.hchunks = (p.hpr + p.hc - 1) / p.hc;
    const long long rows = (long long)B * sel_heads * p.hchunks;
    const long long rows1 = rows > 0 ? rows : 1;
    long long splits = (kTargetWorkgroups + rows1 - 1) / rows1;
    if (splits < 1) splits = 1;
    if (splits > k) splits = k;
    if (rows > kMaxCounters) splits = 1;  // rows beyond the counter area: no split, no counters
    p.spb = int((k + splits - 1) / splits);
    p.splits = (k + p.spb - 1) / p.spb;
    const size_t part_bytes =
        p.splits > 1 ? size_t(rows) * p.splits * p.hc * (size_t(D) + 2) * sizeof(float) : 0;
    p.counters_off = 0;
    p.part_off = kCounterBytes;
    p.bytes = p.part_off + align256(part_bytes);
    return p;
}

hipError_t launch_sparse_attn(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
    const bool qb = a.q_dtype == 1;
    if (a.kv_dtype == 0) { if (qb) launch_hc<0, true>(a, p, s); else launch_hc<0, false>(a, p, s); }
    else if (a.kv_dtype == 1) { if (qb) launch_hc<1, true>(a, p, s); else launch_hc<1, false>(a, p, s); }
    else { if (qb) launch_hc<2, true>(a, p, s); else launch_hc<2, false>(a, p, s); }
    return hipGetLastError();
}

}  // namespace qs

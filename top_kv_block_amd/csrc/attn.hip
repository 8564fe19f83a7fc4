// attn.hip -- exact decode attention over the selected KV blocks only.
//
// Source: "0.8MB 跑通 Qwen | 第 10-2 篇" (page 1), section 2 "对应代码": per-token scores
// on the selected blocks (fp32 KV: float dot; q8 KV: int8 x int8 dot plus scale), max
// subtraction and softmax over the selected tokens only, weighted sum of V; section 1:
// the softmax is renormalised over the selection. "ops-transformer
// select_attention_operators" (page 3), section "quest_block_select_paged": selected
// indices are sequence-relative and are mapped through block_tables.
//
// Design (CDNA4). Decode attention reads every selected K/V row once; the bytes are the
// bound. A workgroup takes one selection row (all query heads sharing a KV head, so
// each K/V row is fetched once for all of them) and a range of its selection slots.
//
// bf16 (or fp16) KV with a query of the same type (the serving path) runs on the matrix
// cores, because with
// G query heads per KV head the work per token is a [G x 128] x [128 x T] product and on
// the vector ALU (no packed fp32 here) it would cost about as many cycles as the HBM
// stream: per 32-token chunk a wave computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16
// (K rows are loaded as whole 256-B rows, 16 lanes each, staged through the wave's LDS
// tile and read back in the A-operand layout: a direct A-operand load would touch 16 rows
// x 64 B per instruction and streams ~2% slower; the heads are the 16 columns), does the
// online softmax on the accumulator registers (each lane owns one
// head, so the running max/sum and the output rescale need no lane exchange), rounds P
// to the operand format and accumulates O^T = V^T P^T with 8 more MFMAs. V^T comes from a per-wave
// LDS tile that the wave writes transposed (8x8 register transposes + 16-byte stores).
// Four waves take interleaved 32-token chunks and merge (max, sum, acc) through LDS.
//
// fp32 and int8 KV, and mixed query / KV types (small, latency-bound workloads), run on
// the vector ALU in fp32: a token row
// is read by LPR lanes with 16-byte loads, dots reduce by shuffles, each lane group is an
// independent online-softmax worker. int8: the query row is quantised in fp32 (absmax /
// 127, half-to-even, clamp +-127) and dots use v_dot4_i32_i8 with exact int32 sums.
//
// When there are too few rows to fill the chip the slots are split over workgroups,
// each writing (max, sum, acc) partials, and a small second kernel merges them in a
// fixed order (no cross-workgroup synchronisation inside a kernel).
#include <math.h>

#include <type_traits>

#include "attn_dev.h"
#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace {

using namespace attn;

constexpr int kTargetWorkgroupsMfma = 1024;
constexpr int kTargetWorkgroupsVec = 2048;
constexpr int kNoSplitRows = 1024;   // rows at which each row gets one workgroup

// the attention kernels: one workgroup per (slot split x head chunk, selection row, request);
// NT: K/V through non-temporal loads
template <int DT, bool NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void attn_mfma_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMfmaLdsBytes];  // 40 KiB
    const uint3 w = xcd_block_index(p.splits > 1);
    const int split = int(w.x) % p.splits, hcix = int(w.x) / p.splits;
    const int s = int(w.y), b = int(w.z);
    const int row = b * p.sel_heads + s;
    mfma_body<DT, NT>(p, split, hcix, s, b, p.sel + size_t(row) * p.k, p.nsel[row], lds, false);
}

template <int KV, int QDT, int HC>
__global__ __launch_bounds__(kThreads) void attn_vec_kernel(AttnParams p) {
    __shared__ float red[vec_red_floats<HC>()];
    const int split = blockIdx.x % p.splits, hcix = blockIdx.x / p.splits;
    const int s = blockIdx.y, b = blockIdx.z;
    const int row = b * p.sel_heads + s;
    vec_body<KV, QDT, HC>(p, split, hcix, s, b, p.sel + size_t(row) * p.k, p.nsel[row], red);
}

// ------------------------------------------------------------------------------------
// combine pass for split rows: merges the splits' partials. Four lanes per output
// element (request, head, channel): lane u merges splits u, u+4, u+8, ... (their loads
// issued together), then the four states are merged across the lanes with two xor
// shuffles. The pairwise merge is symmetric in its operands (max, and sums of products,
// whose fp additions commute), so both lanes of a pair hold bitwise the same state and
// the result does not depend on scheduling.
// ------------------------------------------------------------------------------------
constexpr int kCombineLanes = 4;
constexpr int kCombineBatch = 8;

__global__ __launch_bounds__(kThreads) void attn_combine_kernel(AttnParams p, int hc_cap, int out_dt) {
    const int gid = blockIdx.x * kThreads + threadIdx.x;
    const int e = gid / kCombineLanes, u = gid % kCombineLanes;  // (head, channel) of request b
    const int b = blockIdx.y;
    const bool live = e < p.H * D;  // no early return: the lanes of an element shuffle together
    const int ee = live ? e : 0;
    const int d = ee % D, h = ee / D;
    const int s = h / p.hpr, hh = h % p.hpr;
    const int hcix = hh / hc_cap, g = hh % hc_cap;
    const int row = b * p.sel_heads + s;
    const float* base = p.part + ((size_t(row) * p.hchunks + hcix) * p.splits) * hc_cap * PSTRIDE + size_t(g) * PSTRIDE;
    const size_t sstride = size_t(hc_cap) * PSTRIDE;
    float M = -INFINITY, Ls = 0.f, A = 0.f;
    for (int sp0 = u; sp0 < p.splits; sp0 += kCombineLanes * kCombineBatch) {
        float mv[kCombineBatch], lv[kCombineBatch], av[kCombineBatch];
#pragma unroll
        for (int t = 0; t < kCombineBatch; ++t) {
            const int sp = min(sp0 + t * kCombineLanes, p.splits - 1);
            const float* rec = base + size_t(sp) * sstride;
            mv[t] = rec[D];
            lv[t] = rec[D + 1];
            av[t] = rec[d];
        }
#pragma unroll
        for (int t = 0; t < kCombineBatch; ++t)
            if (sp0 + t * kCombineLanes < p.splits) merge_state(M, Ls, &A, 1, mv[t], lv[t], &av[t]);
    }
#pragma unroll
    for (int o = 1; o < kCombineLanes; o <<= 1) {
        const float m2 = __shfl_xor(M, o, kWave), l2 = __shfl_xor(Ls, o, kWave), a2 = __shfl_xor(A, o, kWave);
        merge_state(M, Ls, &A, 1, m2, l2, &a2);
    }
    if (live && u == 0) store_out(p.out, (size_t(b) * p.H + h) * D + d, (Ls > 0.f) ? A / Ls : 0.f, out_dt);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

template <int KV, int QB>
void launch_vec(const AttnParams& prm, const AttnPlan& pl, dim3 grid, hipStream_t s) {
    switch (pl.hc) {
        case 1: hipLaunchKernelGGL((attn_vec_kernel<KV, QB, 1>), grid, dim3(kThreads), 0, s, prm); break;
        case 2: hipLaunchKernelGGL((attn_vec_kernel<KV, QB, 2>), grid, dim3(kThreads), 0, s, prm); break;
        case 4: hipLaunchKernelGGL((attn_vec_kernel<KV, QB, 4>), grid, dim3(kThreads), 0, s, prm); break;
        default: hipLaunchKernelGGL((attn_vec_kernel<KV, QB, 8>), grid, dim3(kThreads), 0, s, prm); break;
    }
}

}  // namespace

AttnPlan plan_sparse_attn(int B, int H, int N, int D_, int sel_heads, int k, int q_dtype, int kv_dtype) {
    (void)N;
    (void)D_;
    AttnPlan p;
    p.mfma = q_dtype == kv_dtype && (q_dtype == kBF16 || q_dtype == kF16);
    p.hpr = H / sel_heads;
    if (p.mfma)
        p.hc = 16;
    else
        p.hc = p.hpr >= 8 ? 8 : (p.hpr >= 4 ? (p.hpr == 4 ? 4 : 8) : (p.hpr == 1 ? 1 : (p.hpr == 2 ? 2 : 4)));
    p.hchunks = (p.hpr + p.hc - 1) / p.hc;
    const long long rows = (long long)B * sel_heads * p.hchunks;
    long long splits = 1;
    if (rows < kNoSplitRows) {
        const long long rows1 = rows > 0 ? rows : 1;
        const long long target = p.mfma ? kTargetWorkgroupsMfma : kTargetWorkgroupsVec;
        splits = (target + rows1 - 1) / rows1;
        if (splits > k) splits = k;
        if (splits < 1) splits = 1;
    }
    p.spb = int((k + splits - 1) / splits);
    p.splits = (k + p.spb - 1) / p.spb;
    const size_t part_bytes = p.splits > 1 ? size_t(rows) * p.splits * p.hc * PSTRIDE * sizeof(float) : 0;
    p.part_off = 0;
    p.bytes = align256(part_bytes);
    if (p.bytes < 256) p.bytes = 256;
    return p;
}

hipError_t launch_sparse_attn(const AttnArgs& a, const AttnPlan& pl, hipStream_t s) {
    AttnParams prm{(const uint8_t*)a.query, (const uint8_t*)a.k_cache, (const uint8_t*)a.v_cache, a.k_scale,
                   a.v_scale, a.num_kv_blocks, a.block_tables, a.mkbpr, a.seq_lens, a.selected, a.n_selected,
                   a.H, a.N, a.BS, a.sel_heads, a.k, pl.hpr, pl.hchunks, pl.splits, pl.spb, a.scale * kLog2e,
                   (uint8_t*)a.out, (float*)((uint8_t*)a.workspace + pl.part_off)};
    dim3 grid(unsigned(pl.splits * pl.hchunks), unsigned(a.sel_heads), unsigned(a.B));
    if (pl.mfma) {
        // K/V bytes the call streams (upper bound: k full blocks per selection row)
        const size_t kv = size_t(a.B) * a.sel_heads * size_t(a.k) * a.BS * 2 * D * 2;
        auto go = [&](auto ntc) {
            constexpr bool NT = decltype(ntc)::value;
            if (a.q_dtype == kF16) hipLaunchKernelGGL((attn_mfma_kernel<kF16, NT>), grid, dim3(kThreads), 0, s, prm);
            else hipLaunchKernelGGL((attn_mfma_kernel<kBF16, NT>), grid, dim3(kThreads), 0, s, prm);
        };
        if (kv > kNtStreamBytes) go(std::true_type{});
        else go(std::false_type{});
    } else {
        auto by_q = [&](auto kv) {
            constexpr int KV = decltype(kv)::value;
            if (a.q_dtype == kBF16) launch_vec<KV, kBF16>(prm, pl, grid, s);
            else if (a.q_dtype == kF16) launch_vec<KV, kF16>(prm, pl, grid, s);
            else launch_vec<KV, kF32>(prm, pl, grid, s);
        };
        if (a.kv_dtype == kF32) by_q(std::integral_constant<int, kF32>{});
        else if (a.kv_dtype == kBF16) by_q(std::integral_constant<int, kBF16>{});
        else if (a.kv_dtype == kF16) by_q(std::integral_constant<int, kF16>{});
        else by_q(std::integral_constant<int, kI8>{});
    }
    if (pl.splits > 1) return attn::launch_combine(prm, a.B, pl.hc, a.q_dtype, s);
    return hipGetLastError();
}

hipError_t attn::launch_combine(const AttnParams& p, int B, int hc_cap, int out_dt, hipStream_t s) {
    const unsigned per_req = unsigned((size_t(p.H) * D * kCombineLanes + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(attn_combine_kernel, dim3(per_req, unsigned(B)), dim3(kThreads), 0, s, p, hc_cap, out_dt);
    return hipGetLastError();
}

}  // namespace qs

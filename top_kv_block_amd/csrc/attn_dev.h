// attn_dev.h -- device code of the selected-block attention, shared by the attention
// kernels (attn.hip) and the fused select + attention kernel (fused.hip). The design
// notes are at the top of attn.hip.
#pragma once

#include <math.h>

#include <type_traits>

#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace attn {

constexpr float kLog2e = 1.4426950408889634f;
// A call that streams more than this many bytes (K/V plus block metadata) reads them with
// non-temporal loads. Measured on MI355X: a 1.21 GB serving step 218 -> 197 us with them;
// a 286 MB long-context step 52.5 -> 55.3 us (part of it stays in the 256 MB last-level
// cache from one step to the next, and non-temporal loads give that up).
constexpr size_t kNtStreamBytes = size_t(512) << 20;
constexpr int D = 128;
constexpr int PSTRIDE = D + 2;       // partial record: acc[D], max, sum

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void merge_state(float& m, float& l, float* a, int n, float m2, float l2,
                                            const float* a2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    const float c1 = exp2f(m - M), c2 = exp2f(m2 - M);
    l = l * c1 + l2 * c2;
    for (int e = 0; e < n; ++e) a[e] = a[e] * c1 + a2[e] * c2;
    m = M;
}

struct AttnParams {
    const uint8_t* query;
    const uint8_t* kc;
    const uint8_t* vc;
    const float* ksc;
    const float* vsc;
    int num_kv_blocks;
    const int32_t* bt;
    int mkbpr;
    const int32_t* sl;
    const int32_t* sel;
    const int32_t* nsel;
    int H, N, BS, sel_heads, k;
    int hpr, hchunks, splits, spb;
    float scale_log2;
    uint8_t* out;
    float* part;
};

// stores output element o in the query dtype (F32, BF16 or F16; 16-bit: round to nearest even)
__device__ __forceinline__ void store_out(uint8_t* out, size_t o, float v, int out_dt) {
    if (out_dt == kBF16) ((uint16_t*)out)[o] = f32_to_half<kBF16>(v);
    else if (out_dt == kF16) ((uint16_t*)out)[o] = f32_to_half<kF16>(v);
    else ((float*)out)[o] = v;
}

// result of one workgroup for head g, channel d: either the output or a partial record
__device__ __forceinline__ void emit(const AttnParams& p, int b, int row, int hcix, int split, int hc_cap, int h0,
                                     int g, int d, float M, float Ls, float A, int out_dt) {
    if (p.splits == 1) {
        const float v = (Ls > 0.f) ? A / Ls : 0.f;
        store_out(p.out, (size_t(b) * p.H + h0 + g) * D + d, v, out_dt);
    } else {
        float* rec = p.part + (((size_t(row) * p.hchunks + hcix) * p.splits + split) * hc_cap + g) * PSTRIDE;
        rec[d] = A;
        if (d == 0) { rec[D] = M; rec[D + 1] = Ls; }
    }
}

// Slot table of one wave (used when a split has at most 64 slots): lane t resolves slot
// slot0 + t of the selection row into (physical block, valid tokens), or (-1, 0) for a
// slot past the count, a negative or out-of-range entry, or an out-of-range table entry.
// The entry is read before the selection count is known (a selection row always holds k
// entries), so the count, the sequence length and the entries are in flight together and
// only the block-table lookup waits on them; the slot loops then read the table back with
// v_readlane and issue nothing but K/V loads.
__device__ __forceinline__ void slot_table(const AttnParams& p, int b, const int32_t* srow, int slot0, int nsl,
                                           int nb, int L, int lane, int& tab_phys, int& tab_nt) {
    const int blk_raw = (lane < p.spb && slot0 + lane < p.k) ? srow[slot0 + lane] : -1;
    const int blk = lane < nsl ? blk_raw : -1;
    tab_phys = -1;
    tab_nt = 0;
    if (blk >= 0 && blk < nb && blk < p.mkbpr) {
        const int ph = p.bt[size_t(b) * p.mkbpr + blk];
        if (ph >= 0 && ph < p.num_kv_blocks) {
            tab_phys = ph;
            tab_nt = min(p.BS, L - blk * p.BS);
        }
    }
}

// ------------------------------------------------------------------------------------
// matrix-core kernel (bf16 or f16 query and KV)
// ------------------------------------------------------------------------------------
constexpr int kVtPitch = 80;             // bytes per V^T row in LDS: 32 tokens (64 B) + pad
constexpr int kVtBytes = D * kVtPitch;   // one wave's V^T tile

// the MFMA operand type of a 16-bit format, and v_mfma_f32_16x16x32 on it
template <int DT>
using op8 = typename std::conditional<DT == kBF16, bf16x8, f16x8>::type;
template <int DT>
using op1 = typename std::conditional<DT == kBF16, __bf16, _Float16>::type;
template <int DT>
__device__ __forceinline__ op8<DT> as_op8(u32x4 v) {
    u32v4 t = {v.x, v.y, v.z, v.w};
    return __builtin_bit_cast(op8<DT>, t);
}
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(op8<DT> a, op8<DT> b, f32x4 c) {
    if constexpr (DT == kBF16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 128 VGPRs: four workgroups (16 waves) per CU, which the 1024-row serving batch fills
// in one round; LDS is 40 KiB per workgroup, 160 KiB per CU.
// Matrix-core attention of one workgroup: selection row s of request b (entries srow,
// count ns_raw, in global memory or LDS), head chunk hcix, slot range `split`. lds: the
// kMfmaLdsBytes work area. With sync_after_table the workgroup synchronises once every
// wave has read its slot table, so the selection may live inside the work area. NT: K/V
// rows are read with non-temporal loads (see kNtStreamBytes).
template <int DT, bool NT = false>
__device__ __forceinline__ void mfma_body(const AttnParams& p, int split, int hcix, int s, int b,
                                          const int32_t* srow, int ns_raw, uint8_t* lds, bool sync_after_table) {
    const int h0 = s * p.hpr + hcix * 16;
    const int nh = min(16, p.hpr - hcix * 16);
    const int G = p.H / p.N;
    const int kh = (s * p.hpr) / G;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int c16 = lane & 15, j = lane >> 4;

    const int L = max(p.sl[b], 0);
    const int nb = (L + p.BS - 1) / p.BS;
    const int row = b * p.sel_heads + s;
    const int ns = min(max(ns_raw, 0), p.k);
    const int slot0 = split * p.spb, slot1 = min(ns, slot0 + p.spb);
    const int cpb = (p.BS + 31) / 32;                 // 32-token chunks per block
    const int nq = max(0, slot1 - slot0) * cpb;
    const size_t tstride = size_t(p.N) * D;           // elements between tokens of one KV head
    uint8_t* vt = lds + w * kVtBytes;

    // slot table (splits of up to 64 slots; longer ranges look up in the loop)
    const int nsl = max(0, slot1 - slot0);
    const bool use_tab = p.spb <= kWave;
    int tab_phys = -1, tab_nt = 0;
    if (use_tab) slot_table(p, b, srow, slot0, nsl, nb, L, lane, tab_phys, tab_nt);

    // B operand of S^T = K Q^T: lane holds Q[head c16][32*ks + 8*j .. +7]
    op8<DT> qb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        u32x4 v{0u, 0u, 0u, 0u};
        if (c16 < nh) v = ld16(p.query + ((size_t(b) * p.H + h0 + c16) * D + 32 * ks + 8 * j) * 2);
        qb[ks] = as_op8<DT>(v);
    }

    if (sync_after_table) __syncthreads();

    float m = -INFINITY, lsum = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int q = w; q < nq; q += kWaves) {
        const int slot = slot0 + q / cpb, cib = q % cpb;
        int phys, nt;
        if (use_tab) {
            phys = __builtin_amdgcn_readlane(tab_phys, slot - slot0);
            nt = __builtin_amdgcn_readlane(tab_nt, slot - slot0);
            if (phys < 0) continue;
        } else {
            const int blk = srow[slot];
            if (blk < 0 || blk >= nb || blk >= p.mkbpr) continue;
            phys = p.bt[size_t(b) * p.mkbpr + blk];
            if (phys < 0 || phys >= p.num_kv_blocks) continue;
            nt = min(p.BS, L - blk * p.BS);
        }
        const int tb = cib * 32;
        if (tb >= nt) continue;
        const uint16_t* kb = (const uint16_t*)p.kc + (size_t(phys) * p.BS * p.N + kh) * D;
        const uint16_t* vb = (const uint16_t*)p.vc + (size_t(phys) * p.BS * p.N + kh) * D;

        // K: loaded like V (16 lanes per 256-B token row, whole cache lines per instruction)
        // and staged through this wave's LDS tile, from which each lane reads its MFMA A
        // operand. Tile tau row r = c16 is token tb + 8*(r/4) + 4*tau + r%4 (so that lane
        // group j ends up holding tokens tb + 8j .. 8j+7 in its accumulators).
        u32x4 kn[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int t = tb + 8 * j + u;
            const int tl = t < nt ? t : 0;
            kn[u] = NT ? ld16_nt(kb + size_t(tl) * tstride + 8 * c16) : ld16(kb + size_t(tl) * tstride + 8 * c16);
        }
        // V: lane (c16, j) loads tokens tb + 8j + u, channels 8*c16 .. +7
        u32x4 vr[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int t = tb + 8 * j + u;
            const int tl = t < nt ? t : 0;
            vr[u] = NT ? ld16_nt(vb + size_t(tl) * tstride + 8 * c16) : ld16(vb + size_t(tl) * tstride + 8 * c16);
        }

        constexpr int KP = 272;  // K tile pitch: a 256-B token row + 16 B
        static_assert(32 * KP <= kVtBytes, "the K tile fits the wave's LDS tile");
#pragma unroll
        for (int u = 0; u < 8; ++u) st16(vt + (8 * j + u) * KP + 16 * c16, kn[u]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f32x4 sacc[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            sacc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int tr = 8 * (c16 >> 2) + 4 * tau + (c16 & 3);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                sacc[tau] = mfma16x16x32<DT>(as_op8<DT>(ld16(vt + tr * KP + 64 * ks + 16 * j)), qb[ks], sacc[tau]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float sv[8];
        float cmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tau = e >> 2, i = e & 3;
            const float x = sacc[tau][i] * p.scale_log2;
            sv[e] = (tb + 8 * j + e < nt) ? x : -INFINITY;
            cmax = fmaxf(cmax, sv[e]);
        }
        cmax = fmaxf(cmax, __shfl_xor(cmax, 16, kWave));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32, kWave));
        const float mn = fmaxf(m, cmax);
        const float cf = (mn == -INFINITY) ? 1.f : exp2f(m - mn);
        op8<DT> pv;
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pe = (sv[e] == -INFINITY) ? 0.f : exp2f(sv[e] - mn);
            const op1<DT> pb = (op1<DT>)pe;  // P in the operand format; the sum takes the rounded value
            pv[e] = pb;
            psum += (float)pb;
        }
        lsum = lsum * cf + psum;
        m = mn;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] *= cf;

        // V^T tile: row d = 8*c16 + e holds tokens 8j .. 8j+7 at byte 16*j
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int wsel = e >> 1;
            uint32_t x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const u32x4 r = vr[u];
                x[u] = wsel == 0 ? r.x : wsel == 1 ? r.y : wsel == 2 ? r.z : r.w;
            }
            u32x4 t;
            if (e & 1) {
                t.x = (x[0] >> 16) | (x[1] & 0xffff0000u);
                t.y = (x[2] >> 16) | (x[3] & 0xffff0000u);
                t.z = (x[4] >> 16) | (x[5] & 0xffff0000u);
                t.w = (x[6] >> 16) | (x[7] & 0xffff0000u);
            } else {
                t.x = (x[0] & 0xffffu) | (x[1] << 16);
                t.y = (x[2] & 0xffffu) | (x[3] << 16);
                t.z = (x[4] & 0xffffu) | (x[5] << 16);
                t.w = (x[6] & 0xffffu) | (x[7] << 16);
            }
            st16(vt + (8 * c16 + e) * kVtPitch + 16 * j, t);
        }
        // this wave's V^T stores must land before its lanes read other lanes' rows
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // O^T (channels x heads) += V^T P^T
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const u32x4 a = ld16(vt + (16 * dt + c16) * kVtPitch + 16 * j);
            o[dt] = mfma16x16x32<DT>(as_op8<DT>(a), pv, o[dt]);
        }
        // the next chunk overwrites the tile only after every lane has read it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // per-head sum over the four lane groups
    lsum += __shfl_xor(lsum, 16, kWave);
    lsum += __shfl_xor(lsum, 32, kWave);

    // merge the four waves through LDS: red_o[w][head][channel], red_m/red_l[w][head]
    __syncthreads();
    float* red_o = (float*)lds;                        // 4 * 16 * 128 floats = 32 KiB
    float* red_m = red_o + kWaves * 16 * D;
    float* red_l = red_m + kWaves * 16;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_o[(w * 16 + c16) * D + 16 * dt + 4 * j + i] = o[dt][i];
    if (j == 0) { red_m[w * 16 + c16] = m; red_l[w * 16 + c16] = lsum; }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * D; idx += kThreads) {
        const int g = idx / D, d = idx % D;
        if (g >= nh) continue;
        float M = -INFINITY, Ls = 0.f, A = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww)
            merge_state(M, Ls, &A, 1, red_m[ww * 16 + g], red_l[ww * 16 + g], &red_o[(ww * 16 + g) * D + d]);
        emit(p, b, row, hcix, split, 16, h0, g, d, M, Ls, A, DT);
    }
}

// ------------------------------------------------------------------------------------
// vector-ALU kernel (fp32 / bf16 with fp32 query / int8 KV)
// ------------------------------------------------------------------------------------
// Vector-ALU attention of one workgroup (arguments as mfma_body). red: kWaves * HC *
// (D + 2) floats of LDS for the cross-wave merge.
template <int KV, int QDT, int HC>
__device__ __forceinline__ void vec_body(const AttnParams& p, int split, int hcix, int s, int b,
                                         const int32_t* srow, int ns_raw, float* red) {
    constexpr int ke = elem_bytes(KV);
    constexpr int qe = elem_bytes(QDT);
    constexpr int LPR = D * ke / 16;    // lanes per K/V row
    constexpr int EPL = 16 / ke;        // channels per lane
    constexpr int NG = kThreads / LPR;  // independent lane groups per workgroup
    // tokens in flight per lane group: a step covers 32 tokens with fp32 rows (8 groups of
    // 32 lanes), so a 32-token block is one round trip of loads; 16-bit and int8 rows have
    // 16 and 32 groups, and two tokens each already cover a block
    constexpr int U = KV == kF32 ? 4 : 2;

    float* red_m = red;                       // [kWaves][HC]
    float* red_l = red + kWaves * HC;         // [kWaves][HC]
    float* red_a = red + 2 * kWaves * HC;     // [kWaves][HC][D]

    const int h0 = s * p.hpr + hcix * HC;
    const int nh = min(HC, p.hpr - hcix * HC);
    const int G = p.H / p.N;
    const int kh = (s * p.hpr) / G;
    const int tid = threadIdx.x, lr = tid % LPR, grp = tid / LPR;

    const int L = max(p.sl[b], 0);
    const int nb = (L + p.BS - 1) / p.BS;
    const int row = b * p.sel_heads + s;
    const int ns = min(max(ns_raw, 0), p.k);
    const int slot0 = split * p.spb, slot1 = min(ns, slot0 + p.spb);
    const size_t tok_bytes = size_t(p.N) * D * ke;

    // slot table (splits of up to 64 slots; longer ranges look up in the loop)
    const int nsl = max(0, slot1 - slot0);
    const bool use_tab = p.spb <= kWave;
    int tab_phys = -1, tab_nt = 0;
    if (use_tab) slot_table(p, b, srow, slot0, nsl, nb, L, tid & (kWave - 1), tab_phys, tab_nt);

    // query: fp32 (pre-scaled by softmax_scale * log2 e) or int8 codes
    float qf[HC][EPL];
    int32_t q8[HC][EPL / 4 > 0 ? EPL / 4 : 1];
    float qscale[HC];
#pragma unroll
    for (int g = 0; g < HC; ++g) {
        const int hh = h0 + (g < nh ? g : 0);
        const uint8_t* qp = p.query + (size_t(b) * p.H + hh) * D * qe;
        float x[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int d = lr * EPL + e;
            x[e] = load_elem<QDT>(qp, d);
        }
        if constexpr (KV == kI8) {
            float amax = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
            amax = group_max<LPR>(amax);
            const float sq = amax / 127.0f;
            qscale[g] = sq * p.scale_log2;
#pragma unroll
            for (int wd = 0; wd < EPL / 4; ++wd) {
                uint32_t packed = 0;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    float r = 0.f;
                    if (sq != 0.f) r = fminf(fmaxf(rintf(x[4 * wd + jj] / sq), -127.f), 127.f);
                    packed |= (uint32_t(int32_t(r)) & 0xffu) << (8 * jj);
                }
                q8[g][wd] = int32_t(packed);
            }
        } else {
            qscale[g] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) qf[g][e] = x[e] * p.scale_log2;
        }
    }

    float m[HC], l[HC], acc[HC][EPL];
#pragma unroll
    for (int g = 0; g < HC; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }

    for (int slot = slot0; slot < slot1; ++slot) {
        int phys, nt;
        if (use_tab) {
            phys = __builtin_amdgcn_readlane(tab_phys, slot - slot0);
            nt = __builtin_amdgcn_readlane(tab_nt, slot - slot0);
            if (phys < 0) continue;
        } else {
            const int blk = srow[slot];
            if (blk < 0 || blk >= nb || blk >= p.mkbpr) continue;
            phys = p.bt[size_t(b) * p.mkbpr + blk];
            if (phys < 0 || phys >= p.num_kv_blocks) continue;
            nt = min(p.BS, L - blk * p.BS);
        }
        const size_t tok0 = size_t(phys) * p.BS;
        const uint8_t* kb = p.kc + (tok0 * p.N + kh) * D * ke + lr * 16;
        const uint8_t* vb = p.vc + (tok0 * p.N + kh) * D * ke + lr * 16;
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
                if constexpr (KV == kI8) {
                    ks[u] = p.ksc[(tok0 + tt) * p.N + kh];
                    vs[u] = p.vsc[(tok0 + tt) * p.N + kh];
                } else {
                    ks[u] = vs[u] = 1.f;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t kw[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
                const uint32_t vw[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
                float vf[EPL];
                if constexpr (KV == kF32) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) vf[jj] = __uint_as_float(vw[jj]);
                } else if constexpr (KV == kBF16 || KV == kF16) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) { vf[2 * jj] = lo16<KV>(vw[jj]); vf[2 * jj + 1] = hi16<KV>(vw[jj]); }
                } else {
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) vf[jj] = float(int8_t(vw[jj / 4] >> (8 * (jj % 4)))) * vs[u];
                }
#pragma unroll
                for (int g = 0; g < HC; ++g) {
                    float sc;
                    if constexpr (KV == kI8) {
                        int dot = 0;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) dot = __builtin_amdgcn_sdot4(q8[g][jj], int32_t(kw[jj]), dot, false);
                        dot = group_sum_i<LPR>(dot);
                        sc = float(dot) * (qscale[g] * ks[u]);
                    } else {
                        float pp = 0.f;
                        if constexpr (KV == kF32) {
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj) pp += qf[g][jj] * __uint_as_float(kw[jj]);
                        } else {
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj)
                                pp += qf[g][2 * jj] * lo16<KV>(kw[jj]) + qf[g][2 * jj + 1] * hi16<KV>(kw[jj]);
                        }
                        sc = group_sum<LPR>(pp);
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

    // merge the lane groups of each wave (same lr = same channels)
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
            if (lr == 0) { red_m[w * HC + g] = m[g]; red_l[w * HC + g] = l[g]; }
#pragma unroll
            for (int e = 0; e < EPL; ++e) red_a[(w * HC + g) * D + lr * EPL + e] = acc[g][e];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < HC * D; idx += kThreads) {
        const int g = idx / D, d = idx % D;
        if (g >= nh) continue;
        float M = -INFINITY, Ls = 0.f, A = 0.f;
        for (int ww = 0; ww < kWaves; ++ww)
            merge_state(M, Ls, &A, 1, red_m[ww * HC + g], red_l[ww * HC + g], &red_a[(ww * HC + g) * D + d]);
        emit(p, b, row, hcix, split, HC, h0, g, d, M, Ls, A, QDT);
    }
}

constexpr int kMfmaLdsBytes = kWaves * kVtBytes;  // 40 KiB work area of mfma_body
template <int HC>
constexpr int vec_red_floats() { return kWaves * HC * (D + 2); }

// merges split partials into the output (attn.hip)
hipError_t launch_combine(const AttnParams& p, int B, int hc_cap, int out_dt, hipStream_t s);

}  // namespace attn
}  // namespace qs

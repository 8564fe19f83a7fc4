// select_dev.h -- device code of the Quest block selection (scoring, forcing, exact
// top-k), shared by the selection kernels (select.hip) and the fused select + attention
// kernel (fused.hip). The design notes are at the top of select.hip.
#pragma once

#include <math.h>

#include <type_traits>

#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace sel {

constexpr int kLdsScoreCap = 8192;     // row mode keeps up to this many scores in LDS
constexpr int kMtStageCap = 256;       // metadata-table rows up to this long are staged in LDS
static_assert(kMtStageCap <= kThreads, "one staging load per thread");

struct Forced {
    int w_lo;   // blocks >= w_lo are forced (window); nb when none
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
        const long long num = (long long)L - u;
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

struct RowInfo {
    int L, nb;
    Forced F;
};

__device__ __forceinline__ RowInfo row_info(const int32_t* sl, const int32_t* tsmu, uint32_t flags, int k, int b,
                                            int BS, int cap) {
    RowInfo r;
    r.L = max(sl[b], 0);
    r.nb = min((r.L + BS - 1) / BS, cap);
    r.F = forced_set(r.L, r.nb, BS, k, tsmu, b, flags);
    return r;
}

// Scores blocks [i0, i_end) of row (b, n) into dst[i] (LDS or global). Forced blocks are
// skipped (NaN written when nan_forced); an out-of-range metadata entry scores -inf.
// i_lim (i_end <= i_lim <= the row capacity mmbpr * BS) bounds the range's table entries
// without the row length, so the table lookups are issued together with the loads of the
// row length instead of after them; i_end may be <= i0 (nothing scored). qstage: kThreads
// 16-byte LDS slots used to stage the group's query rows; mt_stage: kMtStageCap ints of LDS
// for the metadata-table entries of [i0, i_lim) (MT_LDS: the caller guarantees they fit).
// NT: the metadata rows are read with non-temporal loads (attn::kNtStreamBytes).
// Contains a barrier: every thread of the workgroup must call it.
template <int DT, bool MT_LDS, bool NT = false>
__device__ __forceinline__ void score_range(const uint8_t* __restrict__ query, const uint8_t* __restrict__ maxb,
                                            const uint8_t* __restrict__ minb, int num_meta,
                                            const int32_t* __restrict__ mt, int mmbpr, int H, int N, int BS, int b,
                                            int n, const Forced& F, int i0, int i_end, int i_lim, float* dst,
                                            bool nan_forced, u32x4* qstage, int32_t* mt_stage) {
    constexpr int esize = elem_bytes(DT);
    constexpr int D = 128;
    constexpr int LPR = D * esize / 16;  // lanes per metadata row
    constexpr int EPL = 16 / esize;      // channels per lane
    constexpr int RPP = kThreads / LPR;  // rows per pass
    constexpr int U = 4;                 // passes per batch
    const int tid = threadIdx.x;
    const int lr = tid % LPR, slot = tid / LPR;
    const int G = H / N;
    const size_t row_bytes = size_t(N) * D * esize;

    // One batch = U passes of RPP rows; the next batch's loads are issued before the
    // current batch is consumed. With MT_LDS the range's metadata-table entries are
    // staged in LDS so that the lookups of later batches are LDS reads (a global lookup
    // would have to wait for every load in flight before it); batch 0 looks up in global
    // memory while the staging loads are in flight.
    const int mbase = i0 / BS;
    auto issue = [&](int base, u32x4 (&vmx)[U], u32x4 (&vmn)[U], bool (&ok)[U], auto from_lds) {
        int mrow[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * RPP + slot;
            ok[u] = i < i_end && !F.has(i);
            if constexpr (decltype(from_lds)::value)
                mrow[u] = ok[u] ? mt_stage[i / BS - mbase] : 0;
            else  // not gated on ok: the entry of any i < i_lim is in the table
                mrow[u] = i < i_lim ? mt[size_t(b) * mmbpr + i / BS] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * RPP + slot;
            ok[u] = ok[u] && mrow[u] >= 0 && mrow[u] < num_meta;
            // rows that are not scored read the first row (always valid) and are masked
            const size_t off = ok[u] ? (size_t(mrow[u]) * BS + (i % BS)) * row_bytes + size_t(n) * D * esize + lr * 16
                                     : size_t(lr) * 16;
            vmx[u] = NT ? ld16_nt(maxb + off) : ld16(maxb + off);
            vmn[u] = NT ? ld16_nt(minb + off) : ld16(minb + off);
        }
    };

    // the group's query rows: one 16-byte piece per thread, loaded ahead of batch 0
    const int npieces = G * LPR;
    const bool staged = npieces <= kThreads;
    u32x4 qpiece{0u, 0u, 0u, 0u};
    if (staged && tid < npieces)
        qpiece = ld16(query + ((size_t(b) * H + size_t(n) * G + tid / LPR) * D + (tid % LPR) * EPL) * esize);
    const int n_ent = i0 < i_lim ? (i_lim - 1) / BS - mbase + 1 : 0;  // table entries of [i0, i_lim)
    int32_t mt_piece = 0;
    if (MT_LDS && tid < n_ent) mt_piece = mt[size_t(b) * mmbpr + mbase + tid];
    u32x4 vmx[U], vmn[U];
    bool ok[U];
    // batch 0 is issued even for an empty range (its rows then read the first metadata row
    // and are masked), so that nothing before the loads waits for the row length
    issue(i0, vmx, vmn, ok, std::false_type{});
    if (MT_LDS && tid < n_ent) mt_stage[tid] = mt_piece;

    // grouped query for this lane's channels: mean over the group's G heads
    float gq[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) gq[e] = 0.f;
    auto add_piece = [&](const u32x4& v) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        if constexpr (DT != kF32) {
#pragma unroll
            for (int j = 0; j < 4; ++j) { gq[2 * j] += lo16<DT>(w[j]); gq[2 * j + 1] += hi16<DT>(w[j]); }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) gq[j] += __uint_as_float(w[j]);
        }
    };
    if (staged && tid < npieces) qstage[tid] = qpiece;
    __syncthreads();  // query pieces and the table row are in LDS
    if (staged) {
        for (int g = 0; g < G; ++g) add_piece(qstage[g * LPR + lr]);
    } else {
        for (int g = 0; g < G; ++g)
            add_piece(ld16(query + ((size_t(b) * H + size_t(n) * G + g) * D + lr * EPL) * esize));
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) gq[e] = gq[e] / float(G);

    auto consume = [&](int base, const u32x4 (&vmx)[U], const u32x4 (&vmn)[U], const bool (&ok)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t a[4] = {vmx[u].x, vmx[u].y, vmx[u].z, vmx[u].w};
            const uint32_t z[4] = {vmn[u].x, vmn[u].y, vmn[u].z, vmn[u].w};
            float part = 0.f;
            if constexpr (DT != kF32) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    part += fmaxf(gq[2 * j] * lo16<DT>(a[j]), gq[2 * j] * lo16<DT>(z[j]));
                    part += fmaxf(gq[2 * j + 1] * hi16<DT>(a[j]), gq[2 * j + 1] * hi16<DT>(z[j]));
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
                    dst[i] = s;
                else if (!F.has(i))
                    dst[i] = -INFINITY;
                else if (nan_forced)
                    dst[i] = __builtin_nanf("");
            }
        }
    };

    // ping-pong over two register sets, so a batch's loads are in flight while the other
    // batch is consumed, with no register copies between them
    constexpr int STEP = RPP * U;
    u32x4 wmx[U], wmn[U];
    bool wok[U];
    for (int base = i0; base < i_end; base += 2 * STEP) {
        const bool more1 = base + STEP < i_end;
        if (more1) issue(base + STEP, wmx, wmn, wok, std::integral_constant<bool, MT_LDS>{});
        consume(base, vmx, vmn, ok);
        if (base + 2 * STEP < i_end) issue(base + 2 * STEP, vmx, vmn, ok, std::integral_constant<bool, MT_LDS>{});
        if (more1) consume(base + STEP, wmx, wmn, wok);
    }
}

// Exact top-k of a row from its scores (LDS or global); writes selected / n_selected.
// A threshold select finds the k-th best key T among the fill candidates and how many
// candidates equal to T are taken (the lowest-index ones). Each thread then takes a
// contiguous run of blocks and counts, in its run, the sure picks (forced, or above T)
// and the candidates equal to T; one block-wide scan of the two counts (packed in one
// word while the row is shorter than 65536 blocks) gives every thread its output
// position, and the picks are written in ascending block order.
__device__ __forceinline__ void topk_emit(const float* scores, int nb, const Forced& F, int k, int32_t* out,
                                          int32_t* n_out, uint32_t* hist, int* sh, int* wsum) {
    const int tid = threadIdx.x;
    const int R = max(0, min(k, nb) - F.count);  // fill picks
    const int nc = nb - F.count;                   // fill candidates
    const bool take_all = R >= nc;
    const bool thresh = R > 0 && !take_all;
    uint32_t T = 0;
    int need_eq = 0;
    if (thresh) {
        auto kf = [&](int i, uint32_t& key) -> bool {
            if (F.has(i)) return false;
            key = f2key(scores[i]);
            return true;
        };
        T = block_topk_threshold(nb, R, kf, hist, sh, need_eq);
    }
    // 0: not picked, 1: picked for sure, 2: equal to T (picked while the quota lasts)
    auto cls = [&](int i) -> int {
        if (F.has(i)) return 1;
        if (R == 0) return 0;
        if (take_all) return 1;
        const uint32_t key = f2key(scores[i]);
        return key > T ? 1 : (key == T ? 2 : 0);
    };
    const int E = (nb + kThreads - 1) / kThreads;  // blocks per thread, contiguous
    const int i0 = min(nb, tid * E), i1 = min(nb, i0 + E);
    int sure = 0, eq = 0;
    for (int i = i0; i < i1; ++i) {
        const int c = cls(i);
        sure += c == 1 ? 1 : 0;
        eq += c == 2 ? 1 : 0;
    }
    int sure_before, eq_before, sure_tot, eq_tot;
    if (nb < 65536) {
        int tot;
        const int ex = block_excl_scan((sure << 16) | eq, wsum, tot);
        sure_before = ex >> 16;
        eq_before = ex & 0xffff;
        sure_tot = tot >> 16;
        eq_tot = tot & 0xffff;
    } else {
        sure_before = block_excl_scan(sure, wsum, sure_tot);
        eq_before = block_excl_scan(eq, wsum, eq_tot);
    }
    const int npick = sure_tot + min(eq_tot, need_eq);
    int pos = sure_before + min(eq_before, need_eq);
    for (int i = i0, eq_seen = eq_before; i < i1; ++i) {
        const int c = cls(i);
        bool pick = c == 1;
        if (c == 2) {
            pick = eq_seen < need_eq;
            ++eq_seen;
        }
        if (pick) {
            if (pos < k) out[pos] = i;
            ++pos;
        }
    }
    for (int j = npick + tid; j < k; j += kThreads) out[j] = -1;
    if (tid == 0) *n_out = min(npick, k);
}

// Lanes of this wave below the calling lane whose bit is set in `mask`.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return int(__builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u)));
}

// The same selection as topk_emit, for rows of at most 64 * KPL blocks whose scores are
// in LDS, with a single workgroup barrier. Every wave computes the whole selection on its
// own and writes it, ascending and -1 padded to k, to its `out` (a wave passing null
// writes nothing); every wave returns the count. Lane l holds the keys of blocks l,
// l + 64, ... in registers (forced blocks and blocks past the row hold 0; keys of scores
// are never 0). Steps: the wave finds the candidates' key range [kmin, kmax]; the
// workgroup histograms the keys into 256 bins of that range (wave w adds rounds
// w, w + 4, ..., so every key once), the barrier; each wave finds the bin holding the
// R-th largest key and the R-th largest key T inside it: a bin of at most kRankBin keys
// is ranked in registers (each of its keys broadcast once and compared with the others);
// a larger one (m <= 256, else the workgroup radix select) is gathered into the wave's
// own list in LDS (wlist, 256 entries per wave) and T found by a binary search over the
// bin's low bits, each step counting the list's keys >= a trial value with ballots;
// finally, 64 blocks a round in ascending
// order, it takes forced blocks and keys above T, and keys equal to T while the quota
// lasts (lower blocks first), ballots giving each pick its output position.
// `hist` (512 uint32 of LDS) must be zeroed, and the scores written, before a barrier
// that precedes the call. Every thread of the workgroup must call it.
constexpr int kRankBin = 16;  // boundary bins up to this many keys are ranked in registers

template <int KPL>
__device__ __forceinline__ int topk_waves(const float* scores, int nb, const Forced& F, int k, int32_t* out,
                                          uint32_t* hist, uint32_t* wlist, int* sh) {
    const int lane = lane_id(), wv = wave_id();
    const int R = max(0, min(k, nb) - F.count);  // fill picks
    const int nc = nb - F.count;                   // fill candidates
    uint32_t key[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const int i = kWave * j + lane;
        key[j] = (i < nb && !F.has(i)) ? f2key(scores[i]) : 0u;
    }
    uint32_t T = 0xffffffffu;  // taken for sure: keys above T
    int need_eq = 0;           // and this many keys equal to T
    if (R > 0 && R < nc) {
        uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
        for (int j = 0; j < KPL; ++j)
            if (key[j]) { kmin = min(kmin, key[j]); kmax = max(kmax, key[j]); }
        kmin = wave_min_u32(kmin);
        kmax = wave_max_u32(kmax);
        int shift = 0;
        if (kmin != kmax) {
            shift = max(0, (32 - __clz(kmax - kmin)) - 8);  // (key - kmin) >> shift is in [0, 255]
#pragma unroll
            for (int j = 0; j < KPL; ++j)
                if (j % kWaves == wv && key[j]) atomicAdd(&hist[(key[j] - kmin) >> shift], 1u);
        }
        __syncthreads();
        if (kmin == kmax) {  // every candidate has the same key
            T = kmin;
            need_eq = R;
        } else {
            // the bin holding the R-th largest key: lane l owns bins 255-4l .. 252-4l
            uint32_t c[4], s4 = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) { c[j] = hist[255 - 4 * lane - j]; s4 += c[j]; }
            const uint32_t incl = wave_incl_scan(s4);
            uint32_t run = incl - s4;
            int bin = -1, above = 0;
            if (run < uint32_t(R) && uint32_t(R) <= incl) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (bin < 0 && run + c[j] >= uint32_t(R)) { bin = 255 - 4 * lane - j; above = int(run); }
                    run += c[j];
                }
            }
            const uint64_t owner = __ballot(bin >= 0);
            const int src = __ffsll((unsigned long long)owner) - 1;
            const uint32_t bs = uint32_t(__builtin_amdgcn_readlane(bin, src));
            const int need = R - __builtin_amdgcn_readlane(above, src);  // 1 <= need <= the bin's count
            const int m = int(hist[bs]);
            if (m <= kRankBin) {
                // few keys in the bin: rank them against each other straight from the
                // registers, one broadcast per key of the bin (no LDS round trip). gt / ge:
                // how many keys of the bin are above / at least this lane's key j.
                bool in[KPL];
                uint32_t gt[KPL], ge[KPL];
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    in[j] = key[j] && ((key[j] - kmin) >> shift) == bs;
                    gt[j] = ge[j] = 0u;
                }
#pragma unroll
                for (int j2 = 0; j2 < KPL; ++j2) {
                    uint64_t mk = __ballot(in[j2]);
                    while (mk) {
                        const int src = __ffsll((unsigned long long)mk) - 1;
                        mk &= mk - 1;
                        const uint32_t v = uint32_t(__builtin_amdgcn_readlane(int(key[j2]), src));
#pragma unroll
                        for (int j = 0; j < KPL; ++j) {
                            gt[j] += v > key[j];
                            ge[j] += v >= key[j];
                        }
                    }
                }
                // the need-th largest key of the bin: the key with gt < need <= ge (every lane
                // holding it agrees on gt)
                int found = 0;
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    const uint64_t hm = __ballot(in[j] && gt[j] < uint32_t(need) && uint32_t(need) <= ge[j]);
                    if (!found && hm) {
                        const int src = __ffsll((unsigned long long)hm) - 1;
                        T = uint32_t(__builtin_amdgcn_readlane(int(key[j]), src));
                        need_eq = need - __builtin_amdgcn_readlane(int(gt[j]), src);
                        found = 1;
                    }
                }
            } else if (m > 256) {
                // crowded boundary bin: the workgroup radix select (m is the same in every
                // wave, so every wave gets here; the barrier lets all finish reading hist)
                __syncthreads();
                auto kf = [&](int i, uint32_t& kk) -> bool {
                    if (F.has(i)) return false;
                    kk = f2key(scores[i]);
                    return true;
                };
                T = block_radix_select(nb, R, kf, hist, sh, need_eq);
            } else {
                // the bin's keys into this wave's list (their order does not matter)
                int base = 0;
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    const bool in = key[j] && ((key[j] - kmin) >> shift) == bs;
                    const uint64_t mk = __ballot(in);
                    if (in) wlist[base + lanes_below(mk)] = key[j];
                    base += __popcll(mk);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                uint32_t lk[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) lk[q] = lane + kWave * q < m ? wlist[lane + kWave * q] : 0u;
                // the largest offset o in the bin with at least `need` of its keys >= lo + o
                const uint32_t lo = kmin + (bs << shift);
                const int nq = (m + kWave - 1) / kWave;
                uint32_t o = 0;
                for (int bit = shift - 1; bit >= 0; --bit) {
                    const uint32_t cand = lo + (o | (1u << bit));
                    int cnt = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (q < nq) cnt += __popcll(__ballot(lk[q] >= cand));
                    if (cnt >= need) o |= 1u << bit;
                }
                T = lo + o;
                int gt = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (q < nq) gt += __popcll(__ballot(lk[q] > T));
                need_eq = need - gt;
            }
        }
    }
    // the picks in ascending block order, 64 blocks a round
    const bool all_fill = R > 0 && R >= nc;
    int base = 0, eq_base = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const int i = kWave * j + lane;
        bool sure = false, eqv = false;
        if (i < nb) {
            if (F.has(i) || all_fill) {
                sure = true;
            } else if (R > 0) {
                sure = key[j] > T;
                eqv = key[j] == T;
            }
        }
        const uint64_t em = __ballot(eqv);
        const bool take = sure || (eqv && eq_base + lanes_below(em) < need_eq);
        const uint64_t tm = __ballot(take);
        const int pos = base + lanes_below(tm);
        if (out && take && pos < k) out[pos] = i;
        base += __popcll(tm);
        eq_base += __popcll(em);
    }
    if (out)
        for (int j = base + lane; j < k; j += kWave) out[j] = -1;
    return min(base, k);
}

// The selection of a row whose scores are in LDS: topk_waves for a capacity of at most
// 256 blocks (KPL from the capacity; wave 0 writes `out`, every wave returns the count),
// else the workgroup top-k topk_emit, which writes `out` and *n_out itself (every thread
// takes part) and makes this return -1: the caller then reads the count from *n_out after
// a barrier. `hist` must be zeroed before a barrier that precedes the call.
// KPL > 0 fixes the variant at compile time (the caller guarantees cap <= 64 * KPL);
// KPL = -1 always takes the workgroup top-k; KPL = 0 picks from the capacity at run time.
template <int KPL = 0>
__device__ __forceinline__ int topk_dispatch(const float* scores, int nb, int cap, const Forced& F, int k,
                                             int32_t* out, int32_t* n_out, uint32_t* hist, uint32_t* wlist,
                                             int* sh, int* wsum) {
    int32_t* w0 = wave_id() == 0 ? out : nullptr;
    if constexpr (KPL > 0) {
        return topk_waves<KPL>(scores, nb, F, k, w0, hist, wlist, sh);
    } else if constexpr (KPL < 0) {
        topk_emit(scores, nb, F, k, out, n_out, hist, sh, wsum);
        return -1;
    } else {
        if (cap <= 128) return topk_waves<2>(scores, nb, F, k, w0, hist, wlist, sh);
        if (cap <= 256) return topk_waves<4>(scores, nb, F, k, w0, hist, wlist, sh);
        topk_emit(scores, nb, F, k, out, n_out, hist, sh, wsum);
        return -1;
    }
}

// keys per lane of topk_waves for a row capacity; -1: the workgroup top-k, taken beyond
// 256 blocks: with 16 keys per lane (1024-block rows) and 16 waves per CU selecting at
// once, the per-wave top-k measured slower than the workgroup one (long-context fused
// step 64 -> 67 us), while rows of up to 256 blocks gain from it
inline int topk_kpl(int cap) { return cap <= 128 ? 2 : cap <= 256 ? 4 : -1; }

struct SelParams {
    const uint8_t* query;
    const uint8_t* maxb;
    const uint8_t* minb;
    int num_meta;
    const int32_t* mt;
    int mmbpr;
    const int32_t* sl;
    const int32_t* tsmu;
    uint32_t flags;
    int k, H, N, BS;
    int32_t* selected;
    int32_t* n_selected;
    float* dbg_scores;
    float* ws_scores;
};

}  // namespace sel
}  // namespace qs

// metadata.hip -- Quest block metadata: per-block, per-channel max/min of K.
//
// Source: "ops-transformer select_attention_operators" (page 3), section
// "quest_prefill_metadata: 元数据构建原理": max/min over each KV block's valid tokens,
// BS block rows per metadata block placed by metadata_block_tables, unused rows of a
// request's last metadata block zero-filled.
//
// Design (CDNA4): one workgroup per (request, sequence block). A KV block [BS, N, D]
// is contiguous in HBM, so the workgroup streams it with 16-byte loads in row order:
// lane c of a token row owns 16 bytes of channels, R = 256 / (row bytes / 16) token
// rows are in flight per pass, and each lane keeps running max/min registers. The page's
// Ascend kernel copies one KV head at a time with strided DMA; here all N heads of a
// block move in one coalesced stream. Max/min run on an order-preserving integer image
// of the floats (IEEE total order, -0 < +0), so the result is bit-exact whatever the
// hardware's float max does with signed zeros. Workgroups past a request's last block
// but inside its last metadata block write the +0.0 tail rows.
#include <type_traits>

#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace {

typedef short s16x2 __attribute__((ext_vector_type(2)));

// order-preserving image of two packed bf16 as two signed int16 (an involution)
__device__ __forceinline__ uint32_t ord_bf16x2(uint32_t w) {
    const uint32_t s = (w >> 15) & 0x00010001u;
    return w ^ (s * 0x7fffu);
}
__device__ __forceinline__ uint32_t ord_f32(uint32_t w) {
    return w ^ (uint32_t(int32_t(w) >> 31) & 0x7fffffffu);
}

template <bool BF16>
struct Ext;

template <>
struct Ext<true> {  // packed bf16 pairs in the int16 image
    static constexpr uint32_t lo_init = 0x7fff7fffu;  // min identity
    static constexpr uint32_t hi_init = 0x80008000u;  // max identity
    static __device__ __forceinline__ uint32_t ord(uint32_t w) { return ord_bf16x2(w); }
    static __device__ __forceinline__ uint32_t mx(uint32_t a, uint32_t b) {
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, a),
                                                                      __builtin_bit_cast(s16x2, b)));
    }
    static __device__ __forceinline__ uint32_t mn(uint32_t a, uint32_t b) {
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(s16x2, a),
                                                                      __builtin_bit_cast(s16x2, b)));
    }
};

template <>
struct Ext<false> {  // fp32 in the int32 image
    static constexpr uint32_t lo_init = 0x7fffffffu;
    static constexpr uint32_t hi_init = 0x80000000u;
    static __device__ __forceinline__ uint32_t ord(uint32_t w) { return ord_f32(w); }
    static __device__ __forceinline__ uint32_t mx(uint32_t a, uint32_t b) {
        return uint32_t(max(int32_t(a), int32_t(b)));
    }
    static __device__ __forceinline__ uint32_t mn(uint32_t a, uint32_t b) {
        return uint32_t(min(int32_t(a), int32_t(b)));
    }
};

template <bool BF16>
__device__ __forceinline__ void fold(u32x4& hi, u32x4& lo, u32x4 v) {
    using E = Ext<BF16>;
    const uint32_t a = E::ord(v.x), b = E::ord(v.y), c = E::ord(v.z), d = E::ord(v.w);
    hi.x = E::mx(hi.x, a); hi.y = E::mx(hi.y, b); hi.z = E::mx(hi.z, c); hi.w = E::mx(hi.w, d);
    lo.x = E::mn(lo.x, a); lo.y = E::mn(lo.y, b); lo.z = E::mn(lo.z, c); lo.w = E::mn(lo.w, d);
}

template <bool BF16>
__device__ __forceinline__ u32x4 unord(u32x4 v) {
    using E = Ext<BF16>;
    return u32x4{E::ord(v.x), E::ord(v.y), E::ord(v.z), E::ord(v.w)};
}

// NT: the K rows are read with non-temporal loads (a build over more bytes than the
// last-level cache holds streams them once)
template <bool BF16, bool NT>
__global__ __launch_bounds__(kThreads) void meta_kernel(
    const uint8_t* __restrict__ kc, int num_kv_blocks,
    const int32_t* __restrict__ bt, int mkbpr,
    const int32_t* __restrict__ sl,
    const int32_t* __restrict__ mt, int mmbpr,
    uint8_t* __restrict__ maxb, uint8_t* __restrict__ minb, int num_meta,
    int BS, int row_vecs, const int32_t* __restrict__ first) {
    using E = Ext<BF16>;
    __shared__ u32x4 red_hi[kThreads];
    __shared__ u32x4 red_lo[kThreads];

    const int b = blockIdx.y;
    // sequence block of request b: the grid's x index, offset by the request's first
    // block to refresh when only new blocks are reduced
    const int i = int(blockIdx.x) + (first ? max(first[b], 0) : 0);
    const int L = max(sl[b], 0);
    const int nb = (L + BS - 1) / BS;
    const int nb_round = ((nb + BS - 1) / BS) * BS;
    if (i >= (first ? nb : nb_round) || i / BS >= mmbpr) return;
    const int m = mt[size_t(b) * mmbpr + i / BS];
    if (m < 0 || m >= num_meta) return;
    // this workgroup's slice of the row: columns [c0, c0 + cv) of 16 bytes each
    const int cv = row_vecs / int(gridDim.z);
    const size_t c0b = size_t(blockIdx.z) * cv * 16;
    const size_t row_bytes = size_t(row_vecs) * 16;
    uint8_t* omax = maxb + (size_t(m) * BS + (i % BS)) * row_bytes + c0b;
    uint8_t* omin = minb + (size_t(m) * BS + (i % BS)) * row_bytes + c0b;
    const int tid = threadIdx.x;

    if (i >= nb) {  // tail row of the last metadata block: +0.0
        const u32x4 z{0u, 0u, 0u, 0u};
        for (int v = tid; v < cv; v += kThreads) {
            st16(omax + size_t(v) * 16, z);
            st16(omin + size_t(v) * 16, z);
        }
        return;
    }
    if (i >= mkbpr) return;
    const int phys = bt[size_t(b) * mkbpr + i];
    if (phys < 0 || phys >= num_kv_blocks) return;
    const int nt = min(BS, L - i * BS);
    const uint8_t* src = kc + size_t(phys) * BS * row_bytes + c0b;

    if (cv <= kThreads) {
        const int R = kThreads / cv;  // token rows per pass
        const int col = tid % cv;
        const int r0 = tid / cv;
        u32x4 hi{E::hi_init, E::hi_init, E::hi_init, E::hi_init};
        u32x4 lo{E::lo_init, E::lo_init, E::lo_init, E::lo_init};
        if (r0 < R) {
            const uint8_t* p = src + size_t(col) * 16;
            int t = r0;
            for (; t + 7 * R < nt; t += 8 * R) {
                u32x4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = NT ? ld16_nt(p + size_t(t + u * R) * row_bytes) : ld16(p + size_t(t + u * R) * row_bytes);
#pragma unroll
                for (int u = 0; u < 8; ++u) fold<BF16>(hi, lo, v[u]);
            }
            for (; t < nt; t += R) fold<BF16>(hi, lo, NT ? ld16_nt(p + size_t(t) * row_bytes) : ld16(p + size_t(t) * row_bytes));
        }
        red_hi[tid] = hi;
        red_lo[tid] = lo;
        __syncthreads();
        if (tid < cv) {
            for (int r = 1; r < R; ++r) {
                const u32x4 h2 = red_hi[r * cv + tid];
                const u32x4 l2 = red_lo[r * cv + tid];
                hi.x = E::mx(hi.x, h2.x); hi.y = E::mx(hi.y, h2.y);
                hi.z = E::mx(hi.z, h2.z); hi.w = E::mx(hi.w, h2.w);
                lo.x = E::mn(lo.x, l2.x); lo.y = E::mn(lo.y, l2.y);
                lo.z = E::mn(lo.z, l2.z); lo.w = E::mn(lo.w, l2.w);
            }
            st16(omax + size_t(tid) * 16, unord<BF16>(hi));
            st16(omin + size_t(tid) * 16, unord<BF16>(lo));
        }
    } else {
        for (int col = tid; col < cv; col += kThreads) {
            u32x4 hi{E::hi_init, E::hi_init, E::hi_init, E::hi_init};
            u32x4 lo{E::lo_init, E::lo_init, E::lo_init, E::lo_init};
            const uint8_t* p = src + size_t(col) * 16;
            int t = 0;
            for (; t + 7 < nt; t += 8) {
                u32x4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = NT ? ld16_nt(p + size_t(t + u) * row_bytes) : ld16(p + size_t(t + u) * row_bytes);
#pragma unroll
                for (int u = 0; u < 8; ++u) fold<BF16>(hi, lo, v[u]);
            }
            for (; t < nt; ++t) fold<BF16>(hi, lo, NT ? ld16_nt(p + size_t(t) * row_bytes) : ld16(p + size_t(t) * row_bytes));
            st16(omax + size_t(col) * 16, unord<BF16>(hi));
            st16(omin + size_t(col) * 16, unord<BF16>(lo));
        }
    }
}

// Above this many bytes of K a build reads them with non-temporal loads: measured on the
// serving workload's 8.6 GB rebuild, and for the same reason as the attention's K/V (a plain
// read kernel over 1 GiB streamed 7.0 TB/s with them against 6.2 TB/s without).
constexpr size_t kMetaNtBytes = size_t(512) << 20;

void launch_meta(const MetaArgs& a, dim3 grid, const int32_t* first, hipStream_t s) {
    const int esize = a.bf16 ? 2 : 4;
    const int row_vecs = a.N * a.D * esize / 16;
    // K bytes the grid can read (upper bound: every block of the grid full)
    const size_t bytes = size_t(grid.x) * grid.y * a.BS * size_t(row_vecs) * 16;
    auto go = [&](auto bf, auto nt) {
        constexpr bool BF = decltype(bf)::value, NT = decltype(nt)::value;
        hipLaunchKernelGGL((meta_kernel<BF, NT>), grid, dim3(kThreads), 0, s, (const uint8_t*)a.k_cache,
                           a.num_kv_blocks, a.block_tables, a.mkbpr, a.seq_lens, a.meta_tables, a.mmbpr,
                           (uint8_t*)a.maxb, (uint8_t*)a.minb, a.num_meta, a.BS, row_vecs, first);
    };
    const bool nt = bytes > kMetaNtBytes;
    if (a.bf16) {
        if (nt) go(std::true_type{}, std::true_type{});
        else go(std::true_type{}, std::false_type{});
    } else {
        if (nt) go(std::false_type{}, std::true_type{});
        else go(std::false_type{}, std::false_type{});
    }
}

}  // namespace

hipError_t launch_build_metadata(const MetaArgs& a, hipStream_t s) {
    launch_meta(a, dim3(unsigned(a.mmbpr) * unsigned(a.BS), unsigned(a.B), 1u), nullptr, s);
    return hipGetLastError();
}

int update_col_slices(int B, int N, int D, bool bf16, int max_new_blocks) {
    // A refresh touches few blocks (often one per request): split each block's row into
    // column slices of at least one KV head (256 bytes or more) until the grid fills the chip.
    const int row_vecs = N * D * (bf16 ? 2 : 4) / 16;
    int slices = 1;
    while ((long long)B * max_new_blocks * slices < 2048 && row_vecs / (slices * 2) >= 16 &&
           (row_vecs % (slices * 2)) == 0)
        slices *= 2;
    return slices;
}

hipError_t launch_update_metadata(const MetaArgs& a, const int32_t* first_block, int max_new_blocks,
                                  hipStream_t s) {
    const int slices = update_col_slices(a.B, a.N, a.D, a.bf16, max_new_blocks);
    launch_meta(a, dim3(unsigned(max_new_blocks), unsigned(a.B), unsigned(slices)), first_block, s);
    return hipGetLastError();
}

}  // namespace qs

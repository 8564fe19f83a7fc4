// qs_device.h -- device helpers shared by the qsparse kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qs {

constexpr int kWave = 64;
constexpr int kThreads = 256;            // every kernel runs 4 wave64s per workgroup
constexpr int kWaves = kThreads / kWave;

struct __attribute__((aligned(16))) u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
// 16-byte load marked non-temporal (global_load_dwordx4 ... nt): for data a step streams
// once (K/V rows, block metadata). A plain read kernel over 1 GiB measured 7.0 TB/s with
// it against 6.2 TB/s without on MI355X.
typedef uint32_t u32nt4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
    const u32nt4 v = __builtin_nontemporal_load(reinterpret_cast<const u32nt4*>(p));
    return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// f32 -> bf16 (the upper half of a binary32), round to nearest even
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// Element types (the qs_dtype values) and the two 16-bit float formats: bf16 is the upper
// half of a binary32; f16 is IEEE binary16 (converted by the hardware, round to nearest even).
constexpr int kF32 = 0, kBF16 = 1, kI8 = 2, kF16 = 3;
__host__ __device__ constexpr int elem_bytes(int dt) { return dt == kF32 ? 4 : (dt == kI8 ? 1 : 2); }
template <int DT>
__device__ __forceinline__ float lo16(uint32_t w) {
    static_assert(DT == kBF16 || DT == kF16, "16-bit float formats only");
    if constexpr (DT == kBF16) return __uint_as_float(w << 16);
    else return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
template <int DT>
__device__ __forceinline__ float hi16(uint32_t w) {
    static_assert(DT == kBF16 || DT == kF16, "16-bit float formats only");
    if constexpr (DT == kBF16) return __uint_as_float(w & 0xffff0000u);
    else return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}
template <int DT>
__device__ __forceinline__ float half_to_f32(uint16_t h) { return lo16<DT>(uint32_t(h)); }
template <int DT>
__device__ __forceinline__ uint16_t f32_to_half(float f) {
    if constexpr (DT == kBF16) return f32_to_bf16_rne(f);
    else return __builtin_bit_cast(unsigned short, (_Float16)f);
}
// element e of a row as fp32 (DT f32, bf16 or f16)
template <int DT>
__device__ __forceinline__ float load_elem(const void* row, int e) {
    if constexpr (DT == kF32) return ((const float*)row)[e];
    else return half_to_f32<DT>(((const uint16_t*)row)[e]);
}

// Monotone map from finite floats to uint32: a < b (IEEE total order, -0 < +0)
// iff key(a) < key(b). Used for exact, deterministic top-k on scores.
__device__ __forceinline__ uint32_t f2key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// DPP lane moves inside a row of 16 lanes (all patterns stay within the row)
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within each 16
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

// Sum over aligned groups of `width` lanes (a power of two <= 64); every lane of the
// group ends with the same, bitwise identical sum. Groups of up to 16 lanes reduce with
// DPP row operations (quad swaps, then half-row and row mirrors: after each step all
// lanes of the merged span hold equal values, so a mirror pairs whole spans); wider
// groups finish with cross-row shuffles.
template <int width>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (width >= 2) v += dpp_f<kDppXor1>(v);
    if constexpr (width >= 4) v += dpp_f<kDppXor2>(v);
    if constexpr (width >= 8) v += dpp_f<kDppHalfMirror>(v);
    if constexpr (width >= 16) v += dpp_f<kDppMirror>(v);
#pragma unroll
    for (int o = 16; o < width; o <<= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
template <int width>
__device__ __forceinline__ int group_sum_i(int v) {
    if constexpr (width >= 2) v += dpp_i<kDppXor1>(v);
    if constexpr (width >= 4) v += dpp_i<kDppXor2>(v);
    if constexpr (width >= 8) v += dpp_i<kDppHalfMirror>(v);
    if constexpr (width >= 16) v += dpp_i<kDppMirror>(v);
#pragma unroll
    for (int o = 16; o < width; o <<= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
template <int width>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (width >= 2) v = fmaxf(v, dpp_f<kDppXor1>(v));
    if constexpr (width >= 4) v = fmaxf(v, dpp_f<kDppXor2>(v));
    if constexpr (width >= 8) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    if constexpr (width >= 16) v = fmaxf(v, dpp_f<kDppMirror>(v));
#pragma unroll
    for (int o = 16; o < width; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP (row shifts within each row
// of 16, then the row broadcasts 15 and 31 carry the row totals forward).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false); // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false); // row_bcast:31
    return x;
}

// max / min of a uint32 over the 64 lanes of a wave (every lane active), in every lane
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, uint32_t(dpp_i<kDppXor1>(int(v))));
    v = max(v, uint32_t(dpp_i<kDppXor2>(int(v))));
    v = max(v, uint32_t(dpp_i<kDppHalfMirror>(int(v))));
    v = max(v, uint32_t(dpp_i<kDppMirror>(int(v))));
    uint32_t r = 0u;
#pragma unroll
    for (int row = 0; row < kWave; row += 16) r = max(r, uint32_t(__builtin_amdgcn_readlane(int(v), row)));
    return r;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, uint32_t(dpp_i<kDppXor1>(int(v))));
    v = min(v, uint32_t(dpp_i<kDppXor2>(int(v))));
    v = min(v, uint32_t(dpp_i<kDppHalfMirror>(int(v))));
    v = min(v, uint32_t(dpp_i<kDppMirror>(int(v))));
    uint32_t r = 0xffffffffu;
#pragma unroll
    for (int row = 0; row < kWave; row += 16) r = min(r, uint32_t(__builtin_amdgcn_readlane(int(v), row)));
    return r;
}

// Exclusive prefix sum of a per-thread count over the workgroup in thread order; `total`
// receives the sum. wsum: kWaves ints of LDS. Two barriers.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
    const uint32_t incl = wave_incl_scan(uint32_t(v));
    if (lane_id() == kWave - 1) wsum[wave_id()] = int(incl);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int c = wsum[w];
        off += (w < wave_id()) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return off + int(incl) - v;
}

// Wave 0 scans the 256-bin histogram h from the highest bin down and finds the bin that
// holds the need-th largest element (1 <= need <= total): out[0] = that bin, out[1] = the
// count in the bins above it. Lane l owns bins 255-4l .. 252-4l.
__device__ __forceinline__ void find_desc_bin(const uint32_t* h, int need, int* out) {
    const int l = lane_id();
    uint32_t c[4];
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { c[j] = h[255 - 4 * l - j]; s += c[j]; }
    const uint32_t incl = wave_incl_scan(s);
    uint32_t run = incl - s;
    if (run < uint32_t(need) && uint32_t(need) <= incl) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (run + c[j] >= uint32_t(need)) {
                out[0] = 255 - 4 * l - j;
                out[1] = int(run);
                break;
            }
            run += c[j];
        }
    }
}

// Block-wide radix select over a virtual array of n keys.
// kf(i, &key) returns true if index i is a candidate and sets its key.
// Finds the R-th largest candidate key T (1 <= R <= #candidates); on return `need_eq`
// holds how many candidates equal to T belong to the top R (R minus those above T).
// LDS: hist[512] (two 256-bin histograms used alternately, so clearing the next one
// needs no barrier of its own), sh[4]. Two barriers per 8-bit pass; every thread of the
// workgroup must call it.
template <class KeyFn>
__device__ uint32_t block_radix_select(int n, int R, KeyFn kf, uint32_t* hist, int* sh, int& need_eq) {
    uint32_t prefix = 0, pmask = 0;
    int need = R;
    for (int j = threadIdx.x; j < 512; j += kThreads) hist[j] = 0;
    __syncthreads();
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        uint32_t* h = hist + 256 * (pass & 1);
        for (int i = threadIdx.x; i < n; i += kThreads) {
            uint32_t key;
            if (kf(i, key) && (key & pmask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave_id() == 0) find_desc_bin(h, need, sh + 2 * (pass & 1));
        // the other histogram is free now: clear it for the next pass
        for (int j = threadIdx.x; j < 256; j += kThreads) hist[256 * ((pass + 1) & 1) + j] = 0;
        __syncthreads();
        const uint32_t d = uint32_t(sh[2 * (pass & 1)]);
        need -= sh[2 * (pass & 1) + 1];
        prefix |= d << shift;
        pmask |= 255u << shift;
    }
    need_eq = need;
    return prefix;
}


// The same result as block_radix_select (the R-th largest candidate key T, and need_eq),
// in one histogram pass for keys that are spread out: the block's key range [kmin, kmax]
// is cut into 256 bins by the top 8 significant bits of key - kmin (a monotone map, so
// every key in a higher bin is larger), the bin holding the R-th largest key is found,
// its keys are gathered into a list, and T is the key whose rank in that list is right
// (counted against the whole list). Five barriers and no contended LDS atomics when the
// keys spread over the bins; when more than 256 keys share the boundary bin (heavy
// clustering or ties) it falls back to the radix select. Same LDS as
// block_radix_select: hist[512] (bins in the first half, the boundary list and the
// per-wave range in the second), sh[4]. Every thread of the workgroup must call it.
template <class KeyFn>
__device__ uint32_t block_topk_threshold(int n, int R, KeyFn kf, uint32_t* hist, int* sh, int& need_eq) {
    const int tid = threadIdx.x;
    uint32_t* list = hist + 256;
    for (int j = tid; j < 256; j += kThreads) hist[j] = 0;
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    for (int i = tid; i < n; i += kThreads) {
        uint32_t key;
        if (kf(i, key)) { kmin = min(kmin, key); kmax = max(kmax, key); }
    }
    // wave range: DPP inside each row of 16 lanes (every lane active), then the four row
    // results, so that every lane holds the wave's range
    kmin = min(kmin, uint32_t(dpp_i<kDppXor1>(int(kmin))));
    kmax = max(kmax, uint32_t(dpp_i<kDppXor1>(int(kmax))));
    kmin = min(kmin, uint32_t(dpp_i<kDppXor2>(int(kmin))));
    kmax = max(kmax, uint32_t(dpp_i<kDppXor2>(int(kmax))));
    kmin = min(kmin, uint32_t(dpp_i<kDppHalfMirror>(int(kmin))));
    kmax = max(kmax, uint32_t(dpp_i<kDppHalfMirror>(int(kmax))));
    kmin = min(kmin, uint32_t(dpp_i<kDppMirror>(int(kmin))));
    kmax = max(kmax, uint32_t(dpp_i<kDppMirror>(int(kmax))));
#pragma unroll
    for (int r = 0; r < kWave; r += 16) {
        kmin = min(kmin, uint32_t(__builtin_amdgcn_readlane(int(kmin), r)));
        kmax = max(kmax, uint32_t(__builtin_amdgcn_readlane(int(kmax), r)));
    }
    if (lane_id() == 0) { list[wave_id()] = kmin; list[kWaves + wave_id()] = kmax; }
    if (tid == 0) sh[3] = 0;  // boundary list length
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) { kmin = min(kmin, list[w]); kmax = max(kmax, list[kWaves + w]); }
    if (kmin == kmax) {  // every candidate has the same key
        need_eq = R;
        return kmin;
    }
    const uint32_t d = kmax - kmin;
    const int shift = max(0, (32 - __clz(d)) - 8);  // (key - kmin) >> shift is in [0, 255]
    for (int i = tid; i < n; i += kThreads) {
        uint32_t key;
        if (kf(i, key)) atomicAdd(&hist[(key - kmin) >> shift], 1u);
    }
    __syncthreads();
    if (wave_id() == 0) find_desc_bin(hist, R, sh);
    __syncthreads();
    const uint32_t bs = uint32_t(sh[0]);
    const int need = R - sh[1];  // 1 <= need <= the boundary bin's count
    for (int i = tid; i < n; i += kThreads) {
        uint32_t key;
        if (kf(i, key) && ((key - kmin) >> shift) == bs) {
            const int pos = atomicAdd(&sh[3], 1);
            if (pos < 256) list[pos] = key;
        }
    }
    __syncthreads();
    const int m = sh[3];
    if (m > 256) return block_radix_select(n, R, kf, hist, sh, need_eq);
    if (tid < m) {
        const uint32_t mk = list[tid];
        int gt = 0, ge = 0;
        for (int e = 0; e < m; ++e) {
            const uint32_t o = list[e];
            gt += o > mk ? 1 : 0;
            ge += o >= mk ? 1 : 0;
        }
        // T has fewer than `need` larger keys and at least `need` keys >= it; every thread
        // holding T writes the same two values
        if (gt < need && need <= ge) { sh[0] = int(mk); sh[1] = need - gt; }
    }
    __syncthreads();
    need_eq = sh[1];
    return uint32_t(sh[0]);
}
// Workgroup placement on the 8 XCDs. The dispatcher deals workgroups to the XCDs
// round-robin by linear id, so the slot splits of one row (consecutive in x) land on
// different XCDs, and each XCD re-reads the row's shared inputs (staged scores, metadata,
// table row) into its own L2. With `grouped` and a grid size that is a multiple of 8, the
// workgroup with linear id l instead takes work item (l mod 8)·(total/8) + l/8, so each
// XCD takes one contiguous eighth of the work items in (x, y, z) order: whole rows with
// all their splits. A bijection on the work items, so every item still runs exactly once.
// Rows of one workgroup share nothing, and there the round-robin placement streams
// faster (measured on the serving workload: 221 against 230 us), so callers group only
// split rows. Returns the item's (x, y, z).
constexpr int kXcds = 8;
__device__ __forceinline__ uint3 xcd_block_index(bool grouped) {
    const uint64_t nx = gridDim.x, ny = gridDim.y, total = nx * ny * gridDim.z;
    if (!grouped || total % kXcds) return make_uint3(blockIdx.x, blockIdx.y, blockIdx.z);
    const uint64_t lin = blockIdx.x + nx * (blockIdx.y + ny * uint64_t(blockIdx.z));
    const uint64_t w = (lin % kXcds) * (total / kXcds) + lin / kXcds;
    return make_uint3(unsigned(w % nx), unsigned((w / nx) % ny), unsigned(w / (nx * ny)));
}

}  // namespace qs

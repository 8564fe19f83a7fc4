// importance.hip -- page 1's prefill importance: the attention mass each prompt token
// receives from the causal prefill, per head and summed over heads.
//
// Source: "0.8MB 跑通 Qwen | 第 10-2 篇" (page 1), section 1 "知识点", signal 2 (how much
// attention the prefill actually gave each token, recorded per head and reduced over
// heads) and section 2's closing note (each head's imp_head is added into
// prefill_importance[s] when the prefill ends). With p_h[t][s] the causal softmax weight
// of key s in query row t of head h, imp_head[h][s] = sum over t >= s of p_h[t][s] and
// prefill_importance[s] = sum over heads of imp_head[h][s].
//
// Design (CDNA4). The weights need each row's softmax normaliser before any column can
// be summed, so there are two passes over the causal score matrix. The row pass is a
// dense contraction on the matrix cores; the column pass either repeats it (16-bit
// inputs, or fp32 scores too large to keep) or, for fp32 inputs when the lower triangle
// of 16x16 score tiles fits the workspace (at most 2 GiB), streams the scores that the
// row pass stored:
//   row pass     work item (query tile, key chunk): each wave takes 16 query rows per
//                row tile it holds and walks the chunk's 16-key tiles up to its last row,
//                S = Q K^T on v_mfma_f32_16x16x4_f32 (fp32 inputs) or
//                v_mfma_f32_16x16x32_{bf16,f16}; each lane keeps an online (max, sum) of
//                its key column for its 4 rows of each row tile, and the 16 lanes of a row
//                merge once at the end into the chunk's (max, sum);
//   merge        per row, the chunks' (max, sum) in chunk order -> log2-sum-exp (with
//                one chunk the row pass writes it itself);
//   column pass  work item (key tile, query-row chunk): each wave takes 16 keys per key
//                tile it holds and walks the chunk's 16-row query tiles from its first key
//                on, S^T = K Q^T, adds 2^(x - lse_row) into per-lane column sums, merges
//                the 16 lanes and writes the chunk's column sums;
//   stored scores (fp32) the row pass also writes each causal 16x16 tile of its scaled
//                scores (masked entries as -inf, non-temporal stores: nothing reads them
//                before they leave the cache); the column pass is then one workgroup per
//                (key tile, head, request) whose four waves take every fourth row tile,
//                eight in flight per wave, add 2^(x - lse_row) per key and merge in a fixed
//                order. A fp32 tile costs 32 MFMA steps of 4 channels (about 1000 cycles
//                of one SIMD); a SIMD's share of the HBM rate (about 3.3 bytes a cycle)
//                streams the tile's 1 KB in about 300, so reading the scores back is
//                cheaper than the contraction it replaces, even before the K tile's fetch
//                and LDS staging that the contraction needs as well;
//   reduce       sums the chunks, then the heads, in a fixed order (deterministic).
// A wave holds one 16-row tile with fp32 inputs and two with 16-bit ones (wave_tiles), so
// a workgroup's tile is 64 or 128 query rows (keys). With 16-bit inputs a wave's matrix
// work per fetched tile is short and the per-step work around it (the tile's fetch, LDS
// store, barrier and fragment reads) dominates; two tiles per wave feed each fetched tile
// and each fragment read to twice the MFMAs.
// Chunks: a causal tile's work grows with its distance from the diagonal. With 16-bit
// inputs a wave's matrix work between two barriers is short, so a CU whose short tiles
// have finished cannot keep its matrix pipe fed from the one long tile left; there every
// tile's range is cut into chunks of R tiles (at most 8 chunks), giving several times
// more, bounded items, which the dispatcher hands to CUs as they free up. With fp32
// inputs one wave's matrix work alone keeps the pipe busy and the extra items only cost
// their start-up, so each tile stays one item, as do jobs that already hold enough work
// to balance (>= 8192 x 64 rows x heads x requests); the snake order below evens the
// first items out.
// Operand layout: a lane (row r = lane % 16, group j = lane / 16) holds channels
// 32j .. 32j+31 of its row, contiguous in memory (16-byte loads). The contraction order
// over channels is free, so both operands use that same channel order: at step ks the
// f32 MFMA pairs channel 32j + ks, the 16-bit one channels 32j + 8ks .. 8ks + 7.
#include <float.h>
#include <math.h>

#include "attn_dev.h"
#include "qs_device.h"
#include "qs_internal.h"

namespace qs {
namespace {

constexpr int D = 128;
constexpr float kLog2e = 1.4426950408889634f;

// 16-row tiles per wave: two with 16-bit inputs, whose matrix work per tile is short, so
// that each operand fragment read from LDS and each tile fetched into LDS feed twice the
// MFMAs; one with fp32 inputs, where 64 more registers of query would cost occupancy. A
// workgroup of four waves then covers wave_tiles * 64 query rows (row pass) or keys
// (column pass).
template <int DT>
constexpr int wave_tiles() { return DT == kF32 ? 1 : 2; }
template <int DT>
constexpr int tile_rows() { return 64 * wave_tiles<DT>(); }

struct ImpParams {
    const uint8_t* q;   // [B, max_len, H, D]
    const uint8_t* kc;  // [num_kv_blocks, BS, N, D]
    int num_kv_blocks;
    const int32_t* bt;
    int mkbpr;
    const int32_t* sl;
    int B, H, N, BS, max_len;
    float scale2;  // softmax scale * log2(e)
    int TR;        // rows (keys) of a workgroup's tile: 64 or 128
    int T, R, C;   // tiles of max_len, tiles per chunk, chunks
    float* lse;    // [B, H, max_len] workspace: log2-sum-exp2 of each row
    float* mpart;  // [C, B, H, max_len] workspace: each key chunk's row max (log2 units)
    float* lpart;  // [C, B, H, max_len] workspace: each key chunk's sum of 2^(x - max)
    float* cpart;  // [C, B, H, max_len] workspace: each row chunk's column sums
    float* S;      // fp32 stored-score path: the scores x (log2 units, masked -inf) of each
                   // (b, h) in 16 x 16 blocks, key-tile-major lower triangle; null: recompute
    int T16;       // 16-row tiles of max_len
    size_t sblocks;  // blocks per (b, h): T16 (T16 + 1) / 2
};

// block (key tile kt, row tile rt >= kt) of one (b, h) in the stored-score layout: key tile
// kt's blocks are consecutive, rows kt .. T16 - 1; inside a block, key column c's 16 rows
// are contiguous (element (c, i) at c * 16 + i)
__device__ __forceinline__ size_t sblock(int T16, int kt, int rt) {
    return size_t(kt) * T16 - size_t(kt) * (kt - 1) / 2 + size_t(rt - kt);
}

// chunking of a (B, H, max_len) job with tiles of TR rows
constexpr int kMaxChunks = 8;
struct Split { int T, R, C; };
inline Split imp_split(int B, int H, int max_len, bool chunked, int TR) {
    constexpr long kEnoughRows = 8192L * 64;  // rows x heads x requests that balance unaided
    Split sp;
    sp.T = (max_len + TR - 1) / TR;
    if (sp.T <= 0) return Split{0, 1, 1};
    const long rows = long(sp.T) * TR * H * B;
    const int want = (!chunked || rows >= kEnoughRows) ? 1 : min(kMaxChunks, sp.T);
    sp.R = (sp.T + want - 1) / want;
    sp.C = (sp.T + sp.R - 1) / sp.R;
    return sp;
}
// items of the two passes per (head, request): the diagonal chunk of every tile plus the
// full chunks (row pass: chunks c < i / R of row tile i; column pass: chunks c > j / R of
// key tile j)
inline long row_items(const Split& s) {
    long n = s.T;
    for (int c = 0; c < s.C; ++c) n += max(0, s.T - (c + 1) * s.R);
    return n;
}
inline long col_items(const Split& s) {
    long n = s.T;
    for (int c = 1; c < s.C; ++c) n += long(c) * s.R;
    return n;
}

// one row's channels 32j .. 32j+31 (this lane's operand slice)
template <int DT>
struct Frag {
    static constexpr int kVecs = DT == kF32 ? 8 : 4;  // 16-byte pieces
    u32x4 v[kVecs];
};

template <int DT>
__device__ __forceinline__ void load_frag(Frag<DT>& f, const uint8_t* row, int j) {
    const uint8_t* p = row + size_t(32 * j) * elem_bytes(DT);
#pragma unroll
    for (int i = 0; i < Frag<DT>::kVecs; ++i) f.v[i] = ld16(p + 16 * i);
}

// C[m][n] = sum over the 128 channels of A-row m times B-row n (16 x 16 tile, fp32). Two
// independent accumulation chains (even and odd steps) halve the dependent MFMA latency.
template <int DT>
__device__ __forceinline__ attn::f32x4 dot_tile(const Frag<DT>& a, const Frag<DT>& b) {
    attn::f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t aw[4] = {a.v[i].x, a.v[i].y, a.v[i].z, a.v[i].w};
            const uint32_t bw[4] = {b.v[i].x, b.v[i].y, b.v[i].z, b.v[i].w};
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(aw[e]), __uint_as_float(bw[e]), c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(aw[e + 1]), __uint_as_float(bw[e + 1]), c1,
                                                          0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            c0 = attn::mfma16x16x32<DT>(attn::as_op8<DT>(a.v[i]), attn::as_op8<DT>(b.v[i]), c0);
            c1 = attn::mfma16x16x32<DT>(attn::as_op8<DT>(a.v[i + 1]), attn::as_op8<DT>(b.v[i + 1]), c1);
        }
    }
    return c0 + c1;
}

// two tiles sharing the operand a: four independent accumulation chains
template <int DT>
__device__ __forceinline__ void dot_tile2(const Frag<DT>& a, const Frag<DT>& b0, const Frag<DT>& b1,
                                          attn::f32x4& r0, attn::f32x4& r1) {
    attn::f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, d0 = c0, d1 = c0;
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t aw[4] = {a.v[i].x, a.v[i].y, a.v[i].z, a.v[i].w};
            const uint32_t bw[4] = {b0.v[i].x, b0.v[i].y, b0.v[i].z, b0.v[i].w};
            const uint32_t ew[4] = {b1.v[i].x, b1.v[i].y, b1.v[i].z, b1.v[i].w};
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(aw[e]), __uint_as_float(bw[e]), c0, 0, 0, 0);
                d0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(aw[e]), __uint_as_float(ew[e]), d0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(aw[e + 1]), __uint_as_float(bw[e + 1]), c1, 0, 0, 0);
                d1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(aw[e + 1]), __uint_as_float(ew[e + 1]), d1, 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            c0 = attn::mfma16x16x32<DT>(attn::as_op8<DT>(a.v[i]), attn::as_op8<DT>(b0.v[i]), c0);
            d0 = attn::mfma16x16x32<DT>(attn::as_op8<DT>(a.v[i]), attn::as_op8<DT>(b1.v[i]), d0);
            c1 = attn::mfma16x16x32<DT>(attn::as_op8<DT>(a.v[i + 1]), attn::as_op8<DT>(b0.v[i + 1]), c1);
            d1 = attn::mfma16x16x32<DT>(attn::as_op8<DT>(a.v[i + 1]), attn::as_op8<DT>(b1.v[i + 1]), d1);
        }
    }
    r0 = c0 + c1;
    r1 = d0 + d1;
}

// two tiles sharing the operand b (two row tiles against one key tile in the row pass, two
// key tiles against one query tile in the column pass): four independent chains
template <int DT>
__device__ __forceinline__ void dot_tile2a(const Frag<DT>& a0, const Frag<DT>& a1, const Frag<DT>& b,
                                           attn::f32x4& r0, attn::f32x4& r1) {
    attn::f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, d0 = c0, d1 = c0;
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t aw[4] = {a0.v[i].x, a0.v[i].y, a0.v[i].z, a0.v[i].w};
            const uint32_t ew[4] = {a1.v[i].x, a1.v[i].y, a1.v[i].z, a1.v[i].w};
            const uint32_t bw[4] = {b.v[i].x, b.v[i].y, b.v[i].z, b.v[i].w};
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(aw[e]), __uint_as_float(bw[e]), c0, 0, 0, 0);
                d0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ew[e]), __uint_as_float(bw[e]), d0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(aw[e + 1]), __uint_as_float(bw[e + 1]), c1, 0, 0, 0);
                d1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ew[e + 1]), __uint_as_float(bw[e + 1]), d1, 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            c0 = attn::mfma16x16x32<DT>(attn::as_op8<DT>(a0.v[i]), attn::as_op8<DT>(b.v[i]), c0);
            d0 = attn::mfma16x16x32<DT>(attn::as_op8<DT>(a1.v[i]), attn::as_op8<DT>(b.v[i]), d0);
            c1 = attn::mfma16x16x32<DT>(attn::as_op8<DT>(a0.v[i + 1]), attn::as_op8<DT>(b.v[i + 1]), c1);
            d1 = attn::mfma16x16x32<DT>(attn::as_op8<DT>(a1.v[i + 1]), attn::as_op8<DT>(b.v[i + 1]), d1);
        }
    }
    r0 = c0 + c1;
    r1 = d0 + d1;
}

// Work item of this workgroup: (tile, chunk, head, request). Consecutive ranks take the
// heads and requests of one (tile, chunk), so the items running together share their
// other operand in L2. The full chunks (all of one size) come first, chunk by chunk, then
// the diagonal chunks, longest tile first when there is one chunk. The first 1024 items
// are all resident at once and the dispatcher hands ids to the CUs round-robin (CU c
// holds ids c, c + kCus, ...), so ids map to ranks in a snake order over rounds of kCus
// (forward in even rounds, backward in odd ones): with one chunk per tile every CU then
// holds a mix of long and short tiles instead of four equal ones.
constexpr int kCus = 256;
struct WorkItem { int tile, chunk, h, b; };
__device__ __forceinline__ int snake_rank() {
    const int id = blockIdx.x, total = gridDim.x;
    const int rnd = id / kCus, pos = id % kCus;
    const int cnt = min(kCus, total - rnd * kCus);  // ids in this round
    return rnd * kCus + ((rnd & 1) ? cnt - 1 - pos : pos);
}
__device__ __forceinline__ WorkItem row_item(const ImpParams& p) {
    const int HB = p.H * p.B, rank = snake_rank();
    const int hb = rank % HB;
    int q = rank / HB;
    int tile = -1, chunk = 0;
    for (int c = 0; c < p.C && tile < 0; ++c) {  // row tiles i >= (c + 1) R hold a full chunk c
        const int n = max(0, p.T - (c + 1) * p.R);
        if (q < n) { tile = (c + 1) * p.R + q; chunk = c; } else { q -= n; }
    }
    if (tile < 0) { tile = p.T - 1 - q; chunk = tile / p.R; }
    return WorkItem{tile, chunk, hb % p.H, hb / p.H};
}
__device__ __forceinline__ WorkItem col_item(const ImpParams& p) {
    const int HB = p.H * p.B, rank = snake_rank();
    const int hb = rank % HB;
    int q = rank / HB;
    int tile = -1, chunk = 0;
    for (int c = p.C - 1; c >= 1 && tile < 0; --c) {  // key tiles j < c R see a full chunk c
        const int n = c * p.R;
        if (q < n) { tile = q; chunk = c; } else { q -= n; }
    }
    if (tile < 0) { tile = q; chunk = tile / p.R; }
    return WorkItem{tile, chunk, hb % p.H, hb / p.H};
}

// address of key s >= 0 (head kh) of request b, or nullptr when its block is out of range
__device__ __forceinline__ const uint8_t* key_row(const ImpParams& p, int b, int s, int kh, int esize) {
    const unsigned blk = unsigned(s) / unsigned(p.BS), off = unsigned(s) - blk * unsigned(p.BS);
    const int phys = p.bt[size_t(b) * p.mkbpr + blk];
    if (phys < 0 || phys >= p.num_kv_blocks) return nullptr;
    return p.kc + ((size_t(phys) * p.BS + off) * p.N + kh) * D * esize;
}

// 2^x on the hardware's exp2 (v_exp_f32), without the library's rescaling of results
// below 2^-126: such a term changes none of the sums here (a row's sum is >= 1, and a
// column sum's terms are the weights themselves)
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// A 16-row operand tile shared by the workgroup's four waves through LDS: the workgroup
// loads it once (each thread 16-byte pieces of whole rows), every wave reads its
// fragment from LDS. Rows are padded by 16 B against bank conflicts. The passes take two
// tiles per workgroup barrier (four buffers, two pairs in turn): while a pair is
// multiplied, the next pair is already in flight into registers, and the waves run four
// independent accumulation chains (dot_tile2).
template <int DT>
struct Tile {
    static constexpr int kRowBytes = D * elem_bytes(DT);        // 512 (fp32) or 256
    static constexpr int kPitch = kRowBytes + 16;
    static constexpr int kPieces = 16 * kRowBytes / 16;         // 16-byte pieces per tile
    static constexpr int kPerThread = kPieces / kThreads;       // 2 (fp32) or 1
    static constexpr int kBytes = 16 * kPitch;
    static_assert(kPieces % kThreads == 0, "whole pieces per thread");
};

// this thread's pieces of a 16-row tile whose row i starts at base + i * stride for
// i <= last (later rows repeat row last). The base is wave-uniform and the per-lane
// offset 32-bit (stride <= 65535 * 512 bytes, rows <= 15), so each load is one
// scalar-base global load with no 64-bit lane arithmetic.
template <int DT>
__device__ __forceinline__ void tile_fetch(u32x4 (&v)[Tile<DT>::kPerThread], const uint8_t* base, unsigned stride,
                                           int last) {
    constexpr int ppr = Tile<DT>::kRowBytes / 16;  // pieces per row
#pragma unroll
    for (int u = 0; u < Tile<DT>::kPerThread; ++u) {
        const int piece = threadIdx.x + u * kThreads;
        const unsigned row = unsigned(min(piece / ppr, last));
        v[u] = ld16(base + (row * stride + 16u * unsigned(piece % ppr)));
    }
}
template <int DT>
__device__ __forceinline__ void tile_store(uint8_t* buf, const u32x4 (&v)[Tile<DT>::kPerThread]) {
    constexpr int ppr = Tile<DT>::kRowBytes / 16;
#pragma unroll
    for (int u = 0; u < Tile<DT>::kPerThread; ++u) {
        const int piece = threadIdx.x + u * kThreads;
        st16(buf + (piece / ppr) * Tile<DT>::kPitch + 16 * (piece % ppr), v[u]);
    }
}
// this lane's operand slice (row r, channels 32j .. 32j+31) from an LDS tile
template <int DT>
__device__ __forceinline__ void frag_from_tile(Frag<DT>& f, const uint8_t* buf, int r, int j) {
    const uint8_t* q = buf + r * Tile<DT>::kPitch + 32 * j * elem_bytes(DT);
#pragma unroll
    for (int i = 0; i < Frag<DT>::kVecs; ++i) f.v[i] = ld16(q + 16 * i);
}

// STORE (fp32 stored-score path): every score x of the pass is also written to p.S
template <int DT, bool STORE = false>
__global__ __launch_bounds__(kThreads) void imp_row_kernel(ImpParams p) {
    constexpr int es = elem_bytes(DT);
    constexpr int RW = wave_tiles<DT>(), TR = tile_rows<DT>();
    __shared__ __attribute__((aligned(16))) uint8_t kt[4][Tile<DT>::kBytes];
    const WorkItem wi = row_item(p);
    const int b = wi.b, h = wi.h;
    const int L = min(max(p.sl[b], 0), min(p.max_len, p.mkbpr * p.BS));
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, j = lane >> 4;
    const int tw = wi.tile * TR;  // the workgroup's rows tw .. tw + TR - 1
    if (tw >= L) return;                              // whole workgroup
    const int t0 = tw + 16 * RW * w;                  // this wave's rows t0 .. t0 + 16 RW - 1
    const int s_lo = wi.chunk * p.R * TR;             // the chunk's keys s_lo .. (<= tw since chunk <= tile / R)
    const int kh = h / (p.H / p.N);
    Frag<DT> qf[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
        load_frag<DT>(qf[rr], p.q + ((size_t(b) * p.max_len + min(t0 + 16 * rr + r, L - 1)) * p.H + h) * D * es, j);

    // online max / sum of 2^x over this lane's key column, rows t0 + 16 rr + 4j + i. The max
    // starts at -FLT_MAX, below every finite score, so a masked score (-inf) never meets an
    // infinite max
    float m[RW][4], l[RW][4];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
        for (int i = 0; i < 4; ++i) { m[rr][i] = -FLT_MAX; l[rr][i] = 0.f; }
    const int s_end = min(min(s_lo + p.R * TR, tw + TR), L) - 1;  // last key any wave needs
    // key tile s0 (16 keys in one block, physical block ph): rows past L repeat the last
    // key (masked). The block-table entries are read one step before their tile (bt_at),
    // so no step waits for a lookup between its barrier and its loads.
    // read through the constant address space: nothing writes the block table while the
    // kernel runs, and with the score stores in the loop the compiler can no longer prove it
    // by itself; scalar lookups then keep the step's K loads in flight past them
    typedef const __attribute__((address_space(4))) int32_t* const_i32p;
    const const_i32p btrow = (const_i32p)(p.bt + size_t(b) * p.mkbpr);
    auto bt_at = [&](int s) { return btrow[unsigned(min(s, L - 1)) / unsigned(p.BS)]; };
    auto fetch = [&](int s0, int ph, u32x4 (&v)[Tile<DT>::kPerThread]) -> bool {
        if (ph < 0 || ph >= p.num_kv_blocks) return false;
        const uint8_t* base = p.kc + ((size_t(ph) * p.BS + unsigned(s0) % unsigned(p.BS)) * p.N + kh) * size_t(D * es);
        tile_fetch<DT>(v, base, unsigned(p.N) * D * es, L - 1 - s0);
        return true;
    };
    int pa = bt_at(s_lo), pb = bt_at(s_lo + 16);
    // the softmax update of row tile rr (this lane's 4 rows) with one 16-key tile's scores
    // (key s of this lane), branch-free: a masked score enters as -inf and changes nothing.
    // Tiles whose 16 keys precede all of the tile's rows and L (all) skip the mask.
    float pv[2][4];            // STORE: a step's scores, written early in the next step
    int pblk[2] = {-1, -1};    // their blocks in the stored layout (-1: nothing pending)
    float* const sbh = STORE ? p.S + (size_t(b) * p.H + h) * p.sblocks * 256 + r * 16 + 4 * j : nullptr;
    auto flush = [&]() {
        if constexpr (STORE) {
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                if (pblk[sl] < 0) continue;
                typedef float f4nt __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(f4nt{pv[sl][0], pv[sl][1], pv[sl][2], pv[sl][3]},
                                            reinterpret_cast<f4nt*>(sbh + size_t(pblk[sl]) * 256));
                pblk[sl] = -1;
            }
        }
    };
    auto upd = [&](const attn::f32x4& c, int rr, int s, bool all, int s0k, int sl) {
        float xs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 16 * rr + 4 * j + i;
            xs[i] = (all || (s <= t && s < L)) ? c[i] * p.scale2 : -INFINITY;
        }
        if constexpr (STORE) {  // this lane's key column r, rows 4j .. 4j + 3 of the block
            pblk[sl] = int(sblock(p.T16, s0k >> 4, (t0 + 16 * rr) >> 4));
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[sl][i] = xs[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // one exp2 per score: a new maximum rescales the sum, any other score adds
            const float x = xs[i];
            const float d = x - m[rr][i];
            const float e = exp2_hw(-fabsf(d));
            l[rr][i] = d > 0.f ? fmaf(l[rr][i], e, 1.f) : l[rr][i] + e;
            m[rr][i] = fmaxf(m[rr][i], x);
        }
    };
    auto upd_tile = [&](const attn::f32x4& c, int rr, int s0k, int sl) {
        if (s0k + 15 <= t0 + 16 * rr && s0k + 15 < L) upd(c, rr, s0k + r, true, s0k, sl);
        else upd(c, rr, s0k + r, false, s0k, sl);
    };
    // a step takes two key tiles (32 keys): both go to LDS, one barrier, then the next two
    // are fetched into the freed register sets and the pair is multiplied; four LDS
    // buffers, so a pair's stores never meet the previous pair's reads
    auto step2 = [&](int s0, uint8_t* b0, uint8_t* b1, u32x4 (&va)[Tile<DT>::kPerThread], bool& ha,
                     u32x4 (&vb)[Tile<DT>::kPerThread], bool& hb) {
        // stored whether or not a tile was fetched (an unfetched buffer is never read): every
        // step then waits for its loads here, so the MFMAs below never wait for global loads
        tile_store<DT>(b0, va);
        tile_store<DT>(b1, vb);
        // key tile kk of the pair is needed by row tile rr if it was fetched, its first key
        // is at or before the tile's last row, and the tile has rows before L
        auto need = [&](int kk, int rr) {
            const int tr = t0 + 16 * rr;
            return (kk == 0 ? ha : hb) && s0 + 16 * kk <= tr + 15 && tr < L;
        };
        bool nd[2][RW];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) nd[kk][rr] = need(kk, rr);
        __syncthreads();
        // the previous step's scores: issued before this step's loads, so the wait for those
        // loads at the next step's start never waits on a store issued after them
        flush();
        ha = s0 + 32 <= s_end && fetch(s0 + 32, pa, va);
        hb = s0 + 48 <= s_end && fetch(s0 + 48, pb, vb);
        pa = bt_at(s0 + 64);  // the entries of the next step's tiles
        pb = bt_at(s0 + 80);
        if constexpr (RW == 1) {
            if (nd[0][0] && nd[1][0]) {
                Frag<DT> k0, k1;
                frag_from_tile<DT>(k0, b0, r, j);
                frag_from_tile<DT>(k1, b1, r, j);
                attn::f32x4 r0, r1;
                dot_tile2<DT>(qf[0], k0, k1, r0, r1);
                upd_tile(r0, 0, s0, 0);
                upd_tile(r1, 0, s0 + 16, 1);
            } else if (nd[0][0] || nd[1][0]) {
                Frag<DT> kf;
                frag_from_tile<DT>(kf, nd[0][0] ? b0 : b1, r, j);
                const attn::f32x4 c = dot_tile<DT>(qf[0], kf);
                if (nd[0][0]) upd_tile(c, 0, s0, 0);
                else upd_tile(c, 0, s0 + 16, 1);
            }
        } else {
            // each key fragment read from LDS feeds both row tiles
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (!nd[kk][0] && !nd[kk][1]) continue;
                Frag<DT> kf;
                frag_from_tile<DT>(kf, kk == 0 ? b0 : b1, r, j);
                const int sk = s0 + 16 * kk;
                if (nd[kk][0] && nd[kk][1]) {
                    attn::f32x4 r0, r1;
                    dot_tile2a<DT>(qf[0], qf[1], kf, r0, r1);
                    upd_tile(r0, 0, sk, 0);
                    upd_tile(r1, 1, sk, 0);
                } else if (nd[kk][0]) {  // constant tile indices keep m, l and qf in registers
                    upd_tile(dot_tile<DT>(qf[0], kf), 0, sk, 0);
                } else {
                    upd_tile(dot_tile<DT>(qf[1], kf), 1, sk, 0);
                }
            }
        }
    };
    u32x4 na[Tile<DT>::kPerThread] = {}, nb[Tile<DT>::kPerThread] = {};
    bool ha = fetch(s_lo, pa, na);
    bool hb = s_lo + 16 <= s_end && fetch(s_lo + 16, pb, nb);
    pa = bt_at(s_lo + 32);
    pb = bt_at(s_lo + 48);
    for (int s0 = s_lo, buf = 0; s0 <= s_end; s0 += 32, buf ^= 2) step2(s0, kt[buf], kt[buf + 1], na, ha, nb, hb);
    flush();
    // merge the 16 key columns of each row into the chunk's (max, sum); every row t < L
    // has a key of the chunk (s_lo <= tw), so the max is finite. With one chunk that is
    // the row's log2-sum-exp already.
    const size_t o = ((size_t(wi.chunk) * p.B + b) * p.H + h) * p.max_len;
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float M = group_max<16>(m[rr][i]);
            const float part = l[rr][i] * exp2f(m[rr][i] - M);  // a lane without keys: l = 0
            const float S = group_sum<16>(part);
            const int t = t0 + 16 * rr + 4 * j + i;
            if (r == 0 && t < L) {
                if (p.C == 1) {
                    p.lse[o + t] = M + log2f(S);
                } else {
                    p.mpart[o + t] = M;
                    p.lpart[o + t] = S;
                }
            }
        }
    }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void imp_col_kernel(ImpParams p) {
    constexpr int es = elem_bytes(DT);
    constexpr int RW = wave_tiles<DT>(), TR = tile_rows<DT>();
    __shared__ __attribute__((aligned(16))) uint8_t qt[4][Tile<DT>::kBytes];
    __shared__ float lt_s[4][16];
    const WorkItem wi = col_item(p);
    const int b = wi.b, h = wi.h;
    const int L = min(max(p.sl[b], 0), min(p.max_len, p.mkbpr * p.BS));
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, j = lane >> 4;
    const int sw = wi.tile * TR;  // the workgroup's keys sw .. sw + TR - 1
    // the chunk's query rows t_lo .. t_hi-1 (rows before sw see none of these keys)
    const int t_lo = max(wi.chunk * p.R * TR, sw), t_hi = min((wi.chunk + 1) * p.R * TR, L);
    if (t_lo >= t_hi) return;                         // whole workgroup (sw >= L included)
    const int s0 = sw + 16 * RW * w;  // this wave's keys s0 .. s0 + 16 RW - 1
    const int kh = h / (p.H / p.N);
    const uint8_t* kr[RW];
    Frag<DT> kf[RW];
#pragma unroll
    for (int kk = 0; kk < RW; ++kk) {
        const int sk = s0 + 16 * kk;
        kr[kk] = sk < L ? key_row(p, b, sk, kh, es) : nullptr;
        if (kr[kk] != nullptr) load_frag<DT>(kf[kk], kr[kk] + size_t(min(r, L - 1 - sk)) * p.N * D * es, j);
    }
    const float* lse = p.lse + (size_t(b) * p.H + h) * p.max_len;
    float acc[RW][4];  // keys s0 + 16 kk + 4j + i, partial over this lane's query column
#pragma unroll
    for (int kk = 0; kk < RW; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[kk][i] = 0.f;
    // query tile t0: 16 rows of head h (rows past L repeat the last row, masked) and their lse
    auto fetch = [&](int t0, u32x4 (&v)[Tile<DT>::kPerThread], float& lv) {
        tile_fetch<DT>(v, p.q + ((size_t(b) * p.max_len + t0) * p.H + h) * size_t(D * es), unsigned(p.H) * D * es,
                       L - 1 - t0);
        lv = (threadIdx.x < 16 && t0 + int(threadIdx.x) < L) ? lse[t0 + threadIdx.x] : 0.f;
    };
    // key tile kk's weights 2^(x - lse_t) for this lane's 4 keys and query row t; tiles whose
    // 16 rows follow all of the key tile's keys and end before L (all) skip the mask
    auto upd = [&](const attn::f32x4& c, int kk, int t, float lt, bool all) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = s0 + 16 * kk + 4 * j + i;
            const float wgt = exp2_hw(c[i] * p.scale2 - lt);
            acc[kk][i] += (all || (t >= s && t < L)) ? wgt : 0.f;
        }
    };
    auto upd_tile = [&](const attn::f32x4& c, int kk, int t0q, float lt) {
        if (t0q >= s0 + 16 * kk + 15 && t0q + 15 < L) upd(c, kk, t0q + r, lt, true);
        else upd(c, kk, t0q + r, lt, false);
    };
    // as in the row pass: two query tiles per barrier, four LDS buffers
    auto step2 = [&](int t0, int bi, u32x4 (&va)[Tile<DT>::kPerThread], float& la, u32x4 (&vb)[Tile<DT>::kPerThread],
                     float& lb, bool hb) {
        tile_store<DT>(qt[bi], va);
        tile_store<DT>(qt[bi + 1], vb);
        if (threadIdx.x < 16) {
            lt_s[bi][threadIdx.x] = la;
            lt_s[bi + 1][threadIdx.x] = lb;
        }
        __syncthreads();
        if (t0 + 32 < t_hi) fetch(t0 + 32, va, la);
        if (t0 + 48 < t_hi) fetch(t0 + 48, vb, lb);
        // query tile qq of the pair is needed by key tile kk if it was stored, the key tile
        // has its fragment, and the query tile holds a row at or after the key tile's first key
        bool nd[2][RW];
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int kk = 0; kk < RW; ++kk)
                nd[qq][kk] = (qq == 0 || hb) && kr[kk] != nullptr && t0 + 16 * qq + 15 >= s0 + 16 * kk;
        if constexpr (RW == 1) {
            if (nd[0][0] && nd[1][0]) {
                Frag<DT> q0, q1;
                frag_from_tile<DT>(q0, qt[bi], r, j);
                frag_from_tile<DT>(q1, qt[bi + 1], r, j);
                attn::f32x4 r0, r1;
                dot_tile2<DT>(kf[0], q0, q1, r0, r1);
                upd_tile(r0, 0, t0, lt_s[bi][r]);
                upd_tile(r1, 0, t0 + 16, lt_s[bi + 1][r]);
            } else if (nd[0][0] || nd[1][0]) {
                const int bx = nd[0][0] ? bi : bi + 1;
                Frag<DT> qf;
                frag_from_tile<DT>(qf, qt[bx], r, j);
                upd_tile(dot_tile<DT>(kf[0], qf), 0, nd[0][0] ? t0 : t0 + 16, lt_s[bx][r]);
            }
        } else {
            // each query fragment read from LDS feeds both key tiles
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                if (!nd[qq][0] && !nd[qq][1]) continue;
                Frag<DT> qf;
                frag_from_tile<DT>(qf, qt[bi + qq], r, j);
                const float lt = lt_s[bi + qq][r];
                const int tq = t0 + 16 * qq;
                if (nd[qq][0] && nd[qq][1]) {
                    attn::f32x4 r0, r1;
                    dot_tile2a<DT>(kf[0], kf[1], qf, r0, r1);
                    upd_tile(r0, 0, tq, lt);
                    upd_tile(r1, 1, tq, lt);
                } else if (nd[qq][0]) {  // constant tile indices keep acc and kf in registers
                    upd_tile(dot_tile<DT>(kf[0], qf), 0, tq, lt);
                } else {
                    upd_tile(dot_tile<DT>(kf[1], qf), 1, tq, lt);
                }
            }
        }
    };
    u32x4 na[Tile<DT>::kPerThread] = {}, nb[Tile<DT>::kPerThread] = {};
    float la = 0.f, lb = 0.f;
    fetch(t_lo, na, la);
    if (t_lo + 16 < t_hi) fetch(t_lo + 16, nb, lb);
    for (int t0 = t_lo, buf = 0; t0 < t_hi; t0 += 32, buf ^= 2) step2(t0, buf, na, la, nb, lb, t0 + 16 < t_hi);
    const size_t o = ((size_t(wi.chunk) * p.B + b) * p.H + h) * p.max_len;
#pragma unroll
    for (int kk = 0; kk < RW; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float tot = group_sum<16>(acc[kk][i]);
            const int s = s0 + 16 * kk + 4 * j + i;
            if (r == 0 && s < L) p.cpart[o + s] = tot;
        }
    }
}

// Column sums from the stored scores (fp32 path): work item (16-key tile kt, head, request),
// longest items (first key tiles) first through the snake order. Wave w takes the tile's
// row blocks w, w + 4, ...; a lane takes key column c = lane / 4 and rows 4q .. 4q + 3 of
// each block (q = lane % 4): one non-temporal 16-byte load of scores (read once), the
// block's 16 row normalisers loaded by lanes 0..15 and handed out by lane shuffles, adding
// 2^(x - lse_t) for rows t < L (masked scores are -inf and add 0). The four lanes of a key,
// then the four waves, are added in a fixed order: deterministic.
__global__ __launch_bounds__(kThreads) void imp_colS_kernel(ImpParams p) {
    constexpr int U = 8;  // blocks in flight per wave
    __shared__ float part[kThreads / 64][16];
    const int HB = p.H * p.B, rank = snake_rank();
    const int hb = rank % HB, kt = rank / HB;
    const int h = hb % p.H, b = hb / p.H;
    const int L = min(max(p.sl[b], 0), min(p.max_len, p.mkbpr * p.BS));
    const int s0 = kt * 16;
    if (s0 >= L) return;  // whole workgroup: keys past the prompt get no column sums
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane >> 2, q = lane & 3;
    // a key tile in a block whose table entry is out of range was skipped by the row pass
    // (never stored): its keys get no column sums, as in the recomputing column pass
    const int ph = p.bt[size_t(b) * p.mkbpr + unsigned(s0) / unsigned(p.BS)];
    const bool skipped = ph < 0 || ph >= p.num_kv_blocks;
    const int nrt = skipped ? 0 : (L - 1) / 16 - kt + 1;  // row tiles kt .. (L - 1) / 16
    const float* sb = p.S + ((size_t(b) * p.H + h) * p.sblocks + sblock(p.T16, kt, kt)) * 256 + c * 16 + 4 * q;
    const float* lse = p.lse + (size_t(b) * p.H + h) * p.max_len;
    float acc = 0.f;
    for (int it0 = w; it0 < nrt; it0 += 4 * U) {
        u32x4 x[U];
        float l16[U];  // lane l < 16: the normaliser of row l of the block
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int it = it0 + 4 * u;
            const bool in = it < nrt;
            x[u] = ld16_nt(sb + size_t(in ? it : 0) * 256);
            l16[u] = lse[min((kt + (in ? it : 0)) * 16 + (lane & 15), L - 1)];
        }
        float lt[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) lt[u][i] = __shfl(l16[u], 4 * q + i, kWave);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int it = it0 + 4 * u;
            const float xv[4] = {__uint_as_float(x[u].x), __uint_as_float(x[u].y), __uint_as_float(x[u].z),
                                 __uint_as_float(x[u].w)};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = (kt + it) * 16 + 4 * q + i;
                acc += (it < nrt && t < L) ? exp2_hw(xv[i] - lt[u][i]) : 0.f;
            }
        }
    }
    acc += __shfl_xor(acc, 1, kWave);
    acc += __shfl_xor(acc, 2, kWave);
    if (q == 0) part[w][c] = acc;
    __syncthreads();
    if (threadIdx.x < 16) {
        const int s = s0 + int(threadIdx.x);
        const float tot = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
        if (s < L) p.cpart[(size_t(b) * p.H + h) * p.max_len + s] = tot;
    }
}

// lse[t] = log2 of the sum over the key chunks of row t (chunks 0 .. (t / 64) / R, in
// chunk order) of sum * 2^max
__global__ __launch_bounds__(kThreads) void imp_merge_kernel(ImpParams p) {
    const int t = blockIdx.x * kThreads + threadIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int L = min(max(p.sl[b], 0), min(p.max_len, p.mkbpr * p.BS));
    if (t >= L) return;
    const size_t row = (size_t(b) * p.H + h) * p.max_len + t, cs = size_t(p.B) * p.H * p.max_len;
    const int nc = (t / p.TR) / p.R + 1;  // <= C <= kMaxChunks
    float mv[kMaxChunks], lv[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {  // all loads in flight at once
        mv[c] = c < nc ? p.mpart[c * cs + row] : -INFINITY;
        lv[c] = c < nc ? p.lpart[c * cs + row] : 0.f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) M = fmaxf(M, mv[c]);
    float S = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
        if (c < nc) S += lv[c] * exp2f(mv[c] - M);
    p.lse[row] = M + log2f(S);
}

// importance[b][s] = sum over heads of each head's column sum (its row chunks in chunk
// order), 0 for s >= L. Workgroup = 64 keys of one request; wave w takes heads w, w + 4,
// ... and the four partials are added in wave order (a fixed order: deterministic).
__global__ __launch_bounds__(kThreads) void imp_reduce_kernel(ImpParams p, float* importance, int stride,
                                                              float* head_importance) {
    static_assert(kThreads == 256, "four partials, added in wave order");
    __shared__ float part[kThreads / 64][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int s = blockIdx.x * 64 + lane, b = blockIdx.y;
    const int L = min(max(p.sl[b], 0), min(p.max_len, p.mkbpr * p.BS));
    // key s has the column sums of row chunks s / (TR R) .. those holding rows below L
    const int c_lo = (s / p.TR) / p.R, c_hi = (L + p.TR * p.R - 1) / (p.TR * p.R);
    const size_t cs = size_t(p.B) * p.H * p.max_len;
    float tot = 0.f;
    if (s < stride) {
        for (int h = w; h < p.H; h += kThreads / 64) {
            float v = 0.f;
            if (s < L) {
                const float* src = p.cpart + (size_t(b) * p.H + h) * p.max_len + s;
                float x[kMaxChunks];
#pragma unroll
                for (int c = 0; c < kMaxChunks; ++c) x[c] = (c >= c_lo && c < c_hi) ? src[c * cs] : 0.f;
#pragma unroll
                for (int c = 0; c < kMaxChunks; ++c) v += x[c];
            }
            tot += v;
            if (head_importance) head_importance[(size_t(b) * p.H + h) * stride + s] = v;
        }
    }
    part[w][lane] = tot;
    __syncthreads();
    if (w == 0 && s < stride && importance)
        importance[size_t(b) * stride + s] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

}  // namespace

namespace {
// the stored-score region of the fp32 path: 16 x 16 fp32 blocks of the causal lower
// triangle per (b, h), used when all of them fit in kScoreCap
constexpr size_t kScoreCap = size_t(2) << 30;
size_t score_bytes(int B, int H, int max_len) {
    const size_t t16 = (size_t(max(max_len, 0)) + 15) / 16;
    const size_t bytes = t16 * (t16 + 1) / 2 * 1024 * size_t(B) * size_t(H);
    return bytes <= kScoreCap ? bytes : 0;
}
}  // namespace

size_t prefill_importance_min_workspace_bytes(int B, int H, int max_len) {
    // the larger of the two splits: fp32 (64-row tiles, one chunk) and 16-bit (128-row tiles)
    const int C = max(imp_split(B, H, max_len, false, tile_rows<kF32>()).C,
                      imp_split(B, H, max_len, true, tile_rows<kBF16>()).C);
    size_t bytes = size_t(B) * H * max_len * sizeof(float) * (1 + 3 * size_t(C));
    bytes = (bytes + 255) & ~size_t(255);
    return bytes < 256 ? 256 : bytes;
}

size_t prefill_importance_workspace_bytes(int B, int H, int max_len) {
    return prefill_importance_min_workspace_bytes(B, H, max_len) + score_bytes(B, H, max_len);
}

hipError_t launch_prefill_importance(const ImportanceArgs& a, hipStream_t s) {
    float* ws = (float*)a.workspace;
    const int TR = a.dtype == kF32 ? tile_rows<kF32>() : tile_rows<kBF16>();
    const Split sp = imp_split(a.B, a.H, a.max_len, a.dtype != kF32, TR);
    const size_t plane = size_t(a.B) * a.H * a.max_len;
    const size_t min_bytes = prefill_importance_min_workspace_bytes(a.B, a.H, a.max_len);
    const size_t sbytes = score_bytes(a.B, a.H, a.max_len);
    // fp32 with room for the scores: store them in the row pass and read them back in the
    // column pass instead of recomputing Q K^T (the 16-bit passes recompute faster than the
    // scores stream)
    const bool stored = a.dtype == kF32 && sbytes > 0 && a.workspace_bytes >= min_bytes + sbytes;
    const int T16 = (a.max_len + 15) / 16;
    ImpParams p{(const uint8_t*)a.query, (const uint8_t*)a.k_cache, a.num_kv_blocks, a.block_tables, a.mkbpr,
                a.seq_lens, a.B, a.H, a.N, a.BS, a.max_len, a.scale * kLog2e, TR, sp.T, sp.R, sp.C,
                ws, ws + plane, ws + plane * (1 + sp.C), ws + plane * (1 + 2 * size_t(sp.C)),
                stored ? (float*)((uint8_t*)a.workspace + min_bytes) : nullptr, T16,
                size_t(T16) * (T16 + 1) / 2};
    if (a.max_len > 0) {
        const long hb = long(a.H) * a.B;
        const dim3 rgrid(unsigned(row_items(sp) * hb)), cgrid(unsigned(col_items(sp) * hb));
        const dim3 mgrid(unsigned((a.max_len + kThreads - 1) / kThreads), unsigned(a.H), unsigned(a.B));
        if (a.dtype == kBF16) hipLaunchKernelGGL(imp_row_kernel<kBF16>, rgrid, dim3(kThreads), 0, s, p);
        else if (a.dtype == kF16) hipLaunchKernelGGL(imp_row_kernel<kF16>, rgrid, dim3(kThreads), 0, s, p);
        else if (stored) hipLaunchKernelGGL((imp_row_kernel<kF32, true>), rgrid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL(imp_row_kernel<kF32>, rgrid, dim3(kThreads), 0, s, p);
        if (sp.C > 1) hipLaunchKernelGGL(imp_merge_kernel, mgrid, dim3(kThreads), 0, s, p);
        if (a.dtype == kBF16) hipLaunchKernelGGL(imp_col_kernel<kBF16>, cgrid, dim3(kThreads), 0, s, p);
        else if (a.dtype == kF16) hipLaunchKernelGGL(imp_col_kernel<kF16>, cgrid, dim3(kThreads), 0, s, p);
        else if (stored) hipLaunchKernelGGL(imp_colS_kernel, dim3(unsigned(long(T16) * hb)), dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL(imp_col_kernel<kF32>, cgrid, dim3(kThreads), 0, s, p);
    }
    hipLaunchKernelGGL(imp_reduce_kernel, dim3(unsigned((a.stride + 63) / 64), unsigned(a.B)),
                       dim3(kThreads), 0, s, p, a.importance, a.stride, a.head_importance);
    return hipGetLastError();
}

}  // namespace qs

// qsparse_abi.hip -- the C ABI: argument validation, workspace sizing, launches.
//
// Every check that the host can make happens before the first HIP call, so invalid
// calls return QS_ERR_INVALID / QS_ERR_UNSUPPORTED without touching the device.
// Compiled with QS_CHECKED (libqsparse_checked.so), every call also checks the
// device-resident tables it will use, synchronously, before its own kernels run.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/qsparse.h"
#include "qs_check.h"
#include "qs_internal.h"

namespace {

thread_local char g_err[512] = "";

qs_status fail(qs_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

qs_status ok() {
    g_err[0] = '\0';
    return QS_OK;
}

qs_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(QS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

constexpr int kMaxGrid = 65535;

bool block_size_ok(int bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128; }

// shared size checks; returns QS_OK or an error with the message set
qs_status check_dims(const char* fn, int32_t B, int32_t H, int32_t N, int32_t D, int32_t BS) {
    if (B < 0 || B > kMaxGrid) return fail(QS_ERR_INVALID, "%s: B=%d out of range [0, %d]", fn, B, kMaxGrid);
    if (N < 1 || N > kMaxGrid) return fail(QS_ERR_INVALID, "%s: N=%d must be in [1, %d]", fn, N, kMaxGrid);
    if (H < N || H % N != 0) return fail(QS_ERR_INVALID, "%s: H=%d must be a positive multiple of N=%d", fn, H, N);
    if (D != 128) return fail(QS_ERR_UNSUPPORTED, "%s: only D=128 is implemented (got %d)", fn, D);
    if (!block_size_ok(BS)) return fail(QS_ERR_UNSUPPORTED, "%s: block_size must be 16, 32, 64 or 128 (got %d)", fn, BS);
    return QS_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#ifdef QS_CHECKED
constexpr bool kChecked = true;
#else
constexpr bool kChecked = false;
#endif

// The checked build's device-input check: runs the check kernel on the call's stream, waits
// for it and turns its report into QS_ERR_INVALID with a message naming the first bad entry.
// `word` is device memory for the check's verdict; NULL allocates (and frees) one word.
qs_status device_check(const char* fn, qs::CheckArgs c, hipStream_t s, unsigned long long* word = nullptr) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return hip_status(e, fn);
    if (cs != hipStreamCaptureStatusNone)
        return fail(QS_ERR_UNSUPPORTED, "%s: the checked build waits for its check and cannot be captured", fn);
    unsigned long long* d = word;
    if (!d) e = hipMalloc(reinterpret_cast<void**>(&d), sizeof *d);
    if (e != hipSuccess) return hip_status(e, fn);
    unsigned long long h = ~0ull;
    e = hipMemcpyAsync(d, &h, sizeof h, hipMemcpyHostToDevice, s);
    c.out = d;
    if (e == hipSuccess) e = qs::launch_check(c, s);
    if (e == hipSuccess) e = hipMemcpyAsync(&h, d, sizeof h, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    const hipError_t ef = word ? hipSuccess : hipFree(d);
    if (e == hipSuccess) e = ef;
    if (e != hipSuccess) return hip_status(e, fn);
    if (h == ~0ull) return QS_OK;
    const int b = int(h >> 43), rule = int((h >> 40) & 7u);
    const long long pos = (long long)(h & ((1ull << 40) - 1));
    const int32_t* src = rule == qs::kBadBlockTable ? c.bt + (size_t)b * c.mkbpr + pos
                         : rule == qs::kBadMetaTable ? c.mt + (size_t)b * c.mmbpr + pos
                                                     : c.seq_lens + b;
    int32_t v = 0;
    e = hipMemcpyAsync(&v, src, sizeof v, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, fn);
    switch (rule) {
        case qs::kLenPastMaxLen:
            return fail(QS_ERR_INVALID, "%s: seq_lens[%d] = %d exceeds max_len = %d", fn, b, v, c.max_len);
        case qs::kLenPastBlockTable:
            return fail(QS_ERR_INVALID, "%s: seq_lens[%d] = %d needs more than max_kv_blocks_per_req = %d blocks",
                        fn, b, v, c.mkbpr);
        case qs::kLenPastMetaTable:
            return fail(QS_ERR_INVALID,
                        "%s: seq_lens[%d] = %d needs more than max_meta_blocks_per_req = %d metadata blocks", fn, b,
                        v, c.mmbpr);
        case qs::kBadBlockTable:
            return fail(QS_ERR_INVALID, "%s: block_tables[%d][%lld] = %d is outside [0, num_kv_blocks = %d)", fn, b,
                        pos, v, c.nkv);
        default:
            return fail(QS_ERR_INVALID,
                        "%s: metadata_block_tables[%d][%lld] = %d is outside [0, num_meta_blocks = %d)", fn, b, pos,
                        v, c.nmeta);
    }
}

// Scratch of qs_select_attn_decode_static: a static device array (each GPU the library runs
// on holds its own copy until the process ends), QS_STATIC_SCRATCH_BYTES of workspace and
// 256 bytes for the checked build's verdict word. Host code never uses the array's name
// as an address: its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchTotal = QS_STATIC_SCRATCH_BYTES + 256;
__device__ __align__(256) uint8_t scratch[kScratchTotal];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the device's first call).
qs_status static_scratch(const char* fn, uint8_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, fn);
    if (dev < 0 || dev >= kMaxDevices) return fail(QS_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, fn);
        if (!p) return fail(QS_ERR_HIP, "%s: no device address for the static scratch", fn);
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<uint8_t*>(g_scratch_ptr[dev]);
    return QS_OK;
}

qs::CheckArgs check_args(int B, int BS, uint32_t rules, const int32_t* seq_lens) {
    qs::CheckArgs c{};
    c.B = B;
    c.BS = BS;
    c.rules = rules;
    c.seq_lens = seq_lens;
    return c;
}

}  // namespace

extern "C" {

const char* qs_last_error(void) { return g_err; }

const char* qs_version(void) { return kChecked ? "qsparse 0.1 (gfx950, checked)" : "qsparse 0.1 (gfx950)"; }

int32_t qs_checked_build(void) { return kChecked ? 1 : 0; }

qs_status qs_build_metadata(int32_t B, int32_t N, int32_t D, int32_t block_size, qs_dtype kv_dtype,
                            const void* k_cache, int32_t num_kv_blocks, const int32_t* block_tables,
                            int32_t max_kv_blocks_per_req, const int32_t* seq_lens,
                            const int32_t* metadata_block_tables, int32_t max_meta_blocks_per_req, void* maxblocks,
                            void* minblocks, int32_t num_meta_blocks, void* stream) {
    const char* fn = "qs_build_metadata";
    qs_status st = check_dims(fn, B, N, N, D, block_size);
    if (st != QS_OK) return st;
    if (kv_dtype != QS_F32 && kv_dtype != QS_BF16 && kv_dtype != QS_F16)
        return fail(QS_ERR_UNSUPPORTED, "%s: kv_dtype must be QS_F32, QS_BF16 or QS_F16", fn);
    if (!k_cache || !block_tables || !seq_lens || !metadata_block_tables || !maxblocks || !minblocks)
        return fail(QS_ERR_INVALID, "%s: null pointer argument", fn);
    if (!aligned16(k_cache) || !aligned16(maxblocks) || !aligned16(minblocks))
        return fail(QS_ERR_INVALID, "%s: k_cache, maxblocks and minblocks must be 16-byte aligned", fn);
    if (num_kv_blocks < 1 || num_meta_blocks < 1 || max_kv_blocks_per_req < 1 || max_meta_blocks_per_req < 1)
        return fail(QS_ERR_INVALID, "%s: block counts and table widths must be >= 1", fn);
    if ((long long)max_meta_blocks_per_req * block_size > 0x7fffffffLL)
        return fail(QS_ERR_INVALID, "%s: max_meta_blocks_per_req * block_size overflows", fn);
    if (B == 0) return ok();
    if (kChecked) {
        qs::CheckArgs c = check_args(B, block_size, qs::kRuleNbWithinBt | qs::kRuleNbWithinMt | qs::kRuleBtUsed |
                                                        qs::kRuleMtUsed, seq_lens);
        c.bt = block_tables, c.mkbpr = max_kv_blocks_per_req, c.nkv = num_kv_blocks;
        c.mt = metadata_block_tables, c.mmbpr = max_meta_blocks_per_req, c.nmeta = num_meta_blocks;
        if ((st = device_check(fn, c, (hipStream_t)stream)) != QS_OK) return st;
    }
    qs::MetaArgs a{B, N, D, block_size, kv_dtype != QS_F32, k_cache, num_kv_blocks, block_tables,
                   max_kv_blocks_per_req, seq_lens, metadata_block_tables, max_meta_blocks_per_req,
                   maxblocks, minblocks, num_meta_blocks};
    return hip_status(qs::launch_build_metadata(a, (hipStream_t)stream), fn);
}

qs_status qs_update_metadata(int32_t B, int32_t N, int32_t D, int32_t block_size, qs_dtype kv_dtype,
                             const void* k_cache, int32_t num_kv_blocks, const int32_t* block_tables,
                             int32_t max_kv_blocks_per_req, const int32_t* seq_lens, const int32_t* first_block,
                             int32_t max_new_blocks, const int32_t* metadata_block_tables,
                             int32_t max_meta_blocks_per_req, void* maxblocks, void* minblocks,
                             int32_t num_meta_blocks, void* stream) {
    const char* fn = "qs_update_metadata";
    qs_status st = check_dims(fn, B, N, N, D, block_size);
    if (st != QS_OK) return st;
    if (kv_dtype != QS_F32 && kv_dtype != QS_BF16 && kv_dtype != QS_F16)
        return fail(QS_ERR_UNSUPPORTED, "%s: kv_dtype must be QS_F32, QS_BF16 or QS_F16", fn);
    if (!k_cache || !block_tables || !seq_lens || !first_block || !metadata_block_tables || !maxblocks ||
        !minblocks)
        return fail(QS_ERR_INVALID, "%s: null pointer argument", fn);
    if (!aligned16(k_cache) || !aligned16(maxblocks) || !aligned16(minblocks))
        return fail(QS_ERR_INVALID, "%s: k_cache, maxblocks and minblocks must be 16-byte aligned", fn);
    if (num_kv_blocks < 1 || num_meta_blocks < 1 || max_kv_blocks_per_req < 1 || max_meta_blocks_per_req < 1)
        return fail(QS_ERR_INVALID, "%s: block counts and table widths must be >= 1", fn);
    if (max_new_blocks < 1) return fail(QS_ERR_INVALID, "%s: max_new_blocks=%d must be >= 1", fn, max_new_blocks);
    if ((long long)max_meta_blocks_per_req * block_size > 0x7fffffffLL)
        return fail(QS_ERR_INVALID, "%s: max_meta_blocks_per_req * block_size overflows", fn);
    if (B == 0) return ok();
    if (kChecked) {
        qs::CheckArgs c = check_args(B, block_size, qs::kRuleNbWithinBt | qs::kRuleNbWithinMt | qs::kRuleBtUsed |
                                                        qs::kRuleMtUsed, seq_lens);
        c.bt = block_tables, c.mkbpr = max_kv_blocks_per_req, c.nkv = num_kv_blocks;
        c.mt = metadata_block_tables, c.mmbpr = max_meta_blocks_per_req, c.nmeta = num_meta_blocks;
        c.first_block = first_block, c.max_new = max_new_blocks;
        if ((st = device_check(fn, c, (hipStream_t)stream)) != QS_OK) return st;
    }
    qs::MetaArgs a{B, N, D, block_size, kv_dtype != QS_F32, k_cache, num_kv_blocks, block_tables,
                   max_kv_blocks_per_req, seq_lens, metadata_block_tables, max_meta_blocks_per_req,
                   maxblocks, minblocks, num_meta_blocks};
    return hip_status(qs::launch_update_metadata(a, first_block, max_new_blocks, (hipStream_t)stream), fn);
}

size_t qs_block_select_workspace_bytes(int32_t B, int32_t N, int32_t block_size, int32_t max_meta_blocks_per_req) {
    if (B < 0 || N < 1 || block_size < 1 || max_meta_blocks_per_req < 1) return 0;
    return qs::plan_block_select(B, N, block_size, max_meta_blocks_per_req).bytes;
}

qs_status qs_block_select(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size, qs_dtype dtype,
                          const void* query, const void* maxblocks, const void* minblocks, int32_t num_meta_blocks,
                          const int32_t* metadata_block_tables, int32_t max_meta_blocks_per_req,
                          const int32_t* seq_lens, const int32_t* tokens_since_update, uint32_t flags, int32_t k,
                          int32_t* selected, int32_t* n_selected, float* block_scores, void* workspace,
                          size_t workspace_bytes, void* stream) {
    const char* fn = "qs_block_select";
    qs_status st = check_dims(fn, B, H, N, D, block_size);
    if (st != QS_OK) return st;
    if (dtype != QS_F32 && dtype != QS_BF16 && dtype != QS_F16)
        return fail(QS_ERR_UNSUPPORTED, "%s: dtype must be QS_F32, QS_BF16 or QS_F16", fn);
    if (!query || !maxblocks || !minblocks || !metadata_block_tables || !seq_lens || !selected || !n_selected ||
        !workspace)
        return fail(QS_ERR_INVALID, "%s: null pointer argument", fn);
    if (!aligned16(query) || !aligned16(maxblocks) || !aligned16(minblocks))
        return fail(QS_ERR_INVALID, "%s: query, maxblocks and minblocks must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(QS_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
    if (flags & ~(uint32_t)(QS_FORCE_SINK | QS_FORCE_WINDOW))
        return fail(QS_ERR_INVALID, "%s: flags may only hold QS_FORCE_SINK | QS_FORCE_WINDOW", fn);
    if (k < 1) return fail(QS_ERR_INVALID, "%s: k=%d must be >= 1", fn, k);
    if (num_meta_blocks < 1 || max_meta_blocks_per_req < 1)
        return fail(QS_ERR_INVALID, "%s: num_meta_blocks and max_meta_blocks_per_req must be >= 1", fn);
    if ((long long)max_meta_blocks_per_req * block_size > (1LL << 24))
        return fail(QS_ERR_UNSUPPORTED, "%s: more than 2^24 blocks per request", fn);
    const qs::SelectPlan plan = qs::plan_block_select(B, N, block_size, max_meta_blocks_per_req);
    if (workspace_bytes < plan.bytes)
        return fail(QS_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, plan.bytes);
    if (B == 0) return ok();
    if (kChecked) {
        qs::CheckArgs c = check_args(B, block_size, qs::kRuleNbWithinMt | qs::kRuleMtUsed, seq_lens);
        c.mt = metadata_block_tables, c.mmbpr = max_meta_blocks_per_req, c.nmeta = num_meta_blocks;
        if ((st = device_check(fn, c, (hipStream_t)stream)) != QS_OK) return st;
    }
    qs::SelectArgs a{B, H, N, D, block_size, int(dtype), query, maxblocks, minblocks, num_meta_blocks,
                     metadata_block_tables, max_meta_blocks_per_req, seq_lens, tokens_since_update, flags, k,
                     selected, n_selected, block_scores, workspace};
    return hip_status(qs::launch_block_select(a, plan, (hipStream_t)stream), fn);
}

size_t qs_probe_select_workspace_bytes(int32_t B, int32_t H, int32_t max_kv_blocks_per_req) {
    if (B < 0 || H < 1 || max_kv_blocks_per_req < 1) return 0;
    return qs::probe_workspace_bytes(B, H, max_kv_blocks_per_req);
}

qs_status qs_probe_select(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size, qs_dtype q_dtype,
                          qs_dtype kv_dtype, const void* query, const void* k_cache, int32_t num_kv_blocks,
                          const int32_t* block_tables, int32_t max_kv_blocks_per_req, const int32_t* seq_lens,
                          const float* importance, int32_t importance_stride, int32_t n_probe, int32_t k,
                          uint32_t flags, int32_t* selected, int32_t* n_selected, float* probe_scores,
                          void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "qs_probe_select";
    qs_status st = check_dims(fn, B, H, N, D, block_size);
    if (st != QS_OK) return st;
    if (H > kMaxGrid) return fail(QS_ERR_INVALID, "%s: H=%d exceeds %d", fn, H, kMaxGrid);
    if ((q_dtype != QS_F32 && q_dtype != QS_BF16 && q_dtype != QS_F16) ||
        (kv_dtype != QS_F32 && kv_dtype != QS_BF16 && kv_dtype != QS_F16))
        return fail(QS_ERR_UNSUPPORTED, "%s: query and K must be QS_F32, QS_BF16 or QS_F16", fn);
    if (!query || !k_cache || !block_tables || !seq_lens || !selected || !n_selected || !workspace)
        return fail(QS_ERR_INVALID, "%s: null pointer argument", fn);
    if (!aligned16(k_cache)) return fail(QS_ERR_INVALID, "%s: k_cache must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(QS_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
    if (flags & ~(uint32_t)QS_RECENCY) return fail(QS_ERR_INVALID, "%s: flags may only hold QS_RECENCY", fn);
    if (k < 1) return fail(QS_ERR_INVALID, "%s: k=%d must be >= 1", fn, k);
    if (num_kv_blocks < 1 || max_kv_blocks_per_req < 1)
        return fail(QS_ERR_INVALID, "%s: num_kv_blocks and max_kv_blocks_per_req must be >= 1", fn);
    if (max_kv_blocks_per_req > qs::kProbeMaxBlocks)
        return fail(QS_ERR_UNSUPPORTED, "%s: max_kv_blocks_per_req=%d exceeds %d", fn, max_kv_blocks_per_req,
                    qs::kProbeMaxBlocks);
    if (importance && importance_stride < 1)
        return fail(QS_ERR_INVALID, "%s: importance_stride must be >= 1 when importance is given", fn);
    const size_t need = qs::probe_workspace_bytes(B, H, max_kv_blocks_per_req);
    if (workspace_bytes < need)
        return fail(QS_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    if (B == 0) return ok();
    if (kChecked) {
        qs::CheckArgs c = check_args(B, block_size, qs::kRuleNbWithinBt | qs::kRuleBtUsed, seq_lens);
        c.bt = block_tables, c.mkbpr = max_kv_blocks_per_req, c.nkv = num_kv_blocks;
        if ((st = device_check(fn, c, (hipStream_t)stream)) != QS_OK) return st;
    }
    qs::ProbeArgs a{B, H, N, D, block_size, int(q_dtype), int(kv_dtype), query, k_cache, num_kv_blocks,
                    block_tables, max_kv_blocks_per_req, seq_lens, importance, importance_stride, n_probe, k, flags,
                    selected, n_selected, probe_scores, workspace};
    return hip_status(qs::launch_probe_select(a, (hipStream_t)stream), fn);
}

size_t qs_sparse_attn_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D, int32_t sel_heads, int32_t k) {
    if (B < 0 || N < 1 || H < N || sel_heads < 1 || H % sel_heads != 0 || k < 1 || D < 1) return 0;
    // enough for either kernel family (matrix-core bf16 and vector-ALU)
    const size_t a = qs::plan_sparse_attn(B, H, N, D, sel_heads, k, QS_BF16, QS_BF16).bytes;
    const size_t b = qs::plan_sparse_attn(B, H, N, D, sel_heads, k, QS_F32, QS_F32).bytes;
    return a > b ? a : b;
}

qs_status qs_sparse_attn_decode(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size, qs_dtype q_dtype,
                                qs_dtype kv_dtype, const void* query, const void* k_cache, const void* v_cache,
                                const float* k_scale, const float* v_scale, int32_t num_kv_blocks,
                                const int32_t* block_tables, int32_t max_kv_blocks_per_req, const int32_t* seq_lens,
                                const int32_t* selected, const int32_t* n_selected, int32_t sel_heads, int32_t k,
                                float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
    const char* fn = "qs_sparse_attn_decode";
    qs_status st = check_dims(fn, B, H, N, D, block_size);
    if (st != QS_OK) return st;
    if (q_dtype != QS_F32 && q_dtype != QS_BF16 && q_dtype != QS_F16)
        return fail(QS_ERR_UNSUPPORTED, "%s: q_dtype must be QS_F32, QS_BF16 or QS_F16", fn);
    if (kv_dtype != QS_F32 && kv_dtype != QS_BF16 && kv_dtype != QS_I8 && kv_dtype != QS_F16)
        return fail(QS_ERR_UNSUPPORTED, "%s: kv_dtype must be QS_F32, QS_BF16, QS_F16 or QS_I8", fn);
    if (!query || !k_cache || !v_cache || !block_tables || !seq_lens || !selected || !n_selected || !out ||
        !workspace)
        return fail(QS_ERR_INVALID, "%s: null pointer argument", fn);
    if (kv_dtype == QS_I8 && (!k_scale || !v_scale))
        return fail(QS_ERR_INVALID, "%s: int8 KV needs k_scale and v_scale", fn);
    if (!aligned16(k_cache) || !aligned16(v_cache))
        return fail(QS_ERR_INVALID, "%s: k_cache and v_cache must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(QS_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
    if (sel_heads < N || sel_heads > H || sel_heads % N != 0 || H % sel_heads != 0)
        return fail(QS_ERR_INVALID, "%s: sel_heads=%d must satisfy N | sel_heads | H (N=%d, H=%d)", fn, sel_heads, N, H);
    if (sel_heads > kMaxGrid) return fail(QS_ERR_INVALID, "%s: sel_heads exceeds %d", fn, kMaxGrid);
    if (k < 1) return fail(QS_ERR_INVALID, "%s: k=%d must be >= 1", fn, k);
    if (num_kv_blocks < 1 || max_kv_blocks_per_req < 1)
        return fail(QS_ERR_INVALID, "%s: num_kv_blocks and max_kv_blocks_per_req must be >= 1", fn);
    if (!(softmax_scale == softmax_scale)) return fail(QS_ERR_INVALID, "%s: softmax_scale is NaN", fn);
    const qs::AttnPlan plan = qs::plan_sparse_attn(B, H, N, D, sel_heads, k, int(q_dtype), int(kv_dtype));
    if (workspace_bytes < plan.bytes)
        return fail(QS_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, plan.bytes);
    if ((long long)plan.splits * plan.hchunks > 0x7fffffffLL) return fail(QS_ERR_INVALID, "%s: grid too large", fn);
    if (B == 0) return ok();
    if (kChecked) {
        qs::CheckArgs c = check_args(B, block_size, qs::kRuleBtSelected, seq_lens);
        c.bt = block_tables, c.mkbpr = max_kv_blocks_per_req, c.nkv = num_kv_blocks;
        c.sel = selected, c.nsel = n_selected, c.rows = sel_heads, c.k = k;
        if ((st = device_check(fn, c, (hipStream_t)stream)) != QS_OK) return st;
    }
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(float(D));
    qs::AttnArgs a{B, H, N, D, block_size, int(q_dtype), int(kv_dtype), query, k_cache, v_cache, k_scale, v_scale,
                   num_kv_blocks, block_tables, max_kv_blocks_per_req, seq_lens, selected, n_selected, sel_heads, k,
                   scale, out, workspace};
    return hip_status(qs::launch_sparse_attn(a, plan, (hipStream_t)stream), fn);
}

size_t qs_select_attn_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t block_size,
                                      int32_t max_meta_blocks_per_req, int32_t k, qs_dtype dtype) {
    if (B < 0 || N < 1 || H < N || H % N != 0 || block_size < 1 || max_meta_blocks_per_req < 1 || k < 1 ||
        (dtype != QS_F32 && dtype != QS_BF16 && dtype != QS_F16))
        return 0;
    return qs::plan_select_attn(B, H, N, block_size, max_meta_blocks_per_req, k, int(dtype)).bytes;
}

}  // extern "C"

namespace {

// qs_select_attn_decode with its workspace given (`word`: the checked build's verdict word,
// NULL to allocate one). With static_ws the workspace is the static scratch: it is checked
// against QS_STATIC_SCRATCH_BYTES instead of workspace_bytes and named so in messages.
qs_status select_attn_impl(const char* fn, bool static_ws, int32_t B, int32_t H, int32_t N, int32_t D,
                           int32_t block_size, qs_dtype dtype, const void* query, const void* maxblocks,
                           const void* minblocks, int32_t num_meta_blocks, const int32_t* metadata_block_tables,
                           int32_t max_meta_blocks_per_req, const void* k_cache, const void* v_cache,
                           int32_t num_kv_blocks, const int32_t* block_tables, int32_t max_kv_blocks_per_req,
                           const int32_t* seq_lens, const int32_t* tokens_since_update, uint32_t flags, int32_t k,
                           float softmax_scale, void* out, int32_t* selected, int32_t* n_selected, void* workspace,
                           size_t workspace_bytes, void* stream, unsigned long long* word) {
    qs_status st = check_dims(fn, B, H, N, D, block_size);
    if (st != QS_OK) return st;
    if (dtype != QS_F32 && dtype != QS_BF16 && dtype != QS_F16)
        return fail(QS_ERR_UNSUPPORTED, "%s: dtype must be QS_F32, QS_BF16 or QS_F16", fn);
    if (!query || !maxblocks || !minblocks || !metadata_block_tables || !k_cache || !v_cache || !block_tables ||
        !seq_lens || !out || (!workspace && !static_ws))
        return fail(QS_ERR_INVALID, "%s: null pointer argument", fn);
    if ((selected == nullptr) != (n_selected == nullptr))
        return fail(QS_ERR_INVALID, "%s: selected and n_selected must both be given or both be NULL", fn);
    if (!aligned16(query) || !aligned16(maxblocks) || !aligned16(minblocks) || !aligned16(k_cache) ||
        !aligned16(v_cache))
        return fail(QS_ERR_INVALID, "%s: query, metadata and K/V caches must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(QS_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
    if (flags & ~(uint32_t)(QS_FORCE_SINK | QS_FORCE_WINDOW))
        return fail(QS_ERR_INVALID, "%s: flags may only hold QS_FORCE_SINK | QS_FORCE_WINDOW", fn);
    if (k < 1) return fail(QS_ERR_INVALID, "%s: k=%d must be >= 1", fn, k);
    if (num_meta_blocks < 1 || max_meta_blocks_per_req < 1 || num_kv_blocks < 1 || max_kv_blocks_per_req < 1)
        return fail(QS_ERR_INVALID, "%s: block counts and table widths must be >= 1", fn);
    if ((long long)max_meta_blocks_per_req * block_size > (1LL << 24))
        return fail(QS_ERR_UNSUPPORTED, "%s: more than 2^24 blocks per request", fn);
    if (!(softmax_scale == softmax_scale)) return fail(QS_ERR_INVALID, "%s: softmax_scale is NaN", fn);
    const qs::FusedPlan plan = qs::plan_select_attn(B, H, N, block_size, max_meta_blocks_per_req, k, int(dtype));
    if (static_ws && plan.bytes > QS_STATIC_SCRATCH_BYTES)
        return fail(QS_ERR_INVALID, "%s: these sizes need %zu bytes of scratch, the static scratch holds %zu", fn,
                    plan.bytes, (size_t)QS_STATIC_SCRATCH_BYTES);
    if (!static_ws && workspace_bytes < plan.bytes)
        return fail(QS_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, plan.bytes);
    if ((long long)plan.attn.splits * plan.attn.hchunks > 0x7fffffffLL)
        return fail(QS_ERR_INVALID, "%s: grid too large", fn);
    if (B == 0) return ok();
    if (static_ws) {
        uint8_t* base = nullptr;
        if ((st = static_scratch(fn, &base)) != QS_OK) return st;
        workspace = base;
        word = reinterpret_cast<unsigned long long*>(base + QS_STATIC_SCRATCH_BYTES);
    }
    if (kChecked) {
        qs::CheckArgs c = check_args(B, block_size, qs::kRuleNbWithinMt | qs::kRuleMtUsed | qs::kRuleBtUsed, seq_lens);
        c.bt = block_tables, c.mkbpr = max_kv_blocks_per_req, c.nkv = num_kv_blocks;
        c.mt = metadata_block_tables, c.mmbpr = max_meta_blocks_per_req, c.nmeta = num_meta_blocks;
        if ((st = device_check(fn, c, (hipStream_t)stream, word)) != QS_OK) return st;
    }
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(float(D));
    qs::SelectArgs sa{B, H, N, D, block_size, int(dtype), query, maxblocks, minblocks, num_meta_blocks,
                      metadata_block_tables, max_meta_blocks_per_req, seq_lens, tokens_since_update, flags, k,
                      selected, n_selected, nullptr, workspace};
    qs::AttnArgs aa{B, H, N, D, block_size, int(dtype), int(dtype), query, k_cache, v_cache, nullptr, nullptr,
                    num_kv_blocks, block_tables, max_kv_blocks_per_req, seq_lens, selected, n_selected, N, k,
                    scale, out, workspace};
    return hip_status(qs::launch_select_attn(sa, aa, plan, (hipStream_t)stream), fn);
}

}  // namespace

extern "C" {

qs_status qs_select_attn_decode(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size, qs_dtype dtype,
                                const void* query, const void* maxblocks, const void* minblocks,
                                int32_t num_meta_blocks, const int32_t* metadata_block_tables,
                                int32_t max_meta_blocks_per_req, const void* k_cache, const void* v_cache,
                                int32_t num_kv_blocks, const int32_t* block_tables, int32_t max_kv_blocks_per_req,
                                const int32_t* seq_lens, const int32_t* tokens_since_update, uint32_t flags,
                                int32_t k, float softmax_scale, void* out, int32_t* selected, int32_t* n_selected,
                                void* workspace, size_t workspace_bytes, void* stream) {
    return select_attn_impl("qs_select_attn_decode", false, B, H, N, D, block_size, dtype, query, maxblocks,
                            minblocks, num_meta_blocks, metadata_block_tables, max_meta_blocks_per_req, k_cache,
                            v_cache, num_kv_blocks, block_tables, max_kv_blocks_per_req, seq_lens,
                            tokens_since_update, flags, k, softmax_scale, out, selected, n_selected, workspace,
                            workspace_bytes, stream, nullptr);
}

qs_status qs_select_attn_decode_static(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size,
                                       qs_dtype dtype, const void* query, const void* maxblocks,
                                       const void* minblocks, int32_t num_meta_blocks,
                                       const int32_t* metadata_block_tables, int32_t max_meta_blocks_per_req,
                                       const void* k_cache, const void* v_cache, int32_t num_kv_blocks,
                                       const int32_t* block_tables, int32_t max_kv_blocks_per_req,
                                       const int32_t* seq_lens, const int32_t* tokens_since_update, uint32_t flags,
                                       int32_t k, float softmax_scale, void* out, int32_t* selected,
                                       int32_t* n_selected, void* stream) {
    return select_attn_impl("qs_select_attn_decode_static", true, B, H, N, D, block_size, dtype, query, maxblocks,
                            minblocks, num_meta_blocks, metadata_block_tables, max_meta_blocks_per_req, k_cache,
                            v_cache, num_kv_blocks, block_tables, max_kv_blocks_per_req, seq_lens,
                            tokens_since_update, flags, k, softmax_scale, out, selected, n_selected, nullptr, 0,
                            stream, nullptr);
}

size_t qs_probe_attn_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t max_kv_blocks_per_req, int32_t k) {
    if (B < 0 || N < 1 || H < N || H % N != 0 || max_kv_blocks_per_req < 1 || k < 1) return 0;
    return qs::plan_probe_attn(B, H, N, max_kv_blocks_per_req, k).bytes;
}

qs_status qs_probe_attn_decode(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size, qs_dtype q_dtype,
                               qs_dtype kv_dtype, const void* query, const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale, const void* probe_k_cache,
                               qs_dtype probe_k_dtype,
                               int32_t num_kv_blocks, const int32_t* block_tables, int32_t max_kv_blocks_per_req,
                               const int32_t* seq_lens, const float* importance, int32_t importance_stride,
                               int32_t n_probe, int32_t k, uint32_t flags, float softmax_scale, void* out,
                               int32_t* selected, int32_t* n_selected, void* workspace, size_t workspace_bytes,
                               void* stream) {
    const char* fn = "qs_probe_attn_decode";
    qs_status st = check_dims(fn, B, H, N, D, block_size);
    if (st != QS_OK) return st;
    if (H > kMaxGrid) return fail(QS_ERR_INVALID, "%s: H=%d exceeds %d", fn, H, kMaxGrid);
    const bool q8 = kv_dtype == QS_I8;
    if ((q_dtype != QS_F32 && q_dtype != QS_BF16 && q_dtype != QS_F16) ||
        (kv_dtype != QS_F32 && kv_dtype != QS_BF16 && kv_dtype != QS_F16 && !q8))
        return fail(QS_ERR_UNSUPPORTED, "%s: query must be QS_F32, QS_BF16 or QS_F16 and KV one of those or QS_I8",
                    fn);
    if (q8 && probe_k_dtype != QS_F32 && probe_k_dtype != QS_BF16 && probe_k_dtype != QS_F16)
        return fail(QS_ERR_UNSUPPORTED, "%s: probe_k_dtype must be QS_F32, QS_BF16 or QS_F16", fn);
    if (!query || !k_cache || !v_cache || !block_tables || !seq_lens || !out || !workspace)
        return fail(QS_ERR_INVALID, "%s: null pointer argument", fn);
    if (q8 && (!k_scale || !v_scale || !probe_k_cache))
        return fail(QS_ERR_INVALID, "%s: an int8 cache needs k_scale, v_scale and probe_k_cache", fn);
    if (!q8 && (k_scale || v_scale || probe_k_cache))
        return fail(QS_ERR_INVALID, "%s: k_scale, v_scale and probe_k_cache are for an int8 cache only", fn);
    if ((selected == nullptr) != (n_selected == nullptr))
        return fail(QS_ERR_INVALID, "%s: selected and n_selected must be given together", fn);
    if (!aligned16(k_cache) || !aligned16(v_cache) || (q8 && !aligned16(probe_k_cache)))
        return fail(QS_ERR_INVALID, "%s: k_cache, v_cache and probe_k_cache must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(QS_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
    if (flags & ~(uint32_t)QS_RECENCY) return fail(QS_ERR_INVALID, "%s: flags may only hold QS_RECENCY", fn);
    if (k < 1 || k > qs::kProbeMaxBlocks)
        return fail(QS_ERR_INVALID, "%s: k=%d must be in [1, %d]", fn, k, qs::kProbeMaxBlocks);
    if (num_kv_blocks < 1 || max_kv_blocks_per_req < 1)
        return fail(QS_ERR_INVALID, "%s: num_kv_blocks and max_kv_blocks_per_req must be >= 1", fn);
    if (max_kv_blocks_per_req > qs::kProbeMaxBlocks)
        return fail(QS_ERR_UNSUPPORTED, "%s: max_kv_blocks_per_req=%d exceeds %d", fn, max_kv_blocks_per_req,
                    qs::kProbeMaxBlocks);
    if (importance && importance_stride < 1)
        return fail(QS_ERR_INVALID, "%s: importance_stride must be >= 1 when importance is given", fn);
    if (!(softmax_scale == softmax_scale)) return fail(QS_ERR_INVALID, "%s: softmax_scale is NaN", fn);
    const qs::AttnPlan plan = qs::plan_probe_attn(B, H, N, max_kv_blocks_per_req, k);
    if (workspace_bytes < plan.bytes)
        return fail(QS_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, plan.bytes);
    if (B == 0) return ok();
    if (kChecked) {
        qs::CheckArgs c = check_args(B, block_size, qs::kRuleNbWithinBt | qs::kRuleBtUsed, seq_lens);
        c.bt = block_tables, c.mkbpr = max_kv_blocks_per_req, c.nkv = num_kv_blocks;
        if ((st = device_check(fn, c, (hipStream_t)stream)) != QS_OK) return st;
    }
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(float(D));
    qs::ProbeArgs pa{B, H, N, D, block_size, int(q_dtype), int(q8 ? probe_k_dtype : kv_dtype), query,
                     q8 ? probe_k_cache : k_cache, num_kv_blocks, block_tables, max_kv_blocks_per_req, seq_lens,
                     importance, importance_stride, n_probe, k, flags, selected, n_selected, nullptr, workspace};
    qs::AttnArgs ta{B, H, N, D, block_size, int(q_dtype), int(kv_dtype), query, k_cache, v_cache, k_scale, v_scale,
                    num_kv_blocks, block_tables, max_kv_blocks_per_req, seq_lens, nullptr, nullptr, H, k, scale, out,
                    workspace};
    return hip_status(qs::launch_probe_attn(pa, ta, plan, (hipStream_t)stream), fn);
}

size_t qs_prefill_importance_workspace_bytes(int32_t B, int32_t H, int32_t max_len) {
    if (B < 0 || H < 1 || max_len < 0) return 0;
    return qs::prefill_importance_workspace_bytes(B, H, max_len);
}

qs_status qs_prefill_importance(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block_size, qs_dtype dtype,
                                const void* query, int32_t max_len, const void* k_cache, int32_t num_kv_blocks,
                                const int32_t* block_tables, int32_t max_kv_blocks_per_req, const int32_t* seq_lens,
                                float softmax_scale, float* importance, int32_t importance_stride,
                                float* head_importance, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "qs_prefill_importance";
    qs_status st = check_dims(fn, B, H, N, D, block_size);
    if (st != QS_OK) return st;
    if (H > kMaxGrid) return fail(QS_ERR_INVALID, "%s: H=%d exceeds %d", fn, H, kMaxGrid);
    if (dtype != QS_F32 && dtype != QS_BF16 && dtype != QS_F16)
        return fail(QS_ERR_UNSUPPORTED, "%s: dtype must be QS_F32, QS_BF16 or QS_F16", fn);
    if (!query || !k_cache || !block_tables || !seq_lens || !workspace)
        return fail(QS_ERR_INVALID, "%s: null pointer argument", fn);
    if (!importance && !head_importance)
        return fail(QS_ERR_INVALID, "%s: importance and head_importance are both NULL", fn);
    if (!aligned16(query) || !aligned16(k_cache))
        return fail(QS_ERR_INVALID, "%s: query and k_cache must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(QS_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
    if (max_len < 0 || importance_stride < 1)
        return fail(QS_ERR_INVALID, "%s: max_len must be >= 0 and importance_stride >= 1", fn);
    if (num_kv_blocks < 1 || max_kv_blocks_per_req < 1)
        return fail(QS_ERR_INVALID, "%s: num_kv_blocks and max_kv_blocks_per_req must be >= 1", fn);
    if (!(softmax_scale == softmax_scale)) return fail(QS_ERR_INVALID, "%s: softmax_scale is NaN", fn);
    if ((long long)((max_len + 63) / 64) * H * B > 0x7fffffffLL)
        return fail(QS_ERR_INVALID, "%s: max_len * H * B too large for one grid", fn);
    const size_t need = qs::prefill_importance_min_workspace_bytes(B, H, max_len);
    if (workspace_bytes < need)
        return fail(QS_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    if (B == 0) return ok();
    if (kChecked) {
        qs::CheckArgs c = check_args(B, block_size, qs::kRuleLenWithinMax | qs::kRuleNbWithinBt | qs::kRuleBtUsed,
                                     seq_lens);
        c.bt = block_tables, c.mkbpr = max_kv_blocks_per_req, c.nkv = num_kv_blocks, c.max_len = max_len;
        if ((st = device_check(fn, c, (hipStream_t)stream)) != QS_OK) return st;
    }
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(float(D));
    qs::ImportanceArgs a{B, H, N, D, block_size, int(dtype), query, max_len, k_cache, num_kv_blocks, block_tables,
                         max_kv_blocks_per_req, seq_lens, scale, importance, importance_stride, head_importance,
                         workspace, workspace_bytes};
    return hip_status(qs::launch_prefill_importance(a, (hipStream_t)stream), fn);
}

}  // extern "C"

// qs_internal.h -- launchers behind the C ABI (host side, already-validated arguments).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qs {

// ---- metadata ----------------------------------------------------------------------
struct MetaArgs {
    int B, N, D, BS;
    bool bf16;  // any 16-bit float format (bf16 or f16): the reduction only orders bit patterns
    const void* k_cache;
    int num_kv_blocks;
    const int32_t* block_tables;
    int mkbpr;
    const int32_t* seq_lens;
    const int32_t* meta_tables;
    int mmbpr;
    void* maxb;
    void* minb;
    int num_meta;
};
hipError_t launch_build_metadata(const MetaArgs& a, hipStream_t s);
int update_col_slices(int B, int N, int D, bool bf16, int max_new_blocks);
hipError_t launch_update_metadata(const MetaArgs& a, const int32_t* first_block, int max_new_blocks,
                                  hipStream_t s);

// ---- Quest select ------------------------------------------------------------------
struct SelectPlan {
    bool row_mode;     // one workgroup per (request, KV head); else score grid + top-k kernel
    int chunk;         // blocks per scoring workgroup (split mode)
    int n_chunks;      // scoring workgroups per row (split mode)
    size_t lds_bytes;  // dynamic LDS of the row-mode / top-k kernel (scores kept on chip)
    size_t scores_off, bytes;
};
SelectPlan plan_block_select(int B, int N, int BS, int mmbpr);

struct SelectArgs {
    int B, H, N, D, BS;
    int dtype;  // qs_dtype of the query and metadata (F32, BF16 or F16)
    const void* query;
    const void* maxb;
    const void* minb;
    int num_meta;
    const int32_t* meta_tables;
    int mmbpr;
    const int32_t* seq_lens;
    const int32_t* tsmu;
    uint32_t flags;
    int k;
    int32_t* selected;
    int32_t* n_selected;
    float* block_scores;
    void* workspace;
};
hipError_t launch_block_select(const SelectArgs& a, const SelectPlan& p, hipStream_t s);
// the split-mode scoring grid alone: scores [B, N, mmbpr * BS] (forced blocks not written)
hipError_t launch_select_scores(const SelectArgs& a, const SelectPlan& p, float* scores, hipStream_t s);

// ---- probe select ------------------------------------------------------------------
constexpr int kProbeMaxBlocks = 4096;
struct ProbeArgs {
    int B, H, N, D, BS;
    int q_dtype, kv_dtype;  // F32, BF16 or F16
    const void* query;
    const void* k_cache;
    int num_kv_blocks;
    const int32_t* block_tables;
    int mkbpr;
    const int32_t* seq_lens;
    const float* importance;
    int imp_stride;
    int n_probe;
    int k;
    uint32_t flags;
    int32_t* selected;
    int32_t* n_selected;
    float* probe_scores;
    void* workspace;  // B * H * mkbpr probe keys
};
size_t probe_workspace_bytes(int B, int H, int mkbpr);
hipError_t launch_probe_select(const ProbeArgs& a, hipStream_t s);

// ---- sparse attention --------------------------------------------------------------
struct AttnPlan {
    bool mfma;        // bf16 matrix-core kernel (bf16 query and KV)
    int hpr;          // query heads per selection row
    int hc;           // head capacity of one workgroup (1, 2, 4, 8; 16 for the MFMA kernel)
    int hchunks;      // workgroups across a row's heads
    int splits;       // workgroups across a row's selection slots (1 = no combine pass)
    int spb;          // selection slots per split
    size_t part_off, bytes;
};
AttnPlan plan_sparse_attn(int B, int H, int N, int D, int sel_heads, int k, int q_dtype, int kv_dtype);

struct AttnArgs {
    int B, H, N, D, BS;
    int q_dtype, kv_dtype;  // qs_dtype values
    const void* query;
    const void* k_cache;
    const void* v_cache;
    const float* k_scale;
    const float* v_scale;
    int num_kv_blocks;
    const int32_t* block_tables;
    int mkbpr;
    const int32_t* seq_lens;
    const int32_t* selected;
    const int32_t* n_selected;
    int sel_heads;
    int k;
    float scale;
    void* out;
    void* workspace;
};
hipError_t launch_sparse_attn(const AttnArgs& a, const AttnPlan& p, hipStream_t s);

// ---- fused probe selection + attention ----------------------------------------------
// One row per query head on the vector ALU; the workspace holds the probe keys, then the
// attention partials at part_off (bytes in total).
AttnPlan plan_probe_attn(int B, int H, int N, int mkbpr, int k);
hipError_t launch_probe_attn(const ProbeArgs& a, const AttnArgs& t, const AttnPlan& p, hipStream_t s);

// ---- prefill importance -------------------------------------------------------------
struct ImportanceArgs {
    int B, H, N, D, BS;
    int dtype;  // F32, BF16 or F16 (query and K)
    const void* query;  // [B, max_len, H, D]
    int max_len;
    const void* k_cache;
    int num_kv_blocks;
    const int32_t* block_tables;
    int mkbpr;
    const int32_t* seq_lens;
    float scale;
    float* importance;       // [B, stride] or null
    int stride;
    float* head_importance;  // [B, H, stride] or null
    void* workspace;
    size_t workspace_bytes;  // at least the minimum; the full size lets fp32 store its scores
};
// the two-pass workspace, and the full one (plus the fp32 path's stored scores when they fit)
size_t prefill_importance_min_workspace_bytes(int B, int H, int max_len);
size_t prefill_importance_workspace_bytes(int B, int H, int max_len);
hipError_t launch_prefill_importance(const ImportanceArgs& a, hipStream_t s);

// ---- fused select + attention -------------------------------------------------------
struct FusedPlan {
    // kOneKernel: each workgroup scores its row into LDS, selects and attends;
    // kPrescored: a scoring grid writes the scores, then each attention workgroup selects
    // from them in LDS and attends; kSeparate: the two operations' kernels
    enum Mode { kOneKernel, kPrescored, kSeparate } mode;
    SelectPlan sel;
    AttnPlan attn;
    size_t sel_off, attn_off, idx_off, nidx_off, bytes;  // workspace regions
};
FusedPlan plan_select_attn(int B, int H, int N, int BS, int mmbpr, int k, int dtype);
hipError_t launch_select_attn(const SelectArgs& s, const AttnArgs& a, const FusedPlan& p, hipStream_t st);

}  // namespace qs

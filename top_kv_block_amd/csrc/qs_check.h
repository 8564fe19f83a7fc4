// qs_check.h -- the device-input check of the checked build (see check.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qs {

// rules a call asks for (bit set)
enum : uint32_t {
    kRuleNbWithinBt = 1u,     // ceil(L / BS) <= max_kv_blocks_per_req
    kRuleNbWithinMt = 2u,     // ceil(ceil(L / BS) / BS) <= max_meta_blocks_per_req
    kRuleLenWithinMax = 4u,   // L <= max_len
    kRuleBtUsed = 8u,         // block_tables entries of the used blocks in [0, num_kv_blocks)
    kRuleMtUsed = 16u,        // metadata_block_tables entries of the used blocks in [0, num_meta_blocks)
    kRuleBtSelected = 32u,    // block_tables entries of the selected blocks in [0, num_kv_blocks)
};

// what a report names, in reporting order within one request
enum : int {
    kLenPastMaxLen = 0,
    kLenPastBlockTable = 1,
    kLenPastMetaTable = 2,
    kBadBlockTable = 3,
    kBadMetaTable = 4,
};

struct CheckArgs {
    int B, BS;
    uint32_t rules;
    const int32_t* seq_lens;            // [B]; negative counts as 0
    const int32_t* bt;                  // [B, mkbpr] or null when no block_tables rule
    int mkbpr, nkv;
    const int32_t* mt;                  // [B, mmbpr] or null when no metadata-table rule
    int mmbpr, nmeta;
    int max_len;                        // kRuleLenWithinMax
    const int32_t* first_block;         // [B] or null: used blocks are a refresh's range
    int max_new;
    const int32_t* sel;                 // [B, rows, k] (kRuleBtSelected)
    const int32_t* nsel;                // [B, rows]
    int rows, k;
    unsigned long long* out;            // one word, ~0 on entry; the smallest report key on exit
};

hipError_t launch_check(const CheckArgs& a, hipStream_t s);

}  // namespace qs

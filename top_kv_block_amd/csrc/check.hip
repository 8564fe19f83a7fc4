// check.hip -- validation of the device-resident inputs (sequence lengths, block tables,
// metadata tables, selections) for the checked build of the library.
//
// The kernels of every call skip a table entry that is out of range, so a bad table never
// faults; but a skipped block silently changes the result. The checked build runs this
// kernel before a call's own kernels and refuses the call when any entry the call would
// use is out of range, naming the first such entry (lowest request, then the rule order
// below, then the lowest position). One workgroup per request; each reads only inside the
// shapes the host validated, whatever the values it finds.
#include <hip/hip_runtime.h>

#include "qs_check.h"

namespace qs {
namespace {

constexpr int kThreads = 256;

// packed report key: request (16 bits) | rule (3 bits) | position (40 bits); smaller is first
__device__ __forceinline__ unsigned long long report_key(int b, int rule, long long pos) {
    return (static_cast<unsigned long long>(b) << 43) | (static_cast<unsigned long long>(rule) << 40) |
           static_cast<unsigned long long>(pos);
}

__device__ __forceinline__ bool out_of(int32_t v, int n) { return v < 0 || v >= n; }

__global__ __launch_bounds__(kThreads) void check_kernel(CheckArgs a) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    int32_t L = a.seq_lens[b];
    if (L < 0) L = 0;
    const int nb = L / a.BS + (L % a.BS != 0 ? 1 : 0);  // no overflow near INT32_MAX
    unsigned long long best = ~0ull;

    if (tid == 0) {
        if ((a.rules & kRuleLenWithinMax) && L > a.max_len) best = min(best, report_key(b, kLenPastMaxLen, 0));
        if ((a.rules & kRuleNbWithinBt) && nb > a.mkbpr) best = min(best, report_key(b, kLenPastBlockTable, 0));
        if ((a.rules & kRuleNbWithinMt) && (nb / a.BS + (nb % a.BS != 0 ? 1 : 0)) > a.mmbpr)
            best = min(best, report_key(b, kLenPastMetaTable, 0));
    }

    // the sequence blocks whose entries the call uses: all of them, or a refresh's range
    long long i_lo = 0, i_hi = nb;
    if (a.first_block) {
        i_lo = a.first_block[b] > 0 ? a.first_block[b] : 0;
        i_hi = min(static_cast<long long>(nb), i_lo + a.max_new);
    }
    if (a.rules & kRuleBtUsed) {
        const long long hi = min(i_hi, static_cast<long long>(a.mkbpr));
        const int32_t* row = a.bt + static_cast<size_t>(b) * a.mkbpr;
        for (long long i = i_lo + tid; i < hi; i += kThreads)
            if (out_of(row[i], a.nkv)) best = min(best, report_key(b, kBadBlockTable, i));
    }
    if ((a.rules & kRuleMtUsed) && i_lo < i_hi) {
        const long long j_lo = i_lo / a.BS;
        const long long j_hi = min((i_hi - 1) / a.BS + 1, static_cast<long long>(a.mmbpr));
        const int32_t* row = a.mt + static_cast<size_t>(b) * a.mmbpr;
        for (long long j = j_lo + tid; j < j_hi; j += kThreads)
            if (out_of(row[j], a.nmeta)) best = min(best, report_key(b, kBadMetaTable, j));
    }
    if (a.rules & kRuleBtSelected) {
        // every selected entry the attention reads: slots below the row's clamped count that
        // name one of the request's blocks (other entries are skipped by definition)
        const int lim = min(nb, a.mkbpr);
        const int32_t* row = a.bt + static_cast<size_t>(b) * a.mkbpr;
        const long long n = static_cast<long long>(a.rows) * a.k;
        for (long long e = tid; e < n; e += kThreads) {
            const long long r = e / a.k;
            const int j = static_cast<int>(e - r * a.k);
            int ns = a.nsel[static_cast<size_t>(b) * a.rows + r];
            ns = ns < 0 ? 0 : (ns > a.k ? a.k : ns);
            if (j >= ns) continue;
            const int32_t blk = a.sel[(static_cast<size_t>(b) * a.rows + r) * a.k + j];
            if (blk < 0 || blk >= lim) continue;
            if (out_of(row[blk], a.nkv)) best = min(best, report_key(b, kBadBlockTable, blk));
        }
    }
    if (best != ~0ull) atomicMin(a.out, best);
}

}  // namespace

hipError_t launch_check(const CheckArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(check_kernel, dim3(unsigned(a.B)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace qs

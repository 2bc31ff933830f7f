// gdn_prefill.hip -- the chunked prefill's varlen schedule and dispatch.
//
// The preparation and scan kernels are templates in gdn_prefill.hpp,
// instantiated per (element type, chunk size) in gdn_prefill_inst.hip. This
// file holds the one-workgroup schedule kernel for calls of more sequences
// than the preparation kernel locates by itself, and launch_prefill, which
// picks the instantiation.
#include "gdn_prefill.hpp"

namespace gdn {

// ---------------------------------------------------------------------------
// 1. Varlen schedule (one workgroup)
// ---------------------------------------------------------------------------

constexpr int kSchedThreads = 1024;
constexpr int kMaxRankedSeqs = 4096;

__device__ __forceinline__ int block_scan_incl(int x, int *s_tmp, bool use_max) {
    const int tid = threadIdx.x;
    s_tmp[tid] = x;
    __syncthreads();
    for (int off = 1; off < kSchedThreads; off <<= 1) {
        const int y = tid >= off ? s_tmp[tid - off] : (use_max ? INT32_MIN : 0);
        __syncthreads();
        s_tmp[tid] = use_max ? max(s_tmp[tid], y) : s_tmp[tid] + y;
        __syncthreads();
    }
    const int r = s_tmp[tid];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kSchedThreads) void gdn_schedule_kernel(
    const int32_t *__restrict__ cu, int32_t num_seqs, int32_t total_tokens, int32_t chunk,
    int32_t *__restrict__ bounds, int32_t *__restrict__ seq_chunk0, int32_t *__restrict__ order,
    int32_t *__restrict__ chunk_seq, int32_t *__restrict__ chunk_tok0, int32_t *__restrict__ counters)
{
    __shared__ int s_tmp[kSchedThreads];
    __shared__ int s_carry;
    __shared__ int s_len[kMaxRankedSeqs];
    const int tid = threadIdx.x;

    // bounds[j] = max over i <= j of clamp(cu[i], 0, T): sequences become
    // disjoint, ordered ranges inside [0, T) whatever the input holds.
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base <= num_seqs; base += kSchedThreads) {
        const int j = base + tid;
        int x = 0;
        if (j <= num_seqs) x = min(max(cu[j], 0), total_tokens);
        int pm = block_scan_incl(x, s_tmp, true);
        pm = max(pm, s_carry);
        if (j <= num_seqs) bounds[j] = pm;
        __syncthreads();
        if (tid == kSchedThreads - 1) s_carry = pm;
        __syncthreads();
    }
    __syncthreads();

    // Chunk counts, their exclusive prefix sum, and the chunk table.
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base < num_seqs; base += kSchedThreads) {
        const int n = base + tid;
        int start = 0, len = 0;
        if (n < num_seqs) {
            start = bounds[n];
            len = bounds[n + 1] - start;
        }
        const int nch = (len + chunk - 1) / chunk;
        const int incl = block_scan_incl(nch, s_tmp, false);
        const int first = s_carry + incl - nch;
        if (n < num_seqs) {
            seq_chunk0[n] = first;
            if (n < kMaxRankedSeqs) s_len[n] = len;
            for (int c = 0; c < nch; ++c) {
                chunk_seq[first + c] = n;
                chunk_tok0[first + c] = start + c * chunk;
            }
        }
        __syncthreads();
        if (tid == kSchedThreads - 1) s_carry = first + nch;
        __syncthreads();
    }
    if (tid == 0) {
        seq_chunk0[num_seqs] = s_carry;
        counters[0] = s_carry;
    }
    __syncthreads();

    // Longest sequence first, so the longest chains start earliest. Ties keep
    // index order. Past kMaxRankedSeqs sequences the order is the identity.
    for (int n = tid; n < num_seqs; n += kSchedThreads) {
        int rank = n;
        if (num_seqs <= kMaxRankedSeqs) {
            const int ln = s_len[n];
            rank = 0;
            for (int m = 0; m < num_seqs; ++m) {
                const int lm = s_len[m];
                rank += (lm > ln) || (lm == ln && m < n);
            }
        }
        order[rank] = n;
    }
}

hipError_t launch_schedule(const PrefillArgs &A, hipStream_t st, int32_t *bounds, int32_t *seq_chunk0,
                           int32_t *order, int32_t *chunk_seq, int32_t *chunk_tok0, int32_t *counters) {
    return launch_kernel(kSchedule, gdn_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, st,
                         A.cu, A.num_seqs, (int32_t)A.total_tokens, A.chunk,
                         bounds, seq_chunk0, order, chunk_seq, chunk_tok0, counters);
}

hipError_t launch_prefill(const PrefillArgs &A, hipStream_t st) {
    if (A.io_bf16) {
        switch (A.chunk) {
        case 16: return GDN_PREFILL_INST_FN(1, 16)(A, st);
        case 32: return GDN_PREFILL_INST_FN(1, 32)(A, st);
        case 64: return GDN_PREFILL_INST_FN(1, 64)(A, st);
        default: return hipErrorInvalidValue;
        }
    }
    switch (A.chunk) {
    case 16: return GDN_PREFILL_INST_FN(0, 16)(A, st);
    case 32: return GDN_PREFILL_INST_FN(0, 32)(A, st);
    case 64: return GDN_PREFILL_INST_FN(0, 64)(A, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn

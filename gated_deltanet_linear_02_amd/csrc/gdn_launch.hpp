// gdn_launch.hpp -- internal host-side interface between the C ABI
// (gdn_api.hip) and the kernel launchers. Not installed, not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace gdn {

enum KernelKind {
    kSchedule = 0, kPrep = 1, kScan = 2, kDecode = 3, kTokenScan = 4, kDecodeNorm = 5, kNormApply = 6,
    kKinds = 7
};

// Per-kernel timing (see gdn_timing_start in gdn.h): while it is active,
// each launch claims a pair of events that the dispatch itself stamps with
// the kernel's start and end, so that they time the kernel alone (no marker
// packets around it); otherwise both are null.
struct TimingEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
TimingEvents timing_claim(KernelKind kind);

// Launches `kernel` on `st`, timed as `kind` while timing is active.
template <typename F, typename... Args>
hipError_t launch_kernel(KernelKind kind, F kernel, dim3 grid, dim3 block, size_t smem, hipStream_t st,
                         Args... args) {
    const TimingEvents ev = timing_claim(kind);
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)smem, st, ev.start, ev.stop, 0u, args...);
    return hipGetLastError();
}

struct DecodeArgs {
    const void *q, *k, *v, *g, *beta;
    void *state;  // fp32, or bf16 when state_bf16
    const int32_t *slots;
    int32_t num_slots;
    void *out;
    int32_t batch, hk, hv, d;
    float scale;
    bool io_bf16, gate_bf16;
    bool state_bf16 = false;
    const float *norm_w = nullptr;  // non-null: output normalisation fused in
    float norm_eps = 0.f;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st);

// Workspace of one prefill call, carved from the caller's buffer. Sizes are
// upper bounds known on the host: a sequence of length L has ceil(L/C) <=
// (L + C - 1) / C chunks, so N sequences over at most T tokens have at most
// floor((T + N (C - 1)) / C); for one sequence that is exactly ceil(T/C),
// so the preparation grid launches no workgroup without a chunk.
struct PrefillLayout {
    int64_t max_chunks;
    size_t off_bounds, off_seq_chunk0, off_order;   // int32 [N+1], [N+1], [N]
    size_t off_chunk_seq, off_chunk_tok0, off_counters;            // int32 [max_chunks], [4]
    // Operands of the scan, each in MFMA fragment order (C*C or C*dk
    // elements per chunk and head):
    size_t off_tbmat, off_pmat, off_wmat;  // E, per (chunk, value head)
    size_t off_qmat, off_ktmat;            // E, per (chunk, query/key head)
    size_t off_gates;                      // float [max_chunks][hv][gate_record(C)]
    // Output normalisation fused into the scan: per (chunk, value head, scan
    // workgroup of that head (at most dv/16)), one partial sum of squares per
    // token of the chunk.
    size_t off_norm_part;                  // float [max_chunks][hv][dv / 16][C]
    size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Floats per (chunk, value head) gate record: delta = exp(c_C - c_t) at
// [0, C), scale * gamma_t at [C, 2C), gamma_C at 2C, then 3 floats of
// padding, so that the record is read as C/2 + 1 aligned 16-byte pieces.
constexpr int64_t gate_record(int64_t chunk) { return 2 * chunk + 4; }

inline PrefillLayout prefill_layout(int64_t num_seqs, int64_t total_tokens, int64_t hk, int64_t hv,
                                    int64_t dk, int64_t chunk, size_t elem_bytes) {
    PrefillLayout L;
    L.max_chunks = std::max<int64_t>(1, (total_tokens + num_seqs * (chunk - 1)) / chunk);
    size_t o = 0;
    auto take = [&o](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
    L.off_bounds = take(sizeof(int32_t) * (size_t)(num_seqs + 1));
    L.off_seq_chunk0 = take(sizeof(int32_t) * (size_t)(num_seqs + 1));
    L.off_order = take(sizeof(int32_t) * (size_t)num_seqs);
    L.off_chunk_seq = take(sizeof(int32_t) * (size_t)L.max_chunks);
    L.off_chunk_tok0 = take(sizeof(int32_t) * (size_t)L.max_chunks);
    L.off_counters = take(sizeof(int32_t) * 4);
    const size_t per_mat = (size_t)L.max_chunks * (size_t)hv * (size_t)(chunk * chunk) * elem_bytes;
    L.off_tbmat = take(per_mat);
    L.off_pmat = take(per_mat);
    L.off_wmat = take((size_t)L.max_chunks * (size_t)hv * (size_t)(dk * chunk) * elem_bytes);
    const size_t per_kq = (size_t)L.max_chunks * (size_t)hk * (size_t)(dk * chunk) * elem_bytes;
    L.off_qmat = take(per_kq);
    L.off_ktmat = take(per_kq);
    L.off_gates = take((size_t)L.max_chunks * (size_t)hv * (size_t)gate_record(chunk) * sizeof(float));
    L.off_norm_part = take((size_t)L.max_chunks * (size_t)hv * (size_t)(dk / 16) * (size_t)chunk * sizeof(float));
    L.total = o;
    return L;
}

struct PrefillArgs {
    const void *q, *k, *v, *g, *beta;
    const int32_t *cu;
    int32_t num_seqs;
    int64_t total_tokens;
    int32_t hk, hv, d, chunk;
    float scale;
    bool io_bf16, gate_bf16;
    bool state_bf16 = false;  // states stored in bf16 (fp32 arithmetic)
    int32_t slice_rows = 16;  // state rows per scan workgroup: 16, or 32 (bf16 I/O, d >= 32)
    const void *s0;           // fp32, or bf16 when state_bf16
    void *s_final;
    void *out;
    char *ws;
    PrefillLayout lay;
    // Output normalisation fused into the chunked scan (norm_w non-null):
    // y = o w / sqrt(mean(o^2) + eps) per (token, value head) row.
    const float *norm_w = nullptr;
    float norm_eps = 0.f;
};

// Workgroups of the chunked scan: per (sequence, query/key head) group of
// hv/hk value heads, dv/rows slices each, the groups padded to a multiple of
// 8 (the XCD-aware placement).
inline int64_t scan_grid(int64_t num_seqs, int64_t hk, int64_t hv, int64_t dv, int64_t rows) {
    return ((num_seqs * hk + 7) / 8) * (hv / hk) * (dv / rows) * 8;
}

// Whether a chunked prefill with an output normalisation takes it in the
// scan: when one workgroup holds a head's whole state (rows = dv), which
// normalises its own rows, or when the scan's workgroups fit the device in
// one pass, one per compute unit (`cus`: the device's count, 256 on a whole
// MI355X, fewer on a partition of one). The row slices of a head then
// exchange their partial sums of squares while all of them run; with more
// workgroups than CUs, slices of one head could wait on one another across
// passes, so those calls normalise in a pass after the scan.
inline bool fused_norm_fits(int64_t num_seqs, int64_t hk, int64_t hv, int64_t dv, int64_t rows, int64_t cus) {
    return rows == dv || scan_grid(num_seqs, hk, hv, dv, rows) <= cus;
}
// Compute units of the device that owns `stream` (looked up once per device),
// or 0 if HIP cannot say or the stream's CU mask leaves some of them out.
int32_t stream_device_cus(hipStream_t stream);

// Chunked prefill (chunk 16, 32 or 64): preparation and scan kernels.
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st);
// Token-by-token prefill (chunk 1): one kernel, no workspace.
hipError_t launch_token_scan(const PrefillArgs &a, hipStream_t st);

// Output normalisation of the prefill, in place on `out` after the prefill's
// kernels: rows of tokens in [cu[0], cu[num_seqs]) (clamped into [0, T]).
struct NormArgs {
    void *out;
    const float *norm_w;
    float eps;
    const int32_t *cu;
    int32_t num_seqs;
    int64_t total_tokens;
    int32_t hv, dv;
    bool io_bf16;
};
hipError_t launch_norm_apply(const NormArgs &a, hipStream_t st);

// The chunk gdn_tune_prefill cached for this shape on the current device, or
// 0 (nothing cached, or no device to ask).
// A prefill method: chunk size (1 = token by token) and, for the chunked
// scan, state rows per workgroup (0 = not applicable or not chosen).
struct Method {
    int32_t chunk = 0, rows = 0;
};

// The (chunk, rows) that gdn_tune_prefill cached for this device and shape
// bucket, or chunk 0 when there is none.
Method tuned_method(int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv, int32_t d, int32_t io,
                    int32_t gate, int64_t max_seqlen);

// gdn_prefill with the method given (chunk 1, 16, 32 or 64 and, chunked, 16,
// 32, 64 or 128 state rows per scan workgroup); GDN_ERR_UNSUPPORTED for rows
// that do not fit the call.
int32_t prefill_with_method(const void *q, const void *k, const void *v, const void *g, const void *beta,
                            const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens, int32_t hk,
                            int32_t hv, int32_t dk, int32_t dv, Method m, float scale, int32_t io_dtype,
                            int32_t gate_dtype, const float *initial_state, float *final_state, void *out,
                            void *workspace, size_t workspace_bytes, void *stream);

// gdn_prefill with chunk 0, when nothing is tuned for the shape, picks the
// method from host-known sizes alone (the lengths stay on the device), by
// the mean sequence length L = T / N and the state rows per scan workgroup
// (scan_slice_rows). Measured at HK = 16, HV = 32, d = 128 (whole prefill):
//   token by token   T <= 32, or L <= 10: the chunked path's fixed costs
//                    dominate (one 16-token prompt: 8 vs 13 us; 64 x 8: 93
//                    vs 144 us at best chunked; the crossover lies between
//                    L = 9 and 14 for 8 to 256 sequences);
//   64 or 128 rows   (several sequences) one chunk step per sequence where
//                    it takes one: chunks of 16 for L <= 16, of 32 for
//                    L <= 32 (the step of a wide slice is long, so fewer
//                    steps count: 32 x 24: 62 us with chunks of 32, 67.5
//                    with 16), else of 64;
//   chunks of 16     (16 or 32 rows) L <= 48: the fewest padded rows;
//   chunks of 32     (16 or 32 rows) the scan's workgroups fit the GPU in one
//                    pass (at most one per CU) and L <= 1024: a lone sequence
//                    is bound by its chain's latency, which shorter chunks cut
//                    (1 x 512: 28 vs 32 us);
//   chunks of 64     otherwise: with several passes over the GPU the total
//                    work counts, which the largest chunks minimise.
// fp32 I/O (16-row slices, fp32 MFMA, fewer register stages) crosses over
// later: token by token up to L = 48 (64 x 48: 426 against 496 us at best
// chunked; 16 x 64: 155 against 131), chunks of 32 for one pass and
// L <= 512 (1 x 128: 29 against 40 us with 64), else 64 (1 x 4096: 323
// against 405 us with 32; 8 x 300: 230 against 273).
constexpr int64_t kTokenScanTokens = 32;
constexpr int64_t kTokenScanPerSeq = 10;
constexpr int64_t kChunk16PerSeq = 48;
constexpr int64_t kChunk32PerSeq = 1024;
constexpr int64_t kF32TokenScanPerSeq = 48;
constexpr int64_t kF32Chunk32PerSeq = 512;
constexpr int64_t kScanOnePassWgs = 256;  // gfx950 (MI355X): 256 CUs
// State rows per chunked-scan workgroup: 16, 32, 64 or 128, more than 16
// for bf16 I/O only and at most dv.
inline bool slice_rows_fit(int32_t rows, int64_t dv, bool io_bf16) {
    return rows == 16 || ((rows == 32 || rows == 64 || rows == 128) && io_bf16 && dv >= rows);
}
// Every workgroup of a head loads the head's whole chunk operands, so wider
// slices cut those loads per state row, at the cost of a longer chunk step.
// The scan takes the narrowest slices whose workgroups fit the CUs in one
// pass, else the widest. Measured at HK = 16, HV = 32, d = 128 (whole
// prefill, us, 16 / 32 / 64 / 128 rows): 1 x 4096: 87.5 / 100.8 / 141 / 232;
// 2 x 2048: 89.7 / 76.8 / 89.9 / 133; 4 x 1024: 95.1 / 76.7 / 66.8 / 84.9;
// 8 x 512: 109 / 81.6 / 70.4 / 66.9; 32 x 128: 186 / 128 / 105 / 92.9.
//
// A caller that knows the longest sequence's length on the host may pass it
// (max_seqlen > 0). When the lengths are far from even (the longest above
// 1.25 times the mean), the rows are those that minimise an estimate of the
// scan's time instead: the chunk-step cost of the width times the larger of
// the longest sequence's chain and the batch's work spread over the CUs,
// both counted in tokens with a fixed cost of two 64-token chunk steps per
// workgroup (its state load and store and its launch). Longest sequences
// are scheduled first, so shorter ones fill the CUs beside the longest
// chain, and a narrower slice with a faster step can finish sooner over
// several passes than the one-pass width. Step costs relative to 16 rows,
// fitted to whole-prefill times of twelve uneven batches at HK = 16,
// HV = 32, d = 128, chunk 64, less the preparation: 1, 1.4, 1.9 and 2.9 for
// 16, 32, 64 and 128 rows. The estimate picks the fastest width on eleven of
// them and one within 4% on the last (16 against 32 rows for 16384 + 3 x
// 2048 tokens); the one-pass rule loses 1.1 to 2.1 times on all but the
// even control (4096 + 4 x 512: 259 against 147 us; 8 sequences of 1,541 to
// 14,620 tokens: 1.35 against 1.10 ms). On even batches both agree.
inline double scan_step_cost(int32_t rows) {
    return rows == 16 ? 1.0 : rows == 32 ? 1.4 : rows == 64 ? 1.9 : 2.9;
}
// Whether a max_seqlen hint marks the batch as uneven: several sequences,
// the longest above 1.25 times the mean.
inline bool uneven(int64_t num_seqs, int64_t total_tokens, int64_t max_seqlen) {
    return max_seqlen > 0 && num_seqs > 1 && (double)max_seqlen * (double)num_seqs > 1.25 * (double)total_tokens;
}
inline int32_t scan_slice_rows(int64_t num_seqs, int64_t hv, int64_t dv, bool io_bf16, int64_t total_tokens = 0,
                               int64_t max_seqlen = 0) {
    if (uneven(num_seqs, total_tokens, max_seqlen)) {
        constexpr double kFixedTokens = 128.0;
        const double chain = (double)max_seqlen + kFixedTokens;
        const double work = (double)total_tokens + kFixedTokens * (double)num_seqs;
        int32_t best = 16;
        double best_t = 0.0;
        for (int32_t rows = 16; rows <= 128; rows *= 2) {
            if (!slice_rows_fit(rows, dv, io_bf16)) continue;
            const double spread = (double)hv * (double)(dv / rows) * work / (double)kScanOnePassWgs;
            const double t = scan_step_cost(rows) * std::max(chain, spread);
            if (rows == 16 || t < best_t) {
                best = rows;
                best_t = t;
            }
        }
        return best;
    }
    int32_t rows = 16;
    while (slice_rows_fit(rows * 2, dv, io_bf16) && num_seqs * hv * (dv / rows) > kScanOnePassWgs) rows *= 2;
    return rows;
}

// Under the max_seqlen hint an uneven batch is chunked even where its mean
// length would take it token by token, once its longest sequence exceeds
// kTokenScanLongest + 2 N tokens: that sequence's token chain (about 0.45 us
// a token) then outlasts a chunked pass (about 15 + 0.85 N us at these
// sizes). 500 + 63 x 1 tokens: 79 us chunked against 222 token by token;
// 120 + 20 x 3: 35 against 58; 64 + 63 x 1 stays token by token (36
// against 71). Its chunk follows the longest sequence too: with 64 or 128
// rows, chunks of 16 up to 256 tokens, 32 up to 1,024 (300 + 40 x 8: 55
// against 62 us with 16), else the mean's.
constexpr int64_t kTokenScanLongest = 16;
inline int32_t uneven_chunk(int64_t max_seqlen) {
    return max_seqlen <= 256 ? 16 : max_seqlen <= kChunk32PerSeq ? 32 : 64;
}
inline int32_t rule_chunk(int64_t num_seqs, int64_t total_tokens, int64_t hv, int64_t dv, bool io_bf16,
                          int64_t max_seqlen = 0) {
    const bool skew = uneven(num_seqs, total_tokens, max_seqlen);
    const bool long_chain = skew && max_seqlen > kTokenScanLongest + 2 * num_seqs;
    if ((total_tokens <= kTokenScanTokens || total_tokens <= kTokenScanPerSeq * num_seqs) && !long_chain) return 1;
    if (!io_bf16) {
        if (total_tokens <= kF32TokenScanPerSeq * num_seqs) return 1;
        const bool one_pass = num_seqs * hv * (dv / 16) <= kScanOnePassWgs;
        if (one_pass && (skew ? max_seqlen <= kF32Chunk32PerSeq : total_tokens <= kF32Chunk32PerSeq * num_seqs))
            return 32;
        // uneven, under the hint: its longest chain, as a lone sequence's
        // (300 + 77 + 5 tokens: 64 against 69 us with 64; 500 + 8 x 20:
        // 101 against 113)
        return skew && max_seqlen <= kF32Chunk32PerSeq ? 32 : 64;
    }
    const int64_t rows = scan_slice_rows(num_seqs, hv, dv, io_bf16, total_tokens, max_seqlen);
    if (rows >= 64) {
        const int32_t c = total_tokens <= 16 * num_seqs ? 16 : total_tokens <= 32 * num_seqs ? 32 : 64;
        return skew ? std::max(c, uneven_chunk(max_seqlen)) : c;
    }
    // An uneven batch under the hint is bound by its longest chain as a lone
    // sequence is, so that length decides, over one pass or more (300 + 77 +
    // 5 tokens: 24.4 us with chunks of 32 against 28.3 with 64; 2048 + 1024
    // + 512 + 256 at HV = 16, d = 64, one pass: 44.7 us with 64 against 50.0
    // with 32).
    if (skew) return uneven_chunk(max_seqlen);
    if (total_tokens <= kChunk16PerSeq * num_seqs) return 16;
    // one pass with the slice rows the scan will take (2 x 600: 32-row
    // slices fill the 256 CUs once, and chunks of 32 measure 38.5 against
    // 41 us)
    if (num_seqs * hv * (dv / rows) <= kScanOnePassWgs && total_tokens <= kChunk32PerSeq * num_seqs) return 32;
    return 64;
}

}  // namespace gdn

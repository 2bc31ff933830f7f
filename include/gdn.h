/*
 * gdn.h -- C ABI of libgdn.so: the Gated DeltaNet recurrent layer on AMD
 * Instinct MI355X (gfx950).
 *
 * The layer keeps, per sequence and value head, a fixed-size fp32 matrix state
 * S (dv x dk). For every token a learned gate decides how much of S to keep
 * and a delta update writes the token in ("Optimiser l'inference sur appareil
 * pour Apple Silicon", section "Qwen cree trois formes de charges de travail
 * distinctes"). The gated delta rule computed here:
 *
 *     a_t = exp(g_t)
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * Prefill evaluates it chunk by chunk (the reorganisation into blocks that
 * exposes matrix products, same section); decode advances one token per
 * sequence against resident states. State and gates stay fp32 because the
 * rounding of sequential updates accumulates ("Maintenir l'etat recurrent sur
 * la puce"); a long prompt can be split into fragments whose final state is
 * the next fragment's initial state ("Limiter la memoire temporaire grace au
 * decoupage des prompts").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer to row-major, contiguous memory
 *   that the caller owns. The library allocates no device memory per call and
 *   keeps no pointer after a call returns. q, k, v, out and the states are
 *   read and written in 16-byte pieces and must start on a 16-byte boundary
 *   (GDN_ERR_MISALIGNED); device allocations always do.
 * - Layouts, with T = total tokens, N = sequences, B = decode batch:
 *       q, k            [T][hk][dk]         (decode: [B][hk][dk])
 *       v, out          [T][hv][dv]         (decode: [B][hv][dv])
 *       g, beta         [T][hv]             (decode: [B][hv])
 *       states          [N or slots][hv][dv][dk] fp32; element [i][j] is
 *                       S[i][j], i over values, j over keys.
 *   Value head h reads query/key head h / (hv / hk): consecutive value heads
 *   share one query/key head.
 * - g is the log of the decay (a = exp(g)); it must be finite. beta is used
 *   as given (normally in [0, 1]).
 * - io_dtype applies to q, k, v and out; gate_dtype to g and beta.
 * - `stream` is a hipStream_t (NULL = the null stream). Calls enqueue work on
 *   it and return without synchronising; device-side faults surface at the
 *   caller's next synchronisation.
 * - Argument errors are detected on the host before anything is enqueued and
 *   reported as a status code; no C++ exception or abort crosses the ABI.
 *   After a launch, a HIP launch error is reported as GDN_ERR_HIP.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 5

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL_ARG = 1,    /* a required pointer is NULL */
    GDN_ERR_BAD_SHAPE = 2,   /* negative size, hv % hk != 0, ... */
    GDN_ERR_UNSUPPORTED = 3, /* head size, chunk or dtype outside the built set */
    GDN_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
    GDN_ERR_HIP = 5,         /* a HIP runtime call or launch failed */
    GDN_ERR_ALIAS = 6,       /* an output or the workspace overlaps another buffer */
    GDN_ERR_BAD_VALUE = 7,   /* a scalar argument out of range (norm eps) */
    GDN_ERR_MISALIGNED = 8   /* q, k, v, out or a state not 16-byte aligned */
} gdn_status;

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* Version of this ABI (GDN_ABI_VERSION of the built library). */
int32_t gdn_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *gdn_status_string(int32_t status);

/*
 * Bytes of device workspace gdn_prefill needs for these sizes. Depends only
 * on host-known sizes (never on the contents of cu_seqlens). Returns 0 for
 * arguments gdn_prefill would reject.
 */
size_t gdn_prefill_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                  int32_t hk, int32_t hv, int32_t dk, int32_t dv,
                                  int32_t chunk, int32_t io_dtype);

/*
 * The method gdn_prefill uses for these sizes and this chunk argument: 1
 * (token by token), 16, 32 or 64; for chunk 0, the cached tuned choice or the
 * rule above. Returns 0 for arguments gdn_prefill would reject.
 * slice_rows (may be NULL) receives the chunked scan's state rows per
 * workgroup: 16, 32, 64 or 128 (more than 16 for bf16 I/O only, at most
 * dv), taken from the tuned choice for chunk 0 and otherwise the fewest whose
 * N * hv * dv / rows workgroups fit the GPU's 256 CUs, else the most; 0 for
 * the token-by-token method or a rejected call.
 */
int32_t gdn_prefill_method(int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv,
                           int32_t dk, int32_t dv, int32_t chunk, int32_t io_dtype,
                           int32_t gate_dtype, int32_t *slice_rows);

/*
 * gdn_prefill_method with a host-side hint: max_seqlen, the length of the
 * batch's longest sequence when the caller knows it without reading
 * cu_seqlens back (as varlen attention kernels take it), or 0 for none. A
 * hint must lie between the mean length and total_tokens (else the call
 * returns 0). When the longest sequence is above 1.25 times the mean, the
 * state rows per scan workgroup are those that minimise an estimate of the
 * scan's time, the larger of the longest sequence's chain and the batch's
 * work spread over the CUs, each weighted by the chunk-step cost of the
 * width; otherwise, and without a hint, the rule of gdn_prefill_method.
 * For such batches the chunk size follows the longest sequence too, and a
 * bf16 batch that its mean length would send token by token is chunked
 * once the longest exceeds 16 + 2 num_seqs tokens. Uneven batches gain most
 * (a 4,096-token prompt beside four of 512: 32 rows, 147 us, against 259
 * us with the one-pass rule's 128 rows; 500 tokens beside 63 single ones:
 * chunks of 32, 86 us, against 234 us token by token).
 */
int32_t gdn_prefill_method_hint(int32_t num_seqs, int64_t total_tokens, int64_t max_seqlen,
                                int32_t hk, int32_t hv, int32_t dk, int32_t dv, int32_t chunk,
                                int32_t io_dtype, int32_t gate_dtype, int32_t *slice_rows);

/*
 * Chunked prefill over N packed variable-length sequences.
 *
 * What it computes: the gated delta rule above over every token of every
 * sequence, writing o_t for each token and each sequence's state after its
 * last token. The evaluation is the block form that the first page sets
 * beside the token-by-token one: the same computation reorganised into
 * chunks so that matrix products and token-level parallelism appear
 * ("Optimiser l'inference sur appareil pour Apple Silicon", section "Qwen
 * cree trois formes de charges de travail distinctes"). The state is carried
 * across chunks on chip and handed between calls through initial_state and
 * final_state, so that a long prompt can be fed as fragments whose final
 * state seeds the next (same page, section "Limiter la memoire temporaire
 * grace au decoupage des prompts"); the state stays fp32 (section "Maintenir
 * l'etat recurrent sur la puce").
 *
 * cu_seqlens   int32 [N + 1] DEVICE array of token offsets: sequence n owns
 *              tokens [cu_seqlens[n], cu_seqlens[n+1]). It is read only on the
 *              device. Offsets are clamped into [0, total_tokens] and made
 *              non-decreasing there, so a malformed array cannot cause an
 *              out-of-bounds access (its results are then unspecified).
 *              Zero-length sequences are allowed: their final state equals
 *              their initial state.
 * chunk        how the recurrence is evaluated. 16, 32 or 64: in chunks of that
 *              many tokens (the WY form: a preparation kernel, then the
 *              chunk-recurrent scan). 1: token by token, the state rows held
 *              in registers (one kernel, no workspace), which is faster for
 *              short prompts and multi-token steps. 0: the method that
 *              gdn_tune_prefill cached for this device and shape bucket if
 *              there is one, else by the mean sequence length L = T / N
 *              and the chunked scan's state rows per workgroup (rows: the
 *              fewest of 16, 32, 64, 128 whose N * hv * dv / rows
 *              workgroups fit the GPU's 256 CUs, else the most; more than
 *              16 for bf16 I/O only, at most dv): 1 when T <= 32 or
 *              L <= 10; with 64 or 128 rows 16 when L <= 16, 32 when
 *              L <= 32, else 64; with 16 or 32 rows 16 when L <= 48, 32
 *              when the workgroups fit the GPU's 256 CUs and L <= 1024,
 *              else 64. fp32 I/O: 1 when T <= 32 or L <= 48, 32 when
 *              the 16-row scan fits the CUs in one pass and L <= 512, else
 *              64 (gdn_prefill_method tells which).
 *              The result does not depend on it beyond rounding.
 * dk, dv       16, 32, 64 or 128 each.
 * scale        multiplies every output (1.0 for the plain rule).
 * initial_state  fp32 [N][hv][dv][dk], or NULL for zero states.
 * final_state    fp32 [N][hv][dv][dk], or NULL to skip writing it. It may be
 *                the same pointer as initial_state (updated in place).
 * out          [T][hv][dv] in io_dtype; must not overlap q, k, v, g, beta,
 *              cu_seqlens or the states (GDN_ERR_ALIAS).
 * workspace    device scratch of at least gdn_prefill_workspace_size(...)
 *              bytes, 256-byte aligned; contents need not be initialised and
 *              are meaningless afterwards. It must not overlap q, k, v, g,
 *              beta, cu_seqlens, the norm weight or the states
 *              (GDN_ERR_ALIAS). Calls on different streams need
 *              different workspaces. Token by token (chunk 1, or chunk 0
 *              choosing it) uses none; it may then be NULL. The size for
 *              chunk 0 covers whichever method it picks.
 */
int32_t gdn_prefill(const void *q, const void *k, const void *v,
                    const void *g, const void *beta,
                    const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                    int32_t hk, int32_t hv, int32_t dk, int32_t dv, int32_t chunk,
                    float scale, int32_t io_dtype, int32_t gate_dtype,
                    const float *initial_state, float *final_state, void *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. The
 * arguments are gdn_prefill's without the workspace; the workspace is a
 * fixed array of GDN_NOALLOC_SCRATCH_BYTES in the library's device memory,
 * one per GPU, which the library keeps from the first such call on a GPU
 * until the process ends. The call itself allocates nothing.
 *
 * The array is found on the device of `stream` (the current device for the
 * null stream). A call whose method needs more workspace than the array holds
 * (gdn_prefill_workspace_size of the method gdn_prefill_method reports; the
 * token-by-token method needs none) returns GDN_ERR_WORKSPACE before
 * anything is enqueued; at HK = 16, HV = 32, d = 128 and chunk 64 the array
 * holds one sequence of up to 5,184 bf16 tokens. Every call on a GPU
 * shares that GPU's array, and the array keeps what the last call left in it
 * (each call writes what it reads): calls that may overlap on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 * Results are those of gdn_prefill with the same method, bit for bit.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int32_t gdn_prefill_noalloc(const void *q, const void *k, const void *v,
                            const void *g, const void *beta,
                            const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                            int32_t hk, int32_t hv, int32_t dk, int32_t dv, int32_t chunk,
                            float scale, int32_t io_dtype, int32_t gate_dtype,
                            const float *initial_state, float *final_state, void *out, void *stream);

/*
 * One decode step: one new token for each of `batch` sequences, updating
 * their resident fp32 states in place.
 *
 * What it computes: one application of the gated delta rule above per
 * (sequence, value head), S <- a S (I - b k k^T) + b v k^T and o = scale S q,
 * with the new state written over the old one. Decode produces one new row
 * per step, and its throughput is set by the bytes moved per token
 * ("Optimiser l'inference sur appareil pour Apple Silicon", section
 * "Decodage : minimiser les octets deplaces par token"): each state is read
 * once and written once, and the recurrent update is one fused step (section
 * "Reduire le trafic intermediaire et d'etat").
 *
 * state        fp32 [num_slots][hv][dv][dk], read and written in place.
 * state_slots  int32 [batch] DEVICE array: sequence b uses state slot
 *              state_slots[b]; NULL means slot b (then num_slots >= batch is
 *              required). A slot outside [0, num_slots) makes the kernel skip
 *              that sequence: its state is untouched and its output row is
 *              written as zeros. Two sequences of one call must not share a
 *              slot.
 * dk, dv       16, 32, 64 or 128 each.
 * out          [batch][hv][dv] in io_dtype; must not overlap the inputs.
 */
int32_t gdn_decode_step(const void *q, const void *k, const void *v,
                        const void *g, const void *beta,
                        int32_t batch, int32_t hk, int32_t hv, int32_t dk, int32_t dv,
                        float scale, int32_t io_dtype, int32_t gate_dtype,
                        float *state, const int32_t *state_slots, int32_t num_slots,
                        void *out, void *stream);

/*
 * The same two calls with two options: how states are stored, and the
 * layer's output normalisation. With state_dtype GDN_F32 and norm_weight NULL
 * they are gdn_prefill and gdn_decode_step, and compute what those compute
 * (prefill: "Qwen cree trois formes de charges de travail distinctes" and
 * "Limiter la memoire temporaire grace au decoupage des prompts"; decode:
 * "Decodage : minimiser les octets deplaces par token", all on "Optimiser
 * l'inference sur appareil pour Apple Silicon").
 *
 * state_dtype  GDN_F32 or GDN_BF16: the element type of initial_state,
 *              final_state (prefill) and state (decode), whose layouts are
 *              unchanged. The pages disagree on it: fp32 because rounding
 *              accumulates over sequential updates ("Maintenir l'etat
 *              recurrent sur la puce" of "Optimiser l'inference sur appareil
 *              pour Apple Silicon"), bf16 recurrence states in the engine of
 *              "On descend d'un cran : #004 le meme compilateur sur les puces
 *              d'Apple". With GDN_BF16 all
 *              arithmetic stays fp32: a decode step widens the stored state
 *              and rounds the new one to bf16 (nearest, ties to even); a
 *              prefill widens the initial state, keeps fp32 on chip, and
 *              rounds the final state once. It halves the state traffic of
 *              decode. Built for io_dtype GDN_BF16 only (else
 *              GDN_ERR_UNSUPPORTED); any other value is GDN_ERR_UNSUPPORTED.
 *
 * norm_weight  NULL, or an fp32 [dv] DEVICE array: every output row is then
 *              RMS-normalised. The pages fuse the recurrent update with a
 *              normalisation (section "Reduire le trafic intermediaire et
 *              d'etat" of the same page) but do not give its form; here,
 *              per (token or sequence, value head) row of dv outputs,
 *                  y_i = o_i * norm_weight[i] / sqrt(mean_j o_j^2 + norm_eps)
 *              with one weight per value channel shared by all heads. It must
 *              not overlap out or the states (GDN_ERR_ALIAS).
 * norm_eps     finite and >= 0 when norm_weight is given, else
 *              GDN_ERR_BAD_VALUE. With 0, an all-zero row gives NaN, as the
 *              definition does.
 *
 * Decode with a weight is one kernel: a workgroup owns a whole (sequence,
 * value head) state, so the unnormalised row never goes to memory. A chunked
 * prefill with bf16 I/O normalises inside the scan when a scan workgroup
 * holds whole rows (state rows per workgroup = dv, the widest slices the scan
 * takes for several sequences at d = 128) or when its workgroups, one per
 * compute unit, fit the stream's device in one pass (one sequence at
 * HK = 16, HV = 32, d = 128 on a whole MI355X, for instance; a partition of
 * one counts its own CUs, and a stream whose CU mask leaves some CUs out
 * counts none); in the second case the workgroups holding the parts of a row
 * exchange partial sums of squares through the workspace and wait for one
 * another, so they must all be resident at once. Either way each output is
 * rounded once. Otherwise (fp32 I/O, token by token, or narrower slices over
 * more than one pass or on a masked stream)
 * the prefill's kernels are followed by one pass that rewrites the rows of
 * out in place; rows of tokens outside [cu_seqlens[0], cu_seqlens[N]) are
 * left untouched, and in bf16 a row is then rounded twice (before and after
 * the normalisation). The states are those of the call without a weight.
 */
int32_t gdn_prefill_ex(const void *q, const void *k, const void *v,
                       const void *g, const void *beta,
                       const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                       int32_t hk, int32_t hv, int32_t dk, int32_t dv, int32_t chunk,
                       float scale, int32_t io_dtype, int32_t gate_dtype,
                       const void *initial_state, void *final_state, int32_t state_dtype,
                       const float *norm_weight, float norm_eps, void *out,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill_ex with the max_seqlen hint of gdn_prefill_method_hint (0 for
 * none), which steers the method that chunk 0 and the scan's state rows
 * take; the hint is never checked against cu_seqlens, and a wrong one only
 * costs time. The state rows do not change a result's bits; where the hint
 * also changes the chunk size, results differ by rounding, as between
 * chunk sizes. Errors: as gdn_prefill_ex, plus GDN_ERR_BAD_VALUE for a hint
 * below the mean length or above total_tokens.
 */
int32_t gdn_prefill_hint(const void *q, const void *k, const void *v,
                         const void *g, const void *beta,
                         const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                         int64_t max_seqlen,
                         int32_t hk, int32_t hv, int32_t dk, int32_t dv, int32_t chunk,
                         float scale, int32_t io_dtype, int32_t gate_dtype,
                         const void *initial_state, void *final_state, int32_t state_dtype,
                         const float *norm_weight, float norm_eps, void *out,
                         void *workspace, size_t workspace_bytes, void *stream);

int32_t gdn_decode_step_ex(const void *q, const void *k, const void *v,
                           const void *g, const void *beta,
                           int32_t batch, int32_t hk, int32_t hv, int32_t dk, int32_t dv,
                           float scale, int32_t io_dtype, int32_t gate_dtype,
                           void *state, int32_t state_dtype,
                           const int32_t *state_slots, int32_t num_slots,
                           const float *norm_weight, float norm_eps, void *out, void *stream);

/*
 * Choice of the prefill method by measurement, with a correctness gate.
 *
 * The fastest evaluation (token by token, or chunks of 16, 32 or 64 with 16,
 * 32, 64 or 128 state rows per scan workgroup) depends on the shape and the hardware ("Qwen cree trois formes de charges de
 * travail distinctes" of "Optimiser l'inference sur appareil pour Apple
 * Silicon"); the engine of "On descend d'un cran : #004 le meme compilateur
 * sur les puces d'Apple" measures its options at load time and checks each
 * against a reference, with 1/64 of the largest value as its bar.
 *
 * gdn_tune_prefill runs every method on the caller's inputs (same arguments
 * as gdn_prefill, fp32 initial state or NULL). The GDN_TUNE_CANDIDATES
 * methods, in this order, are (chunk, rows): (64, 16), (64, 32), (64, 64),
 * (64, 128), (32, 16), (32, 32), (32, 64), (32, 128), (16, 16), (16, 32),
 * (16, 64), (16, 128) and (1, -); more than 16 rows only for bf16 I/O with
 * d >= rows. It compares each method's output and final state with those of
 * (64, 16) and rejects it when
 * max |x - ref| / max |ref| exceeds gate_tol, in [0, 1] (1/64 is the pages'
 * bar). It times the rest, each one warm-up plus the mean of five runs on
 * the same inputs, and returns the fastest in *chosen_chunk and *chosen_rows
 * (may be NULL; 0 for the token-by-token method), except that the method of
 * the fixed rule (chunk 0 with nothing cached) is kept unless the fastest
 * is more than 3% faster than it: warm timings on one input set differ by
 * about that much from run to run. For an uneven batch (its longest
 * sequence, read from cu_seqlens, above 1.25 times the mean) that rule is
 * the one given the longest length as a max_seqlen hint. It also caches
 * the choice for (device, driver version, library version, shape bucket,
 * evenness). The bucket is num_seqs and total_tokens each rounded up to a
 * power of two, with hk, hv, d and both dtypes exact; evenness is whether
 * the batch tuned on was uneven. gdn_prefill with chunk 0 then uses the
 * cached choice: a call with a max_seqlen hint (gdn_prefill_hint) the one
 * tuned on a batch of its own evenness, else the hinted rule; a call
 * without the hint the even batches' choice, else the uneven ones'.
 * candidate_ms and candidate_err (may be NULL; GDN_TUNE_CANDIDATES floats
 * each) receive, in the order above, the mean time in ms (-1 when rejected or
 * not applicable) and the gate error (-1 when not run).
 * scratch      device memory of gdn_tune_prefill_scratch_size(...) bytes,
 *              256-byte aligned: outputs, final states and a workspace for
 *              the candidates. The caller's buffers are read, never written.
 * The call synchronises `stream`. Errors: as gdn_prefill, plus
 * GDN_ERR_BAD_VALUE for gate_tol outside [0, 1].
 *
 * The cache lives in the process, shared by all threads, and may be saved
 * to a text file and loaded back, one choice per line: "gdn-tune-v3", the
 * device, driver and library versions, the bucket's sequences, tokens, hk,
 * hv, d, io and gate dtypes, its evenness (0 even, 1 uneven), then the chunk
 * and rows. Entries made on
 * another device, driver or library version are kept but never match.
 * gdn_tune_cache_load returns GDN_ERR_BAD_VALUE when the file cannot be
 * opened, and skips lines it cannot parse; *entries (may be NULL) receives
 * the number loaded.
 */
#define GDN_TUNE_CANDIDATES 13
size_t gdn_tune_prefill_scratch_size(int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv,
                                     int32_t dk, int32_t dv, int32_t io_dtype);
int32_t gdn_tune_prefill(const void *q, const void *k, const void *v,
                         const void *g, const void *beta,
                         const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                         int32_t hk, int32_t hv, int32_t dk, int32_t dv, float scale,
                         int32_t io_dtype, int32_t gate_dtype, const float *initial_state,
                         float gate_tol, void *scratch, size_t scratch_bytes, void *stream,
                         int32_t *chosen_chunk, int32_t *chosen_rows, float *candidate_ms,
                         float *candidate_err);
void gdn_tune_cache_clear(void);
int32_t gdn_tune_cache_size(void);
int32_t gdn_tune_cache_save(const char *path);
int32_t gdn_tune_cache_load(const char *path, int32_t *entries);

/*
 * Per-kernel timing (a profiling aid, not needed for computation).
 *
 * gdn_timing_start(max_launches) makes the library time each of its next
 * kernel launches (up to max_launches) with a pair of HIP events that the
 * kernel's own dispatch on its stream stamps with the kernel's start and end
 * (hipExtLaunchKernelGGL), so that they cover the kernel alone, as a kernel
 * trace does. gdn_timing_stop() waits for those
 * events, writes for each kernel kind k < n_kinds the number of launches
 * timed (counts[k]) and their summed duration in milliseconds (total_ms[k]),
 * releases the events and stops timing. Kinds: 0 = varlen schedule,
 * 1 = chunk preparation, 2 = chunk-recurrent scan, 3 = decode step,
 * 4 = token-by-token prefill, 5 = decode step with output normalisation,
 * 6 = output normalisation pass of the prefill.
 * Not thread-safe with concurrent gdn_* calls from other host threads.
 */
#define GDN_KERNEL_KINDS 7
int32_t gdn_timing_start(int32_t max_launches);
int32_t gdn_timing_stop(int32_t *counts, float *total_ms, int32_t n_kinds);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */

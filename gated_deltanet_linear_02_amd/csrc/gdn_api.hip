// gdn_api.hip -- the C ABI of libgdn.so (declared in include/gdn.h).
//
// Host side only: argument checks (all before any HIP call), workspace
// carving, dispatch to the kernel launchers, and optional per-kernel event
// timing. Nothing here allocates device memory.
#include "gdn.h"
#include "gdn_launch.hpp"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <new>
#include <vector>

namespace gdn {

// ----------------------------------------------------------------- timing

namespace {
struct TimingState {
    std::mutex mu;
    bool active = false;
    int max_launches = 0;
    int used = 0;
    std::vector<hipEvent_t> events;  // 2 per launch
    std::vector<int> kinds;
};
TimingState &timing() {
    static TimingState t;
    return t;
}
}  // namespace

TimingEvents timing_claim(KernelKind kind) {
    TimingState &T = timing();
    std::lock_guard<std::mutex> lk(T.mu);
    TimingEvents ev;
    if (!T.active || T.used >= T.max_launches) return ev;
    ev.start = T.events[2 * T.used];
    ev.stop = T.events[2 * T.used + 1];
    T.kinds[T.used] = kind;
    ++T.used;
    return ev;
}

int32_t stream_device_cus(hipStream_t stream) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int32_t> cached[kMaxDevices] = {};
    hipDevice_t dev = 0;
    const hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) return 0;
    int32_t n = dev < kMaxDevices ? cached[dev].load(std::memory_order_relaxed) : 0;
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
        if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
    }
    // A stream whose CU mask leaves some of them out: which XCDs keep how
    // many is not known here, so it is not counted on to hold a whole grid.
    constexpr int kMaskWords = 32;  // up to 1,024 CUs
    uint32_t mask[kMaskWords] = {};
    const int words = std::min(kMaskWords, (n + 31) / 32);
    if (hipExtStreamGetCUMask(stream, (uint32_t)words, mask) == hipSuccess) {
        int on = 0;
        for (int w = 0; w < words; ++w) on += __builtin_popcount(mask[w]);
        if (on < n) return 0;
    }
    return n;
}

// ----------------------------------------------------------------- checks

static bool valid_head(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
static bool valid_chunk(int32_t c) { return c == 0 || c == 1 || c == 16 || c == 32 || c == 64; }

static bool valid_dtype(int32_t t) { return t == GDN_BF16 || t == GDN_F32; }
static size_t dtype_bytes(int32_t t) { return t == GDN_BF16 ? 2 : 4; }

struct Range {
    uintptr_t lo, hi;
};
static Range span(const void *p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}
// Tensors the kernels read or write in 16-byte pieces must start on a
// 16-byte boundary (their rows are then aligned too: d >= 16).
static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static bool overlaps(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

}  // namespace gdn

using namespace gdn;

extern "C" {

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char *gdn_status_string(int32_t status) {
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case GDN_ERR_BAD_SHAPE: return "invalid sizes (negative, zero where not allowed, or hv not a multiple of hk)";
    case GDN_ERR_UNSUPPORTED: return "head size, chunk size or dtype not supported by the library";
    case GDN_ERR_WORKSPACE: return "workspace is NULL, misaligned or smaller than gdn_prefill_workspace_size()";
    case GDN_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case GDN_ERR_ALIAS: return "an output buffer or the workspace overlaps another buffer";
    case GDN_ERR_BAD_VALUE: return "a scalar argument is out of range (norm eps must be finite and >= 0)";
    case GDN_ERR_MISALIGNED: return "q, k, v, out or a state tensor does not start on a 16-byte boundary";
    default: return "unknown status";
    }
}

// Whether method c (1, 16, 32 or 64) fits the launch limits for this shape.
static bool method_fits(int32_t c, int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv, int32_t dk,
                        int32_t dv, int32_t io_dtype) {
    if (c == 1)  // token scan: one workgroup per (sequence, value head, row slice)
        return (int64_t)num_seqs * hv * dv <= INT32_MAX;
    const PrefillLayout L = prefill_layout(num_seqs, total_tokens, hk, hv, dk, c, dtype_bytes(io_dtype));
    const int64_t scan_grid = (((int64_t)num_seqs * hk + 7) / 8) * (hv / hk) * (dv / 16) * 8;
    return scan_grid <= INT32_MAX && L.max_chunks <= INT32_MAX;
}

static int32_t check_prefill_shape(int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv,
                                   int32_t dk, int32_t dv, int32_t chunk, int32_t io_dtype,
                                   int32_t gate_dtype, int64_t max_seqlen = 0) {
    if (num_seqs < 1 || total_tokens < 0 || total_tokens > INT32_MAX || hk < 1 || hv < 1 || hv % hk != 0)
        return GDN_ERR_BAD_SHAPE;
    if (!valid_head(dk) || dv != dk || !valid_chunk(chunk) || !valid_dtype(io_dtype) ||
        !valid_dtype(gate_dtype) || hk > 65535)
        return GDN_ERR_UNSUPPORTED;
    const int32_t c =
        chunk != 0 ? chunk : rule_chunk(num_seqs, total_tokens, hv, dv, io_dtype == GDN_BF16, max_seqlen);
    return method_fits(c, num_seqs, total_tokens, hk, hv, dk, dv, io_dtype) ? GDN_OK : GDN_ERR_UNSUPPORTED;
}

// The method a call uses: the chunk asked for, or for chunk 0 the choice
// cached by gdn_tune_prefill for this device and shape, else the rule; and
// for a chunked method the scan's state rows per workgroup: `rows` when it is
// given and fits, the tuned rows for chunk 0, else the rule's (which a
// max_seqlen hint, if given, informs).
static Method method_for(int32_t chunk, int32_t rows, int32_t num_seqs, int64_t total_tokens, int32_t hk,
                         int32_t hv, int32_t dk, int32_t dv, int32_t io_dtype, int32_t gate_dtype,
                         int64_t max_seqlen = 0) {
    Method m;
    m.chunk = chunk;
    m.rows = rows;
    if (chunk == 0) {
        m = tuned_method(num_seqs, total_tokens, hk, hv, dk, io_dtype, gate_dtype, max_seqlen);
        if (m.chunk == 0 || !method_fits(m.chunk, num_seqs, total_tokens, hk, hv, dk, dv, io_dtype)) {
            m.chunk = rule_chunk(num_seqs, total_tokens, hv, dv, io_dtype == GDN_BF16, max_seqlen);
            m.rows = 0;
        }
    }
    const bool bf = io_dtype == GDN_BF16;
    if (m.chunk == 1) m.rows = 0;
    else if (!slice_rows_fit(m.rows, dv, bf)) m.rows = scan_slice_rows(num_seqs, hv, dv, bf, total_tokens, max_seqlen);
    return m;
}

// Workspace bytes for chunk c (the token scan needs none; 256 are reported so
// that a size of 0 keeps meaning "rejected"). Chunk 0 may take any method
// (a tuned choice), so it reports the largest chunked need.
static size_t prefill_workspace_bytes(int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv,
                                      int32_t dk, int32_t chunk, int32_t io_dtype) {
    if (chunk == 1) return 256;
    if (chunk != 0) return prefill_layout(num_seqs, total_tokens, hk, hv, dk, chunk, dtype_bytes(io_dtype)).total;
    size_t m = 256;
    for (int32_t c : {16, 32, 64})
        m = std::max(m, prefill_layout(num_seqs, total_tokens, hk, hv, dk, c, dtype_bytes(io_dtype)).total);
    return m;
}

size_t gdn_prefill_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv,
                                  int32_t dk, int32_t dv, int32_t chunk, int32_t io_dtype) {
    if (check_prefill_shape(num_seqs, total_tokens, hk, hv, dk, dv, chunk, io_dtype, GDN_F32) != GDN_OK)
        return 0;
    return prefill_workspace_bytes(num_seqs, total_tokens, hk, hv, dk, chunk, io_dtype);
}

// A max_seqlen hint: 0 (none), or the longest sequence's length, which
// lies between the mean length and the total.
static bool valid_max_seqlen(int64_t max_seqlen, int32_t num_seqs, int64_t total_tokens) {
    return max_seqlen == 0 ||
           (max_seqlen > 0 && max_seqlen <= total_tokens && max_seqlen * (int64_t)num_seqs >= total_tokens);
}

int32_t gdn_prefill_method(int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv, int32_t dk,
                           int32_t dv, int32_t chunk, int32_t io_dtype, int32_t gate_dtype, int32_t *slice_rows) {
    return gdn_prefill_method_hint(num_seqs, total_tokens, 0, hk, hv, dk, dv, chunk, io_dtype, gate_dtype,
                                   slice_rows);
}

int32_t gdn_prefill_method_hint(int32_t num_seqs, int64_t total_tokens, int64_t max_seqlen, int32_t hk,
                                int32_t hv, int32_t dk, int32_t dv, int32_t chunk, int32_t io_dtype,
                                int32_t gate_dtype, int32_t *slice_rows) {
    if (slice_rows) *slice_rows = 0;
    if (check_prefill_shape(num_seqs, total_tokens, hk, hv, dk, dv, chunk, io_dtype, gate_dtype, max_seqlen) !=
            GDN_OK ||
        !valid_max_seqlen(max_seqlen, num_seqs, total_tokens))
        return 0;
    const Method m =
        method_for(chunk, 0, num_seqs, total_tokens, hk, hv, dk, dv, io_dtype, gate_dtype, max_seqlen);
    if (slice_rows) *slice_rows = m.rows;
    return m.chunk;
}

// eps of the output normalisation: finite and not negative.
static bool valid_eps(float eps) { return std::isfinite(eps) && eps >= 0.f; }

// The state storage type and output normalisation of a call, checked
// before anything else of the call: bf16 states need bf16 I/O, a weight
// needs a finite eps >= 0.
static int32_t check_options(int32_t io_dtype, int32_t state_dtype, const float *norm_w, float norm_eps) {
    if (!valid_dtype(state_dtype)) return GDN_ERR_UNSUPPORTED;
    if (state_dtype == GDN_BF16 && io_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (norm_w && !valid_eps(norm_eps)) return GDN_ERR_BAD_VALUE;
    return GDN_OK;
}

// gdn_prefill and gdn_prefill_ex.
static int32_t prefill_impl(const void *q, const void *k, const void *v, const void *g, const void *beta,
                            const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                            int32_t hk, int32_t hv, int32_t dk, int32_t dv, int32_t chunk,
                            float scale, int32_t io_dtype, int32_t gate_dtype,
                            const void *initial_state, void *final_state, int32_t state_dtype,
                            const float *norm_w, float norm_eps, void *out,
                            void *workspace, size_t workspace_bytes, void *stream, int32_t rows = 0,
                            int64_t max_seqlen = 0) {
    const int32_t sc =
        check_prefill_shape(num_seqs, total_tokens, hk, hv, dk, dv, chunk, io_dtype, gate_dtype, max_seqlen);
    if (sc != GDN_OK) return sc;
    if (!valid_max_seqlen(max_seqlen, num_seqs, total_tokens)) return GDN_ERR_BAD_VALUE;
    const int32_t so = check_options(io_dtype, state_dtype, norm_w, norm_eps);
    if (so != GDN_OK) return so;
    if (!cu_seqlens) return GDN_ERR_NULL_ARG;
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !out)) return GDN_ERR_NULL_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(initial_state) ||
        !aligned16(final_state))
        return GDN_ERR_MISALIGNED;

    const size_t eb = dtype_bytes(io_dtype), gb = dtype_bytes(gate_dtype);
    const Method m =
        method_for(chunk, rows, num_seqs, total_tokens, hk, hv, dk, dv, io_dtype, gate_dtype, max_seqlen);
    const int32_t c = m.chunk;
    // The token scan uses no workspace: its buffer is not checked or touched.
    const PrefillLayout L = c == 1 ? PrefillLayout{} : prefill_layout(num_seqs, total_tokens, hk, hv, dk, c, eb);
    if (c != 1 && (!workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255)))
        return GDN_ERR_WORKSPACE;

    const size_t T = (size_t)total_tokens;
    const size_t state_bytes = (size_t)num_seqs * hv * dv * dk * dtype_bytes(state_dtype);
    const Range r_out = span(out, T * hv * dv * eb);
    const Range inputs[] = {span(q, T * hk * dk * eb), span(k, T * hk * dk * eb), span(v, T * hv * dv * eb),
                            span(g, T * hv * gb), span(beta, T * hv * gb),
                            span(cu_seqlens, sizeof(int32_t) * (num_seqs + 1)),
                            span(norm_w, sizeof(float) * (size_t)dv),
                            span(initial_state, state_bytes), span(final_state, state_bytes),
                            span(workspace, L.total)};
    for (const Range &r : inputs)
        if (overlaps(r_out, r)) return GDN_ERR_ALIAS;
    // The final state may be the initial state, but must not overlap any
    // other buffer.
    const Range r_fin = span(final_state, state_bytes);
    for (int i = 0; i < 7; ++i)
        if (overlaps(r_fin, inputs[i])) return GDN_ERR_ALIAS;
    if (overlaps(r_fin, span(workspace, L.total))) return GDN_ERR_ALIAS;
    // The preparation kernel writes the workspace while other workgroups
    // still read the inputs, so the workspace must not overlap any of them.
    const Range r_ws = span(workspace, L.total);
    for (int i = 0; i < 8; ++i)
        if (overlaps(r_ws, inputs[i])) return GDN_ERR_ALIAS;
    if (final_state && initial_state && final_state != initial_state &&
        overlaps(r_fin, span(initial_state, state_bytes)))
        return GDN_ERR_ALIAS;

    PrefillArgs A;
    A.q = q; A.k = k; A.v = v; A.g = g; A.beta = beta;
    A.cu = cu_seqlens; A.num_seqs = num_seqs; A.total_tokens = total_tokens;
    A.hk = hk; A.hv = hv; A.d = dk; A.chunk = c; A.scale = scale;
    A.io_bf16 = io_dtype == GDN_BF16; A.gate_bf16 = gate_dtype == GDN_BF16;
    A.state_bf16 = state_dtype == GDN_BF16;
    A.slice_rows = m.rows;
    A.s0 = initial_state; A.s_final = final_state; A.out = out;
    A.ws = static_cast<char *>(workspace); A.lay = L;
    // With bf16 I/O the chunked scan takes the normalisation itself when one
    // workgroup holds whole rows (rows = dv) or its workgroups fit the
    // stream's device in one pass, so that each output is rounded once (at
    // T = 4096 the fused form adds about 5 us to the scan, the pass 10.5 us);
    // otherwise (fp32 I/O, where the pass reads the same fp32 values, or
    // narrower slices over more than one pass) a pass over out follows.
    const bool fused_norm =
        norm_w && c != 1 && io_dtype == GDN_BF16 &&
        fused_norm_fits(num_seqs, hk, hv, dv, m.rows, stream_device_cus(static_cast<hipStream_t>(stream)));
    if (fused_norm) {
        A.norm_w = norm_w;
        A.norm_eps = norm_eps;
    }
    try {
        const hipStream_t st = static_cast<hipStream_t>(stream);
        if ((c == 1 ? launch_token_scan(A, st) : launch_prefill(A, st)) != hipSuccess) return GDN_ERR_HIP;
        if (norm_w && !fused_norm) {
            NormArgs N;
            N.out = out; N.norm_w = norm_w; N.eps = norm_eps; N.cu = cu_seqlens; N.num_seqs = num_seqs;
            N.total_tokens = total_tokens; N.hv = hv; N.dv = dv; N.io_bf16 = A.io_bf16;
            if (launch_norm_apply(N, st) != hipSuccess) return GDN_ERR_HIP;
        }
        return GDN_OK;
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

int32_t gdn_prefill(const void *q, const void *k, const void *v, const void *g, const void *beta,
                    const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                    int32_t hk, int32_t hv, int32_t dk, int32_t dv, int32_t chunk,
                    float scale, int32_t io_dtype, int32_t gate_dtype,
                    const float *initial_state, float *final_state, void *out,
                    void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, hk, hv, dk, dv, chunk, scale,
                        io_dtype, gate_dtype, initial_state, final_state, GDN_F32, nullptr, 0.f, out, workspace,
                        workspace_bytes, stream);
}

int32_t gdn_prefill_ex(const void *q, const void *k, const void *v, const void *g, const void *beta,
                       const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                       int32_t hk, int32_t hv, int32_t dk, int32_t dv, int32_t chunk,
                       float scale, int32_t io_dtype, int32_t gate_dtype,
                       const void *initial_state, void *final_state, int32_t state_dtype,
                       const float *norm_weight, float norm_eps, void *out,
                       void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, hk, hv, dk, dv, chunk, scale,
                        io_dtype, gate_dtype, initial_state, final_state, state_dtype, norm_weight, norm_eps, out,
                        workspace, workspace_bytes, stream);
}

int32_t gdn_prefill_hint(const void *q, const void *k, const void *v, const void *g, const void *beta,
                         const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens, int64_t max_seqlen,
                         int32_t hk, int32_t hv, int32_t dk, int32_t dv, int32_t chunk,
                         float scale, int32_t io_dtype, int32_t gate_dtype,
                         const void *initial_state, void *final_state, int32_t state_dtype,
                         const float *norm_weight, float norm_eps, void *out,
                         void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, hk, hv, dk, dv, chunk, scale,
                        io_dtype, gate_dtype, initial_state, final_state, state_dtype, norm_weight, norm_eps, out,
                        workspace, workspace_bytes, stream, 0, max_seqlen);
}

}  // extern "C"

// ------------------------------------------------- gdn_prefill_noalloc

// The workspace of gdn_prefill_noalloc: one copy on every GPU the library
// runs on, held until the process ends. In host code `scratch` names a
// host-side stand-in, not the device array: only the address that
// hipGetSymbolAddress returns for the current device is ever used.
static __device__ __align__(256) char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
struct ScratchPtrs {
    std::mutex mu;
    void *ptr[kMaxDevices] = {};
};
ScratchPtrs &scratch_ptrs() {
    static ScratchPtrs s;
    return s;
}
}  // namespace

// The device address of `scratch` on the device of `stream` (the current
// device for the null stream), looked up once per device with that device
// current.
static int32_t scratch_address(hipStream_t stream, void **out) {
    int dev = -1, cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return GDN_ERR_HIP;
    if (stream) {
        hipDevice_t d;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) return GDN_ERR_HIP;
        dev = (int)d;
    } else {
        dev = cur;
    }
    if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
    ScratchPtrs &S = scratch_ptrs();
    std::lock_guard<std::mutex> lk(S.mu);
    if (!S.ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return GDN_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) return GDN_ERR_HIP;
        S.ptr[dev] = p;
    }
    *out = S.ptr[dev];
    return GDN_OK;
}

extern "C" {

int32_t gdn_prefill_noalloc(const void *q, const void *k, const void *v, const void *g, const void *beta,
                            const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                            int32_t hk, int32_t hv, int32_t dk, int32_t dv, int32_t chunk,
                            float scale, int32_t io_dtype, int32_t gate_dtype,
                            const float *initial_state, float *final_state, void *out, void *stream) {
    const int32_t sc = check_prefill_shape(num_seqs, total_tokens, hk, hv, dk, dv, chunk, io_dtype, gate_dtype);
    if (sc != GDN_OK) return sc;
    // What this call needs (the token scan needs nothing), checked against
    // the fixed maximum before any HIP call.
    const Method m = method_for(chunk, 0, num_seqs, total_tokens, hk, hv, dk, dv, io_dtype, gate_dtype);
    const size_t need = m.chunk == 1 ? 0
        : prefill_layout(num_seqs, total_tokens, hk, hv, dk, m.chunk, dtype_bytes(io_dtype)).total;
    if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
    void *ws = nullptr;
    const int32_t sa = scratch_address(static_cast<hipStream_t>(stream), &ws);
    if (sa != GDN_OK) return sa;
    return prefill_impl(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, hk, hv, dk, dv, m.chunk, scale,
                        io_dtype, gate_dtype, initial_state, final_state, GDN_F32, nullptr, 0.f, out, ws,
                        GDN_NOALLOC_SCRATCH_BYTES, stream, m.rows);
}

// gdn_decode_step and gdn_decode_step_ex.
static int32_t decode_impl(const void *q, const void *k, const void *v, const void *g, const void *beta,
                           int32_t batch, int32_t hk, int32_t hv, int32_t dk, int32_t dv, float scale,
                           int32_t io_dtype, int32_t gate_dtype, void *state, int32_t state_dtype,
                           const int32_t *state_slots, int32_t num_slots, const float *norm_w, float norm_eps,
                           void *out, void *stream) {
    if (batch < 0 || hk < 1 || hv < 1 || hv % hk != 0 || num_slots < 0) return GDN_ERR_BAD_SHAPE;
    if (!valid_head(dk) || dv != dk || !valid_dtype(io_dtype) || !valid_dtype(gate_dtype))
        return GDN_ERR_UNSUPPORTED;
    const int32_t so = check_options(io_dtype, state_dtype, norm_w, norm_eps);
    if (so != GDN_OK) return so;
    if (batch == 0) return GDN_OK;
    if ((int64_t)batch * hv > INT32_MAX) return GDN_ERR_UNSUPPORTED;
    if (!state_slots && num_slots < batch) return GDN_ERR_BAD_SHAPE;
    if (!q || !k || !v || !g || !beta || !state || !out) return GDN_ERR_NULL_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(state))
        return GDN_ERR_MISALIGNED;

    const size_t eb = dtype_bytes(io_dtype), gb = dtype_bytes(gate_dtype), B = (size_t)batch;
    const Range r_out = span(out, B * hv * dv * eb);
    const Range r_state = span(state, (size_t)num_slots * hv * dv * dk * dtype_bytes(state_dtype));
    const Range inputs[] = {span(q, B * hk * dk * eb), span(k, B * hk * dk * eb), span(v, B * hv * dv * eb),
                            span(g, B * hv * gb), span(beta, B * hv * gb),
                            span(state_slots, B * sizeof(int32_t)), span(norm_w, sizeof(float) * (size_t)dv),
                            r_state};
    for (const Range &r : inputs)
        if (overlaps(r_out, r)) return GDN_ERR_ALIAS;
    for (int i = 0; i < 7; ++i)
        if (overlaps(r_state, inputs[i])) return GDN_ERR_ALIAS;

    DecodeArgs A;
    A.q = q; A.k = k; A.v = v; A.g = g; A.beta = beta;
    A.state = state; A.slots = state_slots; A.num_slots = num_slots; A.out = out;
    A.batch = batch; A.hk = hk; A.hv = hv; A.d = dk; A.scale = scale;
    A.io_bf16 = io_dtype == GDN_BF16; A.gate_bf16 = gate_dtype == GDN_BF16;
    A.state_bf16 = state_dtype == GDN_BF16;
    A.norm_w = norm_w; A.norm_eps = norm_eps;
    try {
        const hipStream_t st = static_cast<hipStream_t>(stream);
        const hipError_t e = launch_decode(A, st);
        return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

int32_t gdn_decode_step(const void *q, const void *k, const void *v, const void *g, const void *beta,
                        int32_t batch, int32_t hk, int32_t hv, int32_t dk, int32_t dv, float scale,
                        int32_t io_dtype, int32_t gate_dtype, float *state, const int32_t *state_slots,
                        int32_t num_slots, void *out, void *stream) {
    return decode_impl(q, k, v, g, beta, batch, hk, hv, dk, dv, scale, io_dtype, gate_dtype, state, GDN_F32,
                       state_slots, num_slots, nullptr, 0.f, out, stream);
}

int32_t gdn_decode_step_ex(const void *q, const void *k, const void *v, const void *g, const void *beta,
                           int32_t batch, int32_t hk, int32_t hv, int32_t dk, int32_t dv, float scale,
                           int32_t io_dtype, int32_t gate_dtype, void *state, int32_t state_dtype,
                           const int32_t *state_slots, int32_t num_slots, const float *norm_weight,
                           float norm_eps, void *out, void *stream) {
    return decode_impl(q, k, v, g, beta, batch, hk, hv, dk, dv, scale, io_dtype, gate_dtype, state, state_dtype,
                       state_slots, num_slots, norm_weight, norm_eps, out, stream);
}

int32_t gdn_timing_start(int32_t max_launches) {
    if (max_launches < 1) return GDN_ERR_BAD_SHAPE;
    TimingState &T = timing();
    std::lock_guard<std::mutex> lk(T.mu);
    try {
        for (hipEvent_t e : T.events) (void)hipEventDestroy(e);
        T.events.assign(2 * (size_t)max_launches, nullptr);
        T.kinds.assign((size_t)max_launches, -1);
        for (hipEvent_t &e : T.events) {
            if (hipEventCreate(&e) != hipSuccess) {
                e = nullptr;
                T.active = false;
                return GDN_ERR_HIP;
            }
        }
    } catch (...) {
        T.active = false;
        return GDN_ERR_HIP;
    }
    T.max_launches = max_launches;
    T.used = 0;
    T.active = true;
    return GDN_OK;
}

int32_t gdn_timing_stop(int32_t *counts, float *total_ms, int32_t n_kinds) {
    TimingState &T = timing();
    std::lock_guard<std::mutex> lk(T.mu);
    if (!T.active) return GDN_ERR_BAD_SHAPE;
    T.active = false;
    int32_t status = GDN_OK;
    for (int32_t i = 0; i < n_kinds; ++i) {
        if (counts) counts[i] = 0;
        if (total_ms) total_ms[i] = 0.f;
    }
    for (int i = 0; i < T.used; ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(T.events[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, T.events[2 * i], T.events[2 * i + 1]) != hipSuccess) {
            status = GDN_ERR_HIP;
            continue;
        }
        const int kd = T.kinds[i];
        if (kd >= 0 && kd < n_kinds) {
            if (counts) counts[kd] += 1;
            if (total_ms) total_ms[kd] += ms;
        }
    }
    for (hipEvent_t e : T.events)
        if (e) (void)hipEventDestroy(e);
    T.events.clear();
    T.kinds.clear();
    T.used = 0;
    return status;
}

}  // extern "C"

namespace gdn {

int32_t prefill_with_method(const void *q, const void *k, const void *v, const void *g, const void *beta,
                            const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens, int32_t hk,
                            int32_t hv, int32_t dk, int32_t dv, Method m, float scale, int32_t io_dtype,
                            int32_t gate_dtype, const float *initial_state, float *final_state, void *out,
                            void *workspace, size_t workspace_bytes, void *stream) {
    if (m.chunk == 0) return GDN_ERR_UNSUPPORTED;
    if (m.chunk != 1 && !slice_rows_fit(m.rows, dv, io_dtype == GDN_BF16)) return GDN_ERR_UNSUPPORTED;
    return prefill_impl(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, hk, hv, dk, dv, m.chunk, scale,
                        io_dtype, gate_dtype, initial_state, final_state, GDN_F32, nullptr, 0.f, out, workspace,
                        workspace_bytes, stream, m.rows);
}

}  // namespace gdn

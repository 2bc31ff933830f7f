// gdn_tune.hip -- choice of the prefill method by measurement, with a
// correctness gate (gfx950).
//
// Which evaluation of the recurrence is fastest, token by token or chunked
// with C = 16, 32 or 64 and 16, 32, 64 or 128 state rows per scan workgroup, depends
// on the shape and the hardware ("Optimiser
// l'inference sur appareil pour Apple Silicon", section "Qwen cree trois
// formes de charges de travail distinctes"). The engine of "On descend d'un
// cran : #004 le meme compilateur sur les puces d'Apple" measures its options
// when it loads and keeps the winners, and checks each variant against a
// reference, where a wrong result counts when it differs by more than 1/64
// of the largest value. Here, gdn_tune_prefill runs every method on the
// caller's inputs, rejects any whose output or final state differs from the
// (chunk 64, 16 rows) result by more than gate_tol of the largest magnitude,
// times the others, and caches the fastest per (device, driver, library
// version, shape bucket). gdn_prefill with chunk 0 then takes the cached choice for
// its shape when there is one, else its fixed rule.
#include "gdn.h"
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

namespace gdn {

// ----------------------------------------------------------------- gate

// max |a - ref| and max |ref| over n elements, as the bits of non-negative
// floats (which order as unsigned integers), combined with atomicMax into
// res[0] and res[1]: each workgroup reduces in registers and LDS first, so
// that the atomics (which serialise on their two words) are one pair per
// workgroup. A NaN or infinite difference counts as +inf, so that it fails
// any gate.
template <typename E>
__global__ __launch_bounds__(256) void gdn_gate_kernel(const E *__restrict__ a, const E *__restrict__ ref,
                                                       int64_t n, unsigned *__restrict__ res) {
    __shared__ float s_d[4], s_r[4];
    float dmax = 0.f, rmax = 0.f;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const float x = to_f32(a[i]), r = to_f32(ref[i]);
        float d = fabsf(x - r);
        if (!(d <= 3.4028235e38f)) d = __builtin_huge_valf();
        dmax = fmaxf(dmax, d);
        const float ar = fabsf(r);
        if (ar <= 3.4028235e38f) rmax = fmaxf(rmax, ar);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        dmax = fmaxf(dmax, __shfl_xor(dmax, off));
        rmax = fmaxf(rmax, __shfl_xor(rmax, off));
    }
    if ((threadIdx.x & 63) == 0) {
        s_d[threadIdx.x >> 6] = dmax;
        s_r[threadIdx.x >> 6] = rmax;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        atomicMax(res, __float_as_uint(fmaxf(fmaxf(s_d[0], s_d[1]), fmaxf(s_d[2], s_d[3]))));
        atomicMax(res + 1, __float_as_uint(fmaxf(fmaxf(s_r[0], s_r[1]), fmaxf(s_r[2], s_r[3]))));
    }
}

template <typename E>
static hipError_t launch_gate(const void *a, const void *ref, int64_t n, unsigned *res, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
    gdn_gate_kernel<E><<<dim3((unsigned)blocks), dim3(256), 0, st>>>((const E *)a, (const E *)ref, n, res);
    return hipGetLastError();
}

// ----------------------------------------------------------------- cache

// Cached choices, keyed by device, driver, library version and shape bucket
// (sequence count and total tokens rounded up to powers of two; head counts,
// head size and dtypes exact), and whether the batch tuned on was uneven (its
// longest sequence above 1.25 times the mean, the test of the max_seqlen
// hint): the fastest method differs between even and uneven batches of one
// bucket by up to 1.8 times.
struct TuneKey {
    std::string device;
    int driver = 0, version = 0;
    int n2 = 0, t2 = 0, hk = 0, hv = 0, d = 0, io = 0, gate = 0, uneven = 0;
    bool operator<(const TuneKey &o) const {
        return std::tie(device, driver, version, n2, t2, hk, hv, d, io, gate, uneven) <
               std::tie(o.device, o.driver, o.version, o.n2, o.t2, o.hk, o.hv, o.d, o.io, o.gate, o.uneven);
    }
};

constexpr int kTuneRevision = 2;  // bump when the candidate set or the kernels' speeds change

namespace {
std::mutex &tune_mu() {
    static std::mutex m;
    return m;
}
std::map<TuneKey, Method> &tune_cache() {
    static std::map<TuneKey, Method> c;
    return c;
}
}  // namespace

static int64_t pow2_at_least(int64_t x) {
    int64_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

// The current device's part of the key (name with spaces replaced, compute
// units, driver version); false where no device can be queried.
static bool device_key(TuneKey &k) {
    int dev = 0, drv = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    static std::mutex mu;
    static std::map<int, std::pair<std::string, int>> known;
    std::lock_guard<std::mutex> lk(mu);
    auto it = known.find(dev);
    if (it == known.end()) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess || hipDriverGetVersion(&drv) != hipSuccess) return false;
        std::string name = std::string(p.gcnArchName) + "/" + std::to_string(p.multiProcessorCount) + "cu";
        for (char &c : name)
            if (c == ' ' || c == '\t' || c == '\n') c = '_';
        it = known.emplace(dev, std::make_pair(name, drv)).first;
    }
    k.device = it->second.first;
    k.driver = it->second.second;
    k.version = GDN_ABI_VERSION * 1000 + kTuneRevision;
    return true;
}

static bool shape_key(TuneKey &k, int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv, int32_t d,
                      int32_t io, int32_t gate, bool is_uneven) {
    if (!device_key(k)) return false;
    k.n2 = (int)pow2_at_least(num_seqs);
    k.t2 = (int)pow2_at_least(std::max<int64_t>(total_tokens, 1));
    k.hk = hk; k.hv = hv; k.d = d; k.io = io; k.gate = gate;
    k.uneven = is_uneven ? 1 : 0;
    return true;
}

// A call with a max_seqlen hint takes the choice tuned on a batch of its own
// kind (even or uneven); one without takes the even batches' choice, else
// the uneven ones'.
Method tuned_method(int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv, int32_t d, int32_t io,
                    int32_t gate, int64_t max_seqlen) {
    {
        std::lock_guard<std::mutex> lk(tune_mu());
        if (tune_cache().empty()) return Method{};  // nothing tuned: no device query
    }
    TuneKey k;
    if (!shape_key(k, num_seqs, total_tokens, hk, hv, d, io, gate, uneven(num_seqs, total_tokens, max_seqlen)))
        return Method{};
    std::lock_guard<std::mutex> lk(tune_mu());
    auto it = tune_cache().find(k);
    if (it == tune_cache().end() && max_seqlen == 0) {
        k.uneven = 1;
        it = tune_cache().find(k);
    }
    return it == tune_cache().end() ? Method{} : it->second;
}

// ----------------------------------------------------------------- scratch

struct TuneLayout {
    size_t off_res, off_ref_out, off_out, off_ref_fin, off_fin, off_ws, ws_bytes, total;
};

static TuneLayout tune_layout(int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv, int32_t d,
                              size_t eb) {
    TuneLayout L;
    size_t o = 0;
    auto take = [&o](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
    const size_t out_bytes = (size_t)total_tokens * hv * d * eb;
    const size_t fin_bytes = (size_t)num_seqs * hv * d * d * sizeof(float);
    L.off_res = take(8 * sizeof(unsigned));
    L.off_ref_out = take(out_bytes);
    L.off_out = take(out_bytes);
    L.off_ref_fin = take(fin_bytes);
    L.off_fin = take(fin_bytes);
    L.ws_bytes = 256;
    for (int c : {16, 32, 64})
        L.ws_bytes = std::max(L.ws_bytes, prefill_layout(num_seqs, total_tokens, hk, hv, d, c, eb).total);
    L.off_ws = take(L.ws_bytes);
    L.total = o;
    return L;
}

}  // namespace gdn

using namespace gdn;

// How much faster than the fixed rule's method another must measure to be
// chosen instead (see gdn_tune_prefill).
constexpr float kTuneMargin = 0.03f;

extern "C" {

size_t gdn_tune_prefill_scratch_size(int32_t num_seqs, int64_t total_tokens, int32_t hk, int32_t hv,
                                     int32_t dk, int32_t dv, int32_t io_dtype) {
    if (gdn_prefill_workspace_size(num_seqs, total_tokens, hk, hv, dk, dv, 64, io_dtype) == 0) return 0;
    return tune_layout(num_seqs, total_tokens, hk, hv, dk, io_dtype == GDN_BF16 ? 2 : 4).total;
}

int32_t gdn_tune_prefill(const void *q, const void *k, const void *v, const void *g, const void *beta,
                         const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                         int32_t hk, int32_t hv, int32_t dk, int32_t dv, float scale,
                         int32_t io_dtype, int32_t gate_dtype, const float *initial_state, float gate_tol,
                         void *scratch, size_t scratch_bytes, void *stream,
                         int32_t *chosen_chunk, int32_t *chosen_rows, float *candidate_ms,
                         float *candidate_err) {
    // (chunk, state rows per scan workgroup), the reference first
    static const Method kCandidates[GDN_TUNE_CANDIDATES] = {{64, 16}, {64, 32}, {64, 64}, {64, 128}, {32, 16},
                                                            {32, 32}, {32, 64}, {32, 128}, {16, 16}, {16, 32},
                                                            {16, 64}, {16, 128}, {1, 0}};
    constexpr int NC = GDN_TUNE_CANDIDATES;
    if (!chosen_chunk) return GDN_ERR_NULL_ARG;
    if (!(gate_tol >= 0.f) || !(gate_tol <= 1.f)) return GDN_ERR_BAD_VALUE;
    const size_t need = gdn_tune_prefill_scratch_size(num_seqs, total_tokens, hk, hv, dk, dv, io_dtype);
    if (need == 0) return GDN_ERR_BAD_SHAPE;
    if (!scratch || scratch_bytes < need || (reinterpret_cast<uintptr_t>(scratch) & 255)) return GDN_ERR_WORKSPACE;
    if (!cu_seqlens || (total_tokens > 0 && (!q || !k || !v || !g || !beta))) return GDN_ERR_NULL_ARG;
    const size_t eb = io_dtype == GDN_BF16 ? 2 : 4;
    const TuneLayout L = tune_layout(num_seqs, total_tokens, hk, hv, dk, eb);
    char *base = static_cast<char *>(scratch);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // The batch's longest sequence (bounds clamped into [0, T] and made
    // non-decreasing, as the kernels read them): whether it is uneven keys
    // the cached choice, and the rule it is weighed against takes it as the
    // max_seqlen hint.
    int64_t longest = 0;
    {
        std::vector<int32_t> cu(num_seqs + 1);
        if (hipMemcpyAsync(cu.data(), cu_seqlens, cu.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
                hipSuccess ||
            hipStreamSynchronize(st) != hipSuccess)
            return GDN_ERR_HIP;
        int64_t lo = std::min<int64_t>(std::max<int64_t>(cu[0], 0), total_tokens);
        for (int32_t n = 0; n < num_seqs; ++n) {
            const int64_t hi = std::max(std::min<int64_t>(std::max<int64_t>(cu[n + 1], 0), total_tokens), lo);
            longest = std::max(longest, hi - lo);
            lo = hi;
        }
    }
    const bool is_uneven = uneven(num_seqs, total_tokens, longest);
    const int64_t hint = is_uneven ? longest : 0;
    unsigned *res = reinterpret_cast<unsigned *>(base + L.off_res);
    const int64_t n_out = total_tokens * hv * dv, n_fin = (int64_t)num_seqs * hv * dv * dk;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int32_t status = GDN_OK;
    float ms[NC], err[NC];
    for (int i = 0; i < NC; ++i) ms[i] = err[i] = -1.f;

    auto run = [&](Method c, bool ref) -> int32_t {
        void *out = base + (ref ? L.off_ref_out : L.off_out);
        float *fin = reinterpret_cast<float *>(base + (ref ? L.off_ref_fin : L.off_fin));
        return prefill_with_method(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, hk, hv, dk, dv, c, scale,
                                   io_dtype, gate_dtype, initial_state, fin, out, base + L.off_ws, L.ws_bytes,
                                   stream);
    };
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        status = GDN_ERR_HIP;
    } else {
        // Rows of tokens outside every sequence are not written: zero both
        // outputs so that they compare equal there.
        if (hipMemsetAsync(base + L.off_ref_out, 0, (size_t)n_out * eb, st) != hipSuccess) status = GDN_ERR_HIP;
        if (status == GDN_OK) status = run(kCandidates[0], true);
        for (int i = 0; i < NC && status == GDN_OK; ++i) {
            const Method c = kCandidates[i];
            // more than 16 state rows per workgroup: bf16 I/O with d >= rows only
            if (c.chunk != 1 && !slice_rows_fit(c.rows, dv, io_dtype == GDN_BF16)) continue;
            // correctness gate against the (64, 16) result
            if (hipMemsetAsync(base + L.off_out, 0, (size_t)n_out * eb, st) != hipSuccess ||
                hipMemsetAsync(res, 0, 8 * sizeof(unsigned), st) != hipSuccess) {
                status = GDN_ERR_HIP;
                break;
            }
            if ((status = run(c, false)) != GDN_OK) {
                // a method this shape is outside of (its grid limits) is not a candidate
                if (status == GDN_ERR_UNSUPPORTED && i > 0) {
                    status = GDN_OK;
                    continue;
                }
                break;
            }
            hipError_t e = eb == 2 ? launch_gate<bf16>(base + L.off_out, base + L.off_ref_out, n_out, res, st)
                                   : launch_gate<float>(base + L.off_out, base + L.off_ref_out, n_out, res, st);
            if (e == hipSuccess)
                e = launch_gate<float>(base + L.off_fin, base + L.off_ref_fin, n_fin, res + 2, st);
            unsigned h[4] = {0, 0, 0, 0};
            if (e == hipSuccess) e = hipMemcpyAsync(h, res, sizeof(h), hipMemcpyDeviceToHost, st);
            if (e == hipSuccess) e = hipStreamSynchronize(st);
            if (e != hipSuccess) {
                status = GDN_ERR_HIP;
                break;
            }
            float f[4];
            memcpy(f, h, sizeof(f));
            const float eo = f[1] > 0.f ? f[0] / f[1] : f[0];
            const float es = f[3] > 0.f ? f[2] / f[3] : f[2];
            err[i] = std::max(eo, es);
            if (!(err[i] <= gate_tol)) continue;  // rejected: never timed, never chosen
            // timing: one more warm-up, then the mean of five runs
            constexpr int kReps = 5;
            if ((status = run(c, false)) != GDN_OK) break;
            if (hipEventRecord(e0, st) != hipSuccess) { status = GDN_ERR_HIP; break; }
            for (int r = 0; r < kReps && status == GDN_OK; ++r) status = run(c, false);
            if (status != GDN_OK) break;
            float t = 0.f;
            if (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                hipEventElapsedTime(&t, e0, e1) != hipSuccess) {
                status = GDN_ERR_HIP;
                break;
            }
            ms[i] = t / kReps;
        }
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (status != GDN_OK) return status;

    int best = 0;  // the reference always passes its own gate
    for (int i = 1; i < NC; ++i)
        if (ms[i] >= 0.f && ms[i] < ms[best]) best = i;
    // The fixed rule's method (given the batch's longest length when the
    // batch is uneven) keeps the choice unless another is faster by more
    // than kTuneMargin: the candidates are timed warm on the caller's
    // inputs, and differences within the run-to-run scatter would otherwise
    // decide, and can reverse with cold caches (one 4096-token sequence: 32
    // rows per scan workgroup 1% faster warm, 11% slower cold).
    const bool bf = io_dtype == GDN_BF16;
    Method rule;
    rule.chunk = rule_chunk(num_seqs, total_tokens, hv, dv, bf, hint);
    rule.rows = rule.chunk == 1 ? 0 : scan_slice_rows(num_seqs, hv, dv, bf, total_tokens, hint);
    for (int i = 0; i < NC; ++i)
        if (kCandidates[i].chunk == rule.chunk && kCandidates[i].rows == rule.rows && ms[i] >= 0.f &&
            ms[best] >= ms[i] * (1.f - kTuneMargin))
            best = i;
    *chosen_chunk = kCandidates[best].chunk;
    if (chosen_rows) *chosen_rows = kCandidates[best].rows;
    for (int i = 0; i < NC; ++i) {
        if (candidate_ms) candidate_ms[i] = ms[i];
        if (candidate_err) candidate_err[i] = err[i];
    }
    TuneKey key;
    if (shape_key(key, num_seqs, total_tokens, hk, hv, dk, io_dtype, gate_dtype, is_uneven)) {
        std::lock_guard<std::mutex> lk(tune_mu());
        tune_cache()[key] = kCandidates[best];
    }
    return GDN_OK;
}

void gdn_tune_cache_clear(void) {
    std::lock_guard<std::mutex> lk(tune_mu());
    tune_cache().clear();
}

int32_t gdn_tune_cache_size(void) {
    std::lock_guard<std::mutex> lk(tune_mu());
    return (int32_t)tune_cache().size();
}

int32_t gdn_tune_cache_save(const char *path) {
    if (!path) return GDN_ERR_NULL_ARG;
    std::lock_guard<std::mutex> lk(tune_mu());
    FILE *f = fopen(path, "w");
    if (!f) return GDN_ERR_BAD_VALUE;
    for (const auto &kv : tune_cache()) {
        const TuneKey &k = kv.first;
        fprintf(f, "gdn-tune-v3 %s %d %d %d %d %d %d %d %d %d %d %d %d\n", k.device.c_str(), k.driver,
                k.version, k.n2, k.t2, k.hk, k.hv, k.d, k.io, k.gate, k.uneven, kv.second.chunk, kv.second.rows);
    }
    return fclose(f) == 0 ? GDN_OK : GDN_ERR_BAD_VALUE;
}

int32_t gdn_tune_cache_load(const char *path, int32_t *entries) {
    if (!path) return GDN_ERR_NULL_ARG;
    FILE *f = fopen(path, "r");
    if (!f) return GDN_ERR_BAD_VALUE;
    int32_t n = 0;
    char line[512];
    std::lock_guard<std::mutex> lk(tune_mu());
    while (fgets(line, sizeof(line), f)) {
        char tag[16], dev[256];
        TuneKey k;
        Method m;
        if (sscanf(line, "%15s %255s %d %d %d %d %d %d %d %d %d %d %d %d", tag, dev, &k.driver, &k.version, &k.n2,
                   &k.t2, &k.hk, &k.hv, &k.d, &k.io, &k.gate, &k.uneven, &m.chunk, &m.rows) != 14)
            continue;
        if (strcmp(tag, "gdn-tune-v3") != 0) continue;
        const bool ok = (k.uneven == 0 || k.uneven == 1) &&
                        (m.chunk == 1 ? m.rows == 0
                                      : (m.chunk == 16 || m.chunk == 32 || m.chunk == 64) &&
                                            (m.rows == 16 || m.rows == 32 || m.rows == 64 || m.rows == 128));
        if (!ok) continue;
        k.device = dev;
        tune_cache()[k] = m;
        ++n;
    }
    fclose(f);
    if (entries) *entries = n;
    return GDN_OK;
}

}  // extern "C"

// gdn_norm.hip -- output normalisation pass of the prefill (gfx950).
//
// The layer's output rows are normalised after the recurrent update, which
// the pages fuse with that normalisation ("Optimiser l'inference sur
// appareil pour Apple Silicon", section "Reduire le trafic intermediaire et
// d'etat"): per
// (token, value head), with the dv outputs o and one weight per value channel
//     y_i = o_i w_i / sqrt(mean_j o_j^2 + eps).
// Decode fuses this into its kernel (gdn_decode.hip). The prefill kernels
// cannot: the chunked scan and the token scan split a head's value rows over
// workgroups that run independently and must never wait for one another, so
// no workgroup holds a whole output row. This pass runs after them on the
// same stream and rewrites `out` in place. It is memory-bound: each row is
// read once and written once, in 16-byte pieces, LPR lanes per row, with the
// row's sum of squares finished by butterfly shuffles inside the row's lanes.
// Nontemporal loads and stores (the rows are touched once) and two rows per
// lane group gave the best rate measured (6.5 TB/s at T = 4096; four rows,
// or plain accesses, 5.9 to 6.2).
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

#include <algorithm>

namespace gdn {

template <typename E> struct Piece;
template <> struct Piece<bf16> {
    typedef bf16x8 type;
    static constexpr int N = 8;
};
template <> struct Piece<float> {
    typedef f32x4 type;
    static constexpr int N = 4;
};

constexpr int kNormThreads = 256;
constexpr int kNormRowsPerGroup = 2;  // rows per lane group per iteration

template <typename E, int DV> struct NormShape {
    static constexpr int EPL = Piece<E>::N;            // elements per lane
    static constexpr int LPR = DV / EPL;               // lanes per row
    static constexpr int RPB = kNormThreads / LPR;     // rows per workgroup pass
    static constexpr int STEP = RPB * kNormRowsPerGroup;  // rows per workgroup iteration
};

template <typename E, int DV>
__global__ __launch_bounds__(kNormThreads) void gdn_norm_apply_kernel(
    E *__restrict__ out, const float *__restrict__ norm_w, const int32_t *__restrict__ cu,
    int32_t num_seqs, int32_t total_tokens, int32_t hv, float eps)
{
    typedef NormShape<E, DV> SH;
    typedef typename Piece<E>::type P;
    constexpr int EPL = SH::EPL, LPR = SH::LPR, RPB = SH::RPB, STEP = SH::STEP;

    const int tid = threadIdx.x;
    const int lr = tid % LPR;
    // Tokens inside sequences: [cu[0], cu[N]) clamped into [0, T]; rows of
    // tokens outside every sequence are left as they are.
    const int64_t lo = (int64_t)min(max(cu[0], 0), total_tokens) * hv;
    const int64_t hi = (int64_t)min(max(cu[num_seqs], 0), total_tokens) * hv;

    float w[EPL];  // once per workgroup, so plain loads (no alignment asked of the weight)
#pragma unroll
    for (int j = 0; j < EPL; ++j) w[j] = norm_w[lr * EPL + j];

    for (int64_t base = (lo / STEP + blockIdx.x) * STEP; base < hi; base += (int64_t)gridDim.x * STEP) {
        P x[kNormRowsPerGroup];
        bool live[kNormRowsPerGroup];
#pragma unroll
        for (int i = 0; i < kNormRowsPerGroup; ++i) {
            const int64_t row = base + i * RPB + tid / LPR;
            live[i] = row >= lo && row < hi;
            if (live[i]) x[i] = __builtin_nontemporal_load(reinterpret_cast<const P *>(out + row * DV + lr * EPL));
            else x[i] = P{};
        }
#pragma unroll
        for (int i = 0; i < kNormRowsPerGroup; ++i) {
            float f[EPL];
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                f[j] = static_cast<float>(x[i][j]);
                ss = __builtin_fmaf(f[j], f[j], ss);
            }
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off);
            const float r = 1.0f / sqrtf(ss * (1.0f / DV) + eps);
            P y;
#pragma unroll
            for (int j = 0; j < EPL; ++j) y[j] = from_f32<E>(f[j] * r * w[j]);
            const int64_t row = base + i * RPB + tid / LPR;
            if (live[i]) __builtin_nontemporal_store(y, reinterpret_cast<P *>(out + row * DV + lr * EPL));
        }
    }
}

template <typename E, int D>
static hipError_t launch_norm_apply_t(const NormArgs &A, hipStream_t st) {
    typedef NormShape<E, D> SH;
    const int64_t rows = A.total_tokens * (int64_t)A.hv;
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((rows + SH::STEP - 1) / SH::STEP, 1 << 16));
    return launch_kernel(kNormApply, gdn_norm_apply_kernel<E, D>, dim3((unsigned)blocks), dim3(kNormThreads), 0, st,
                         (E *)A.out, A.norm_w, A.cu, A.num_seqs, (int32_t)A.total_tokens, A.hv, A.eps);
}

template <typename E>
static hipError_t launch_norm_apply_d(const NormArgs &A, hipStream_t st) {
    switch (A.dv) {
    case 16: return launch_norm_apply_t<E, 16>(A, st);
    case 32: return launch_norm_apply_t<E, 32>(A, st);
    case 64: return launch_norm_apply_t<E, 64>(A, st);
    case 128: return launch_norm_apply_t<E, 128>(A, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_norm_apply(const NormArgs &A, hipStream_t st) {
    if (A.total_tokens == 0) return hipSuccess;
    return A.io_bf16 ? launch_norm_apply_d<bf16>(A, st) : launch_norm_apply_d<float>(A, st);
}

}  // namespace gdn

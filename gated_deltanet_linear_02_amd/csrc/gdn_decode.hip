// gdn_decode.hip -- one decode step of the Gated DeltaNet layer (gfx950).
//
// Decode advances every sequence by one token. Its speed is set by the bytes
// moved per token ("Optimiser l'inference sur appareil pour Apple Silicon",
// section "Decodage : minimiser les octets deplaces par token"); here almost
// all of them are the fp32 state, read once and written once. The whole step
// (reductions, update, output) is one fused launch, as in the fused recurrent
// update of section "Reduire le trafic intermediaire et d'etat", and adjacent
// lanes touch adjacent bytes so the memory system can merge their accesses
// (section "Fusionner les lectures du cache d'attention").
//
// Per (sequence b, value head h) with a = exp(g), over the OLD state S:
//     sk = S k,  sq = S q,  kq = k.q
//     u  = b (v - a sk)
//     o  = scale (a sq + kq u)          ( = scale S_new q )
//     S_new = a S + u k^T               ( = a S (I - b k k^T) + b v k^T )
//
// Mapping: the rows of one (b, h) state are independent, so they are split
// over several 256-thread workgroups of ROWS rows each: small workgroups keep
// more of them in flight, which is what an in-place read-then-write stream
// needs to approach the HBM rate. A state row (dk fp32) is split over
// LPR = dk/8 consecutive lanes; lane lr holds 8 elements of the row as two
// 16-byte pieces at columns 4*lr + 4*LPR*m (m = 0, 1), so that for each load
// the LPR lanes of a row read 16*LPR contiguous bytes. Row dot products finish
// with log2(LPR) butterfly shuffles. Each workgroup recomputes k.q (dk
// products), which is negligible.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <typename E> __device__ __forceinline__ void load4(const E *p, float *dst);
template <> __device__ __forceinline__ void load4<float>(const float *p, float *dst) {
    const f32x4 x = *reinterpret_cast<const f32x4 *>(p);
    dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2]; dst[3] = x[3];
}
template <> __device__ __forceinline__ void load4<bf16>(const bf16 *p, float *dst) {
    const bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
    dst[0] = static_cast<float>(x[0]); dst[1] = static_cast<float>(x[1]);
    dst[2] = static_cast<float>(x[2]); dst[3] = static_cast<float>(x[3]);
}

template <int DK, int DV> struct DecodeShape {
    static constexpr int EPL = 8;                  // state elements per lane
    static constexpr int LPR = DK / EPL;           // lanes per state row
    static constexpr int ROWS = 256 / LPR;         // rows per workgroup
    static constexpr int SLICES = (DV + ROWS - 1) / ROWS;  // workgroups per (b, h)
};

template <typename E, typename G, int DK, int DV>
__global__ __launch_bounds__(256) void gdn_decode_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const G *__restrict__ gate_g, const G *__restrict__ gate_b,
    float *__restrict__ state, const int32_t *__restrict__ slots, int32_t num_slots,
    E *__restrict__ out, int32_t hk, int32_t hv, float scale)
{
    typedef DecodeShape<DK, DV> SH;
    constexpr int LPR = SH::LPR, ROWS = SH::ROWS, SLICES = SH::SLICES;

    const int bhs = blockIdx.x;
    const int bh = bhs / SLICES;
    const int row0 = (bhs - bh * SLICES) * ROWS;
    const int b = bh / hv;
    const int h = bh - b * hv;
    const int kh = h / (hv / hk);
    const int tid = threadIdx.x;
    const int lr = tid % LPR;
    const int row = row0 + tid / LPR;
    const bool live = row < DV;

    const int slot = slots ? slots[b] : b;
    E *o_row = out + ((size_t)b * hv + h) * DV;
    if (slot < 0 || slot >= num_slots) {
        if (live && lr == 0) o_row[row] = from_f32<E>(0.0f);
        return;
    }
    float *S = state + ((size_t)slot * hv + h) * (size_t)(DV * DK);

    // State row pieces first: the bulk of the bytes, all loads in flight.
    f32x4 s[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
        s[m] = live ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (size_t)row * DK + 4 * lr + 4 * LPR * m))
                    : f32x4{0.f, 0.f, 0.f, 0.f};

    float kk[8], qq[8];
    const E *kp = k + ((size_t)b * hk + kh) * DK;
    const E *qp = q + ((size_t)b * hk + kh) * DK;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        load4<E>(kp + 4 * lr + 4 * LPR * m, kk + 4 * m);
        load4<E>(qp + 4 * lr + 4 * LPR * m, qq + 4 * m);
    }
    const float a = expf(static_cast<float>(gate_g[(size_t)b * hv + h]));
    const float beta = static_cast<float>(gate_b[(size_t)b * hv + h]);
    const float vv = live ? static_cast<float>(v[((size_t)b * hv + h) * DV + row]) : 0.f;

    float kq = 0.f, sk = 0.f, sq = 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kq += kk[4 * m + e] * qq[4 * m + e];
            sk += s[m][e] * kk[4 * m + e];
            sq += s[m][e] * qq[4 * m + e];
        }
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) {
        kq += __shfl_xor(kq, off);
        sk += __shfl_xor(sk, off);
        sq += __shfl_xor(sq, off);
    }
    if (live) {
        const float u = beta * (vv - a * sk);
        if (lr == 0) o_row[row] = from_f32<E>(scale * (a * sq + kq * u));
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = a * s[m][e] + u * kk[4 * m + e];
            __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(S + (size_t)row * DK + 4 * lr + 4 * LPR * m));
        }
    }
}

template <typename E, typename G, int D>
static hipError_t launch_decode_t(const DecodeArgs &A, hipStream_t st) {
    const dim3 grid((unsigned)A.batch * (unsigned)A.hv * (unsigned)DecodeShape<D, D>::SLICES), block(256);
    return launch_kernel(kDecode, gdn_decode_kernel<E, G, D, D>, grid, block, 0, st,
                         (const E *)A.q, (const E *)A.k, (const E *)A.v,
                         (const G *)A.g, (const G *)A.beta, A.state, A.slots, A.num_slots,
                         (E *)A.out, A.hk, A.hv, A.scale);
}

template <typename E, typename G>
static hipError_t launch_decode_d(const DecodeArgs &A, hipStream_t st) {
    switch (A.d) {
    case 16: return launch_decode_t<E, G, 16>(A, st);
    case 32: return launch_decode_t<E, G, 32>(A, st);
    case 64: return launch_decode_t<E, G, 64>(A, st);
    case 128: return launch_decode_t<E, G, 128>(A, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs &A, hipStream_t st) {
    if (A.io_bf16) {
        return A.gate_bf16 ? launch_decode_d<bf16, bf16>(A, st) : launch_decode_d<bf16, float>(A, st);
    }
    return A.gate_bf16 ? launch_decode_d<float, bf16>(A, st) : launch_decode_d<float, float>(A, st);
}

}  // namespace gdn

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
// needs to approach the HBM rate. A state row (dk elements) is split over
// LPR = dk/8 consecutive lanes, 8 elements per lane (StateLane below gives
// their columns: two 16-byte pieces of fp32, or one of bf16), and each group
// of LPR lanes holds NRL rows. Row dot products finish with log2(LPR)
// butterfly shuffles. Each workgroup recomputes k.q (dk products), which is
// negligible.
//
// States are fp32, or bf16 with fp32 arithmetic (widened on load, rounded to
// nearest even on store): the storage variant that halves the bytes per
// token, whose accuracy the pages argue about.
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

// Workgroup shape of the plain decode kernel, by storage type, measured at
// batch 64, d = 128 (kernel us):
//   fp32 states: 256 threads, one row per lane group (16 rows per
//     workgroup), nontemporal loads and stores: 43.2-43.9 us. Two rows per
//     group, or 512 and 1024 threads, are no faster; plain loads are slower
//     (46.6-48.7 us).
//   bf16 states: a whole (sequence, value head) state per workgroup, 1024
//     threads with two rows per lane group, plain loads and nontemporal
//     stores: 22.8-23.0 us. The same shape with nontemporal loads takes
//     24.6 us; 512 threads with four rows per group 23.1 us; 256 threads with
//     four rows per group (64 rows per workgroup) 26.0-26.4 us.
// Half the bytes per row make a bf16 row's pieces small, so a lane takes
// more rows and a workgroup more of the state to keep the bytes in flight.
template <typename SE> constexpr int kDecodeThreads = 256;
template <> constexpr int kDecodeThreads<bf16> = 1024;
template <typename SE> constexpr int kDecodeRowsPerLane = 1;
template <> constexpr int kDecodeRowsPerLane<bf16> = 2;

template <typename SE, int DK, int DV> struct DecodeShape {
    static constexpr int EPL = 8;                  // state elements per lane
    static constexpr int LPR = DK / EPL;           // lanes per state row
    // threads per workgroup: at most what NRL rows per lane group of one
    // state need (small d), at least one wave
    static constexpr int TMAX = DV * LPR / kDecodeRowsPerLane<SE>;
    static constexpr int THREADS = kDecodeThreads<SE> < TMAX ? kDecodeThreads<SE> : (TMAX < 64 ? 64 : TMAX);
    static constexpr int RPP = THREADS / LPR;      // rows per pass of the workgroup
    // rows per lane group
    static constexpr int NRL = RPP >= DV ? 1 : (kDecodeRowsPerLane<SE> < DV / RPP ? kDecodeRowsPerLane<SE> : DV / RPP);
    static constexpr int ROWS = RPP * NRL;         // rows per workgroup
    static constexpr int SLICES = (DV + ROWS - 1) / ROWS;  // workgroups per (b, h)
};

// A lane's share of one state row: 8 elements, held as floats whatever the
// storage type SE. fp32 storage: two 16-byte pieces at columns 4 lr and
// 4 lr + 4 LPR, so that the LPR lanes of a row read 16 LPR contiguous bytes
// per load; bf16 storage: one 16-byte piece at columns 8 lr .. 8 lr + 7.
// Element j of the lane sits at column col(lr, j); columns 4m .. 4m + 3 of
// the lane are consecutive in both layouts. States are read and written
// once per step, so the stores are nontemporal, and so are the fp32 loads;
// bf16 rows load faster with the default policy (see kDecodeThreads).
template <typename SE, int LPR> struct StateLane;
template <int LPR> struct StateLane<float, LPR> {
    static __device__ __forceinline__ int col(int lr, int j) { return 4 * lr + 4 * LPR * (j >> 2) + (j & 3); }
    static __device__ __forceinline__ void load(const float *row, int lr, float (&s)[8]) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + col(lr, 4 * m)));
#pragma unroll
            for (int e = 0; e < 4; ++e) s[4 * m + e] = x[e];
        }
    }
    static __device__ __forceinline__ void store(float *row, int lr, const float (&w)[8]) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const f32x4 x = {w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]};
            __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(row + col(lr, 4 * m)));
        }
    }
};
template <int LPR> struct StateLane<bf16, LPR> {
    static __device__ __forceinline__ int col(int lr, int j) { return 8 * lr + j; }
    static __device__ __forceinline__ void load(const bf16 *row, int lr, float (&s)[8]) {
        const bf16x8 x = *reinterpret_cast<const bf16x8 *>(row + 8 * lr);
#pragma unroll
        for (int j = 0; j < 8; ++j) s[j] = static_cast<float>(x[j]);
    }
    static __device__ __forceinline__ void store(bf16 *row, int lr, const float (&w)[8]) {
        bf16x8 x;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = static_cast<bf16>(w[j]);  // round to nearest even
        __builtin_nontemporal_store(x, reinterpret_cast<bf16x8 *>(row + 8 * lr));
    }
};

// Sum of x over the LPR consecutive lanes of a row (LPR = 2, 4, 8 or 16; rows
// aligned to LPR), on DPP lane moves (no trip through the LDS crossbar, as
// a shuffle takes). Each step adds the value of a partner lane from a group
// whose lanes all hold the same partial sum: quads by xor 1 and xor 2, then
// half-rows by mirroring within 8 lanes, then rows by mirroring within 16.
template <int Ctrl> __device__ __forceinline__ float dpp_mov(float y) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, y), Ctrl, 0xf, 0xf, false));
}
template <int LPR> __device__ __forceinline__ float row_sum(float x) {
    static_assert(LPR == 2 || LPR == 4 || LPR == 8 || LPR == 16, "row width");
    x += dpp_mov<0xB1>(x);                         // quad_perm [1, 0, 3, 2]: lane ^ 1
    if constexpr (LPR >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]: lane ^ 2
    if constexpr (LPR >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror: lane i <- 7 - i
    if constexpr (LPR >= 16) x += dpp_mov<0x140>(x); // row_mirror: lane i <- 15 - i
    return x;
}

// The arithmetic below is shared by both decode kernels (with explicit fused
// multiply-adds, so that the compiler cannot contract it differently in
// each): they leave bit-identical states.
template <int LPR> __device__ __forceinline__ float lane_group_sum(float x) { return row_sum<LPR>(x); }
template <int LPR>
__device__ __forceinline__ float row_dot(const float (&s)[8], const float (&x)[8]) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_fmaf(s[j], x[j], acc);
    return lane_group_sum<LPR>(acc);
}
template <int LPR>
__device__ __forceinline__ float key_query_dot(const float (&kk)[8], const float (&qq)[8]) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_fmaf(kk[j], qq[j], acc);
    return lane_group_sum<LPR>(acc);
}
// u = b (v - a sk);  o = scale (a sq + kq u);  S_new = a S + u k^T (stored).
__device__ __forceinline__ float write_strength(float beta, float a, float vv, float sk) {
    return beta * __builtin_fmaf(-a, sk, vv);
}
__device__ __forceinline__ float row_output(float scale, float a, float sq, float kq, float u) {
    return scale * __builtin_fmaf(a, sq, kq * u);
}
template <typename SE, int LPR>
__device__ __forceinline__ void store_row(SE *row, int lr, const float (&s)[8], const float (&kk)[8], float a,
                                          float u) {
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = __builtin_fmaf(a, s[j], u * kk[j]);
    StateLane<SE, LPR>::store(row, lr, w);
}

// k and q at the lane's state columns.
template <typename E, typename SE, int LPR>
__device__ __forceinline__ void load_kq(const E *kp, const E *qp, int lr, float (&kk)[8], float (&qq)[8]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int c = StateLane<SE, LPR>::col(lr, 4 * m);
        load4<E>(kp + c, kk + 4 * m);
        load4<E>(qp + c, qq + 4 * m);
    }
}

// kSlots: state_slots given. Without them sequence b uses slot b (the host
// has checked num_slots >= batch), so the kernel neither reads a slot nor
// branches on one before its state loads.
template <typename E, typename G, typename SE, int DK, int DV, bool kSlots>
__global__ __launch_bounds__((DecodeShape<SE, DK, DV>::THREADS)) void gdn_decode_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const G *__restrict__ gate_g, const G *__restrict__ gate_b,
    SE *__restrict__ state, const int32_t *__restrict__ slots, int32_t num_slots,
    E *__restrict__ out, int32_t hk, int32_t hv, float scale)
{
    typedef DecodeShape<SE, DK, DV> SH;
    typedef StateLane<SE, SH::LPR> SL;
    constexpr int LPR = SH::LPR, RPP = SH::RPP, NRL = SH::NRL, ROWS = SH::ROWS, SLICES = SH::SLICES;

    const int bhs = blockIdx.x;
    const int bh = bhs / SLICES;
    const int row0 = (bhs - bh * SLICES) * ROWS;
    const int b = bh / hv;
    const int h = bh - b * hv;
    const int kh = h / (hv / hk);
    const int tid = threadIdx.x;
    const int lr = tid % LPR;
    const int r0 = row0 + tid / LPR;  // this lane group's rows: r0 + p RPP, p < NRL

    const int slot = kSlots ? slots[b] : b;
    E *o_row = out + ((size_t)b * hv + h) * DV;
    if (kSlots && (slot < 0 || slot >= num_slots)) {
#pragma unroll
        for (int p = 0; p < NRL; ++p)
            if (r0 + p * RPP < DV && lr == 0) o_row[r0 + p * RPP] = from_f32<E>(0.0f);
        return;
    }
    SE *S = state + ((size_t)slot * hv + h) * (size_t)(DV * DK);

    // State row pieces first: the bulk of the bytes, all loads in flight.
    float s[NRL][8];
#pragma unroll
    for (int p = 0; p < NRL; ++p) {
#pragma unroll
        for (int j = 0; j < 8; ++j) s[p][j] = 0.f;
        if (r0 + p * RPP < DV) SL::load(S + (size_t)(r0 + p * RPP) * DK, lr, s[p]);
    }

    float kk[8], qq[8];
    load_kq<E, SE, LPR>(k + ((size_t)b * hk + kh) * DK, q + ((size_t)b * hk + kh) * DK, lr, kk, qq);
    const float a = expf(static_cast<float>(gate_g[(size_t)b * hv + h]));
    const float beta = static_cast<float>(gate_b[(size_t)b * hv + h]);
    float vv[NRL];
#pragma unroll
    for (int p = 0; p < NRL; ++p)
        vv[p] = r0 + p * RPP < DV ? static_cast<float>(v[((size_t)b * hv + h) * DV + r0 + p * RPP]) : 0.f;

    const float kq = key_query_dot<LPR>(kk, qq);
#pragma unroll
    for (int p = 0; p < NRL; ++p) {
        const int row = r0 + p * RPP;
        const float sk = row_dot<LPR>(s[p], kk);
        const float sq = row_dot<LPR>(s[p], qq);
        if (row < DV) {
            const float u = write_strength(beta, a, vv[p], sk);
            if (lr == 0) o_row[row] = from_f32<E>(row_output(scale, a, sq, kq, u));
            store_row<SE, LPR>(S + (size_t)row * DK, lr, s[p], kk, a, u);
        }
    }
}

// ---------------------------------------------------------------------------
// Decode with the output normalisation fused in
// ---------------------------------------------------------------------------
//
// The recurrent update and the normalisation that follows it, in one launch
// (the pages fuse the two: section "Reduire le trafic intermediaire et
// d'etat"): per (sequence, value head)
// the output row o (dv values) becomes
//     y_i = o_i w_i / sqrt(mean_j o_j^2 + eps),
// which needs every row of that head's state. So one workgroup owns a whole
// (b, h) state: its lanes form groups of LPR lanes as in the plain kernel,
// and each group holds NRL rows, RPP rows apart (d = 128: 1024 threads, two
// rows per group; measured at B = 64 as fast as the plain kernel, where 512
// threads with four rows each, or 256 with eight, hold more registers per
// lane, fewer waves per CU, and run 10 to 17% slower). The row work and the
// memory pattern are the plain kernel's; the row outputs stay in registers
// while the workgroup sums their squares (wave butterflies, then LDS across
// waves, one barrier), and only the normalised row is written. The
// unnormalised output never goes to memory.
template <int DK, int DV> struct DecodeNormShape {
    static constexpr int LPR = DK / 8;                                  // lanes per state row
    static constexpr int NRL = DV * LPR > 1024 ? DV * LPR / 1024 : 1;   // rows per lane group
    static constexpr int THREADS = DV * LPR / NRL < 64 ? 64 : DV * LPR / NRL;
    static constexpr int RPP = THREADS / LPR;                           // rows per pass
    static constexpr int WAVES = THREADS / 64;
    static_assert(RPP * NRL >= DV, "every row has a lane group");
};

template <typename E, typename G, typename SE, int DK, int DV, bool kSlots>
__global__ __launch_bounds__((DecodeNormShape<DK, DV>::THREADS)) void gdn_decode_norm_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const G *__restrict__ gate_g, const G *__restrict__ gate_b,
    SE *__restrict__ state, const int32_t *__restrict__ slots, int32_t num_slots,
    E *__restrict__ out, int32_t hk, int32_t hv, float scale,
    const float *__restrict__ norm_w, float eps)
{
    typedef DecodeNormShape<DK, DV> SH;
    typedef StateLane<SE, SH::LPR> SL;
    constexpr int LPR = SH::LPR, NRL = SH::NRL, RPP = SH::RPP, WAVES = SH::WAVES;
    __shared__ float s_part[WAVES];

    const int bh = blockIdx.x;
    const int b = bh / hv;
    const int h = bh - b * hv;
    const int kh = h / (hv / hk);
    const int tid = threadIdx.x;
    const int lr = tid % LPR;
    const int r0 = tid / LPR;

    const int slot = kSlots ? slots[b] : b;
    E *o_row = out + ((size_t)b * hv + h) * DV;
    if (kSlots && (slot < 0 || slot >= num_slots)) {  // the same for the whole workgroup
#pragma unroll
        for (int p = 0; p < NRL; ++p)
            if (r0 + p * RPP < DV && lr == 0) o_row[r0 + p * RPP] = from_f32<E>(0.0f);
        return;
    }
    SE *S = state + ((size_t)slot * hv + h) * (size_t)(DV * DK);

    float s[NRL][8];
#pragma unroll
    for (int p = 0; p < NRL; ++p) {
        const int row = r0 + p * RPP;
#pragma unroll
        for (int j = 0; j < 8; ++j) s[p][j] = 0.f;
        if (row < DV) SL::load(S + (size_t)row * DK, lr, s[p]);
    }

    float kk[8], qq[8];
    load_kq<E, SE, LPR>(k + ((size_t)b * hk + kh) * DK, q + ((size_t)b * hk + kh) * DK, lr, kk, qq);
    const float a = expf(static_cast<float>(gate_g[(size_t)b * hv + h]));
    const float beta = static_cast<float>(gate_b[(size_t)b * hv + h]);
    float vv[NRL];
#pragma unroll
    for (int p = 0; p < NRL; ++p)
        vv[p] = r0 + p * RPP < DV ? static_cast<float>(v[((size_t)b * hv + h) * DV + r0 + p * RPP]) : 0.f;

    const float kq = key_query_dot<LPR>(kk, qq);
    float o[NRL];
    float part = 0.f;  // sum of squares of this lane group's outputs (lane lr == 0 only)
#pragma unroll
    for (int p = 0; p < NRL; ++p) {
        const int row = r0 + p * RPP;
        const float sk = row_dot<LPR>(s[p], kk);
        const float sq = row_dot<LPR>(s[p], qq);
        const float u = write_strength(beta, a, vv[p], sk);
        o[p] = row_output(scale, a, sq, kq, u);
        if (row < DV) {
            store_row<SE, LPR>(S + (size_t)row * DK, lr, s[p], kk, a, u);
            if (lr == 0) part = __builtin_fmaf(o[p], o[p], part);
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) part += __shfl_xor(part, off);
    if ((tid & 63) == 0) s_part[tid >> 6] = part;
    __syncthreads();
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) total += s_part[w];
    const float r = 1.0f / sqrtf(total * (1.0f / DV) + eps);
#pragma unroll
    for (int p = 0; p < NRL; ++p) {
        const int row = r0 + p * RPP;
        if (row < DV && lr == 0) o_row[row] = from_f32<E>(o[p] * r * norm_w[row]);
    }
}

template <typename E, typename G, typename SE, int D, bool kSlots>
static hipError_t launch_decode_s(const DecodeArgs &A, hipStream_t st) {
    SE *state = static_cast<SE *>(A.state);
    if (A.norm_w) {
        typedef DecodeNormShape<D, D> SH;
        const dim3 grid((unsigned)A.batch * (unsigned)A.hv), block(SH::THREADS);
        return launch_kernel(kDecodeNorm, gdn_decode_norm_kernel<E, G, SE, D, D, kSlots>, grid, block, 0, st,
                             (const E *)A.q, (const E *)A.k, (const E *)A.v,
                             (const G *)A.g, (const G *)A.beta, state, A.slots, A.num_slots,
                             (E *)A.out, A.hk, A.hv, A.scale, A.norm_w, A.norm_eps);
    }
    typedef DecodeShape<SE, D, D> SH;
    const dim3 grid((unsigned)A.batch * (unsigned)A.hv * (unsigned)SH::SLICES), block(SH::THREADS);
    return launch_kernel(kDecode, gdn_decode_kernel<E, G, SE, D, D, kSlots>, grid, block, 0, st,
                         (const E *)A.q, (const E *)A.k, (const E *)A.v,
                         (const G *)A.g, (const G *)A.beta, state, A.slots, A.num_slots,
                         (E *)A.out, A.hk, A.hv, A.scale);
}

template <typename E, typename G, typename SE, int D>
static hipError_t launch_decode_t(const DecodeArgs &A, hipStream_t st) {
    return A.slots ? launch_decode_s<E, G, SE, D, true>(A, st) : launch_decode_s<E, G, SE, D, false>(A, st);
}

template <typename E, typename G, typename SE>
static hipError_t launch_decode_d(const DecodeArgs &A, hipStream_t st) {
    switch (A.d) {
    case 16: return launch_decode_t<E, G, SE, 16>(A, st);
    case 32: return launch_decode_t<E, G, SE, 32>(A, st);
    case 64: return launch_decode_t<E, G, SE, 64>(A, st);
    case 128: return launch_decode_t<E, G, SE, 128>(A, st);
    default: return hipErrorInvalidValue;
    }
}

// bf16 state storage is built for bf16 I/O only (fp32 I/O is the accuracy
// mode, where a rounded state would defeat its purpose).
hipError_t launch_decode(const DecodeArgs &A, hipStream_t st) {
    if (A.io_bf16) {
        if (A.state_bf16)
            return A.gate_bf16 ? launch_decode_d<bf16, bf16, bf16>(A, st) : launch_decode_d<bf16, float, bf16>(A, st);
        return A.gate_bf16 ? launch_decode_d<bf16, bf16, float>(A, st) : launch_decode_d<bf16, float, float>(A, st);
    }
    if (A.state_bf16) return hipErrorInvalidValue;
    return A.gate_bf16 ? launch_decode_d<float, bf16, float>(A, st) : launch_decode_d<float, float, float>(A, st);
}

// ---------------------------------------------------------------------------
// Token-by-token prefill (chunk = 1)
// ---------------------------------------------------------------------------
//
// The recurrence evaluated one token at a time, the first of the two
// evaluations the pages name ("Qwen cree trois formes de charges de travail
// distinctes"): it exposes no matrix products, but it has no fixed costs
// either (no preparation pass, no workspace), so short prompts and
// multi-token steps finish sooner than through the chunked form. A workgroup
// holds ROWS rows of one (sequence, value head) state in registers and
// applies the decode update for every token of the sequence in order,
// writing each token's output and, at the end, the final state. Row sums use
// DPP within the LPR lanes of a row. Vector-memory instructions bound it, as
// they bound the chunked scan: per token a wave loads only its 16-byte pieces
// of k and q (kNext tokens ahead); gates and v come in one load per lane for
// 64 tokens at a time and are broadcast with readlane.


// A lane's 8 consecutive elements of one token's k or q, as loaded.
template <typename E> struct Vec8;
template <> struct Vec8<bf16> {
    bf16x8 x;
    __device__ __forceinline__ void load(const bf16 *p) { x = *reinterpret_cast<const bf16x8 *>(p); }
    __device__ __forceinline__ float operator[](int i) const { return static_cast<float>(x[i]); }
};
template <> struct Vec8<float> {
    f32x4 x[2];
    __device__ __forceinline__ void load(const float *p) {
        x[0] = *reinterpret_cast<const f32x4 *>(p);
        x[1] = *reinterpret_cast<const f32x4 *>(p + 4);
    }
    __device__ __forceinline__ float operator[](int i) const { return x[i >> 2][i & 3]; }
};

// A workgroup covers ROWS rows of one (sequence, value head) state; a row's
// DK elements are spread over LPR = DK / 8 consecutive lanes, 8 consecutive
// elements each, so that a lane's part of k or q is one 16-byte load (bf16).
// Rows: each group of LPR lanes holds NRL rows, RPP rows apart. With two,
// a lane converts its k and q pieces and forms k.q once for both rows, which
// cuts the VALU work per row and token by about a third; it halves the
// workgroups, so it pays when there are many (batches of sequences) and not
// for one sequence, where the per-token latency of one workgroup is the
// time (launch_token_scan chooses).
template <int DK, int DV, int NRL_> struct TokenScanShape {
    static constexpr int LPR = DK / 8;
    static constexpr int RPP = 256 / LPR;  // rows per pass of the workgroup
    static constexpr int NRL = RPP * NRL_ > DV ? (DV + RPP - 1) / RPP : NRL_;  // rows per lane group
    static constexpr int ROWS = RPP * NRL;  // rows per workgroup
    static constexpr int RPW = 64 / LPR;    // rows per wave and pass
    static constexpr int SLICES = (DV + ROWS - 1) / ROWS;
};

template <typename E, typename G, typename SE, int DK, int DV, int NRL_>
__global__ __launch_bounds__(256) void gdn_token_scan_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const G *__restrict__ gate_g, const G *__restrict__ gate_b,
    const int32_t *__restrict__ cu, int32_t num_seqs, int32_t total_tokens,
    const SE *__restrict__ s0, SE *__restrict__ sfin, E *__restrict__ out,
    int32_t hk, int32_t hv, float scale)
{
    typedef TokenScanShape<DK, DV, NRL_> SH;
    constexpr int LPR = SH::LPR, RPP = SH::RPP, NRL = SH::NRL, ROWS = SH::ROWS, RPW = SH::RPW,
                  SLICES = SH::SLICES;
    constexpr int kNext = 3;  // tokens whose k and q are in flight ahead of the one applied

    const int bhs = blockIdx.x;
    const int bh = bhs / SLICES;
    const int row0 = (bhs - bh * SLICES) * ROWS;
    const int n = bh / hv;
    const int h = bh - n * hv;
    const int kh = h / (hv / hk);
    const int tid = threadIdx.x, lane = tid & 63;
    const int lr = tid % LPR;
    const int r1 = row0 + tid / LPR;            // this lane group's rows: r1 + p RPP, p < NRL
    const int wrow0 = row0 + (tid >> 6) * RPW;  // first row of this wave in pass 0

    // The state rows first: they do not depend on the sequence's bounds, so
    // their latency overlaps that of cu_seqlens.
    const size_t sbase = ((size_t)n * hv + h) * (size_t)(DV * DK) + 8 * lr;
    f32x4 s[NRL][2];
#pragma unroll
    for (int p = 0; p < NRL; ++p) {
        s[p][0] = s[p][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s0 && r1 + p * RPP < DV) {
            s[p][0] = load4f<SE>(s0 + sbase + (size_t)(r1 + p * RPP) * DK);
            s[p][1] = load4f<SE>(s0 + sbase + (size_t)(r1 + p * RPP) * DK + 4);
        }
    }

    // Sequence n's tokens [lo, hi): offsets clamped into [0, T] and made
    // non-decreasing, as on the chunked path. Each wave reduces the maxima
    // itself (strided over the lanes, then a butterfly).
    auto clampT = [&](int x) { return min(max(x, 0), total_tokens); };
    const int b0 = clampT(cu[0]);
    int hi = b0, lo = b0;
    for (int j = lane; j <= n; j += 64) {
        const int e = clampT(cu[j + 1]);
        hi = max(hi, e);
        if (j < n) lo = max(lo, e);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        hi = max(hi, __shfl_xor(hi, off));
        lo = max(lo, __shfl_xor(lo, off));
    }
    // uniform across the wave; saying so keeps the token loop's branches scalar
    hi = __builtin_amdgcn_readfirstlane(hi);
    lo = __builtin_amdgcn_readfirstlane(lo);

    // Per block of 64 tokens, lane l loads token tb + l's gates and, for each
    // of the wave's RPW rows of every pass, its v; a token's values are then
    // read with readlane. Loads are unconditional (tokens clamped into
    // [lo, hi)) so that the compiler counts outstanding loads exactly.
    struct Block {
        G g, b;
        E vr[NRL][RPW];
    };
    auto load_block = [&](Block &bl, int tb) {
        const int t = min(tb + lane, hi - 1);
        bl.g = gate_g[(size_t)t * hv + h];
        bl.b = gate_b[(size_t)t * hv + h];
#pragma unroll
        for (int p = 0; p < NRL; ++p)
#pragma unroll
            for (int r = 0; r < RPW; ++r)
                bl.vr[p][r] = v[((size_t)t * hv + h) * DV + min(wrow0 + p * RPP + r, DV - 1)];
    };
    auto lane_f = [](float x, int i) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), i));
    };
    const int myr = lane / LPR;  // this lane's row within the wave

    struct KQ {
        Vec8<E> k, q;
    };
    auto load_kq = [&](KQ &x, int t) {
        const size_t tk = ((size_t)t * hk + kh) * DK + 8 * lr;
        x.k.load(k + tk);
        x.q.load(q + tk);
    };
    // One token: k, q converted and k.q formed once for the lane's rows.
    auto apply = [&](const KQ &x, float a, float beta, const float (&vv)[NRL], int t) {
        float kk[8], qq[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kk[e] = x.k[e];
            qq[e] = x.q[e];
        }
        float kq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) kq += kk[e] * qq[e];
        kq = row_sum<LPR>(kq);
#pragma unroll
        for (int p = 0; p < NRL; ++p) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sk += s[p][e >> 2][e & 3] * kk[e];
                sq += s[p][e >> 2][e & 3] * qq[e];
            }
            sk = row_sum<LPR>(sk);
            sq = row_sum<LPR>(sq);
            const float u = beta * (vv[p] - a * sk);
            const int row = r1 + p * RPP;
            if (row < DV && lr == 0) out[((size_t)t * hv + h) * DV + row] = from_f32<E>(scale * (a * sq + kq * u));
#pragma unroll
            for (int e = 0; e < 8; ++e) s[p][e >> 2][e & 3] = a * s[p][e >> 2][e & 3] + u * kk[e];
        }
    };

    // Sequences of up to kShort tokens (multi-token steps): each token's
    // inputs loaded directly, all before the first is applied, with a load
    // count fixed per length; the 64-token blocks and the prefetch ring would
    // load mostly duplicates here.
    constexpr int kShort = 4;
    auto short_run = [&](auto lc) {
        constexpr int L = decltype(lc)::value;
        KQ in[L];
        float ga[L], gb[L], gv[L][NRL];
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int t = lo + i;
            load_kq(in[i], t);
            ga[i] = static_cast<float>(gate_g[(size_t)t * hv + h]);
            gb[i] = static_cast<float>(gate_b[(size_t)t * hv + h]);
#pragma unroll
            for (int p = 0; p < NRL; ++p)
                gv[i][p] = static_cast<float>(v[((size_t)t * hv + h) * DV + min(r1 + p * RPP, DV - 1)]);
        }
#pragma unroll
        for (int i = 0; i < L; ++i) apply(in[i], expf(ga[i]), gb[i], gv[i], lo + i);
    };
    const int len = hi - lo;
    if (len > 0 && len <= kShort) {
        if (len == 1) short_run(std::integral_constant<int, 1>());
        else if (len == 2) short_run(std::integral_constant<int, 2>());
        else if (len == 3) short_run(std::integral_constant<int, 3>());
        else short_run(std::integral_constant<int, 4>());
    } else if (len > kShort) {
        constexpr int R = kNext + 1;
        KQ in[R];
        Block cur, nxt;
        load_block(cur, lo);
        __builtin_amdgcn_sched_barrier(0);
        // In stage order: the loop's waits assume stage 0 was issued first.
#pragma unroll
        for (int i = 0; i < kNext; ++i) {
            load_kq(in[i], min(lo + i, hi - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int tb = lo; tb < hi; tb += 64) {
            load_block(nxt, min(tb + 64, hi - 1));
            // this block's gates and v as floats, per lane
            float ga = 0.f, gb = 0.f, gv[NRL][RPW];
            ga = expf(static_cast<float>(cur.g));
            gb = static_cast<float>(cur.b);
#pragma unroll
            for (int p = 0; p < NRL; ++p)
#pragma unroll
                for (int r = 0; r < RPW; ++r) gv[p][r] = static_cast<float>(cur.vr[p][r]);
            // 64 tokens (16 groups of R = 4), stage u % R holding token t + u
            for (int t = tb; t < min(tb + 64, hi); t += R) {
#pragma unroll
                for (int u = 0; u < R; ++u) {
                    load_kq(in[(u + kNext) % R], min(t + u + kNext, hi - 1));
                    if (t + u < hi) {
                        const int i = t + u - tb;
                        float vv[NRL];
#pragma unroll
                        for (int p = 0; p < NRL; ++p) {
                            vv[p] = lane_f(gv[p][0], i);
#pragma unroll
                            for (int r = 1; r < RPW; ++r) {
                                const float vr = lane_f(gv[p][r], i);
                                vv[p] = myr == r ? vr : vv[p];
                            }
                        }
                        apply(in[u], lane_f(ga, i), lane_f(gb, i), vv, t + u);
                    }
                }
            }
            cur = nxt;
        }
    }

    if (sfin) {
#pragma unroll
        for (int p = 0; p < NRL; ++p) {
            if (r1 + p * RPP < DV) {
                store4<SE>(sfin + sbase + (size_t)(r1 + p * RPP) * DK, s[p][0]);
                store4<SE>(sfin + sbase + (size_t)(r1 + p * RPP) * DK + 4, s[p][1]);
            }
        }
    }
}

// Rows per lane group of the token scan: two when the call has at least
// kTokenScanPairedWgs workgroups with one (about two per CU), else one.
constexpr int64_t kTokenScanPairedWgs = 1024;

template <typename E, typename G, typename SE, int D, int NRL>
static hipError_t launch_token_scan_n(const PrefillArgs &A, hipStream_t st) {
    const dim3 grid((unsigned)A.num_seqs * (unsigned)A.hv * (unsigned)TokenScanShape<D, D, NRL>::SLICES), block(256);
    return launch_kernel(kTokenScan, gdn_token_scan_kernel<E, G, SE, D, D, NRL>, grid, block, 0, st,
                         (const E *)A.q, (const E *)A.k, (const E *)A.v, (const G *)A.g, (const G *)A.beta,
                         A.cu, A.num_seqs, (int32_t)A.total_tokens, (const SE *)A.s0, (SE *)A.s_final,
                         (E *)A.out, A.hk, A.hv, A.scale);
}

template <typename E, typename G, typename SE, int D>
static hipError_t launch_token_scan_t(const PrefillArgs &A, hipStream_t st) {
    if constexpr (TokenScanShape<D, D, 2>::NRL == 2) {
        const int64_t wgs = (int64_t)A.num_seqs * A.hv * TokenScanShape<D, D, 1>::SLICES;
        if (wgs >= kTokenScanPairedWgs) return launch_token_scan_n<E, G, SE, D, 2>(A, st);
    }
    return launch_token_scan_n<E, G, SE, D, 1>(A, st);
}

template <typename E, typename G, typename SE>
static hipError_t launch_token_scan_d(const PrefillArgs &A, hipStream_t st) {
    switch (A.d) {
    case 16: return launch_token_scan_t<E, G, SE, 16>(A, st);
    case 32: return launch_token_scan_t<E, G, SE, 32>(A, st);
    case 64: return launch_token_scan_t<E, G, SE, 64>(A, st);
    case 128: return launch_token_scan_t<E, G, SE, 128>(A, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_token_scan(const PrefillArgs &A, hipStream_t st) {
    if (A.io_bf16) {
        if (A.state_bf16)
            return A.gate_bf16 ? launch_token_scan_d<bf16, bf16, bf16>(A, st)
                               : launch_token_scan_d<bf16, float, bf16>(A, st);
        return A.gate_bf16 ? launch_token_scan_d<bf16, bf16, float>(A, st)
                           : launch_token_scan_d<bf16, float, float>(A, st);
    }
    if (A.state_bf16) return hipErrorInvalidValue;
    return A.gate_bf16 ? launch_token_scan_d<float, bf16, float>(A, st) : launch_token_scan_d<float, float, float>(A, st);
}

}  // namespace gdn

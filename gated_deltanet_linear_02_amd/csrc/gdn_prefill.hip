// gdn_prefill.hip -- chunked prefill of the Gated DeltaNet layer (gfx950).
//
// The recurrence can be evaluated token by token or reorganised into chunks
// that expose matrix products and token-level parallelism ("Optimiser
// l'inference sur appareil pour Apple Silicon", section "Qwen cree trois
// formes de charges de travail distinctes"). This file does the latter.
//
// Chunk form. Inside a chunk of C tokens that starts from state S0, with the
// cumulative log-decay c_t = g_1 + ... + g_t and gamma_t = exp(c_t):
//     A[t][s] = b_t exp(c_t - c_s) (k_t . k_s)          (s < t)
//     T       = (I + A)^-1                                (unit lower triangular)
//     U       = T (diag(b) V - diag(b gamma) K S0^T)      (row t is the write u_t)
//     O       = scale diag(gamma) Q S0^T + P U,   P[t][s] = scale exp(c_t - c_s) (q_t . k_s), s <= t
//     S_end^T = gamma_C S0^T + K^T diag(exp(c_C - c)) U
// which follows from unrolling S_t = a_t S_{t-1} + u_t k_t^T with
// u_t = b_t (v_t - a_t S_{t-1} k_t).
//
// Three kernels, enqueued back to back on the caller's stream:
//   1. schedule  cu_seqlens -> clamped monotone sequence bounds, chunk table,
//                sequences ordered longest first (all on the device: no host
//                read of cu_seqlens, as in the GPU-resident routing of section
//                "Maintenir le routage des experts sur le GPU").
//   2. prep      per (chunk, query/key head), fully parallel: K K^T and Q K^T
//                on MFMA, then per value head the gate prefix sums, A, the
//                blocked triangular inverse T and P. Writes T, P, the gate
//                vectors and the scan's K, Q, K^T operands (fragment order).
//   3. scan      per (sequence, value head, slice of R value rows): the only
//                sequential part. The state slice stays on chip (registers for
//                the fp32 master, LDS for the MFMA operand copy) for the whole
//                sequence and is written once at the end, the design of
//                section "Maintenir l'etat recurrent sur la puce"; per-chunk
//                states never go to memory. Value rows of S evolve
//                independently, which is what allows the slicing.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

#include <atomic>

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

// ---------------------------------------------------------------------------
// 2. Chunk preparation
// ---------------------------------------------------------------------------
//
// One workgroup per (chunk, value head). It computes the chunk's gate
// vectors, A and P from K K^T and Q K^T (MFMA), and T = (I + A)^-1 by blocks
// of 16:
//   diagonal blocks    (I + A_bb)^-1 by forward substitution, one wave each;
//   blocks below       T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj, one wave per
//                      block column j, on fp32 MFMA,
// which is (I + A) T = I written blockwise. All operands the scan needs are
// written in MFMA fragment order (see frag_off), so that every fragment the
// scan loads is one contiguous run: T and P per value head, and (by the first
// value head of each query/key head) K, Q and K^T.

template <typename E> struct IsBf16 { static constexpr bool value = false; };
template <> struct IsBf16<bf16> { static constexpr bool value = true; };

// Element offset of lane `lane`'s part of fragment f in fragment order: a
// matrix A [M][K] is stored as fragments f = rt * (K / KW) + kb, each holding
// for lane l the KPL elements A[16 rt + l%16][kb KW + KPL (l/16) + j].
template <typename MM> __device__ __forceinline__ size_t frag_off(int f, int lane) {
    return ((size_t)f * 64 + lane) * MM::KPL;
}

template <typename E, int C, int DK>
struct PrepSmem {
    static constexpr int PE = Pad<E>::value;
    static constexpr int LDK = DK + PE;  // staged K and Q rows (E)
    static constexpr int LDC = C + 4;    // fp32 C x C arrays, 16-byte aligned rows
    // Region X: K and Q tiles (phases 1-3), then A and T (phase 4).
    static constexpr size_t off_K = 0;
    static constexpr size_t off_Q = off_K + (size_t)C * LDK * sizeof(E);
    static constexpr size_t kq_end = off_Q + (size_t)C * LDK * sizeof(E);
    static constexpr size_t off_A = 0;
    static constexpr size_t off_T = off_A + (size_t)C * LDC * sizeof(float);
    static constexpr size_t at_end = off_T + (size_t)C * LDC * sizeof(float);
    // Region Y: raw K K^T and Q K^T.
    static constexpr size_t off_G = ((kq_end > at_end ? kq_end : at_end) + 15) & ~(size_t)15;
    static constexpr size_t off_P0 = off_G + (size_t)C * LDC * sizeof(float);
    static constexpr size_t off_c = off_P0 + (size_t)C * LDC * sizeof(float);
    static constexpr size_t off_b = off_c + (size_t)C * sizeof(float);
    static constexpr size_t bytes = off_b + (size_t)C * sizeof(float);
};

template <typename M> __device__ __forceinline__ typename M::Frag zero_frag() {
    typename M::Frag z;
    if constexpr (std::is_same<typename M::Frag, float>::value) {
        z = 0.f;
    } else {
#pragma unroll
        for (int i = 0; i < (int)(sizeof(z) / 2); ++i) z[i] = static_cast<bf16>(0.f);
    }
    return z;
}

template <typename G> __device__ __forceinline__ float gate_load(const G *p, size_t i) {
    return static_cast<float>(p[i]);
}

// acc += X[xr.., xc..] (16x16) * Y[yr.., yc..] (16x16), fp32 LDS operands
// with row stride ld, on v_mfma_f32_16x16x4_f32.
__device__ __forceinline__ f32x4 mm16_f32(f32x4 acc, const float *X, int xr, int xc, const float *Y, int yr,
                                          int yc, int ld, int lane) {
    const int ln = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[(xr + ln) * ld + xc + 4 * kb + g],
                                                   Y[(yr + 4 * kb + g) * ld + yc + ln], acc, 0, 0, 0);
    return acc;
}

template <typename MM> __device__ __forceinline__ void frag_set(typename MM::Frag &f, int e, float x) {
    if constexpr (MM::KPL == 1) f = x; else f[e] = static_cast<bf16>(x);
}

template <typename E, typename G, int C, int DK>
__global__ __launch_bounds__(256) void gdn_prep_kernel(
    const E *__restrict__ q, const E *__restrict__ k,
    const G *__restrict__ gate_g, const G *__restrict__ gate_b,
    const int32_t *__restrict__ bounds, const int32_t *__restrict__ chunk_seq,
    const int32_t *__restrict__ chunk_tok0, const int32_t *__restrict__ counters,
    E *__restrict__ tmat, E *__restrict__ pmat, E *__restrict__ kmat, E *__restrict__ qmat,
    E *__restrict__ ktmat, f32x4 *__restrict__ gates, float *__restrict__ gammac,
    int32_t hk, int32_t hv, float scale)
{
    typedef PrepSmem<E, C, DK> L;
    typedef Mma<E, DK> MD;
    typedef Mma<E, C> MC;
    constexpr int NB = C / 16, MT = DK / 16;
    constexpr int KBD = DK / MD::KW, KBC = C / MC::KW;
    constexpr int LDK = L::LDK, LDC = L::LDC;
    constexpr int EPV = 16 / sizeof(E), VPR = DK / EPV;

    extern __shared__ __align__(16) char smem[];
    E *sK = reinterpret_cast<E *>(smem + L::off_K);
    E *sQ = reinterpret_cast<E *>(smem + L::off_Q);
    float *sA = reinterpret_cast<float *>(smem + L::off_A);
    float *sT = reinterpret_cast<float *>(smem + L::off_T);
    float *sGk = reinterpret_cast<float *>(smem + L::off_G);
    float *sP0 = reinterpret_cast<float *>(smem + L::off_P0);
    float *sc = reinterpret_cast<float *>(smem + L::off_c);
    float *sb = reinterpret_cast<float *>(smem + L::off_b);

    const int ci = blockIdx.x, kh = blockIdx.y;
    if (ci >= counters[0]) return;
    const int group = hv / hk;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, ln = lane & 15;
    const int n = chunk_seq[ci];
    const int t0 = chunk_tok0[ci];
    const int len = min(C, bounds[n + 1] - t0);
    const size_t kq0 = ((size_t)ci * hk + kh) * (size_t)(C * DK);
    const size_t ld = (size_t)hk * DK;

    // ---- 1. K and Q rows into LDS (zero past the end of the sequence)
    for (int i = tid; i < C * VPR; i += 256) {
        const int r = i / VPR, cv = i - r * VPR;
        const size_t src = (size_t)(t0 + r) * ld + (size_t)kh * DK + cv * EPV;
        st16(sK + r * LDK + cv * EPV, r < len ? ld16(k + src) : zero16());
        st16(sQ + r * LDK + cv * EPV, r < len ? ld16(q + src) : zero16());
    }
    __syncthreads();

    // ---- 2. K, Q and K^T in fragment order for the scan
    for (int f = wave; f < NB * KBD; f += 4) {
        const int rt = f / KBD, kb = f - rt * KBD;
        *reinterpret_cast<typename MD::Frag *>(kmat + kq0 + frag_off<MD>(f, lane)) =
            load_frag<MD>(sK, LDK, 16 * rt, kb * MD::KW, lane);
        *reinterpret_cast<typename MD::Frag *>(qmat + kq0 + frag_off<MD>(f, lane)) =
            load_frag<MD>(sQ, LDK, 16 * rt, kb * MD::KW, lane);
    }
    for (int f = wave; f < MT * KBC; f += 4) {
        const int mt = f / KBC, kb = f - mt * KBC;
        typename MC::Frag fr;
#pragma unroll
        for (int e = 0; e < MC::KPL; ++e)  // K^T[m][t] = K[t][m]
            frag_set<MC>(fr, e, to_f32(sK[(kb * MC::KW + MC::KPL * g4 + e) * LDK + 16 * mt + ln]));
        *reinterpret_cast<typename MC::Frag *>(ktmat + kq0 + frag_off<MC>(f, lane)) = fr;
    }

    // ---- 3. Raw K K^T and Q K^T on the lower-triangular 16x16 tiles
    constexpr int NT = NB * (NB + 1) / 2;
    for (int t = wave; t < 2 * NT; t += 4) {
        const int which = t / NT;  // 0: Gram, 1: scores
        int tt = t - which * NT, ti = 0;
        while ((ti + 1) * (ti + 2) / 2 <= tt) ++ti;
        const int tj = tt - ti * (ti + 1) / 2;
        const E *Am = which ? sQ : sK;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb)
            acc = MD::mma(load_frag<MD>(Am, LDK, 16 * ti, kb * MD::KW, lane),
                          load_frag<MD>(sK, LDK, 16 * tj, kb * MD::KW, lane), acc);
        float *dst = which ? sP0 : sGk;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * ti + 4 * g4 + r) * LDC + 16 * tj + ln] = acc[r];
    }
    __syncthreads();

    // ---- 4. Per value head of the group
    for (int hh = 0; hh < group; ++hh) {
        const int h = kh * group + hh;
        const size_t mat0 = ((size_t)ci * hv + h) * (size_t)(C * C);

        // gate prefix sums c_t = g_1 + ... + g_t (C <= 64: one wave); rows past
        // the end of the sequence act as a = 1, b = 0
        if (wave == 0) {
            const bool valid = lane < len;
            float x = valid ? gate_load(gate_g, (size_t)(t0 + lane) * hv + h) : 0.f;
            const float bv = valid ? gate_load(gate_b, (size_t)(t0 + lane) * hv + h) : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (lane >= off) x += y;
            }
            if (lane < C) {
                sc[lane] = x;
                sb[lane] = bv;
            }
        }
        __syncthreads();
        if (tid < C) {
            const float last = sc[C - 1];
            const float gam = expf(sc[tid]);
            gates[((size_t)ci * hv + h) * C + tid] =
                f32x4{scale * gam, sb[tid], sb[tid] * gam, expf(last - sc[tid])};
            if (tid == 0) gammac[(size_t)ci * hv + h] = expf(last);
        }

        // A = strict_lower(b_i exp(c_i - c_j) (K K^T)_ij) into LDS
        for (int e = tid; e < C * C; e += 256) {
            const int i = e / C, j = e - i * C;
            sA[i * LDC + j] = j < i ? sb[i] * expf(sc[i] - sc[j]) * sGk[i * LDC + j] : 0.f;
        }
        // P = lower(scale exp(c_i - c_j) (Q K^T)_ij), straight to fragment order
        for (int f = wave; f < NB * KBC; f += 4) {
            const int rt = f / KBC, kb = f - rt * KBC;
            const int i = 16 * rt + ln;
            typename MC::Frag fr;
#pragma unroll
            for (int e = 0; e < MC::KPL; ++e) {
                const int j = kb * MC::KW + MC::KPL * g4 + e;
                frag_set<MC>(fr, e, j <= i ? scale * expf(sc[i] - sc[j]) * sP0[i * LDC + j] : 0.f);
            }
            *reinterpret_cast<typename MC::Frag *>(pmat + mat0 + frag_off<MC>(f, lane)) = fr;
        }
        __syncthreads();

        // diagonal blocks: wave b inverts (I + A_bb) by right-looking forward
        // substitution, lane = column (the four lane groups compute the same
        // columns; the first writes them)
        if (wave < NB) {
            const int base = 16 * wave, col = ln;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = i == col ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < 16; ++s2) {
#pragma unroll
                for (int i = s2 + 1; i < 16; ++i) x[i] -= sA[(base + i) * LDC + base + s2] * x[s2];
            }
            if (g4 == 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sT[(base + i) * LDC + base + col] = x[i];
            }
        }
        __syncthreads();

        // blocks below the diagonal, one wave per block column j:
        //   Z = sum_{m=j}^{i-1} A_im T_mj,  T_ij = -T_ii Z   for i = j+1, ...
        // Z stays in registers: its accumulator layout is used directly as the
        // B operand by pairing contraction index 4g + r with k-step r.
        if (wave < NB - 1) {
            const int j = wave;
            for (int i = j + 1; i < NB; ++i) {
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                for (int m = j; m < i; ++m) z = mm16_f32(z, sA, 16 * i, 16 * m, sT, 16 * m, 16 * j, LDC, lane);
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    t = __builtin_amdgcn_mfma_f32_16x16x4f32(-sT[(16 * i + ln) * LDC + 16 * i + 4 * g4 + r], z[r],
                                                             t, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) sT[(16 * i + 4 * g4 + r) * LDC + 16 * j + ln] = t[r];
            }
        }
        __syncthreads();

        // T in fragment order (blocks above the diagonal are zero)
        for (int f = wave; f < NB * KBC; f += 4) {
            const int rt = f / KBC, kb = f - rt * KBC;
            const int i = 16 * rt + ln;
            typename MC::Frag fr;
#pragma unroll
            for (int e = 0; e < MC::KPL; ++e) {
                const int j = kb * MC::KW + MC::KPL * g4 + e;
                frag_set<MC>(fr, e, (j >> 4) <= rt ? sT[i * LDC + j] : 0.f);
            }
            *reinterpret_cast<typename MC::Frag *>(tmat + mat0 + frag_off<MC>(f, lane)) = fr;
        }
    }
}

// ---------------------------------------------------------------------------
// 3. Chunk-recurrent scan over one (sequence, value head, 16 value rows)
// ---------------------------------------------------------------------------
//
// Four waves per workgroup. Wave w owns the token tiles rt = w, w+4, .. of
// the chunk (for X = K S0^T, Q S0^T, Y, U = T Y and the output) and the
// key tiles mt = w, w+4, .. of the state slice (for its update). Every MFMA
// A operand (K, Q, T, P, K^T) is one contiguous fragment load from the
// workspace, issued two chunks ahead into one of three register stages
// (bf16; fp32 fragments are four times larger and use one); LDS only carries the
// small per-chunk exchanges between waves (the state's operand copy, Y, U,
// diag(delta) U, the gates and the output tile).

constexpr int kSliceRows = 16;

template <typename E, int C, int DK>
struct ScanSmem {
    static constexpr int PE = Pad<E>::value;
    static constexpr int R = kSliceRows;
    static constexpr int LDK = DK + PE;  // rows of length DK
    static constexpr int LDC = C + PE;   // rows of length C
    static constexpr size_t off_S = 0;                                   // [R][LDK]
    static constexpr size_t off_Yt = off_S + (size_t)R * LDK * sizeof(E);  // [R][LDC]
    static constexpr size_t off_Ut = off_Yt + (size_t)R * LDC * sizeof(E);
    static constexpr size_t off_DUt = off_Ut + (size_t)R * LDC * sizeof(E);
    static constexpr size_t off_O = off_DUt + (size_t)R * LDC * sizeof(E);  // [C][R]
    static constexpr size_t off_G = (off_O + (size_t)C * R * sizeof(E) + 15) & ~(size_t)15;  // [2][C] f32x4
    static constexpr size_t bytes = off_G + 2 * (size_t)C * 16;
};

// One wave's operands for one chunk, in registers.
template <typename E, int C, int DK>
struct WaveStage {
    typedef Mma<E, DK> MD;  // contractions over keys
    typedef Mma<E, C> MC;   // contractions over the tokens of a chunk
    static constexpr int RT = C / 16, MT = DK / 16;
    static constexpr int NRW = (RT + 3) / 4, NMW = (MT + 3) / 4;  // tiles per wave
    static constexpr int KBD = DK / MD::KW, KBC = C / MC::KW;

    f32x4 gate;  // gate vector of token row min(lane, C - 1)
    typename MD::Frag kf[NRW][KBD], qf[NRW][KBD];
    typename MC::Frag tf[NRW][KBC], pf[NRW][KBC], ktf[NMW][KBC];
    E vv[NRW][4];
    float gc;

    // All loads are unconditional (tiles and rows clamped into range) so that
    // the compiler counts outstanding loads exactly across the loop; rows past
    // the end of the sequence are masked where they are used. The gate load
    // comes first: it is the first one waited for.
    __device__ __forceinline__ void load(const E *__restrict__ v, const E *__restrict__ tmat,
                                         const E *__restrict__ pmat, const E *__restrict__ kmat,
                                         const E *__restrict__ qmat, const E *__restrict__ ktmat,
                                         const f32x4 *__restrict__ gates, const float *__restrict__ gammac,
                                         int tok0, int clen, int ci, int hk, int kh, int hv, int h, int col0,
                                         int wave, int lane) {
        const int g4 = lane >> 4, ln = lane & 15;
        const size_t ci_h = (size_t)ci * hv + h;
        const size_t mat0 = ci_h * (size_t)(C * C);
        const size_t kq0 = ((size_t)ci * hk + kh) * (size_t)(C * DK);
        gate = gates[ci_h * C + min(lane, C - 1)];
#pragma unroll
        for (int r = 0; r < NRW; ++r) {
            const int rt = min(wave + 4 * r, RT - 1);
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) {
                kf[r][kb] = *reinterpret_cast<const typename MD::Frag *>(kmat + kq0 + frag_off<MD>(rt * KBD + kb, lane));
                qf[r][kb] = *reinterpret_cast<const typename MD::Frag *>(qmat + kq0 + frag_off<MD>(rt * KBD + kb, lane));
            }
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) {
                tf[r][kb] = *reinterpret_cast<const typename MC::Frag *>(tmat + mat0 + frag_off<MC>(rt * KBC + kb, lane));
                pf[r][kb] = *reinterpret_cast<const typename MC::Frag *>(pmat + mat0 + frag_off<MC>(rt * KBC + kb, lane));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int vrow = min(16 * rt + 4 * g4 + i, clen - 1);
                vv[r][i] = v[((size_t)(tok0 + vrow) * hv + h) * DK + col0 + ln];
            }
        }
#pragma unroll
        for (int j = 0; j < NMW; ++j) {
            const int mt = min(wave + 4 * j, MT - 1);
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb)
                ktf[j][kb] = *reinterpret_cast<const typename MC::Frag *>(ktmat + kq0 + frag_off<MC>(mt * KBC + kb, lane));
        }
        gc = gammac[ci_h];
    }

    // This wave's share (rows 16 w .. 16 w + 15) of the gate vectors into LDS.
    __device__ __forceinline__ void put_gates(f32x4 *sG, int wave, int lane) const {
        if (lane >= 16 * wave && lane < 16 * wave + 16 && lane < C) sG[lane] = gate;
    }
};

// Write the staged output tile of one chunk ([C][R] in LDS) with 16-byte
// stores; rows at or beyond clen are skipped.
template <typename E, int C, int R>
__device__ __forceinline__ void flush_out(const E *sO, E *__restrict__ out, int tok0, int clen, int hv, int h,
                                          int dv, int col0, int tid) {
    constexpr int EPV = 16 / sizeof(E);
    constexpr int VPRO = R / EPV;
    constexpr int NO = C * VPRO;
#pragma unroll
    for (int it = 0; it < (NO + 255) / 256; ++it) {
        const int id = tid + 256 * it;
        if (NO % 256 == 0 || id < NO) {
            const int r = id / VPRO, cv = id - r * VPRO;
            if (r < clen)
                st16(out + ((size_t)(tok0 + r) * hv + h) * dv + col0 + cv * EPV, ld16(sO + r * R + cv * EPV));
        }
    }
}

template <typename M> __device__ __forceinline__ typename M::Frag mask_frag(typename M::Frag f, bool keep) {
    return keep ? f : zero_frag<M>();
}

template <typename E, int C, int DK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gdn_scan_kernel(
    const E *__restrict__ v,
    const int32_t *__restrict__ bounds, const int32_t *__restrict__ seq_chunk0,
    const int32_t *__restrict__ order,
    const E *__restrict__ tmat, const E *__restrict__ pmat, const E *__restrict__ kmat,
    const E *__restrict__ qmat, const E *__restrict__ ktmat,
    const f32x4 *__restrict__ gates, const float *__restrict__ gammac,
    const float *__restrict__ s0, float *__restrict__ sfin, E *__restrict__ out,
    int32_t num_seqs, int32_t hk, int32_t hv)
{
    typedef ScanSmem<E, C, DK> L;
    typedef WaveStage<E, C, DK> WS;
    typedef typename WS::MD MD;
    typedef typename WS::MC MC;
    constexpr int R = kSliceRows;
    constexpr int DV = DK;
    constexpr int NS = DV / R;  // value-row slices per head
    constexpr int LDK = L::LDK, LDC = L::LDC;
    constexpr int RT = WS::RT, MT = WS::MT, NRW = WS::NRW, NMW = WS::NMW;
    constexpr int KBD = WS::KBD, KBC = WS::KBC;
    constexpr bool kThreeStages = IsBf16<E>::value;  // fp32 fragments are 4x larger

    extern __shared__ __align__(16) char smem[];
    E *sS = reinterpret_cast<E *>(smem + L::off_S);
    E *sYt = reinterpret_cast<E *>(smem + L::off_Yt);
    E *sUt = reinterpret_cast<E *>(smem + L::off_Ut);
    E *sDUt = reinterpret_cast<E *>(smem + L::off_DUt);
    E *sO = reinterpret_cast<E *>(smem + L::off_O);
    f32x4 *sG = reinterpret_cast<f32x4 *>(smem + L::off_G);

    // Workgroup -> (sequence rank, query/key head, value head in group, slice).
    // Dispatch places workgroup b on XCD b % 8; all value heads and slices
    // of one query/key head land on one XCD, so their shared operands are
    // served by that XCD's L2.
    const int group = hv / hk;
    const int per_kh = group * NS;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int gk = (slot / per_kh) * 8 + xcd;
    if (gk >= num_seqs * hk) return;
    const int within = slot - (slot / per_kh) * per_kh;
    const int rank = gk / hk, kh = gk - rank * hk;
    const int h = kh * group + within / NS;
    const int col0 = (within % NS) * R;
    const int n = order[rank];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, ln = lane & 15;
    const int start = bounds[n];
    const int len = bounds[n + 1] - start;
    const int nch = (len + C - 1) / C;
    const int c0 = seq_chunk0[n];
    const size_t state0 = ((size_t)n * hv + h) * (size_t)(DV * DK);

    // fp32 master copy of this wave's S^T tiles (key tiles mt); operand copy
    // (S[value][key]) in LDS.
    f32x4 sacc[NMW];
#pragma unroll
    for (int j = 0; j < NMW; ++j) {
        const int mt = wave + 4 * j;
        sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (mt < MT) {
            if (s0)
                sacc[j] = *reinterpret_cast<const f32x4 *>(s0 + state0 + (size_t)(col0 + ln) * DK + 16 * mt + 4 * g4);
            store_acc_t<E>(sS, LDK, 16 * mt, 0, lane, sacc[j]);
        }
    }

    WS st0, st1, st2;
    auto issue = [&](WS &st, int c) {
        st.load(v, tmat, pmat, kmat, qmat, ktmat, gates, gammac, start + c * C, min(C, len - c * C), c0 + c,
                hk, kh, hv, h, col0, wave, lane);
    };

    // One chunk c with its operands in `st`. The gate vectors of chunk c are
    // in sG[c & 1] when it starts.
    //   kThree: `fut` (which held chunk c - 1) is refilled with chunk c + 2 at
    //           the start, so each load has two chunk-times to land; `nxt`
    //           holds chunk c + 1, whose gates are staged before the last
    //           barrier.
    //   otherwise (one stage): `st` is refilled with chunk c + 1 at the end.
    auto body = [&](WS &st, WS &nxt, WS &fut, int c, auto three) {
        constexpr bool kThree = decltype(three)::value;
        if constexpr (kThree) issue(fut, min(c + 2, nch - 1));  // past the end: reload the last chunk (ignored)
        const int tok0 = start + c * C;
        const int clen = min(C, len - c * C);
        // This wave's gate rows, read once before any LDS store of this chunk
        // (later reads would be ordered behind those stores).
        f32x4 gr[NRW][4];
#pragma unroll
        for (int r = 0; r < NRW; ++r) {
            const int rt = min(wave + 4 * r, RT - 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) gr[r][i] = sG[(c & 1) * C + 16 * rt + 4 * g4 + i];
        }

        // ---- X = K S0^T, O1 = Q S0^T, Y = diag(b) V - diag(b gamma) X
        f32x4 o1[NRW];
#pragma unroll
        for (int r = 0; r < NRW; ++r) {
            const int rt = wave + 4 * r;
            o1[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (rt < RT) {
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KBD; ++kb) {
                    const typename MD::Frag bs = load_frag<MD>(sS, LDK, 0, kb * MD::KW, lane);
                    x = MD::mma(st.kf[r][kb], bs, x);
                    o1[r] = MD::mma(st.qf[r][kb], bs, o1[r]);
                }
                f32x4 y;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * rt + 4 * g4 + i;
                    y[i] = gr[r][i][1] * (row < clen ? to_f32(st.vv[r][i]) : 0.f) - gr[r][i][2] * x[i];
                }
                store_acc_t<E>(sYt, LDC, 16 * rt, 0, lane, y);
            }
        }
        __syncthreads();

        // ---- U = T Y; diag(delta) U
#pragma unroll
        for (int r = 0; r < NRW; ++r) {
            const int rt = wave + 4 * r;
            if (rt < RT) {
                f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb)
                    u = MC::mma(st.tf[r][kb], load_frag<MC>(sYt, LDC, 0, kb * MC::KW, lane), u);
                store_acc_t<E>(sUt, LDC, 16 * rt, 0, lane, u);
                f32x4 du;
#pragma unroll
                for (int i = 0; i < 4; ++i) du[i] = gr[r][i][3] * u[i];
                store_acc_t<E>(sDUt, LDC, 16 * rt, 0, lane, du);
            }
        }
        __syncthreads();

        // ---- O = diag(scale gamma) Q S0^T + P U, staged in LDS
#pragma unroll
        for (int r = 0; r < NRW; ++r) {
            const int rt = wave + 4 * r;
            if (rt < RT) {
                f32x4 o2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb)
                    o2 = MC::mma(st.pf[r][kb], load_frag<MC>(sUt, LDC, 0, kb * MC::KW, lane), o2);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * rt + 4 * g4 + i;
                    sO[row * R + ln] = from_f32<E>(gr[r][i][0] * o1[r][i] + o2[i]);
                }
            }
        }

        // ---- S^T <- gamma_C S^T + K^T (diag(delta) U)
#pragma unroll
        for (int j = 0; j < NMW; ++j) {
            const int mt = wave + 4 * j;
            if (mt < MT) {
                f32x4 acc = sacc[j];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] *= st.gc;
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb)
                    acc = MC::mma(st.ktf[j][kb], load_frag<MC>(sDUt, LDC, 0, kb * MC::KW, lane), acc);
                sacc[j] = acc;
                store_acc_t<E>(sS, LDK, 16 * mt, 0, lane, acc);
            }
        }
        if constexpr (kThree) nxt.put_gates(sG + ((c + 1) & 1) * C, wave, lane);
        __syncthreads();

        if constexpr (!kThree) issue(st, min(c + 1, nch - 1));
        // this chunk's output tile; sO is only rewritten after two more barriers
        flush_out<E, C, R>(sO, out, tok0, clen, hv, h, DV, col0, tid);
    };

    if (nch > 0) {
        issue(st0, 0);
        if constexpr (kThreeStages) {
            issue(st1, min(1, nch - 1));
            st0.put_gates(sG, wave, lane);
            __syncthreads();
            int c = 0;
            for (; c + 2 < nch; c += 3) {
                body(st0, st1, st2, c, std::true_type());
                body(st1, st2, st0, c + 1, std::true_type());
                body(st2, st0, st1, c + 2, std::true_type());
            }
            if (c < nch) body(st0, st1, st2, c, std::true_type());
            if (c + 1 < nch) body(st1, st2, st0, c + 1, std::true_type());
        } else {
            for (int c = 0; c < nch; ++c) {
                st0.put_gates(sG + (c & 1) * C, wave, lane);
                __syncthreads();
                body(st0, st0, st0, c, std::false_type());
            }
        }
    }

    if (sfin) {
#pragma unroll
        for (int j = 0; j < NMW; ++j) {
            const int mt = wave + 4 * j;
            if (mt < MT)
                *reinterpret_cast<f32x4 *>(sfin + state0 + (size_t)(col0 + ln) * DK + 16 * mt + 4 * g4) = sacc[j];
        }
    }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

template <typename KernelT>
static hipError_t allow_smem(KernelT kernel, size_t bytes, std::atomic<bool> &done) {
    if (done.load(std::memory_order_acquire)) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) done.store(true, std::memory_order_release);
    return e;
}

template <typename E, typename G, int C, int D>
static hipError_t launch_prefill_t(const PrefillArgs &A, hipStream_t st) {
    const PrefillLayout &Y = A.lay;
    char *ws = A.ws;
    int32_t *bounds = reinterpret_cast<int32_t *>(ws + Y.off_bounds);
    int32_t *seq_chunk0 = reinterpret_cast<int32_t *>(ws + Y.off_seq_chunk0);
    int32_t *order = reinterpret_cast<int32_t *>(ws + Y.off_order);
    int32_t *chunk_seq = reinterpret_cast<int32_t *>(ws + Y.off_chunk_seq);
    int32_t *chunk_tok0 = reinterpret_cast<int32_t *>(ws + Y.off_chunk_tok0);
    int32_t *counters = reinterpret_cast<int32_t *>(ws + Y.off_counters);
    E *tmat = reinterpret_cast<E *>(ws + Y.off_tmat);
    E *pmat = reinterpret_cast<E *>(ws + Y.off_pmat);
    E *kmat = reinterpret_cast<E *>(ws + Y.off_kmat);
    E *qmat = reinterpret_cast<E *>(ws + Y.off_qmat);
    E *ktmat = reinterpret_cast<E *>(ws + Y.off_ktmat);
    f32x4 *gates = reinterpret_cast<f32x4 *>(ws + Y.off_gates);
    float *gammac = reinterpret_cast<float *>(ws + Y.off_gammac);

    timing_begin(kSchedule, st);
    hipLaunchKernelGGL(gdn_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, st,
                       A.cu, A.num_seqs, (int32_t)A.total_tokens, A.chunk,
                       bounds, seq_chunk0, order, chunk_seq, chunk_tok0, counters);
    timing_end(kSchedule, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    typedef PrepSmem<E, C, D> PL;
    static std::atomic<bool> prep_ok{false};
    auto prep = gdn_prep_kernel<E, G, C, D>;
    if ((e = allow_smem(prep, PL::bytes, prep_ok)) != hipSuccess) return e;
    timing_begin(kPrep, st);
    hipLaunchKernelGGL(prep, dim3((unsigned)Y.max_chunks, (unsigned)A.hk), dim3(256), PL::bytes, st,
                       (const E *)A.q, (const E *)A.k, (const G *)A.g, (const G *)A.beta,
                       bounds, chunk_seq, chunk_tok0, counters, tmat, pmat, kmat, qmat, ktmat, gates, gammac,
                       A.hk, A.hv, A.scale);
    timing_end(kPrep, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    typedef ScanSmem<E, C, D> SL;
    static std::atomic<bool> scan_ok{false};
    auto scan = gdn_scan_kernel<E, C, D>;
    if ((e = allow_smem(scan, SL::bytes, scan_ok)) != hipSuccess) return e;
    const int64_t per_kh = (int64_t)(A.hv / A.hk) * (D / kSliceRows);
    const int64_t groups = (int64_t)A.num_seqs * A.hk;
    const int64_t grid = ((groups + 7) / 8) * per_kh * 8;
    timing_begin(kScan, st);
    hipLaunchKernelGGL(scan, dim3((unsigned)grid), dim3(256), SL::bytes, st,
                       (const E *)A.v, bounds, seq_chunk0, order, tmat, pmat, kmat, qmat, ktmat, gates, gammac,
                       A.s0, A.s_final, (E *)A.out, A.num_seqs, A.hk, A.hv);
    timing_end(kScan, st);
    return hipGetLastError();
}

template <typename E, typename G, int C>
static hipError_t launch_prefill_c(const PrefillArgs &A, hipStream_t st) {
    switch (A.d) {
    case 16: return launch_prefill_t<E, G, C, 16>(A, st);
    case 32: return launch_prefill_t<E, G, C, 32>(A, st);
    case 64: return launch_prefill_t<E, G, C, 64>(A, st);
    case 128: return launch_prefill_t<E, G, C, 128>(A, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename E, typename G>
static hipError_t launch_prefill_g(const PrefillArgs &A, hipStream_t st) {
    switch (A.chunk) {
    case 16: return launch_prefill_c<E, G, 16>(A, st);
    case 32: return launch_prefill_c<E, G, 32>(A, st);
    case 64: return launch_prefill_c<E, G, 64>(A, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill(const PrefillArgs &A, hipStream_t st) {
    if (A.io_bf16)
        return A.gate_bf16 ? launch_prefill_g<bf16, bf16>(A, st) : launch_prefill_g<bf16, float>(A, st);
    return A.gate_bf16 ? launch_prefill_g<float, bf16>(A, st) : launch_prefill_g<float, float>(A, st);
}

}  // namespace gdn

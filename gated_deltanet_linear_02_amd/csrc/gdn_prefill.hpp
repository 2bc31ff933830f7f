// gdn_prefill.hpp -- chunked prefill of the Gated DeltaNet layer (gfx950).
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
#pragma once

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

#include <atomic>

namespace gdn {

// The varlen schedule's launch (gdn_prefill.hip): cu_seqlens -> clamped
// bounds, first chunk per sequence, longest-first order and the chunk table.
hipError_t launch_schedule(const PrefillArgs &A, hipStream_t st, int32_t *bounds, int32_t *seq_chunk0,
                           int32_t *order, int32_t *chunk_seq, int32_t *chunk_tok0, int32_t *counters);

// The kernels of one (element type, chunk size), built from
// gdn_prefill_inst.hip once per pair so that they compile in parallel.
#define GDN_PREFILL_INST_FN(B, C) launch_prefill_inst_b##B##_c##C
#define GDN_PREFILL_INST_DECL(B, C) hipError_t GDN_PREFILL_INST_FN(B, C)(const PrefillArgs &A, hipStream_t st)
GDN_PREFILL_INST_DECL(1, 16);
GDN_PREFILL_INST_DECL(1, 32);
GDN_PREFILL_INST_DECL(1, 64);
GDN_PREFILL_INST_DECL(0, 16);
GDN_PREFILL_INST_DECL(0, 32);
GDN_PREFILL_INST_DECL(0, 64);

// ---------------------------------------------------------------------------
// 2. Chunk preparation
// ---------------------------------------------------------------------------
//
// One workgroup per (chunk, query/key head). It computes K K^T and Q K^T on
// MFMA once, keeps them in registers, and then for each value head of the
// group applies that head's gates and builds the per-head operands of the
// scan:
//   Tb = T diag(b),   W = T diag(b gamma) K   (so that U = Tb V - W S0^T),
//   P,  and the gate record (delta = exp(c_C - c), scale*gamma, gamma_C),
// with T = (I + A)^-1 by blocks of 16:
//   diagonal blocks    (I + A_bb)^-1 by forward substitution, one wave each;
//   blocks below       T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj, one wave per
//                      block column j, on fp32 MFMA,
// which is (I + A) T = I written blockwise. Q and K^T (shared by the value
// heads of the group) are written once.
//
// Every operand goes to the workspace in MFMA fragment order (frag_off), so
// that each fragment the scan loads is one contiguous 1 KB run, and with its
// contraction index in accumulator order (acc_k), so that accumulator tiles
// become fragments without a transpose.

template <typename E> struct IsBf16 { static constexpr bool value = false; };
template <> struct IsBf16<bf16> { static constexpr bool value = true; };

// Element offset of lane `lane`'s part of fragment f in fragment order: a
// matrix [M][K] is stored as fragments f = rt * (K / KW) + kb, each holding
// KPL elements per lane for rows 16 rt + l%16.
template <typename MM> __device__ __forceinline__ size_t frag_off(int f, int lane) {
    return ((size_t)f * 64 + lane) * MM::KPL;
}

// Tb = T diag(b) and P are lower triangular, so in row tile rt (rows
// 16 rt .. 16 rt + 15) the contraction blocks kb with kb * KW >= 16 (rt + 1)
// are zero. The scan reads only blocks kb < tri_read_blocks(rt) of a tile and
// the preparation kernel writes only those: the row tiles whose nonzero
// blocks are as few as in row tile 0 skip the rest (C = 64 bf16: tiles 0
// and 1 read one of two blocks); other tiles read all blocks, zero or not.
template <typename MC, int C> __host__ __device__ constexpr int tri_read_blocks(int rt) {
    return (16 * (rt + 1) + MC::KW - 1) / MC::KW == (16 + MC::KW - 1) / MC::KW ? (16 + MC::KW - 1) / MC::KW
                                                                               : C / MC::KW;
}

template <typename E, int C, int DK>
struct PrepSmem {
    static constexpr int PE = Pad<E>::value;
    static constexpr int LDK = DK + PE;  // staged K and Q rows (E)
    static constexpr int LDC = C + 4;    // fp32 C x C arrays, 16-byte aligned rows
    // K and Q tiles (phases 1-4), then A and T (per value head).
    static constexpr size_t off_K = 0;
    static constexpr size_t off_Q = off_K + (size_t)C * LDK * sizeof(E);
    static constexpr size_t kq_end = off_Q + (size_t)C * LDK * sizeof(E);
    static constexpr size_t off_A = 0;
    static constexpr size_t off_T = off_A + (size_t)C * LDC * sizeof(float);
    static constexpr size_t at_end = off_T + (size_t)C * LDC * sizeof(float);
    // Gate prefixes c, b and b gamma of two value heads ([2][C] each): the
    // first two heads' are computed while K and Q load.
    static constexpr size_t off_c = ((kq_end > at_end ? kq_end : at_end) + 15) & ~(size_t)15;
    static constexpr size_t off_b = off_c + 2 * (size_t)C * sizeof(double);
    static constexpr size_t off_bg = off_b + 2 * (size_t)C * sizeof(float);
    // Chunk location when the kernel schedules itself: sequence ends and
    // lengths (256 each), 4 wave partials and 4 results.
    static constexpr size_t off_loc = off_bg + 2 * (size_t)C * sizeof(float);
    static constexpr size_t bytes = off_loc + (2 * 256 + 8) * sizeof(int);
};

// Up to this many sequences the chunk-preparation kernel locates its own
// chunk from cu_seqlens (and publishes the scan's tables), so no separate
// schedule launch is needed.
constexpr int kFoldMaxSeqs = 256;

// An empty slot of the fused normalisation's partial sums of squares.
constexpr float kNormPartEmpty = -1.0f;

// Inclusive scan (sum, or max) over a 256-thread workgroup: shuffle scans
// within each wave, then the wave totals through LDS (s_part[4]).
__device__ __forceinline__ int wg256_scan_incl(int x, bool use_max, int *s_part) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x = use_max ? max(x, y) : x + y;
    }
    if (lane == 63) s_part[wave] = x;
    __syncthreads();
    int carry = use_max ? INT32_MIN : 0;
    for (int w = 0; w < wave; ++w) carry = use_max ? max(carry, s_part[w]) : carry + s_part[w];
    __syncthreads();  // s_part is reused by the next scan
    return use_max ? max(x, carry) : x + carry;
}

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

// 2^x on the hardware instruction (arguments here are <= 0 for decaying
// gates; results below the fp32 range flush to 0).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr double kLog2eD = 1.4426950408889634;

template <typename MM> __device__ __forceinline__ void frag_set(typename MM::Frag &f, int e, float x) {
    if constexpr (MM::KPL == 1) f = x; else f[e] = static_cast<bf16>(x);
}

// The 16x16 tiles at or below the diagonal of a C x C product (NB = C/16
// row tiles) owned by the waves of parity PAR: with NB = 4, row tiles {0, 3}
// and {1, 2} (five tiles each, balanced); with NB <= 2, row tile PAR. Slot
// first(r) + tj holds tile (row(r), tj), tj <= row(r). Everything is
// compile-time so that the tiles stay in registers.
template <int NB, int PAR> struct TileSet {
    static constexpr int NR = NB == 4 ? 2 : (PAR < NB ? 1 : 0);  // owned row tiles
    static constexpr int row(int r) { return NB == 4 ? (PAR == 0 ? (r == 0 ? 0 : 3) : (r == 0 ? 1 : 2)) : PAR; }
    static constexpr int first(int r) { return r == 0 ? 0 : row(0) + 1; }
    static constexpr int N = NR == 0 ? 0 : (NR == 1 ? row(0) + 1 : row(0) + row(1) + 2);
};

template <typename E, typename G, int C, int DK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(IsBf16<E>::value ? 4 : 2, IsBf16<E>::value ? 4 : 2))) void gdn_prep_kernel(
    const E *__restrict__ q, const E *__restrict__ k,
    const G *__restrict__ gate_g, const G *__restrict__ gate_b,
    const int32_t *__restrict__ cu, int32_t num_seqs, int32_t total_tokens,
    int32_t *__restrict__ bounds, int32_t *__restrict__ seq_chunk0, int32_t *__restrict__ order,
    const int32_t *__restrict__ chunk_seq, const int32_t *__restrict__ chunk_tok0,
    const int32_t *__restrict__ counters,
    E *__restrict__ tbmat, E *__restrict__ pmat, E *__restrict__ wmat, E *__restrict__ qmat,
    E *__restrict__ ktmat, float *__restrict__ gates, int32_t hk, int32_t hv, float scale,
    float *__restrict__ norm_part, int32_t norm_slices)
{
    typedef PrepSmem<E, C, DK> L;
    typedef Mma<E, DK> MD;  // contractions over keys
    typedef Mma<E, C> MC;   // contractions over the tokens of a chunk
    constexpr int NB = C / 16, MT = DK / 16;
    constexpr int KBD = DK / MD::KW, KBC = C / MC::KW;
    constexpr int LDK = L::LDK, LDC = L::LDC;
    constexpr int EPV = 16 / sizeof(E), VPR = DK / EPV;
    // Key tiles are handled in groups that make up whole W fragments: two
    // for the 32-deep bf16 MFMA, one otherwise.
    constexpr int DG = MD::KW >= 32 ? 2 : 1;
    constexpr int NDG = MT / DG, NDGW = (NDG + 3) / 4;

    extern __shared__ __align__(16) char smem[];
    E *sK = reinterpret_cast<E *>(smem + L::off_K);
    E *sQ = reinterpret_cast<E *>(smem + L::off_Q);
    float *sA = reinterpret_cast<float *>(smem + L::off_A);
    float *sT = reinterpret_cast<float *>(smem + L::off_T);
    double *sc = reinterpret_cast<double *>(smem + L::off_c);  // c_t log2(e), fp64 (see the gate prefix)
    float *sb = reinterpret_cast<float *>(smem + L::off_b);    // b_t
    float *sbg = reinterpret_cast<float *>(smem + L::off_bg);  // b_t gamma_t

    const int ci = blockIdx.x, kh = blockIdx.y;
    const int group = hv / hk;
    // readfirstlane: the wave index is uniform, and saying so makes the
    // role branches, wave-strided loops and their addresses scalar.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, ln = lane & 15;
    const size_t ld = (size_t)hk * DK;

    // The inputs of a chunk starting at token tb: waves 0 and 1 first load
    // the gate inputs of its tokens for value head `wave` of the group (their
    // prefix sums are formed while the rest arrives), then every thread its
    // K and Q rows (16 bytes per pass). Rows are clamped into [0, T); rows
    // past the chunk are masked where they are used. All loads are issued
    // before any is waited for.
    constexpr int NIT = (C * VPR + 255) / 256;
    constexpr int kGatePrefetch = 2;  // value heads whose prefix is formed early, one per wave
    Vec16 kr[NIT], qr[NIT];
    float gx_pre = 0.f, gb_pre = 0.f;
    auto load_inputs = [&](int tb) {
        if (wave < kGatePrefetch) {
            const size_t gi = (size_t)min(tb + lane, total_tokens - 1) * hv + kh * group + min(wave, group - 1);
            gx_pre = gate_load(gate_g, gi);
            gb_pre = gate_load(gate_b, gi);
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int i = min(tid + 256 * it, C * VPR - 1);
            const int r = i / VPR, cv = i - r * VPR;
            const size_t src = (size_t)min(tb + r, total_tokens - 1) * ld + (size_t)kh * DK + cv * EPV;
            kr[it] = ld16(k + src);
            qr[it] = ld16(q + src);
        }
    };
    // Most prefills are one sequence from token 0, where chunk ci starts at
    // token ci * C. The inputs are loaded for that guess before the chunk is
    // located, so that their latency overlaps the locating; they are loaded
    // again if the guess turns out wrong.
    const int t_guess = ci * C;
    const bool guessed = t_guess < total_tokens;
    if (guessed) load_inputs(t_guess);

    int t0, len;
    if (cu != nullptr) {
        // ---- 0. Locate this chunk (num_seqs <= 256): thread j owns sequence j.
        //         Bounds are cu clamped into [0, T] and made non-decreasing, so a
        //         malformed cu_seqlens cannot send any access out of range.
        int *s_end = reinterpret_cast<int *>(smem + L::off_loc);
        int *s_len = s_end + 256;
        int *s_part = s_len + 256;
        int *s_res = s_part + 4;
        const int j = tid;
        const int b0 = min(max(cu[0], 0), total_tokens);
        const int e = j < num_seqs ? max(min(max(cu[j + 1], 0), total_tokens), b0) : b0;
        const int hi = wg256_scan_incl(e, true, s_part);  // end of sequence j
        s_end[j] = hi;
        __syncthreads();
        const int lo = j == 0 ? b0 : s_end[j - 1];
        const int lenj = j < num_seqs ? hi - lo : 0;
        const int nchj = (lenj + C - 1) / C;
        const int first = wg256_scan_incl(nchj, false, s_part) - nchj;
        if (j < num_seqs && ci >= first && ci < first + nchj) {
            s_res[0] = lo + (ci - first) * C;
            s_res[1] = hi;
        }
        if (j == 255) s_res[2] = first + nchj;  // chunks in total
        if (ci == 0 && kh == 0) {
            // the scan's tables: bounds, first chunk per sequence, longest first
            s_len[j] = lenj;
            if (j == 0) bounds[0] = b0;
            if (j < num_seqs) {
                bounds[j + 1] = hi;
                seq_chunk0[j] = first;
            }
            if (j == 255) seq_chunk0[num_seqs] = first + nchj;
        }
        __syncthreads();
        if (ci == 0 && kh == 0 && j < num_seqs) {
            int rank = 0;
            for (int m = 0; m < num_seqs; ++m) {
                const int lm = s_len[m];
                rank += (lm > lenj) || (lm == lenj && m < j);
            }
            order[rank] = j;
        }
        if (ci >= s_res[2]) return;
        t0 = s_res[0];
        len = min(C, s_res[1] - t0);
    } else {
        if (ci >= counters[0]) return;
        const int n = chunk_seq[ci];
        t0 = chunk_tok0[ci];
        len = min(C, bounds[n + 1] - t0);
    }
    const size_t kq0 = ((size_t)ci * hk + kh) * (size_t)(C * DK);
    if (!guessed || t0 != t_guess) load_inputs(t0);

    // A scan with the output normalisation fused in exchanges partial sums of
    // squares through norm_part, laid out [chunk][value head][row slice][C]:
    // each slot starts as kNormPartEmpty (no partial is negative). The block
    // of this chunk and the group's value heads is contiguous.
    if (norm_part) {
        f32x4 *blk = reinterpret_cast<f32x4 *>(norm_part + ((size_t)ci * hv + (size_t)kh * group) * norm_slices * C);
        const f32x4 e = {kNormPartEmpty, kNormPartEmpty, kNormPartEmpty, kNormPartEmpty};
        for (int i = tid; i < group * norm_slices * C / 4; i += 256) blk[i] = e;
    }

    // Gate prefix sums c_t = g_1 + ... + g_t of value head hh (one wave;
    // C <= 64) into prefix buffer hh % 2, and the chunk's gate record for the
    // scan. Rows past the end of the sequence act as a = 1, b = 0. The sums
    // are kept in fp64: every decay factor below is exp of a difference
    // c_i - c_j, and where some g are huge (a decay that underflows to 0,
    // g = -1e4) the sums reach -1e5 and more, where fp32 spacing (0.01) would
    // wipe out the differences between nearby tokens.
    auto gate_prefix = [&](int hh, float x, float bv) {
        const bool valid = lane < len;
        if (!valid) x = bv = 0.f;
        double xd = x;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(xd, off);
            if (lane >= off) xd += y;
        }
        const double last = __shfl(xd, C - 1);
        if (lane < C) {
            const int buf = hh & 1;
            const float gam = exp2_hw(static_cast<float>(xd * kLog2eD));
            sc[buf * C + lane] = xd * kLog2eD;
            sb[buf * C + lane] = bv;
            sbg[buf * C + lane] = bv * gam;
            float *rec = gates + ((size_t)ci * hv + kh * group + hh) * (size_t)gate_record(C);
            rec[lane] = exp2_hw(static_cast<float>((last - xd) * kLog2eD));
            rec[C + lane] = scale * gam;
            if (lane == C - 1) rec[2 * C] = exp2_hw(static_cast<float>(last * kLog2eD));
        }
    };
    // the first value heads' prefixes, while K and Q are still arriving
    if (wave < kGatePrefetch && wave < group) gate_prefix(wave, gx_pre, gb_pre);

    // ---- 1. K and Q rows into LDS (zero past the end of the sequence)
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i = tid + 256 * it;
        if (i < C * VPR) {
            const int r = i / VPR, cv = i - r * VPR;
            st16(sK + r * LDK + cv * EPV, r < len ? kr[it] : zero16());
            st16(sQ + r * LDK + cv * EPV, r < len ? qr[it] : zero16());
        }
    }
    __syncthreads();

    // ---- 2. Q fragments (keys in accumulator order)
    for (int f = wave; f < NB * KBD; f += 4) {
        const int rt = f / KBD, kb = f - rt * KBD;
        *reinterpret_cast<typename MD::Frag *>(qmat + kq0 + frag_off<MD>(f, lane)) =
            load_frag_acc<MD>(sQ, LDK, 16 * rt, kb, lane);
    }

    // ---- 3. K^T fragments (tokens in accumulator order) of this wave's key
    //         groups; kept in registers as the A operand of W
    typename MC::Frag ktr[NDGW][DG][KBC];
#pragma unroll
    for (int gi = 0; gi < NDGW; ++gi) {
        const int dg = wave + 4 * gi;
        if (dg < NDG) {
#pragma unroll
            for (int t = 0; t < DG; ++t) {
                const int mt = dg * DG + t;
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) {
                    typename MC::Frag fr;
#pragma unroll
                    for (int e = 0; e < MC::KPL; ++e)  // K^T[m][j] = K[j][m]
                        frag_set<MC>(fr, e, to_f32(sK[acc_k<MC>(kb, g4, e) * LDK + 16 * mt + ln]));
                    *reinterpret_cast<typename MC::Frag *>(ktmat + kq0 + frag_off<MC>(mt * KBC + kb, lane)) = fr;
                    ktr[gi][t][kb] = fr;
                }
            }
        }
    }

    // ---- 4. K K^T (waves 0, 1) and Q K^T (waves 2, 3) on the tiles at or
    //         below the diagonal, computed as K_j K_i^T and K_j Q_i^T so that
    //         lane l holds row 16 ti + l%16, columns 16 tj + 4 (l/16) + r.
    //         The tiles of the wave's TileSet stay in registers.
    const bool score_wave = wave >= 2;
    const int par = wave & 1;
    constexpr int NTS = TileSet<NB, 0>::N > TileSet<NB, 1>::N ? TileSet<NB, 0>::N : TileSet<NB, 1>::N;
    f32x4 til[NTS > 0 ? NTS : 1];
    // Each role and tile set is its own instantiation (ROLE: 0 Gram, 1 scores).
    auto by_role = [&](auto &&fn) {
        if (score_wave) {
            if (par) fn(std::integral_constant<int, 1>(), std::true_type());
            else fn(std::integral_constant<int, 0>(), std::true_type());
        } else {
            if (par) fn(std::integral_constant<int, 1>(), std::false_type());
            else fn(std::integral_constant<int, 0>(), std::false_type());
        }
    };
    auto gram = [&](auto parc, auto scorec) {
        typedef TileSet<NB, decltype(parc)::value> TS;
        constexpr bool kScore = decltype(scorec)::value;
        const E *Bm = kScore ? sQ : sK;
#pragma unroll
        for (int r = 0; r < TS::NR; ++r) {
            const int ti = TS::row(r);
#pragma unroll
            for (int tj = 0; tj <= TS::row(r); ++tj) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KBD; ++kb)
                    acc = MD::mma(load_frag<MD>(sK, LDK, 16 * tj, kb * MD::KW, lane),
                                  load_frag<MD>(Bm, LDK, 16 * ti, kb * MD::KW, lane), acc);
                til[TS::first(r) + tj] = acc;
            }
        }
    };
    by_role(gram);
    __syncthreads();  // the K / Q region becomes A / T

    // ---- 5. Per value head of the group
    for (int hh = 0; hh < group; ++hh) {
        const int h = kh * group + hh;
        const size_t ch = (size_t)ci * hv + h;
        const size_t mat0 = ch * (size_t)(C * C);
        const size_t w0 = ch * (size_t)(C * DK);

        // the gate prefix of the heads beyond the first two (one wave)
        if (hh >= kGatePrefetch) {
            if (wave == 0) {
                const int row = t0 + (lane < len ? lane : 0);
                gate_prefix(hh, gate_load(gate_g, (size_t)row * hv + h), gate_load(gate_b, (size_t)row * hv + h));
            }
            __syncthreads();
        }
        const double *sc_h = sc + (hh & 1) * C;
        const float *sb_h = sb + (hh & 1) * C;
        const float *sbg_h = sbg + (hh & 1) * C;

        // A = strict_lower(b_i exp(c_i - c_j) (K K^T)_ij) into LDS (waves 0, 1);
        // P = lower(scale exp(c_i - c_j) (Q K^T)_ij) to fragments (waves 2, 3)
        auto decay = [&](auto parc, auto scorec) {
            typedef TileSet<NB, decltype(parc)::value> TS;
            constexpr bool score_wave = decltype(scorec)::value;
#pragma unroll
            for (int r = 0; r < TS::NR; ++r) {
                const int ti = TS::row(r);
                const int i = 16 * ti + ln;
                const double cI = sc_h[i];
                const float mI = score_wave ? scale : sb_h[i];
                f32x4 val[NB];
#pragma unroll
                for (int tj = 0; tj < NB; ++tj) {
                    val[tj] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (tj <= TS::row(r)) {
                        const f32x4 t = til[TS::first(r) + (tj <= TS::row(r) ? tj : 0)];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int j = 16 * tj + 4 * g4 + e;
                            const bool keep = score_wave ? j <= i : j < i;
                            const float dc = static_cast<float>(cI - sc_h[j]);  // fp64 difference, then fp32
                            val[tj][e] = keep ? mI * exp2_hw(dc) * t[e] : 0.f;
                        }
                        if constexpr (!score_wave) *reinterpret_cast<f32x4 *>(sA + i * LDC + 16 * tj + 4 * g4) = val[tj];
                    }
                }
                if constexpr (score_wave) {
#pragma unroll
                    for (int kb = 0; kb < KBC; ++kb) {
                        if (kb >= tri_read_blocks<MC, C>(ti)) continue;  // zero, never read
                        typename MC::Frag fr;
#pragma unroll
                        for (int e = 0; e < MC::KPL; ++e)
                            frag_set<MC>(fr, e, val[acc_tile<MC>(kb, e)][acc_slot<MC>(kb, e)]);
                        *reinterpret_cast<typename MC::Frag *>(pmat + mat0 + frag_off<MC>(ti * KBC + kb, lane)) = fr;
                    }
                }
            }
        };
        by_role(decay);
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
        // The column stays in registers. An accumulator tile (lane: column
        // l%16, rows 4 (l/16) + r) is the B operand of the next product when
        // k-step r takes contraction index 4 (l/16) + r, so Z and each new
        // T_mj feed the following MFMAs directly; A_im and T_ii are read
        // from LDS once, as the matching 4 contiguous values per lane.
        if (wave < NB - 1) {
            const int j = wave;
            f32x4 tcol[NB];  // T_mj, m >= j, in accumulator layout
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                tcol[m] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (m == j) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) tcol[m][r] = sT[(16 * j + 4 * g4 + r) * LDC + 16 * j + ln];
                }
            }
#pragma unroll
            for (int i = 1; i < NB; ++i) {
                if (i <= j) continue;
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < i; ++m) {
                    if (m < j) continue;
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(sA + (16 * i + ln) * LDC + 16 * m + 4 * g4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) z = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], tcol[m][r], z, 0, 0, 0);
                }
                const f32x4 d = *reinterpret_cast<const f32x4 *>(sT + (16 * i + ln) * LDC + 16 * i + 4 * g4);
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < 4; ++r) t = __builtin_amdgcn_mfma_f32_16x16x4f32(-d[r], z[r], t, 0, 0, 0);
                tcol[i] = t;
#pragma unroll
                for (int r = 0; r < 4; ++r) sT[(16 * i + 4 * g4 + r) * LDC + 16 * j + ln] = t[r];
            }
        }
        __syncthreads();

        // Tb = T diag(b) in fragments to the workspace, and the B operand of W,
        // T diag(b gamma), in the same fragment order to LDS (over A, which is
        // not read after the inverse), both from one read of T. Blocks above the
        // diagonal are zero; those the scan does not read are not written, and
        // the product for W skips them too.
        typename MC::Frag *sBW = reinterpret_cast<typename MC::Frag *>(sA);
        for (int f = wave; f < NB * KBC; f += 4) {
            const int rt = f / KBC, kb = f - rt * KBC;
            if (kb >= tri_read_blocks<MC, C>(rt)) continue;
            const int i = 16 * rt + ln;
            typename MC::Frag fr, fw;
#pragma unroll
            for (int e = 0; e < MC::KPL; ++e) {
                const int j = acc_k<MC>(kb, g4, e);
                const float t = (j >> 4) <= rt ? sT[i * LDC + j] : 0.f;
                frag_set<MC>(fr, e, t * sb_h[j]);
                frag_set<MC>(fw, e, t * sbg_h[j]);
            }
            *reinterpret_cast<typename MC::Frag *>(tbmat + mat0 + frag_off<MC>(f, lane)) = fr;
            sBW[f * 64 + lane] = fw;
        }
        __syncthreads();

        // -W = -T diag(b gamma) K: per key group and token tile, K^T (registers)
        // times (T diag(b gamma))^T from LDS; the accumulators (lane: token
        // 16 ti + l%16, keys 16 mt + 4 (l/16) + r) are W's fragments with keys
        // in accumulator order.
#pragma unroll
        for (int gi = 0; gi < NDGW; ++gi) {
            const int dg = wave + 4 * gi;
            if (dg >= NDG) continue;
            for (int ti = 0; ti < NB; ++ti) {
                const int nkb = tri_read_blocks<MC, C>(ti);
                typename MC::Frag bfr[KBC];
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) bfr[kb] = kb < nkb ? sBW[(ti * KBC + kb) * 64 + lane] : zero_frag<MC>();
                f32x4 w[DG];
#pragma unroll
                for (int t = 0; t < DG; ++t) {
                    w[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < KBC; ++kb)
                        if (kb < nkb) w[t] = MC::mma(ktr[gi][t][kb], bfr[kb], w[t]);
                }
                if constexpr (MD::KPL == 1) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        wmat[w0 + frag_off<MD>(ti * KBD + 4 * dg + r, lane)] = -w[0][r];
                } else {
                    typename MD::Frag fr;
#pragma unroll
                    for (int e = 0; e < MD::KPL; ++e) frag_set<MD>(fr, e, -w[e >> 2][e & 3]);
                    *reinterpret_cast<typename MD::Frag *>(wmat + w0 + frag_off<MD>(ti * KBD + dg, lane)) = fr;
                }
            }
        }
        __syncthreads();  // sc, sb, sbg, A and T are rewritten for the next value head
    }
}

// ---------------------------------------------------------------------------
// 3. Chunk-recurrent scan over one (sequence, value head, 16, 32, 64 or 128
//    value rows)
// ---------------------------------------------------------------------------
//
// Eight waves per workgroup, two per SIMD, in two roles. With S0 the slice at
// a chunk's start and q = wave % 4:
//   recurrence waves (0-3)  phase 1: U = Tb V - W S0^T on token tile q, then
//                           U and diag(delta) U to LDS;
//                           phase 2: S^T = gamma_C S0^T + K^T diag(delta) U on
//                           key tiles q, q+4, .., operand copy of S to LDS;
//   output waves (4-7)      phase 1: the next chunk's gate record and V rows
//                           to LDS; O1^T = S0 Q^T on token tile q;
//                           phase 2: O^T = O1^T diag(scale gamma) + U^T P^T,
//                           stored from registers.
// One barrier ends each phase. Only the recurrence waves are on the chain
// from one chunk's state to the next; the output waves' work fills the other
// wave slot of each SIMD. Every A operand (Tb, W, K^T; Q, P) is read from the
// workspace as contiguous 1 KB fragments and the gate record with one load,
// issued up to three (recurrence) or four (output) chunks ahead into
// register stages used round robin (fewer stages for the wider slices,
// whose registers hold more rows, and for fp32 fragments, which are four
// times larger: two and three). At 16 rows the chunk step is about as long as
// the CU takes to accept its vector-memory instructions, so their number per
// chunk is kept small.

constexpr int kScanThreads = 512;

// Steps from a chunk's outputs to its normalised rows in the fused
// normalisation's exchange (and steps after the last chunk in which it
// writes the last chunks' rows).
constexpr int kNormLag = 4;
static_assert((kNormLag & (kNormLag - 1)) == 0, "the pending outputs are a ring of kNormLag chunks");

// R: value rows of the state per workgroup (16, or 32, 64, 128 on bf16 I/O).
// kPend: the fused normalisation exchanges partial sums between the slices
// of a head, and keeps each output wave's unnormalised outputs of the last
// kNormLag chunks.
template <typename E, int C, int DK, int R, bool kPend = false>
struct ScanSmem {
    static constexpr int PE = Pad<E>::value;
    static constexpr int LDK = DK + PE;  // rows of length DK
    static constexpr int LDC = C + PE;   // rows of length C
    // Rows in fragment-contiguous order (lds_pos: keys for MD, tokens for MC).
    static constexpr size_t off_S = 0;                                       // [R][LDK] S (value row, key)
    static constexpr size_t off_Ut = off_S + (size_t)R * LDK * sizeof(E);    // [R][LDC] U^T
    static constexpr size_t off_DUt = off_Ut + (size_t)R * LDC * sizeof(E);  // [R][LDC] (diag(delta) U)^T
    static constexpr size_t off_Vt = off_DUt + (size_t)R * LDC * sizeof(E);  // [2][R][LDC] V^T
    static constexpr size_t off_Dl = (off_Vt + 2 * (size_t)R * LDC * sizeof(E) + 15) & ~(size_t)15;  // [2][C] delta
    static constexpr size_t off_Sg = off_Dl + 2 * (size_t)C * sizeof(float);  // [2][C] scale gamma
    static constexpr size_t off_Gc = off_Sg + 2 * (size_t)C * sizeof(float);  // [2][4] gamma_C (first of 4)
    // fused output normalisation: this slice's partial sums of squares of a
    // chunk, the head's block of every slice's partials, their totals
    static constexpr size_t off_Np = off_Gc + 8 * sizeof(float);                   // [C]
    static constexpr size_t off_Nb = off_Np + (size_t)C * sizeof(float);           // [DK / R][C]
    static constexpr size_t off_Nt = off_Nb + (size_t)(DK / R) * C * sizeof(float);  // [C]
    static constexpr size_t off_Nw = off_Nt + (size_t)C * sizeof(float);              // [R] weights
    // [kNormLag][4 output waves][R / 16][64 lanes] f32x4: a ring by chunk
    static constexpr size_t off_Pd = (off_Nw + (size_t)R * sizeof(float) + 15) & ~(size_t)15;
    static constexpr size_t bytes = off_Pd + (kPend ? (size_t)kNormLag * 4 * (R / 16) * 64 * 16 : 0);
};

template <typename E> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

// Where one chunk's operands live in the workspace, for one workgroup.
struct ChunkRef {
    int tok0, clen;  // first token, tokens in the chunk
    size_t ch;       // chunk * hv + value head
    size_t kq;       // (chunk * hk + query/key head)
};

template <typename E, int C, int DK>
struct ScanShape {
    typedef Mma<E, DK> MD;  // contractions over keys
    typedef Mma<E, C> MC;   // contractions over the tokens of a chunk
    typedef typename Vec4<E>::type E4;
    static constexpr int RT = C / 16, MT = DK / 16;
    static constexpr int NMW = (MT + 3) / 4;  // key tiles per recurrence wave
    static constexpr int KBD = DK / MD::KW, KBC = C / MC::KW;
};

// A recurrence wave's operands for one chunk. Loads are unconditional (tiles
// and rows clamped into range) so that the compiler counts outstanding loads
// exactly across the loop; rows past the end of a sequence are masked where
// they are used.
template <typename E, int C, int DK, int NT>
struct RStage {
    typedef ScanShape<E, C, DK> S;
    typename S::MD::Frag wf[S::KBD];
    typename S::MC::Frag tf[NT], ktf[S::NMW][S::KBC];  // Tb: the NT blocks read (tri_read_blocks)

    __device__ __forceinline__ void load(const E *__restrict__ tbmat, const E *__restrict__ wmat,
                                         const E *__restrict__ ktmat, const ChunkRef &r, int q, int lane) {
        const int rt = min(q, S::RT - 1);
        const size_t mat0 = r.ch * (size_t)(C * C), w0 = r.ch * (size_t)(C * DK), kq0 = r.kq * (size_t)(C * DK);
#pragma unroll
        for (int kb = 0; kb < NT; ++kb)
            tf[kb] = *reinterpret_cast<const typename S::MC::Frag *>(tbmat + mat0 + frag_off<typename S::MC>(rt * S::KBC + kb, lane));
#pragma unroll
        for (int kb = 0; kb < S::KBD; ++kb)
            wf[kb] = *reinterpret_cast<const typename S::MD::Frag *>(wmat + w0 + frag_off<typename S::MD>(rt * S::KBD + kb, lane));
#pragma unroll
        for (int j = 0; j < S::NMW; ++j) {
            const int mt = min(q + 4 * j, S::MT - 1);
#pragma unroll
            for (int kb = 0; kb < S::KBC; ++kb)
                ktf[j][kb] = *reinterpret_cast<const typename S::MC::Frag *>(ktmat + kq0 + frag_off<typename S::MC>(mt * S::KBC + kb, lane));
        }
    }
};

struct NoAux {};
template <int N> struct VRows { f32x4 x[N]; };

// An output wave's operands for one chunk (and that chunk's V rows, which
// the wave stages one chunk earlier).
template <typename E, int C, int DK, int NT, int R>
struct OStage {
    typedef ScanShape<E, C, DK> S;
    typename S::MD::Frag qf[S::KBD];
    typename S::MC::Frag pf[NT];  // P: the NT blocks read (tri_read_blocks)
    typename S::E4 vr;  // fp32: V[16 q + l/4][4 (l%4) ..]
    f32x4 aux = {0.f, 0.f, 0.f, 0.f};  // auxiliary load (see the output role of the scan)
    // Slices of 32 rows or more: the V rows 16 q .. 16 q + 15 of the slice,
    // 8 values per lane and load, R / 32 loads
    typename std::conditional<(R > 16), VRows<R / 32>, NoAux>::type vaux;

    __device__ __forceinline__ void load(const E *__restrict__ v, const E *__restrict__ pmat,
                                         const E *__restrict__ qmat, const ChunkRef &r, int hv, int h,
                                         int col0, int q, int lane) {
        const int rt = min(q, S::RT - 1);
        const size_t mat0 = r.ch * (size_t)(C * C), kq0 = r.kq * (size_t)(C * DK);
        if constexpr (!IsBf16<E>::value) {  // bf16: V comes through the auxiliary loads
            const int vrow = min(16 * rt + (lane >> 2), r.clen - 1);
            vr = *reinterpret_cast<const typename S::E4 *>(v + ((size_t)(r.tok0 + vrow) * hv + h) * DK + col0 + 4 * (lane & 3));
        }
#pragma unroll
        for (int kb = 0; kb < S::KBD; ++kb)
            qf[kb] = *reinterpret_cast<const typename S::MD::Frag *>(qmat + kq0 + frag_off<typename S::MD>(rt * S::KBD + kb, lane));
#pragma unroll
        for (int kb = 0; kb < NT; ++kb)
            pf[kb] = *reinterpret_cast<const typename S::MC::Frag *>(pmat + mat0 + frag_off<typename S::MC>(rt * S::KBC + kb, lane));
    }
};

// Runs body(st, nxt, fut, c, idx) for chunks c = 0 .. nch-1 over N register
// stages used round robin: chunk c sits in st[c % N], `nxt` holds chunk c + 1
// and `fut` (which held chunk c - 1) is refilled with chunk c + N - 1. The
// loop is unrolled by N so that every stage index is a compile-time
// constant (the stages stay in registers); idx is that index, I (so c + I
// has I's parity when N is even). st[0 .. N-2] must hold chunks 0 .. N-2 on
// entry.
template <int N, int I = 0, typename St, typename Body>
__device__ __forceinline__ void pipeline_step(St (&st)[N], int c, Body &body) {
    body(st[I], st[(I + 1) % N], st[(I + N - 1) % N], c + I, std::integral_constant<int, I>());
    if constexpr (I + 1 < N) pipeline_step<N, I + 1>(st, c, body);
}
template <int N, int I = 0, typename St, typename Body>
__device__ __forceinline__ void pipeline_tail(St (&st)[N], int c, int nch, Body &body) {
    if constexpr (I + 1 < N) {
        if (c + I < nch)
            body(st[I], st[(I + 1) % N], st[(I + N - 1) % N], c + I, std::integral_constant<int, I>());
        pipeline_tail<N, I + 1>(st, c, nch, body);
    }
}
template <int N, typename St, typename Body>
__device__ __forceinline__ void run_pipeline(St (&st)[N], int nch, Body &body) {
    int c = 0;
    for (; c + N - 1 < nch; c += N) pipeline_step<N>(st, c, body);
    pipeline_tail<N>(st, c, nch, body);
}

// Keeps a loaded value alive without using it (the load of an L2 touch).
__device__ __forceinline__ void keep_alive(float x) { asm volatile("" ::"v"(x)); }

// Chunks ahead of the scan at which its operands are pulled into L2.
constexpr int kTouchAhead = 8;

// Spin limit of the fused normalisation's wait for the other row slices'
// partial sums (each retry is an s_sleep 2 and a device-coherent load, about
// a microsecond, so roughly a second in all). Every slice of the grid runs
// once CUs free up, so a wait ends unless something holds CUs that long (a
// persistent kernel on another stream, say); past the limit the rows are
// written as NaN rather than wrong, and the kernel still ends.
constexpr int kNormSpinMax = 1 << 20;

// Word 3 of a raw buffer resource on gfx9-family GPUs (gfx950 included).
constexpr int kBufferWord3 = 0x00020000;

template <typename E, int C, int DK, typename SE, int R, bool kNorm>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gdn_scan_kernel(
    const E *__restrict__ v,
    const int32_t *__restrict__ bounds, const int32_t *__restrict__ seq_chunk0,
    const int32_t *__restrict__ order,
    const E *__restrict__ tbmat, const E *__restrict__ pmat, const E *__restrict__ wmat,
    const E *__restrict__ qmat, const E *__restrict__ ktmat,
    const float *__restrict__ gates,
    const SE *__restrict__ s0, SE *__restrict__ sfin, E *__restrict__ out,
    int32_t num_seqs, int32_t hk, int32_t hv,
    const float *__restrict__ norm_w, float norm_eps, float *__restrict__ norm_part)
{
    static_assert(R == 16 || ((R == 32 || R == 64 || R == 128) && IsBf16<E>::value && DK >= R),
                  "slices of 32 rows or more: bf16, d >= rows");
    typedef ScanSmem<E, C, DK, R, kNorm && (DK / R > 1)> L;
    typedef ScanShape<E, C, DK> SH;
    typedef typename SH::MD MD;
    typedef typename SH::MC MC;
    typedef typename SH::E4 E4;
    constexpr int DV = DK;
    constexpr int NS = DV / R;  // value-row slices per head
    constexpr int RW = R / 16;  // 16-row tiles per slice
    constexpr int LDK = L::LDK, LDC = L::LDC;
    constexpr int RT = SH::RT, MT = SH::MT, NMW = SH::NMW;
    constexpr int KBD = SH::KBD, KBC = SH::KBC;
    // Register stages per role; fp32 fragments are 4x larger and take fewer.
    // The fused normalisation's exchange alternates two register slots by
    // chunk parity, which the unrolled pipeline keeps compile-time when the
    // output stages are even.
    constexpr int kRStages = !IsBf16<E>::value ? 2 : R == 16 ? 4 : R <= 64 ? 3 : 2,
                  kOStages = !IsBf16<E>::value ? (kNorm ? 4 : 3) : R == 16 && !kNorm ? 5 : R <= 32 ? 4 : 3;
    // The fused normalisation: with several slices per head they exchange
    // partial sums (kNormX); a slice that holds the whole head (R = DV)
    // normalises its rows in the output wave that computes them (kNormW).
    constexpr bool kNormX = kNorm && NS > 1, kNormW = kNorm && NS == 1;

    extern __shared__ __align__(16) char smem[];
    E *sS = reinterpret_cast<E *>(smem + L::off_S);
    E *sUt = reinterpret_cast<E *>(smem + L::off_Ut);
    E *sDUt = reinterpret_cast<E *>(smem + L::off_DUt);
    E *sVt = reinterpret_cast<E *>(smem + L::off_Vt);
    float *sDl = reinterpret_cast<float *>(smem + L::off_Dl);
    float *sSg = reinterpret_cast<float *>(smem + L::off_Sg);
    float *sGc = reinterpret_cast<float *>(smem + L::off_Gc);

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

    // readfirstlane: the wave index is uniform across the wave, and saying so
    // makes role and wave branches scalar.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = wave & 3;
    const bool recurrence = wave < 4;
    const int g4 = lane >> 4, ln = lane & 15;
    const int start = bounds[n];
    const int len = bounds[n + 1] - start;
    const int nch = (len + C - 1) / C;
    const int c0 = seq_chunk0[n];
    const size_t state0 = ((size_t)n * hv + h) * (size_t)(DV * DK);

    auto chunk = [&](int c) {
        ChunkRef r;
        r.tok0 = start + c * C;
        r.clen = min(C, len - c * C);
        r.ch = (size_t)(c0 + c) * hv + h;
        r.kq = (size_t)(c0 + c) * hk + kh;
        return r;
    };

    // Each role runs as one of two instantiations, by the number NT of Tb or P
    // blocks its token tile reads (tri_read_blocks), so that every load count
    // in its loop is a compile-time constant.
    constexpr int kNtLo = tri_read_blocks<MC, C>(0);
    auto by_tile = [&](auto &&role) {
        if constexpr (kNtLo == KBC) {
            role(std::integral_constant<int, KBC>());
        } else {
            if (tri_read_blocks<MC, C>(min(q, RT - 1)) == kNtLo) role(std::integral_constant<int, kNtLo>());
            else role(std::integral_constant<int, KBC>());
        }
    };

    if (recurrence) by_tile([&](auto ntc) {
        constexpr int NT = decltype(ntc)::value;
        typedef RStage<E, C, DK, NT> RS;
        // fp32 master copy of this wave's S^T tiles (key tiles q + 4 j, row
        // tiles rr); operand copy (S[value][key]) in LDS.
        f32x4 sacc[NMW][RW];
#pragma unroll
        for (int j = 0; j < NMW; ++j) {
            const int mt = q + 4 * j;
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                sacc[j][rr] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (mt < MT) {
                    if (s0) sacc[j][rr] = load4f<SE>(s0 + state0 + (size_t)(col0 + 16 * rr + ln) * DK + 16 * mt + 4 * g4);
                    store_acc_p<MD>(sS, LDK, 16 * mt, 16 * rr, lane, sacc[j][rr]);
                }
            }
        }
        __syncthreads();  // S0 and chunk 0's V rows staged

        auto body = [&](RS &st, RS &, RS &fut, int c, auto) {
            // ---- phase 1: U = Tb V - W S0^T (W is stored negated). Token and
            // key contractions accumulate separately: with d = 16 they use
            // MFMAs of different shapes, which must not be chained through
            // one accumulator; two key chains shorten the dependency.
            if (q < RT) {
                const f32x4 dl = *reinterpret_cast<const f32x4 *>(sDl + (c & 1) * C + 16 * q + 4 * g4);
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) {
                    typename MC::Frag vf[NT];
                    typename MD::Frag sf[KBD];
#pragma unroll
                    for (int kb = 0; kb < NT; ++kb)
                        vf[kb] = load_frag_p<MC>(sVt + (c & 1) * (R * LDC), LDC, 16 * rr, kb, lane);
#pragma unroll
                    for (int kb = 0; kb < KBD; ++kb) sf[kb] = load_frag_p<MD>(sS, LDK, 16 * rr, kb, lane);
                    f32x4 ut = {0.f, 0.f, 0.f, 0.f}, uk0 = {0.f, 0.f, 0.f, 0.f}, uk1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < NT; ++kb) ut = MC::mma(st.tf[kb], vf[kb], ut);
#pragma unroll
                    for (int kb = 0; kb < KBD; ++kb) {
                        if (kb & 1) uk1 = MD::mma(st.wf[kb], sf[kb], uk1);
                        else uk0 = MD::mma(st.wf[kb], sf[kb], uk0);
                    }
                    const f32x4 u = ut + uk0 + uk1;
                    store_acc_p<MC>(sUt, LDC, 16 * q, 16 * rr, lane, u);
                    f32x4 du;
#pragma unroll
                    for (int i = 0; i < 4; ++i) du[i] = dl[i] * u[i];
                    store_acc_p<MC>(sDUt, LDC, 16 * q, 16 * rr, lane, du);
                }
            }
            __syncthreads();
            // ---- phase 2: S^T <- gamma_C S^T + K^T (diag(delta) U)
            // The prefetch is issued here rather than at the chunk start: phase 1
            // bounds the chunk through these waves, phase 2 through the output
            // waves, so a load queue that is full costs less here.
            fut.load(tbmat, wmat, ktmat, chunk(min(c + kRStages - 1, nch - 1)), q, lane);
            const float gc = sGc[4 * (c & 1)];
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                typename MC::Frag duf[KBC];
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) duf[kb] = load_frag_p<MC>(sDUt, LDC, 16 * rr, kb, lane);
#pragma unroll
                for (int j = 0; j < NMW; ++j) {
                    const int mt = q + 4 * j;
                    if (mt < MT) {
                        f32x4 acc = sacc[j][rr];
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[i] *= gc;
#pragma unroll
                        for (int kb = 0; kb < KBC; ++kb) acc = MC::mma(st.ktf[j][kb], duf[kb], acc);
                        sacc[j][rr] = acc;
                        store_acc_p<MD>(sS, LDK, 16 * mt, 16 * rr, lane, acc);
                    }
                }
            }
            __syncthreads();
        };

        if (nch > 0) {
            RS st[kRStages];
#pragma unroll
            for (int i = 0; i + 1 < kRStages; ++i) st[i].load(tbmat, wmat, ktmat, chunk(min(i, nch - 1)), q, lane);
            run_pipeline<kRStages>(st, nch, body);
        }

        if constexpr (kNormX) {
            if (nch > 0) {  // the output waves' drain
                for (int st = 0; st < 2 * kNormLag; ++st) __syncthreads();
            }
        }
        if (sfin) {
#pragma unroll
            for (int j = 0; j < NMW; ++j) {
                const int mt = q + 4 * j;
#pragma unroll
                for (int rr = 0; rr < RW; ++rr)
                    if (mt < MT)
                        store4<SE>(sfin + state0 + (size_t)(col0 + 16 * rr + ln) * DK + 16 * mt + 4 * g4, sacc[j][rr]);
            }
        }
    });
    else by_tile([&](auto ntc) {
        constexpr int NT = decltype(ntc)::value;
        typedef OStage<E, C, DK, NT, R> OS;
        // Besides its Q and P fragments, each output wave issues one auxiliary
        // 16-byte-per-lane load per chunk (bf16):
        //   wave 0     the chunk's gate record (delta and gamma_C for the
        //              recurrence waves, scale gamma for the outputs),
        //              staged in LDS;
        //   wave 1     16-row slices: an L2 touch of the chunk kTouchAhead
        //              ahead: the 16 workgroups of the query/key head split
        //              that chunk's operands (Q, K^T, and Tb, P, W of each
        //              value head of the group) and its V rows (128-byte
        //              lines) 64 lines each, one line per lane, so that the
        //              workgroups' own loads later hit L2; the value is only
        //              kept alive until the stage is refilled;
        //   waves 2-3  16-row slices: the chunk's V rows 32 (q - 2) .. + 31
        //              (8 values per lane), staged in LDS.
        // With wider slices waves 1-3 load the gate record again (no touch,
        // below), and every output wave loads the V rows 16 q .. 16 q + 15
        // of its R columns besides (R / 32 loads).
        // Memory instructions, not bytes, bound the scan, so these small
        // loads are folded into as few instructions as possible. fp32 I/O
        // loads V in every output wave with its fragments, and waves 1-3
        // touch (16-row slices) or load the gate record again.
        constexpr int kRunQ = (int)((size_t)C * DK * sizeof(E) / 1024);
        constexpr int kRunM = (int)((size_t)C * C * sizeof(E) / 1024);
        // The L2 touch serves 16-row slices only: wider slices share each
        // line among fewer workgroups, and their touches, which wait on HBM
        // in the issuing wave's load queue, measured slower than none (scan
        // at 2 x 2048, 32 rows: 62.5 against 55.3 us; 4 x 1024, 64 rows:
        // 50.9 against 45.8 us; 4 rotated buffer sets).
        constexpr bool kTouch = (size_t)C * DK * sizeof(E) % 1024 == 0 &&
                                (size_t)C * C * sizeof(E) % 1024 == 0 && R == 16;
        auto gate_ptr = [&](const ChunkRef &r) {
            // the chunk's gate record, 4 floats per lane: lanes [0, C/4)
            // delta, [C/4, C/2) scale gamma, C/2 gamma_C
            return reinterpret_cast<const f32x4 *>(gates + r.ch * (size_t)gate_record(C) + 4 * min(lane, C / 2));
        };
        auto touch_ptr = [&](int cc) {
            const size_t kq = (size_t)(c0 + cc) * hk + kh;
            const size_t ch0 = (size_t)(c0 + cc) * hv + (size_t)kh * group;
            const int per_head = 2 * kRunM + kRunQ;
            const int nops = 8 * (2 * kRunQ + group * per_head);
            // then the chunk's V rows of each value head of the group, from
            // the caller's tensor (cold in HBM, unlike the workspace the
            // preparation kernel has just written)
            constexpr int kLinesPerRow = DK * (int)sizeof(E) >= 128 ? DK * (int)sizeof(E) / 128 : 1;
            const int nlines = nops + C * group * kLinesPerRow;
            const int line = (within * 64 + lane) % nlines;
            if (line >= nops) {
                const int vl = line - nops, per_tok = group * kLinesPerRow;
                const ChunkRef rc = chunk(cc);
                const int t = min(vl / per_tok, rc.clen - 1), rem = vl % per_tok;
                const int hh = rem / kLinesPerRow, hf = rem - hh * kLinesPerRow;
                return reinterpret_cast<const f32x4 *>(v + ((size_t)(rc.tok0 + t) * hv + (size_t)kh * group + hh) * DK +
                                                       (size_t)hf * (128 / sizeof(E)));
            }
            int r = line >> 3;
            const size_t off = (size_t)(line & 7) * (128 / sizeof(E));
            const E *run;
            if (r < kRunQ) {
                run = qmat + kq * (size_t)(C * DK) + (size_t)r * (1024 / sizeof(E));
            } else if (r < 2 * kRunQ) {
                run = ktmat + kq * (size_t)(C * DK) + (size_t)(r - kRunQ) * (1024 / sizeof(E));
            } else {
                r -= 2 * kRunQ;
                const int hh = r / (per_head > 0 ? per_head : 1);
                r -= hh * per_head;
                const size_t chh = ch0 + hh;
                if (r < kRunM) run = tbmat + chh * (size_t)(C * C) + (size_t)r * (1024 / sizeof(E));
                else if (r < 2 * kRunM) run = pmat + chh * (size_t)(C * C) + (size_t)(r - kRunM) * (1024 / sizeof(E));
                else run = wmat + chh * (size_t)(C * DK) + (size_t)(r - 2 * kRunM) * (1024 / sizeof(E));
            }
            return reinterpret_cast<const f32x4 *>(run + off);
        };
        auto aux_ptr = [&](int c_aux, int c_touch) {
            const ChunkRef r = chunk(c_aux);
            if (q == 0) return gate_ptr(r);
            if (q == 1 || R > 16 || !IsBf16<E>::value) return kTouch ? touch_ptr(c_touch) : gate_ptr(r);
            const int vrow = min(32 * (q - 2) + (lane >> 1), r.clen - 1);
            return reinterpret_cast<const f32x4 *>(v + ((size_t)(r.tok0 + vrow) * hv + h) * DK + col0 + 8 * (lane & 1));
        };
        // The load is unconditional; only its address depends on the wave.
        auto load_aux = [&](OS &st, int c_aux, int c_touch) {
            keep_alive(st.aux[0]);  // wave 1: the touch issued when this stage was last filled
            st.aux = *aux_ptr(c_aux, c_touch);
            if constexpr (R > 16) {
                const ChunkRef r = chunk(c_aux);
                const int vrow = min(16 * q + (lane >> 2), r.clen - 1);
                const E *src = v + ((size_t)(r.tok0 + vrow) * hv + h) * DK + col0 + 8 * (lane & 3);
#pragma unroll
                for (int j = 0; j < R / 32; ++j) st.vaux.x[j] = *reinterpret_cast<const f32x4 *>(src + 32 * j);
            }
        };
        // A chunk's staged inputs into LDS buffer `buf`: the gate vectors
        // (wave 0) and, bf16, the V rows (waves 2, 3) from the auxiliary load;
        // fp32, each wave's V rows.
        auto put_chunk = [&](const OS &st, const E4 &vr, int buf) {
            if (q == 0 && lane <= C / 2) {
                if (lane < C / 2) {
                    float *dst = lane < C / 4 ? sDl + buf * C + 4 * lane : sSg + buf * C + 4 * (lane - C / 4);
                    *reinterpret_cast<f32x4 *>(dst) = st.aux;
                } else {
                    sGc[4 * buf] = st.aux[0];
                }
            }
            if constexpr (R > 16) {
                const int t = 16 * q + (lane >> 2);
                if (t < C) {
                    E *dst = sVt + buf * (R * LDC) + lds_pos<MC>(t);
#pragma unroll
                    for (int j = 0; j < R / 32; ++j) {
                        const bf16x8 x = __builtin_bit_cast(bf16x8, st.vaux.x[j]);
#pragma unroll
                        for (int i = 0; i < 8; ++i) dst[(32 * j + 8 * (lane & 3) + i) * LDC] = x[i];
                    }
                }
            } else if constexpr (IsBf16<E>::value) {
                if (q >= 2) {
                    const int t = 32 * (q - 2) + (lane >> 1);
                    if (t < C) {
                        const bf16x8 x = __builtin_bit_cast(bf16x8, st.aux);
                        E *dst = sVt + buf * (R * LDC) + lds_pos<MC>(t);
#pragma unroll
                        for (int i = 0; i < 8; ++i) dst[(8 * (lane & 1) + i) * LDC] = x[i];
                    }
                }
            } else if (q < RT) {
                E *dst = sVt + buf * (R * LDC) + lds_pos<MC>(16 * q + (lane >> 2));
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(4 * (lane & 3) + i) * LDC] = vr[i];
            }
        };
        // ---- output normalisation fused in (kNorm). A slice of the whole
        // head (NS = 1) normalises each row in the output wave that computes
        // it. Otherwise a (token, value head) output row spans the NS row
        // slices of the head, each its own workgroup. Per chunk c, in the
        // workgroup's step
        //   c      every output wave computes its tokens' partial sums of
        //          squares (its columns, then the token's four lane groups)
        //          into LDS, after its outputs, which it keeps in an LDS ring
        //          of kNormLag chunks;
        //   c + 1  output wave 0 publishes the chunk's C partials in the slot
        //          block (chunk, head, slice) with one device-coherent store
        //          (each slot holds kNormPartEmpty until then, set by the
        //          preparation kernel);
        //   c + 2  output wave 1 loads the head's block of the chunk, every
        //          slice's partials, device-coherent: a step and a half after
        //          the slices published them, if they run together;
        //   c + 4  output wave 1 adds each token's NS partials in slice order
        //          (the same sum in every slice) into LDS, and every output
        //          wave writes its rows o w / sqrt(mean + eps): one rounding
        //          of the unrounded outputs kept in the ring.
        // Three memory instructions per workgroup and chunk in all. Each slot
        // is written once per call, so a value other than kNormPartEmpty is
        // that call's partial; the rare wait for a slice behind spins with
        // s_sleep, bounded.
        const int slice = within % NS;
        float *sNp = reinterpret_cast<float *>(smem + L::off_Np);
        float *sNb = reinterpret_cast<float *>(smem + L::off_Nb);
        float *sNt = reinterpret_cast<float *>(smem + L::off_Nt);
        // the slice's normalisation weights, staged in LDS before the first
        // barrier; weight(rr): this lane's four columns of row tile rr
        float *sNw = reinterpret_cast<float *>(smem + L::off_Nw);
        if constexpr (kNorm) {
            const int ot = tid - 256;  // this output wave's thread
            if (ot >= 0 && ot < R) sNw[ot] = norm_w[col0 + ot];
        }
        auto weight = [&](int rr) { return *reinterpret_cast<const f32x4 *>(sNw + 16 * rr + 4 * g4); };
        auto chunk_rows = [&](int cc) { return min(C, len - cc * C); };
        // The head's block of chunk cc's partials, NS x C floats, through a
        // buffer resource: 16-byte loads and stores that bypass the CU's
        // cache (sc1, device coherence), with reads past the block giving 0.
        constexpr int kBlkPieces = NS * C / 4, kBlkLoads = (kBlkPieces + 63) / 64;
        constexpr int kCoherent = 16;  // sc1
        auto part_rsrc = [&](int cc, int first_slice, int slices) {
            return __builtin_amdgcn_make_buffer_rsrc(
                norm_part + (((size_t)(c0 + cc) * hv + h) * NS + first_slice) * C, (short)0, slices * C * 4,
                kBufferWord3);
        };
        // Two register slots for blocks in flight, by chunk step parity: a
        // block is loaded two steps before it is summed, as device-coherent
        // loads reach the other slices' stores only through the L2s' backing
        // (agent scope) and take about a step to return.
        f32x4 blk0[kBlkLoads], blk1[kBlkLoads];
        auto load_into = [&](f32x4 (&b)[kBlkLoads], int cc) {
            const auto rs = part_rsrc(cc, 0, NS);
#pragma unroll
            for (int i = 0; i < kBlkLoads; ++i)
                b[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (64 * i + lane) * 16, 0,
                                                                                       kCoherent));
        };
        auto load_block = [&](int cc, int par) {
            if (par) load_into(blk1, cc);
            else load_into(blk0, cc);
        };
        // Whether every slot of chunk cc's block holds a partial. Evaluated
        // without short-circuit branches: a branch here would leave some of
        // the block's loads possibly outstanding where the paths meet, and
        // the compiler would then wait for every load in flight, the operand
        // prefetches included.
        auto block_ready = [&](const f32x4 (&b)[kBlkLoads], int cc) {
            const int rows = chunk_rows(cc);
            int ok = 1;
#pragma unroll
            for (int i = 0; i < kBlkLoads; ++i) {
                const int pc = 64 * i + lane, t0 = (pc % (C / 4)) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ok &= (int)(pc >= kBlkPieces) | (int)(t0 + e >= rows) | (int)(b[i][e] != kNormPartEmpty);
            }
            return __all(ok);
        };
        // Output wave 1: chunk cc's totals into LDS, from the block in slot
        // par. The first check is straight-line code, so that waiting for
        // these loads does not wait for the later operand prefetches; only
        // the rare retry loop (a slice behind) waits for everything, and
        // after kNormSpinMax retries the totals are NaN (the rows are written
        // as NaN rather than wrong).
        auto sum_from = [&](f32x4 (&b)[kBlkLoads], int cc) {
            bool ok = true;
            if (!block_ready(b, cc)) {
                for (int spin = 0;; ++spin) {
                    if (spin >= kNormSpinMax) {
                        ok = false;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                    // The loop stores nothing; without this compiler barrier
                    // its loads are hoisted out of it, and a slice that found
                    // a slot empty would test the same registers until the
                    // spin limit.
                    asm volatile("" ::: "memory");
                    load_into(b, cc);
                    if (block_ready(b, cc)) break;
                }
            }
#pragma unroll
            for (int i = 0; i < kBlkLoads; ++i)
                if (64 * i + lane < kBlkPieces) *reinterpret_cast<f32x4 *>(sNb + 4 * (64 * i + lane)) = b[i];
            if (lane < C) {  // the wave reads back its own LDS writes
                float tot = 0.f;
#pragma unroll
                for (int sl = 0; sl < NS; ++sl) tot += sNb[sl * C + lane];
                sNt[lane] = ok ? tot : __builtin_nanf("");
            }
        };
        auto sum_block = [&](int cc, int par) {
            if (par) sum_from(blk1, cc);
            else sum_from(blk0, cc);
        };
        // Output wave 0: chunk cc's partials from LDS to its slots.
        auto publish_block = [&](int cc) {
            const auto rs = part_rsrc(cc, slice, 1);
            if (lane < C / 4)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4 *>(sNp + 4 * lane)), rs, lane * 16, 0,
                    kCoherent);
        };
        // This wave's partial sums of squares of chunk cc's outputs po.
        auto put_partials = [&](int cc, const f32x4 (&po)[RW]) {
            float sq = 0.f;
#pragma unroll
            for (int rr = 0; rr < RW; ++rr)
#pragma unroll
                for (int i = 0; i < 4; ++i) sq = __builtin_fmaf(po[rr][i], po[rr][i], sq);
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
            if (g4 == 0) sNp[16 * q + ln] = sq;
        };
        // The exchange's work in the two phases of step st (par: st's
        // parity): publish chunk st - 1, sum chunk st - kNormLag (phase 1);
        // write chunk st - kNormLag's rows and load chunk st + 2 - kNormLag's
        // block (phase 2, after this step's outputs), into the slot just
        // summed. The loop's steps load unconditionally (a clamped chunk),
        // so that its load count is fixed; the drain's steps past the last
        // chunk skip what does not exist.
        auto norm_phase1 = [&](int st, int par) {
            if (q == 0 && st >= 1 && st - 1 < nch) publish_block(st - 1);
            if (q == 1 && st >= kNormLag && st - kNormLag < nch) sum_block(st - kNormLag, par);
        };
        // The wave's unnormalised outputs of chunk cc, in the LDS ring (each
        // lane reads back only what it wrote).
        auto pend_at = [&](int cc, int rr) -> f32x4 * {
            return reinterpret_cast<f32x4 *>(smem + L::off_Pd) +
                   ((((cc & (kNormLag - 1)) * 4 + q) * RW + rr) * 64 + lane);
        };
        auto stash = [&](int cc, const f32x4 (&oc)[RW]) {
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) *pend_at(cc, rr) = oc[rr];
        };
        // Normalise and store chunk cc's outputs (its totals in LDS).
        auto finish = [&](int cc) {
            const int row = 16 * q + ln;
            const float r = 1.0f / sqrtf(sNt[row] * (1.0f / DV) + norm_eps);
            if (row < chunk_rows(cc)) {
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) {
                    const f32x4 po = *pend_at(cc, rr), wr = weight(rr);
                    E4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(po[i] * r * wr[i]);
                    *reinterpret_cast<E4 *>(out + ((size_t)(start + cc * C + row) * hv + h) * DV + col0 + 16 * rr +
                                            4 * g4) = w;
                }
            }
        };

        OS st[kOStages];
        if (nch > 0) {
            st[0].load(v, pmat, qmat, chunk(0), hv, h, col0, q, lane);
            load_aux(st[0], 0, min(kTouchAhead, nch - 1));
            put_chunk(st[0], st[0].vr, 0);
        }
        __syncthreads();  // S0 and chunk 0's V rows staged

        // One chunk c with its operands in `st`; `nxt` holds chunk c + 1,
        // whose V rows are staged here, and `fut` is refilled with chunk
        // c + kOStages - 1.
        auto body = [&](OS &st, OS &nxt, OS &fut, int c, auto idx) {
            const int cf = min(c + kOStages - 1, nch - 1);
            load_aux(fut, cf, min(c + kTouchAhead, nch - 1));
            fut.load(v, pmat, qmat, chunk(cf), hv, h, col0, q, lane);
            // The next chunk's V rows and gate vectors go to LDS now, while
            // this wave would wait for the recurrence waves anyway (their
            // buffers were last read before the previous barrier).
            put_chunk(nxt, nxt.vr, (c + 1) & 1);
            // the step's parity: compile-time in the unrolled pipeline
            constexpr int kIdx = decltype(idx)::value;
            const int par = kOStages % 2 == 0 ? (kIdx & 1) : (c & 1);
            if constexpr (kNormX) norm_phase1(c, par);
            // ---- phase 1: O1^T = S0 Q^T
            f32x4 o1[RW];
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                o1[rr] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (q < RT) {
#pragma unroll
                    for (int kb = 0; kb < KBD; ++kb)
                        o1[rr] = MD::mma(load_frag_p<MD>(sS, LDK, 16 * rr, kb, lane), st.qf[kb], o1[rr]);
                }
            }
            __syncthreads();
            // ---- phase 2: O^T = O1^T diag(scale gamma) + U^T P^T; lane: token
            // 16 q + l%16, value columns 4 (l/16) .. + 3
            const int tok0 = start + c * C;
            const int clen = min(C, len - c * C);
            if (q < RT) {
                const int row = 16 * q + ln;
                const float sg = sSg[(c & 1) * C + row];
                f32x4 oc[RW];
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) {
                    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < NT; ++kb) o = MC::mma(load_frag_p<MC>(sUt, LDC, 16 * rr, kb, lane), st.pf[kb], o);
#pragma unroll
                    for (int i = 0; i < 4; ++i) oc[rr][i] = sg * o1[rr][i] + o[i];
                    if constexpr (!kNorm) {
                        if (row < clen) {
                            E4 w;
#pragma unroll
                            for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(oc[rr][i]);
                            *reinterpret_cast<E4 *>(out + ((size_t)(tok0 + row) * hv + h) * DV + col0 + 16 * rr + 4 * g4) = w;
                        }
                    }
                }
                if constexpr (kNormX) {
                    put_partials(c, oc);
                    if (c >= kNormLag) finish(c - kNormLag);  // its slot, then this chunk's
                    stash(c, oc);
                }
                if constexpr (kNormW) {
                    // the whole row: this lane's columns, then its 4 lane groups
                    float sq = 0.f;
#pragma unroll
                    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
                        for (int i = 0; i < 4; ++i) sq = __builtin_fmaf(oc[rr][i], oc[rr][i], sq);
                    sq += __shfl_xor(sq, 16);
                    sq += __shfl_xor(sq, 32);
                    const float rs = 1.0f / sqrtf(sq * (1.0f / DV) + norm_eps);
                    if (row < clen) {
#pragma unroll
                        for (int rr = 0; rr < RW; ++rr) {
                            const f32x4 wr = weight(rr);
                            E4 w;
#pragma unroll
                            for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(oc[rr][i] * rs * wr[i]);
                            *reinterpret_cast<E4 *>(out + ((size_t)(tok0 + row) * hv + h) * DV + col0 + 16 * rr +
                                                    4 * g4) = w;
                        }
                    }
                }
            }
            if constexpr (kNormX) {
                if (q == 1) load_block(max(c + 2 - kNormLag, 0), par);
            }
            __syncthreads();
        };

        if (nch > 0) {
#pragma unroll
            for (int i = 1; i + 1 < kOStages; ++i) {
                st[i].load(v, pmat, qmat, chunk(min(i, nch - 1)), hv, h, col0, q, lane);
                load_aux(st[i], min(i, nch - 1), min(i + kTouchAhead, nch - 1));
            }
            run_pipeline<kOStages>(st, nch, body);
            if constexpr (kNormX) {
                // the last kNormLag chunks' outputs, in kNormLag more steps
                // of two barriers (the recurrence waves take part)
                for (int st = nch; st < nch + kNormLag; ++st) {
                    norm_phase1(st, st & 1);
                    __syncthreads();
                    if (q < RT && st - kNormLag >= 0) finish(st - kNormLag);
                    if (q == 1 && st + 2 - kNormLag >= 0 && st + 2 - kNormLag < nch) load_block(st + 2 - kNormLag, st & 1);
                    __syncthreads();
                }
            }
        }
    });
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

// The scan, with states stored as SE (fp32, or bf16 with fp32 arithmetic)
// and R state rows per workgroup.
template <typename E, int C, int D, typename SE, int R, bool kNorm>
static hipError_t launch_scan_n(const PrefillArgs &A, hipStream_t st, int32_t *bounds, int32_t *seq_chunk0,
                                int32_t *order, E *tbmat, E *pmat, E *wmat, E *qmat, E *ktmat, float *gates,
                                float *norm_part) {
    typedef ScanSmem<E, C, D, R, kNorm && (D / R > 1)> SL;
    static std::atomic<bool> scan_ok{false};
    auto scan = gdn_scan_kernel<E, C, D, SE, R, kNorm>;
    hipError_t e;
    if ((e = allow_smem(scan, SL::bytes, scan_ok)) != hipSuccess) return e;
    const int64_t grid = scan_grid(A.num_seqs, A.hk, A.hv, D, R);
    return launch_kernel(kScan, scan, dim3((unsigned)grid), dim3(kScanThreads), SL::bytes, st,
                         (const E *)A.v, (const int32_t *)bounds, (const int32_t *)seq_chunk0,
                         (const int32_t *)order, (const E *)tbmat, (const E *)pmat, (const E *)wmat,
                         (const E *)qmat, (const E *)ktmat, (const float *)gates, (const SE *)A.s0,
                         (SE *)A.s_final, (E *)A.out, A.num_seqs, A.hk, A.hv, A.norm_w, A.norm_eps, norm_part);
}

// With A.norm_w the normalisation is fused in (the caller has checked that
// the grid fits one pass, fused_norm_fits).
template <typename E, int C, int D, typename SE, int R>
static hipError_t launch_scan_r(const PrefillArgs &A, hipStream_t st, int32_t *bounds, int32_t *seq_chunk0,
                                int32_t *order, E *tbmat, E *pmat, E *wmat, E *qmat, E *ktmat, float *gates,
                                float *norm_part) {
    if (A.norm_w)
        return launch_scan_n<E, C, D, SE, R, true>(A, st, bounds, seq_chunk0, order, tbmat, pmat, wmat, qmat, ktmat,
                                                   gates, norm_part);
    return launch_scan_n<E, C, D, SE, R, false>(A, st, bounds, seq_chunk0, order, tbmat, pmat, wmat, qmat, ktmat,
                                                gates, norm_part);
}

// Every slice loads the head's whole chunk operands, so wider slices cut
// those loads per state row at the cost of a longer chunk step. That pays
// once narrower slices take more than one pass over the CUs (several
// sequences, or many heads); a single pass keeps the shorter step. The caller
// picks (scan_slice_rows, or a tuned choice).
template <typename E, int C, int D, typename SE>
static hipError_t launch_scan(const PrefillArgs &A, hipStream_t st, int32_t *bounds, int32_t *seq_chunk0,
                              int32_t *order, E *tbmat, E *pmat, E *wmat, E *qmat, E *ktmat, float *gates,
                              float *norm_part) {
    if constexpr (IsBf16<E>::value && D >= 32) {
        if (A.slice_rows == 32)
            return launch_scan_r<E, C, D, SE, 32>(A, st, bounds, seq_chunk0, order, tbmat, pmat, wmat, qmat, ktmat,
                                                  gates, norm_part);
    }
    if constexpr (IsBf16<E>::value && D >= 64) {
        if (A.slice_rows == 64)
            return launch_scan_r<E, C, D, SE, 64>(A, st, bounds, seq_chunk0, order, tbmat, pmat, wmat, qmat, ktmat,
                                                  gates, norm_part);
    }
    if constexpr (IsBf16<E>::value && D >= 128) {
        if (A.slice_rows == 128)
            return launch_scan_r<E, C, D, SE, 128>(A, st, bounds, seq_chunk0, order, tbmat, pmat, wmat, qmat, ktmat,
                                                   gates, norm_part);
    }
    return launch_scan_r<E, C, D, SE, 16>(A, st, bounds, seq_chunk0, order, tbmat, pmat, wmat, qmat, ktmat, gates,
                                          norm_part);
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
    E *tbmat = reinterpret_cast<E *>(ws + Y.off_tbmat);
    E *pmat = reinterpret_cast<E *>(ws + Y.off_pmat);
    E *wmat = reinterpret_cast<E *>(ws + Y.off_wmat);
    E *qmat = reinterpret_cast<E *>(ws + Y.off_qmat);
    E *ktmat = reinterpret_cast<E *>(ws + Y.off_ktmat);
    float *gates = reinterpret_cast<float *>(ws + Y.off_gates);
    float *norm_part = reinterpret_cast<float *>(ws + Y.off_norm_part);
    // state rows per scan workgroup (launch_scan takes 32 only where it fits)
    const int scan_rows = IsBf16<E>::value && A.slice_rows > 16 && A.slice_rows <= D ? A.slice_rows : 16;

    // Up to kFoldMaxSeqs sequences the preparation kernel schedules itself.
    const bool fold = A.num_seqs <= kFoldMaxSeqs;
    hipError_t e = hipSuccess;
    if (!fold) {
        e = launch_schedule(A, st, bounds, seq_chunk0, order, chunk_seq, chunk_tok0, counters);
        if (e != hipSuccess) return e;
    }

    typedef PrepSmem<E, C, D> PL;
    static std::atomic<bool> prep_ok{false};
    auto prep = gdn_prep_kernel<E, G, C, D>;
    if ((e = allow_smem(prep, PL::bytes, prep_ok)) != hipSuccess) return e;
    e = launch_kernel(kPrep, prep, dim3((unsigned)Y.max_chunks, (unsigned)A.hk), dim3(256), PL::bytes, st,
                      (const E *)A.q, (const E *)A.k, (const G *)A.g, (const G *)A.beta,
                      fold ? A.cu : nullptr, A.num_seqs, (int32_t)A.total_tokens, bounds, seq_chunk0, order,
                      (const int32_t *)chunk_seq, (const int32_t *)chunk_tok0, (const int32_t *)counters,
                      tbmat, pmat, wmat, qmat, ktmat, gates, A.hk, A.hv, A.scale,
                      A.norm_w && scan_rows < D ? norm_part : nullptr,
                      A.norm_w && scan_rows < D ? (int32_t)(D / scan_rows) : 0);
    if (e != hipSuccess) return e;

    if constexpr (IsBf16<E>::value) {
        if (A.state_bf16)
            return launch_scan<E, C, D, bf16>(A, st, bounds, seq_chunk0, order, tbmat, pmat, wmat, qmat, ktmat, gates,
                                              norm_part);
    } else if (A.state_bf16) {
        return hipErrorInvalidValue;  // bf16 states are built for bf16 I/O only
    }
    return launch_scan<E, C, D, float>(A, st, bounds, seq_chunk0, order, tbmat, pmat, wmat, qmat, ktmat, gates,
                                       norm_part);
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

}  // namespace gdn

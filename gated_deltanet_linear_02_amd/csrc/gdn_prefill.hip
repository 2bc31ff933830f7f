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
//                blocked triangular inverse T and P. Writes T, P and the gate
//                vectors to the workspace.
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
// 2. Chunk preparation: T = (I + A)^-1, P and the gate vectors
// ---------------------------------------------------------------------------

template <typename E, int C, int DK>
struct PrepSmem {
    static constexpr int PE = Pad<E>::value;
    static constexpr int LDK = DK + PE;  // K, Q rows (elements)
    static constexpr int LDC = C + 1;    // fp32 C x C arrays
    static constexpr size_t kq_bytes = 2 * (size_t)C * LDK * sizeof(E);
    static constexpr size_t atz_bytes = 3 * (size_t)C * LDC * sizeof(float);
    static constexpr size_t region0 = ((kq_bytes > atz_bytes ? kq_bytes : atz_bytes) + 15) & ~(size_t)15;
    static constexpr size_t gp_bytes = 2 * (size_t)C * LDC * sizeof(float);
    static constexpr size_t bytes = region0 + gp_bytes + 2 * C * sizeof(float);
};

template <typename G> __device__ __forceinline__ float gate_load(const G *p, size_t i) {
    return static_cast<float>(p[i]);
}

template <typename E, typename G, int C, int DK>
__global__ __launch_bounds__(256) void gdn_prep_kernel(
    const E *__restrict__ q, const E *__restrict__ k,
    const G *__restrict__ gate_g, const G *__restrict__ gate_b,
    const int32_t *__restrict__ bounds, const int32_t *__restrict__ chunk_seq,
    const int32_t *__restrict__ chunk_tok0, const int32_t *__restrict__ counters,
    E *__restrict__ tmat, E *__restrict__ pmat, f32x4 *__restrict__ gates,
    float *__restrict__ gammac, int32_t hk, int32_t hv, float scale)
{
    typedef PrepSmem<E, C, DK> L;
    typedef Mma<E, DK> M;
    constexpr int NB = C / 16;
    constexpr int LDK = L::LDK, LDC = L::LDC;
    constexpr int EPV = 16 / sizeof(E);  // elements per 16-byte vector
    constexpr int VPR = DK / EPV;        // vectors per K/Q row

    extern __shared__ __align__(16) char smem[];
    E *sK = reinterpret_cast<E *>(smem);
    E *sQ = sK + C * LDK;
    float *sA = reinterpret_cast<float *>(smem);  // reuses the K/Q region
    float *sT = sA + C * LDC;
    float *sZ = sT + C * LDC;
    float *sG = reinterpret_cast<float *>(smem + L::region0);
    float *sP0 = sG + C * LDC;
    float *sc = sP0 + C * LDC;
    float *sb = sc + C;

    const int ci = blockIdx.x;
    const int kh = blockIdx.y;
    if (ci >= counters[0]) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = chunk_seq[ci];
    const int t0 = chunk_tok0[ci];
    const int len = min(C, bounds[n + 1] - t0);

    for (int i = tid; i < C * VPR; i += 256) {
        const int r = i / VPR, cv = i - r * VPR;
        const size_t src = ((size_t)(t0 + r) * hk + kh) * DK + cv * EPV;
        st16(sK + r * LDK + cv * EPV, r < len ? ld16(k + src) : zero16());
        st16(sQ + r * LDK + cv * EPV, r < len ? ld16(q + src) : zero16());
    }
    __syncthreads();

    // Gram K K^T and scores Q K^T on the lower-triangular 16x16 tiles.
    constexpr int NT = NB * (NB + 1) / 2;
    for (int t = wave; t < 2 * NT; t += 4) {
        const int which = t / NT;
        int tt = t - which * NT, ti = 0;
        while ((ti + 1) * (ti + 2) / 2 <= tt) ++ti;
        const int tj = tt - ti * (ti + 1) / 2;
        const E *Am = which ? sQ : sK;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < DK / M::KW; ++kb)
            acc = M::mma(load_frag<M>(Am, LDK, 16 * ti, kb * M::KW, lane),
                         load_frag<M>(sK, LDK, 16 * tj, kb * M::KW, lane), acc);
        float *dst = which ? sP0 : sG;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dst[(16 * ti + 4 * (lane >> 4) + i) * LDC + 16 * tj + (lane & 15)] = acc[i];
    }
    __syncthreads();

    const int group = hv / hk;
    for (int hh = 0; hh < group; ++hh) {
        const int h = kh * group + hh;
        const size_t mat0 = ((size_t)ci * hv + h) * (size_t)(C * C);

        // Gate prefix sums (C <= 64: the first wave holds all rows).
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

        // A (strictly lower), P (lower with diagonal), gate vectors.
        for (int e = tid; e < C * C; e += 256) {
            const int i = e / C, j = e - i * C;
            const float d = j <= i ? expf(sc[i] - sc[j]) : 0.f;
            sA[i * LDC + j] = j < i ? sb[i] * d * sG[i * LDC + j] : 0.f;
            pmat[mat0 + e] = from_f32<E>(j <= i ? scale * d * sP0[i * LDC + j] : 0.f);
        }
        if (tid < C) {
            const float last = sc[C - 1];
            const float gam = expf(sc[tid]);
            gates[((size_t)ci * hv + h) * C + tid] =
                f32x4{scale * gam, sb[tid], sb[tid] * gam, expf(last - sc[tid])};
            if (tid == 0) gammac[(size_t)ci * hv + h] = expf(last);
        }
        __syncthreads();

        // Diagonal 16x16 blocks by forward substitution, one lane per column.
        if (wave == 0 && lane < NB * 16) {
            const int base = 16 * (lane >> 4), col = lane & 15;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = i == col ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < i; ++s) acc -= sA[(base + i) * LDC + base + s] * x[s];
                x[i] = acc;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sT[(base + i) * LDC + base + col] = x[i];
        }
        // Blocks above the diagonal are zero.
        for (int e = tid; e < C * C; e += 256) {
            const int i = e / C, j = e - i * C;
            if ((j >> 4) > (i >> 4)) sT[i * LDC + j] = 0.f;
        }
        __syncthreads();

        // Off-diagonal blocks, one block diagonal at a time:
        //   T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj      (i = j + dist)
        for (int dist = 1; dist < NB; ++dist) {
            const int nblk = NB - dist;
            for (int e = tid; e < nblk * 256; e += 256) {
                const int j = e >> 8, i = j + dist;
                const int r = (e >> 4) & 15, c = e & 15;
                float z = 0.f;
                for (int m = j; m < i; ++m) {
#pragma unroll
                    for (int s = 0; s < 16; ++s)
                        z += sA[(16 * i + r) * LDC + 16 * m + s] * sT[(16 * m + s) * LDC + 16 * j + c];
                }
                sZ[(16 * i + r) * LDC + 16 * j + c] = z;
            }
            __syncthreads();
            for (int e = tid; e < nblk * 256; e += 256) {
                const int j = e >> 8, i = j + dist;
                const int r = (e >> 4) & 15, c = e & 15;
                float t = 0.f;
#pragma unroll
                for (int s = 0; s < 16; ++s)
                    t -= sT[(16 * i + r) * LDC + 16 * i + s] * sZ[(16 * i + s) * LDC + 16 * j + c];
                sT[(16 * i + r) * LDC + 16 * j + c] = t;
            }
            __syncthreads();
        }

        for (int e = tid; e < C * C; e += 256) {
            const int i = e / C, j = e - i * C;
            tmat[mat0 + e] = from_f32<E>(sT[i * LDC + j]);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// 3. Chunk-recurrent scan over one (sequence, value head, R value rows)
// ---------------------------------------------------------------------------

template <typename E> struct IsBf16 { static constexpr bool value = false; };
template <> struct IsBf16<bf16> { static constexpr bool value = true; };

template <typename E, int C, int DK, int R>
struct ScanSmem {
    static constexpr int PE = Pad<E>::value;
    static constexpr int LDK = DK + PE;  // rows of length DK
    static constexpr int LDC = C + PE;   // rows of length C
    static constexpr bool kKt = IsBf16<E>::value;  // K^T copy (bf16 fragments need it)
    static constexpr size_t off_K = 0;
    static constexpr size_t off_Q = off_K + (size_t)C * LDK * sizeof(E);
    static constexpr size_t off_Kt = off_Q + (size_t)C * LDK * sizeof(E);
    static constexpr size_t off_T = off_Kt + (kKt ? (size_t)DK * LDC * sizeof(E) : 0);
    static constexpr size_t off_P = off_T + (size_t)C * LDC * sizeof(E);
    static constexpr size_t off_Vt = off_P + (size_t)C * LDC * sizeof(E);
    static constexpr size_t off_Yt = off_Vt + (size_t)R * LDC * sizeof(E);
    static constexpr size_t off_Ut = off_Yt + (size_t)R * LDC * sizeof(E);
    static constexpr size_t off_DUt = off_Ut + (size_t)R * LDC * sizeof(E);
    static constexpr size_t off_S = off_DUt + (size_t)R * LDC * sizeof(E);
    static constexpr size_t off_gate = (off_S + (size_t)R * LDK * sizeof(E) + 15) & ~(size_t)15;
    static constexpr size_t bytes = off_gate + (size_t)C * 16 + 16;
};

template <typename E> __device__ __forceinline__ E vec_elem(const Vec16 &v, int e);
template <> __device__ __forceinline__ bf16 vec_elem<bf16>(const Vec16 &v, int e) {
    const uint16_t bits = (uint16_t)(v.w[e >> 1] >> (16 * (e & 1)));
    return __builtin_bit_cast(bf16, bits);
}
template <> __device__ __forceinline__ float vec_elem<float>(const Vec16 &v, int e) {
    return __builtin_bit_cast(float, v.w[e]);
}

template <typename E, int C, int DK, int R>
__global__ __launch_bounds__(256) void gdn_scan_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const int32_t *__restrict__ bounds, const int32_t *__restrict__ seq_chunk0,
    const int32_t *__restrict__ order,
    const E *__restrict__ tmat, const E *__restrict__ pmat,
    const f32x4 *__restrict__ gates, const float *__restrict__ gammac,
    const float *__restrict__ s0, float *__restrict__ sfin, E *__restrict__ out,
    int32_t num_seqs, int32_t hk, int32_t hv)
{
    typedef ScanSmem<E, C, DK, R> L;
    typedef Mma<E, DK> MD;  // contractions over the key dimension
    typedef Mma<E, C> MC;   // contractions over the tokens of a chunk
    constexpr int DV = DK;
    constexpr int NS = DV / R;          // value-row slices per head
    constexpr int LDK = L::LDK, LDC = L::LDC;
    constexpr int EPV = 16 / sizeof(E);
    constexpr int VPR = DK / EPV;
    constexpr int RT = C / 16, NT = R / 16, MT = DK / 16;
    constexpr int NP = RT * NT, NPW = (NP + 3) / 4;   // (token tile, value tile) pairs
    constexpr int ST = MT * NT, STW = (ST + 3) / 4;   // state tiles

    extern __shared__ __align__(16) char smem[];
    E *sK = reinterpret_cast<E *>(smem + L::off_K);
    E *sQ = reinterpret_cast<E *>(smem + L::off_Q);
    E *sKt = reinterpret_cast<E *>(smem + L::off_Kt);
    E *sT = reinterpret_cast<E *>(smem + L::off_T);
    E *sP = reinterpret_cast<E *>(smem + L::off_P);
    E *sVt = reinterpret_cast<E *>(smem + L::off_Vt);
    E *sYt = reinterpret_cast<E *>(smem + L::off_Yt);
    E *sUt = reinterpret_cast<E *>(smem + L::off_Ut);
    E *sDUt = reinterpret_cast<E *>(smem + L::off_DUt);
    E *sS = reinterpret_cast<E *>(smem + L::off_S);
    f32x4 *sGate = reinterpret_cast<f32x4 *>(smem + L::off_gate);
    float *sGC = reinterpret_cast<float *>(smem + L::off_gate + (size_t)C * 16);

    // Workgroup -> (sequence rank, query/key head, value head in group, slice).
    // Dispatch places workgroup b on XCD b % 8; all value heads and slices
    // of one query/key head land on one XCD, so K, Q, T and P are shared
    // through that XCD's L2.
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

    // fp32 master copy of this wave's S^T tiles; operand copy in LDS.
    f32x4 sacc[STW];
#pragma unroll
    for (int jj = 0; jj < STW; ++jj) {
        const int j = wave + 4 * jj;
        sacc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j < ST) {
            const int mt = j % MT, nt = j / MT;
            if (s0)
                sacc[jj] = *reinterpret_cast<const f32x4 *>(
                    s0 + state0 + (size_t)(col0 + 16 * nt + ln) * DK + 16 * mt + 4 * g4);
            store_acc_t<E>(sS, LDK, 16 * mt, 16 * nt, lane, sacc[jj]);
        }
    }

    for (int c = 0; c < nch; ++c) {
        const int ci = c0 + c;
        const int tok0 = start + c * C;
        const int clen = min(C, len - c * C);
        const size_t mat0 = ((size_t)ci * hv + h) * (size_t)(C * C);

        // ---- stage this chunk's operands
        for (int i = tid; i < C * VPR; i += 256) {
            const int r = i / VPR, cv = i - r * VPR;
            const size_t src = ((size_t)(tok0 + r) * hk + kh) * DK + cv * EPV;
            const Vec16 kv = r < clen ? ld16(k + src) : zero16();
            const Vec16 qv = r < clen ? ld16(q + src) : zero16();
            st16(sK + r * LDK + cv * EPV, kv);
            st16(sQ + r * LDK + cv * EPV, qv);
            if constexpr (L::kKt) {
#pragma unroll
                for (int e = 0; e < EPV; ++e) sKt[(cv * EPV + e) * LDC + r] = vec_elem<E>(kv, e);
            }
        }
        for (int i = tid; i < C * C / EPV; i += 256) {
            const int r = i / (C / EPV), cv = i - r * (C / EPV);
            st16(sT + r * LDC + cv * EPV, ld16(tmat + mat0 + (size_t)i * EPV));
            st16(sP + r * LDC + cv * EPV, ld16(pmat + mat0 + (size_t)i * EPV));
        }
        for (int i = tid; i < C * R; i += 256) {
            const int r = i / R, cc = i - r * R;
            sVt[cc * LDC + r] = r < clen ? v[((size_t)(tok0 + r) * hv + h) * DV + col0 + cc] : from_f32<E>(0.f);
        }
        if (tid < C) sGate[tid] = gates[((size_t)ci * hv + h) * C + tid];
        if (tid == 0) *sGC = gammac[(size_t)ci * hv + h];
        __syncthreads();

        // ---- X = K S0^T and Q S0^T; Y = diag(b) V - diag(b gamma) X
        f32x4 o1[NPW];
#pragma unroll
        for (int pp = 0; pp < NPW; ++pp) {
            const int p = wave + 4 * pp;
            o1[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p < NP) {
                const int rt = p % RT, nt = p / RT;
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < DK / MD::KW; ++kb) {
                    const typename MD::Frag bs = load_frag<MD>(sS, LDK, 16 * nt, kb * MD::KW, lane);
                    x = MD::mma(load_frag<MD>(sK, LDK, 16 * rt, kb * MD::KW, lane), bs, x);
                    o1[pp] = MD::mma(load_frag<MD>(sQ, LDK, 16 * rt, kb * MD::KW, lane), bs, o1[pp]);
                }
                f32x4 y;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * rt + 4 * g4 + i;
                    const f32x4 gt = sGate[row];
                    y[i] = gt[1] * to_f32(sVt[(16 * nt + ln) * LDC + row]) - gt[2] * x[i];
                }
                store_acc_t<E>(sYt, LDC, 16 * rt, 16 * nt, lane, y);
            }
        }
        __syncthreads();

        // ---- U = T Y
#pragma unroll
        for (int pp = 0; pp < NPW; ++pp) {
            const int p = wave + 4 * pp;
            if (p < NP) {
                const int rt = p % RT, nt = p / RT;
                f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < C / MC::KW; ++kb)
                    u = MC::mma(load_frag<MC>(sT, LDC, 16 * rt, kb * MC::KW, lane),
                                load_frag<MC>(sYt, LDC, 16 * nt, kb * MC::KW, lane), u);
                store_acc_t<E>(sUt, LDC, 16 * rt, 16 * nt, lane, u);
                f32x4 du;
#pragma unroll
                for (int i = 0; i < 4; ++i) du[i] = sGate[16 * rt + 4 * g4 + i][3] * u[i];
                store_acc_t<E>(sDUt, LDC, 16 * rt, 16 * nt, lane, du);
            }
        }
        __syncthreads();

        // ---- O = diag(scale gamma) Q S0^T + P U, written out
#pragma unroll
        for (int pp = 0; pp < NPW; ++pp) {
            const int p = wave + 4 * pp;
            if (p < NP) {
                const int rt = p % RT, nt = p / RT;
                f32x4 o2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < C / MC::KW; ++kb)
                    o2 = MC::mma(load_frag<MC>(sP, LDC, 16 * rt, kb * MC::KW, lane),
                                 load_frag<MC>(sUt, LDC, 16 * nt, kb * MC::KW, lane), o2);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * rt + 4 * g4 + i;
                    if (row < clen)
                        out[((size_t)(tok0 + row) * hv + h) * DV + col0 + 16 * nt + ln] =
                            from_f32<E>(sGate[row][0] * o1[pp][i] + o2[i]);
                }
            }
        }

        // ---- S^T <- gamma_C S^T + K^T (diag(delta) U)
        const float gc = *sGC;
#pragma unroll
        for (int jj = 0; jj < STW; ++jj) {
            const int j = wave + 4 * jj;
            if (j < ST) {
                const int mt = j % MT, nt = j / MT;
                f32x4 acc = sacc[jj];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] *= gc;
#pragma unroll
                for (int kb = 0; kb < C / MC::KW; ++kb) {
                    typename MC::Frag a;
                    if constexpr (L::kKt)
                        a = load_frag<MC>(sKt, LDC, 16 * mt, kb * MC::KW, lane);
                    else
                        a = sK[(kb * MC::KW + g4) * LDK + 16 * mt + ln];
                    acc = MC::mma(a, load_frag<MC>(sDUt, LDC, 16 * nt, kb * MC::KW, lane), acc);
                }
                sacc[jj] = acc;
                store_acc_t<E>(sS, LDK, 16 * mt, 16 * nt, lane, acc);
            }
        }
        __syncthreads();
    }

    if (sfin) {
#pragma unroll
        for (int jj = 0; jj < STW; ++jj) {
            const int j = wave + 4 * jj;
            if (j < ST) {
                const int mt = j % MT, nt = j / MT;
                *reinterpret_cast<f32x4 *>(sfin + state0 + (size_t)(col0 + 16 * nt + ln) * DK + 16 * mt + 4 * g4) =
                    sacc[jj];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------

constexpr int kSliceRows = 16;

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
                       bounds, chunk_seq, chunk_tok0, counters, tmat, pmat, gates, gammac,
                       A.hk, A.hv, A.scale);
    timing_end(kPrep, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    typedef ScanSmem<E, C, D, kSliceRows> SL;
    static std::atomic<bool> scan_ok{false};
    auto scan = gdn_scan_kernel<E, C, D, kSliceRows>;
    if ((e = allow_smem(scan, SL::bytes, scan_ok)) != hipSuccess) return e;
    const int64_t per_kh = (int64_t)(A.hv / A.hk) * (D / kSliceRows);
    const int64_t groups = (int64_t)A.num_seqs * A.hk;
    const int64_t grid = ((groups + 7) / 8) * per_kh * 8;
    timing_begin(kScan, st);
    hipLaunchKernelGGL(scan, dim3((unsigned)grid), dim3(256), SL::bytes, st,
                       (const E *)A.q, (const E *)A.k, (const E *)A.v,
                       bounds, seq_chunk0, order, tmat, pmat, gates, gammac,
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

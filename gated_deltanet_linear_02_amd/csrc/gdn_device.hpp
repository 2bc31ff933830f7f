// gdn_device.hpp -- device helpers for the gfx950 (CDNA4) kernels of libgdn.
//
// Element types: operands are either bf16 (MFMA v_mfma_f32_16x16x32_bf16,
// fp32 accumulate) or fp32 (v_mfma_f32_16x16x4_f32). Both instructions work
// on 16x16 output tiles with the same accumulator layout:
//
//   D/C  lane l holds D[4*(l/16) + i][l%16], i = 0..3   (float4)
//   A    lane l holds A[l%16][k0 + KPL*(l/16) + j], j < KPL
//   B    lane l holds B[k0 + KPL*(l/16) + j][l%16], j < KPL
//
// with KPL = 8 (bf16, 32-deep), 4 (bf16, 16-deep: v_mfma_f32_16x16x16_bf16)
// or 1 (fp32) consecutive contraction elements per lane.
// Whatever physical contraction order the hardware uses, A and B are always
// loaded with the same (lane group, slot) -> k mapping, so the product is
// the mathematical one.
//
// In LDS every operand is kept so that a lane's KPL elements are contiguous:
// A operands row-major [M][K], B operands transposed [N][K]. Accumulator
// tiles are written back transposed (4 contiguous elements per lane), which
// is exactly the [N][K] layout the next product reads as its B operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Mma<E, K>: the MFMA used for a contraction of length K (a multiple of 16).
// bf16 contractions of 32 or more use the 32-deep gfx950 instruction; a
// contraction of exactly 16 uses the 16-deep one.
template <typename E, int K> struct Mma;

template <int K> struct Mma<bf16, K> {
    static constexpr bool kDeep = K % 32 == 0;
    static constexpr int KW = kDeep ? 32 : 16;  // contraction length per instruction
    static constexpr int KPL = KW / 4;          // contraction elements held per lane
    typedef typename std::conditional<kDeep, bf16x8, bf16x4>::type Frag;
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
        if constexpr (kDeep) {
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
        } else {
            return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                             __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
        }
    }
};

template <int K> struct Mma<float, K> {
    static constexpr int KW = 4;
    static constexpr int KPL = 1;
    typedef float Frag;
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// LDS row padding (elements) that keeps rows 16-byte aligned and spreads the
// 16 rows of a fragment load over distinct banks.
template <typename E> struct Pad { static constexpr int value = 16 / sizeof(E); };

// Fragment of a row-major [rows][ld] LDS array: row r0 + l%16, contraction
// elements k0 + KPL*(l/16) ...
template <typename M, typename E>
__device__ __forceinline__ typename M::Frag load_frag(const E *base, int ld, int r0, int k0, int lane) {
    const E *p = base + (r0 + (lane & 15)) * ld + k0 + M::KPL * (lane >> 4);
    return *reinterpret_cast<const typename M::Frag *>(p);
}

// Accumulator order of a contraction index. An accumulator tile gives each
// lane 4 consecutive elements of one row (columns 4 (l/16) + r of a 16-wide
// tile). Fragments in accumulator order take their KPL elements in those
// runs: slot e of lane group g of fragment kb holds contraction index
// acc_k(kb, g, e). Because the MFMA sums over k in any order as long as A
// and B agree, a product whose operands both use this order is the same
// product; it lets one product's accumulators be stored, or read back from
// LDS, as the next product's fragments without a transpose.
template <typename MM> __device__ __forceinline__ int acc_k(int kb, int g, int e) {
    if constexpr (MM::KPL == 1) return 16 * (kb >> 2) + 4 * g + (kb & 3);
    else return kb * MM::KW + 16 * (e >> 2) + 4 * g + (e & 3);
}
// The 16-wide tile and the slot within the lane's run of acc_k(kb, g, e).
template <typename MM> __device__ __forceinline__ constexpr int acc_tile(int kb, int e) {
    return MM::KPL == 1 ? (kb >> 2) : (kb * MM::KW) / 16 + (e >> 2);
}
template <typename MM> __device__ __forceinline__ constexpr int acc_slot(int kb, int e) {
    return MM::KPL == 1 ? (kb & 3) : (e & 3);
}

// Fragment of a row-major [rows][ld] LDS array in accumulator order: row
// r0 + l%16, contraction elements acc_k(kb, l/16, .).
template <typename M, typename E>
__device__ __forceinline__ typename M::Frag load_frag_acc(const E *base, int ld, int r0, int kb, int lane) {
    const int g = lane >> 4;
    const E *row = base + (r0 + (lane & 15)) * ld;
    if constexpr (M::KPL == 1) {
        return row[16 * (kb >> 2) + 4 * g + (kb & 3)];
    } else if constexpr (M::KPL == 4) {
        return *reinterpret_cast<const bf16x4 *>(row + kb * 16 + 4 * g);
    } else {
        const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(row + kb * 32 + 4 * g);
        const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(row + kb * 32 + 16 + 4 * g);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// Four accumulator values to 4 contiguous elements.
template <typename E> __device__ __forceinline__ void store4(E *p, f32x4 v);
template <> __device__ __forceinline__ void store4<bf16>(bf16 *p, f32x4 v) {
    bf16x4 w;
    w[0] = static_cast<bf16>(v[0]);
    w[1] = static_cast<bf16>(v[1]);
    w[2] = static_cast<bf16>(v[2]);
    w[3] = static_cast<bf16>(v[3]);
    *reinterpret_cast<bf16x4 *>(p) = w;
}
template <> __device__ __forceinline__ void store4<float>(float *p, f32x4 v) { *reinterpret_cast<f32x4 *>(p) = v; }

// Four consecutive elements read as floats.
template <typename E> __device__ __forceinline__ f32x4 load4f(const E *p);
template <> __device__ __forceinline__ f32x4 load4f<float>(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
template <> __device__ __forceinline__ f32x4 load4f<bf16>(const bf16 *p) {
    const bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{static_cast<float>(x[0]), static_cast<float>(x[1]), static_cast<float>(x[2]), static_cast<float>(x[3])};
}

// Write an accumulator tile transposed: element D[m0 + 4g + i][n0 + n] goes to
// dst[(n0 + n) * ld + m0 + 4g + i] (4 contiguous elements per lane).
template <typename E> __device__ __forceinline__ void store_acc_t(E *dst, int ld, int m0, int n0, int lane, f32x4 v) {
    store4<E>(dst + (n0 + (lane & 15)) * ld + m0 + 4 * (lane >> 4), v);
}

// Fragment-contiguous LDS rows. In rows that are read back as 32-deep
// accumulator-order fragments (KPL = 8), contraction index k is stored at
// lds_pos(k): within each 32-element block the eight indices one lane reads,
// acc_k(kb, g, 0..7), sit at 8 g .. 8 g + 7, so that a fragment is one 16-byte
// LDS read instead of two 8-byte ones (16-byte reads move about 1.7 times the
// bytes per cycle). The four indices an accumulator tile gives a lane
// (4 g .. 4 g + 3 of a 16-wide tile) stay contiguous, so stores are 8 bytes.
// Other fragment shapes keep the natural order.
template <typename MM> __device__ __forceinline__ constexpr int lds_pos(int k) {
    if constexpr (MM::KPL == 8) return (k & ~31) | ((k & 12) << 1) | ((k & 16) >> 2) | (k & 3);
    else return k;
}

// store_acc_t into rows laid out by lds_pos<MM> (m0 is a multiple of 16):
// element D[m0 + 4g + i][n0 + n] goes to dst[(n0 + n) * ld + lds_pos(m0 + 4g) + i].
template <typename MM, typename E>
__device__ __forceinline__ void store_acc_p(E *dst, int ld, int m0, int n0, int lane, f32x4 v) {
    store4<E>(dst + (n0 + (lane & 15)) * ld + lds_pos<MM>(m0 + 4 * (lane >> 4)), v);
}

// load_frag_acc from rows laid out by lds_pos<M>.
template <typename M, typename E>
__device__ __forceinline__ typename M::Frag load_frag_p(const E *base, int ld, int r0, int kb, int lane) {
    if constexpr (M::KPL == 8) {
        return *reinterpret_cast<const bf16x8 *>(base + (r0 + (lane & 15)) * ld + kb * 32 + 8 * (lane >> 4));
    } else {
        return load_frag_acc<M>(base, ld, r0, kb, lane);
    }
}

// 16-byte vector of elements (8 bf16 or 4 fp32) for global <-> LDS staging.
struct alignas(16) Vec16 { uint32_t w[4]; };

__device__ __forceinline__ Vec16 ld16(const void *p) { return *reinterpret_cast<const Vec16 *>(p); }
__device__ __forceinline__ void st16(void *p, const Vec16 &v) { *reinterpret_cast<Vec16 *>(p) = v; }
__device__ __forceinline__ Vec16 zero16() { Vec16 z; z.w[0] = z.w[1] = z.w[2] = z.w[3] = 0u; return z; }

}  // namespace gdn

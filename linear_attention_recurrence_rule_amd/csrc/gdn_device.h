// Device-side building blocks shared by the gated-delta-rule kernels (gfx950).
//
// Matrix-core tiles.  Every product uses 16x16 output tiles, with a
// contraction split into blocks of 32.  A lane's operand fragment holds 8
// elements of one row of A, or one column of B.  Lane l has row/column
// i = l % 16 and group q = l / 16.  Element e < 4 sits at contraction index
// 4q + e, and element e >= 4 at 16 + 4q + (e - 4).  A and B use the same
// (lane, element) -> index map, so the instruction's own internal k order
// does not matter.  The 16x16 fp32 accumulator gives lane l the rows
// 4q + r (r = 0..3) of column l % 16.  Hence two vertically adjacent
// accumulator tiles are, element for element, the B fragment of the next
// product that contracts over those rows.  The kernels chain products this
// way without moving data between lanes.
//
//   fp16 operands: one v_mfma_f32_16x16x32_f16 per 32-block.
//   fp32 operands: eight v_mfma_f32_16x16x4_f32 per 32-block.  Instruction e
//                  contracts the index set {4q + e'} over the lane groups.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int CHUNK = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bfloat16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Load 4 consecutive input elements as fp32 (bf16 bit patterns or fp32).
template <bool BF16>
__device__ __forceinline__ void load4(const void* base, size_t idx, float x[4]) {
    if constexpr (BF16) {
        uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + idx);
        x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
        x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
        float4 w = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
        x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
    }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, size_t idx) {
    if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
    else return reinterpret_cast<const float*>(base)[idx];
}

template <bool BF16>
__device__ __forceinline__ void store1(void* base, size_t idx, float x) {
    if constexpr (BF16) reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16(x);
    else reinterpret_cast<float*>(base)[idx] = x;
}

// ---- operand fragments ----------------------------------------------------------------
template <typename OP> struct Frag;
template <> struct Frag<_Float16> { h8_t v; };
template <> struct Frag<float> { f4_t lo, hi; };

__device__ __forceinline__ void frag_set(Frag<_Float16>& f, int e, float x) { f.v[e] = (_Float16)x; }
__device__ __forceinline__ void frag_set(Frag<float>& f, int e, float x) {
    if (e < 4) f.lo[e] = x; else f.hi[e - 4] = x;
}

__device__ __forceinline__ void frag_set_raw(Frag<_Float16>& f, int e, _Float16 x) { f.v[e] = x; }
__device__ __forceinline__ void frag_set_raw(Frag<float>& f, int e, float x) {
    if (e < 4) f.lo[e] = x; else f.hi[e - 4] = x;
}
__device__ __forceinline__ float frag_get(const Frag<_Float16>& f, int e) { return (float)f.v[e]; }
__device__ __forceinline__ float frag_get(const Frag<float>& f, int e) { return e < 4 ? f.lo[e] : f.hi[e - 4]; }

__device__ __forceinline__ void mma(f4_t& acc, const Frag<_Float16>& a, const Frag<_Float16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f4_t& acc, const Frag<float>& a, const Frag<float>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], acc, 0, 0, 0);
}

// Column fragment of a row-major matrix M: the contraction runs down the rows
// 32*kb + (4q + e) for e < 4 and 32*kb + 16 + 4q + (e - 4) for e >= 4, at
// column 16*cb + (lane % 16).  It serves as a B fragment of M, or as an A
// fragment of M^T.
//
// In LDS with 2-byte elements it takes two transposing reads
// (ds_read_b64_tr_b16).  Within each group of 16 lanes such a read hands lane
// 4a + c element c of the 8 bytes that lanes a, a + 4, a + 8 and a + 12
// addressed.  So lane s of group q addresses row 32*kb + 4q + (s >> 2), columns
// 16*cb + 4(s & 3) .. + 3, and lane (i, q) receives column 16*cb + i of rows
// 32*kb + 4q .. + 3; the second read does the same 16 rows down.  M, ld and
// 16*cb keep every address 8-byte aligned (ld even, M 8-byte aligned).
template <typename OP>
__device__ __forceinline__ Frag<OP> frag_colmajor(const OP* M, int ld, int cb, int kb, int lane) {
    Frag<OP> f;
    if constexpr (sizeof(OP) == 2) {
        typedef short s4_t __attribute__((ext_vector_type(4)));
        typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s4_t* lds_s4;
        const int s = lane & 15, q = lane >> 4;
        const OP* p = M + (size_t)(32 * kb + 4 * q + (s >> 2)) * ld + 16 * cb + 4 * (s & 3);
        const h4_t a = __builtin_bit_cast(h4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)p));
        const h4_t b = __builtin_bit_cast(h4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(p + 16 * ld)));
        f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        const int i = lane & 15, q = lane >> 4;
        const OP* p = M + (size_t)(32 * kb + 4 * q) * ld + 16 * cb + i;
#pragma unroll
        for (int e = 0; e < 8; ++e) frag_set_raw(f, e, p[(size_t)((e & 3) + 16 * (e >> 2)) * ld]);
    }
    return f;
}

// B fragment from two accumulator tiles stacked along the contraction:
// `top` holds contraction rows 0..15 of the block, `bot` rows 16..31.
template <typename OP>
__device__ __forceinline__ Frag<OP> frag_from_acc(const f4_t& top, const f4_t& bot) {
    Frag<OP> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { frag_set(f, e, top[e]); frag_set(f, e + 4, bot[e]); }
    return f;
}

// A stored fragment (fragment-major layout: 64 lanes x 8 elements, contiguous).
template <typename OP>
__device__ __forceinline__ Frag<OP> frag_stored(const OP* base, int frag, int lane) {
    const OP* p = base + ((size_t)frag * WAVE + lane) * 8;
    Frag<OP> f;
    if constexpr (sizeof(OP) == 2) {
        f.v = *reinterpret_cast<const h8_t*>(p);
    } else {
        f.lo = *reinterpret_cast<const f4_t*>(p);
        f.hi = *reinterpret_cast<const f4_t*>(p + 4);
    }
    return f;
}

template <typename OP>
__device__ __forceinline__ void frag_store(OP* base, int frag, int lane, const Frag<OP>& f) {
    OP* p = base + ((size_t)frag * WAVE + lane) * 8;
    if constexpr (sizeof(OP) == 2) {
        *reinterpret_cast<h8_t*>(p) = f.v;
    } else {
        *reinterpret_cast<f4_t*>(p) = f.lo;
        *reinterpret_cast<f4_t*>(p + 4) = f.hi;
    }
}

// Cross-lane moves inside a row of 16 lanes (DPP, no LDS round trip).
// CTRL: quad_perm(1,0,3,2) = 0xB1, quad_perm(2,3,0,1) = 0x4E, row_ror:4 = 0x124,
// row_ror:8 = 0x128, row_half_mirror = 0x141.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Workgroup barrier that orders LDS accesses only: each wave waits for its own
// LDS operations, not for its global stores or loads in flight (a workgroup
// release fence would wait for those too).  The signal fences keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Sum / max over aligned groups of N lanes (N = 8 or 16), result in every lane.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    if constexpr (N == 16) {
        x += dpp<0x124>(x);
        x += dpp<0x128>(x);
    } else {
        x += dpp<0x141>(x);
    }
    return x;
}
template <int N>
__device__ __forceinline__ float group_max(float x) {
    static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    if constexpr (N == 16) {
        x = fmaxf(x, dpp<0x124>(x));
        x = fmaxf(x, dpp<0x128>(x));
    } else {
        x = fmaxf(x, dpp<0x141>(x));
    }
    return x;
}

// Lanes i and i ^ 16 trade values across the two 16-lane rows of each
// 32-lane half (v_permlane16_swap: the odd rows of the first operand trade
// places with the even rows of the second).  With a in every lane and b in
// every lane, an even-row lane gets (its own a, its partner's a) and an
// odd-row lane gets (its partner's b, its own b).
struct F2 {
    float x, y;
};
__device__ __forceinline__ F2 permlane16_swap(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Lanes i and i ^ 32 trade values (v_permlane32_swap: the upper half of the
// first operand trades places with the lower half of the second).  With a in
// every lane and b in every lane, a lower-half lane gets (its own a, its
// partner's a) and an upper-half lane gets (its partner's b, its own b).
__device__ __forceinline__ F2 permlane32_swap(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Partner lane of a butterfly step inside a row of 16 lanes (DPP): lane
// i ^ H for H = 8, 2, 1, and the mirror lane (i & ~7) | (7 - (i & 7)) for
// H = 4, which differs from i in bit 2 (all a butterfly step needs).
template <int H>
__device__ __forceinline__ float row_partner(float x) {
    static_assert(H == 8 || H == 4 || H == 2 || H == 1, "butterfly step inside a row");
    if constexpr (H == 8) return dpp<0x128>(x);
    else if constexpr (H == 4) return dpp<0x141>(x);
    else if constexpr (H == 2) return dpp<0x4E>(x);
    else return dpp<0xB1>(x);
}

// One butterfly step of reduce_scatter inside a row of 16 lanes.
template <int H, int N>
__device__ __forceinline__ void rs_step(float (&x)[N], int c) {
    const bool upper = (c & H) != 0;
#pragma unroll
    for (int i = 0; i < H; ++i) {
        const float lo = x[i] + row_partner<H>(x[i]);
        const float hi = x[i + H] + row_partner<H>(x[i + H]);
        x[i] = upper ? hi : lo;
    }
}

// Sum over aligned groups of N = 16 or 32 lanes, result in every lane.
template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
    static_assert(N == 16 || N == 32, "group of 16 or 32 lanes");
    x = group_sum<16>(x);
    if constexpr (N == 32) {
        const F2 r = permlane16_swap(x, x);
        x = r.x + r.y;
    }
    return x;
}

// Reduce-scatter over aligned groups of N = 16 or 32 lanes: lane c of a group
// (c = lane % N) holds x[0..N-1]; afterwards x[0] is the group's sum of
// element c.  Each step halves the elements a lane carries: the lane whose
// step bit is clear keeps the lower half and the other the upper half, and
// each adds its partner's copy of the half it keeps.
template <int N>
__device__ __forceinline__ float reduce_scatter(float (&x)[N], int c) {
    static_assert(N == 16 || N == 32, "group of 16 or 32 lanes");
    if constexpr (N == 32) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const F2 r = permlane16_swap(x[i], x[i + 16]);
            x[i] = r.x + r.y;
        }
    }
    rs_step<8>(x, c);
    rs_step<4>(x, c);
    rs_step<2>(x, c);
    rs_step<1>(x, c);
    return x[0];
}

}  // namespace gdn

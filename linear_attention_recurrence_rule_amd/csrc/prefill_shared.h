// Device helpers shared by the blocked prefill kernels (prefill.hip: fp32
// inputs; prefill_bf16.hip: bf16 inputs).
#pragma once
#include "gdn_device.h"
#include "gdn.h"  // gdn_prefill_status_flag

namespace gdn {

// Token range and first block slot of one packed sequence.
struct SeqInfo {
    int32_t begin, len, slot_base, pad;
};

// Write 4 accumulator values (one lane's share of a 16x16 tile) as half of a
// stored fragment: part 0 = elements 0..3, part 1 = elements 4..7.
template <typename OP>
__device__ __forceinline__ void store_part(OP* base, int frag, int part, int lane, const f4_t& x) {
    OP* p = base + ((size_t)frag * WAVE + lane) * 8 + 4 * part;
    if constexpr (sizeof(OP) == 2) {
        typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
        h4_t h = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
        *reinterpret_cast<h4_t*>(p) = h;
    } else {
        *reinterpret_cast<f4_t*>(p) = x;
    }
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers (DPP):
// Hillis-Steele inside each row of 16 lanes (row_shr 1, 2, 4, 8), then the
// row totals are carried forward with row_bcast 15 (rows 1, 3) and
// row_bcast 31 (rows 2, 3).  Lanes without a source add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add_src(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += dpp_add_src<0x111, 0xF>(x);  // row_shr:1
    x += dpp_add_src<0x112, 0xF>(x);  // row_shr:2
    x += dpp_add_src<0x114, 0xF>(x);  // row_shr:4
    x += dpp_add_src<0x118, 0xF>(x);  // row_shr:8
    x += dpp_add_src<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_add_src<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}
// The same in fp64: each DPP move carries both 32-bit halves.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_add_src64(double x) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(x);
    const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, ROW_MASK, 0xF, false);
    const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, ROW_MASK, 0xF, false);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ double wave_inclusive_sum(double x) {
    x += dpp_add_src64<0x111, 0xF>(x);
    x += dpp_add_src64<0x112, 0xF>(x);
    x += dpp_add_src64<0x114, 0xF>(x);
    x += dpp_add_src64<0x118, 0xF>(x);
    x += dpp_add_src64<0x142, 0xA>(x);
    x += dpp_add_src64<0x143, 0xC>(x);
    return x;
}

// C + X Y for 16x16 fp32 matrices, X^T and Y (and C) in accumulator layout:
// lane (j, q) holds M[4q + r][j] in element r.  Instruction e contracts over
// k = 4q + e, taking X[i][4q + e] = X^T[4q + e][i] and Y[4q + e][j].
__device__ __forceinline__ f4_t mm16(const f4_t& xt, const f4_t& y, f4_t c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[e], y[e], c, 0, 0, 0);
    return c;
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Sets `bit` in the prefill status word (when there is one) if any lane of the
// wave has `bad` set: one vector atomic per wave.
__device__ __forceinline__ void report_status(unsigned* status, bool bad, unsigned bit) {
    if (status && __any(bad) && (threadIdx.x % WAVE) == 0) atomicOr(status, bit);
}

__device__ __forceinline__ bool any_nonfinite(const f4_t& x) {
    return !__builtin_isfinite(x[0]) || !__builtin_isfinite(x[1]) || !__builtin_isfinite(x[2]) ||
           !__builtin_isfinite(x[3]);
}

}  // namespace gdn

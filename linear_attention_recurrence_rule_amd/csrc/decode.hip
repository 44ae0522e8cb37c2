// Fused decode step of the gated delta rule: one new token per sequence.
//
// This is the direct token scan from "Optimizing on-device inference for Apple
// Silicon", section "Qwen creates three distinct workload shapes".  It is
// fused with the q/k normalisation and the exponential gate, as the section
// "Reduce intermediate traffic and state traffic" fuses the recurrent update
// with its normalisation.  The fp32 state of each (sequence, v-head) is read
// from HBM once and written back once.  That is the whole of the step's
// unavoidable traffic (section "Decode: minimise bytes moved per token").
//
// Per (sequence, v-head), with S the d x d state (row i = value index i):
//   k^ = k / sqrt(|k|^2 + 1e-6), q^ likewise times `scale` (if qk_l2norm)
//   alpha = exp(g);  p = S k^;  u = beta (v - alpha p)
//   S <- alpha S + u k^T;   o = S q^ = alpha (S q^) + u (k^ . q^)
// Both dot products S k^ and S q^ are taken from the state as loaded, in one
// pass.
//
// Layout: one workgroup per (sequence, v-head), d/32 waves.  Each wave owns
// 32 state rows.  A lane holds 4 consecutive entries (16 bytes) of one row,
// so d/4 lanes cover a row, and each wave-wide load reads 1 KiB of contiguous
// state.  The loads are issued before any other work.  The row sums are a
// reduce-scatter across the d/4 lanes of a row.  After it, lane c of a row
// group holds either S k^ or S q^ of one row.
#include "gdn_device.h"

namespace gdn {

template <int D, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(2 * D) void decode_step_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    void* __restrict__ out, int h_k, int h_v, int l2norm, float scale) {
    constexpr int LPR = D / 4;      // lanes per state row
    constexpr int RPI = WAVE / LPR;  // rows covered by one wave-wide load
    constexpr int NL = LPR / 2;      // loads per lane (32 rows per wave)
    static_assert(RPI * NL == 32, "each wave owns 32 rows");

    const int unit = blockIdx.x;  // sequence * h_v + v-head
    const int n = unit / h_v, h = unit - n * h_v;
    const int hk = h / (h_v / h_k);
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    const int c = lane % LPR, sub = lane / LPR;

    float* S = state + (size_t)unit * D * D;
    float4 s[NL];
#pragma unroll
    for (int m = 0; m < NL; ++m) {
        const int row = wave * 32 + m * RPI + sub;
        s[m] = *reinterpret_cast<const float4*>(S + (size_t)row * D + 4 * c);
    }

    float kx[4], qx[4];
    load4<IN_BF16>(k, ((size_t)n * h_k + hk) * D + 4 * c, kx);
    load4<IN_BF16>(q, ((size_t)n * h_k + hk) * D + 4 * c, qx);
    const float alpha = expf(g[unit]);
    const float bt = beta[unit];

    float ssk = kx[0] * kx[0] + kx[1] * kx[1] + kx[2] * kx[2] + kx[3] * kx[3];
    float ssq = qx[0] * qx[0] + qx[1] * qx[1] + qx[2] * qx[2] + qx[3] * qx[3];
#pragma unroll
    for (int mask = LPR / 2; mask >= 1; mask >>= 1) {
        ssk += shfl_xor(ssk, mask);
        ssq += shfl_xor(ssq, mask);
    }
    const float rk = l2norm ? 1.0f / sqrtf(ssk + 1e-6f) : 1.0f;
    const float rq = (l2norm ? 1.0f / sqrtf(ssq + 1e-6f) : 1.0f) * scale;
#pragma unroll
    for (int e = 0; e < 4; ++e) { kx[e] *= rk; qx[e] *= rq; }
    float kq = kx[0] * qx[0] + kx[1] * qx[1] + kx[2] * qx[2] + kx[3] * qx[3];
#pragma unroll
    for (int mask = LPR / 2; mask >= 1; mask >>= 1) kq += shfl_xor(kq, mask);

    // partial row sums: x[m] = (S k^) part, x[NL + m] = (S q^) part
    float x[LPR];
#pragma unroll
    for (int m = 0; m < NL; ++m) {
        x[m] = s[m].x * kx[0] + s[m].y * kx[1] + s[m].z * kx[2] + s[m].w * kx[3];
        x[NL + m] = s[m].x * qx[0] + s[m].y * qx[1] + s[m].z * qx[2] + s[m].w * qx[3];
    }
    // reduce-scatter over the LPR lanes of each row group: afterwards lane c holds x[c] summed
#pragma unroll
    for (int half = LPR / 2; half >= 1; half >>= 1) {
        const bool upper = (c & half) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float send = upper ? x[i] : x[i + half];
            const float keep = upper ? x[i + half] : x[i];
            x[i] = keep + shfl_xor(send, half);
        }
    }
    const float red = x[0];
    // lanes c < NL: row (c) has p = S k^ ; lanes c >= NL: row (c - NL) has S q^
    const int mrow = (c < NL) ? c : c - NL;
    const int row = wave * 32 + mrow * RPI + sub;
    const size_t vo = ((size_t)n * h_v + h) * D + row;
    float u = 0.f;
    if (c < NL) u = bt * (load1<IN_BF16>(v, vo) - alpha * red);
    const float u_pair = shfl_xor(u, NL);
    if (c >= NL) store1<OUT_BF16>(out, vo, alpha * red + u_pair * kq);

    // rank-1 update; u of row m lives in lane (group base + m)
    const int base = lane - c;
#pragma unroll
    for (int m = 0; m < NL; ++m) {
        const float um = __shfl(u, base + m, WAVE);
        s[m].x = alpha * s[m].x + um * kx[0];
        s[m].y = alpha * s[m].y + um * kx[1];
        s[m].z = alpha * s[m].z + um * kx[2];
        s[m].w = alpha * s[m].w + um * kx[3];
    }
#pragma unroll
    for (int m = 0; m < NL; ++m) {
        const int r2 = wave * 32 + m * RPI + sub;
        *reinterpret_cast<float4*>(S + (size_t)r2 * D + 4 * c) = s[m];
    }
}

template <int D, bool IB, bool OB>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, float* state, void* out, int units, int h_k,
                                  int h_v, int l2norm, float scale, hipStream_t stream) {
    hipLaunchKernelGGL((decode_step_kernel<D, IB, OB>), dim3(units), dim3(2 * D), 0, stream, q, k, v,
                       g, beta, state, out, h_k, h_v, l2norm, scale);
    return hipGetLastError();
}

hipError_t launch_decode(int d, bool in_bf16, bool out_bf16, const void* q, const void* k,
                         const void* v, const float* g, const float* beta, float* state, void* out,
                         int units, int h_k, int h_v, int l2norm, float scale, hipStream_t stream) {
#define GDN_DEC(D, IB, OB)                                                                        \
    if (d == D && in_bf16 == IB && out_bf16 == OB)                                                \
        return launch_decode_t<D, IB, OB>(q, k, v, g, beta, state, out, units, h_k, h_v, l2norm, \
                                          scale, stream);
    GDN_DEC(128, true, true) GDN_DEC(128, true, false) GDN_DEC(128, false, true)
    GDN_DEC(128, false, false) GDN_DEC(64, true, true) GDN_DEC(64, true, false)
    GDN_DEC(64, false, true) GDN_DEC(64, false, false)
#undef GDN_DEC
    return hipErrorInvalidValue;
}

}  // namespace gdn

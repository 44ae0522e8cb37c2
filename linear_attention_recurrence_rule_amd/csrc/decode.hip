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
// Two per-token operations beside the update can be folded in (flags `fuse`):
// the gate activations, alpha = 1 / (1 + exp(x_g)) (that is exp(-softplus(x_g)))
// and beta = 1 / (1 + exp(-x_beta)) from raw inputs, and the normalisation of
// each head's output, o / sqrt(mean(o^2) + eps) * w over d_v.  The latter needs
// the head's d outputs, which are spread over the workgroup's waves: each wave
// sums its 32 rows, and one LDS exchange combines them.  The barrier the
// exchange needs comes after the state update and the state stores, so that
// waiting for the other waves overlaps them.
//
// Layout: a workgroup has d/32 waves, and each wave owns 32 state rows.  A
// lane holds 4 consecutive entries (16 bytes) of one row, so d/4 lanes cover a
// row, and each wave-wide load reads 1 KiB of contiguous state.  The row sums
// are a reduce-scatter across the d/4 lanes of a row (DPP inside 16-lane rows,
// v_permlane16_swap between them).  After it, lane c of a row group holds
// either S k^ or S q^ of one row.  Each workgroup takes one (sequence,
// v-head) unit: it loads the unit's state and token inputs, computes, stores
// and exits, and the dispatcher starts the next unit's workgroup in its place,
// two at a time per compute unit at d = 128 (see kDecodeResidencyLds).
// Measured cache-cold on MI355X, this moves the state ~9% faster than a few
// workgroups per compute unit that walk several units each with the next
// unit's loads in flight, and it needs fewer registers.
//
// Cache policy (fuse bit 2, GDN_STREAM_STATE): the state is loaded and stored
// either as ordinary accesses, which leave it in the last-level cache for a
// step that comes back to it while it is still there, or as nontemporal ones
// (the `nt` bit), which do not.  A model steps every layer's state in turn,
// far more than the cache holds, and there the nontemporal form moves the
// state ~8% faster from HBM.
#include "gdn_device.h"

namespace gdn {

// One lane's 16 bytes of state; NT: the nontemporal cache policy.
template <bool NT>
__device__ __forceinline__ float4 state_ld(const float* p) {
    if constexpr (NT) {
        const f4_t t = __builtin_nontemporal_load(reinterpret_cast<const f4_t*>(p));
        return make_float4(t[0], t[1], t[2], t[3]);
    } else {
        return *reinterpret_cast<const float4*>(p);
    }
}

template <bool NT>
__device__ __forceinline__ void state_st(float* p, float4 x) {
    if constexpr (NT) {
        const f4_t t = {x.x, x.y, x.z, x.w};
        __builtin_nontemporal_store(t, reinterpret_cast<f4_t*>(p));
    } else {
        *reinterpret_cast<float4*>(p) = x;
    }
}

// Everything one unit needs, loaded together before any of it is used.
template <int D>
struct DecodeIn {
    float4 s[D / 8];  // this lane's state slices (D/8 = LPR/2 rows)
    float kx[4], qx[4];
    float v, g, b;
    float w;   // output-norm weight of this lane's row
    int slot;  // state slot of the unit's sequence; -1: skip the unit
};

// Sequence n's state is slot slots[n] of the state array (slot n when slots is
// NULL); a slot outside [0, num_slots) skips the unit.
template <int D, bool IN_BF16, bool NT>
__device__ __forceinline__ void decode_load(DecodeIn<D>& in, const float* __restrict__ state,
                                            const int32_t* __restrict__ slots, int num_slots, const void* q,
                                            const void* k, const void* v, const float* g, const float* beta,
                                            const float* __restrict__ norm_w, int unit, int h_k, int h_v, int wave,
                                            int lane) {
    constexpr int LPR = D / 4, RPI = WAVE / LPR, NL = LPR / 2;
    const int n = unit / h_v, h = unit - n * h_v;
    const int hk = h / (h_v / h_k);
    const int c = lane % LPR, sub = lane / LPR;
    const int slot = slots ? slots[n] : n;
    in.slot = (slot >= 0 && slot < num_slots) ? slot : -1;
    const float* S = state + ((size_t)max(in.slot, 0) * h_v + h) * D * D;
#pragma unroll
    for (int m = 0; m < NL; ++m) {
        const int row = wave * 32 + m * RPI + sub;
        in.s[m] = in.slot >= 0 ? state_ld<NT>(S + (size_t)row * D + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    load4<IN_BF16>(k, ((size_t)n * h_k + hk) * D + 4 * c, in.kx);
    load4<IN_BF16>(q, ((size_t)n * h_k + hk) * D + 4 * c, in.qx);
    const int mrow = (c < NL) ? c : c - NL;
    in.v = load1<IN_BF16>(v, (size_t)unit * D + wave * 32 + mrow * RPI + sub);
    in.w = norm_w ? norm_w[wave * 32 + mrow * RPI + sub] : 1.f;
    in.g = g[unit];
    in.b = beta[unit];
}

// Decay and write strength of one token: from g and beta as given, or from
// raw gate inputs (alpha = 1 / (1 + e^x_g), beta = 1 / (1 + e^-x_beta)).  Both
// kernels take them from here, so a token is computed the same way in each.
__device__ __forceinline__ void token_gates(float g, float b, bool raw_gates, float& alpha, float& beta) {
    if (raw_gates) {
        alpha = 1.0f / (1.0f + expf(g));
        beta = 1.0f / (1.0f + expf(-b));
    } else {
        alpha = expf(g);
        beta = b;
    }
}

// One token of the recurrence on the register-resident state slices `sr`
// (updated in place), with decay alpha and write strength bin; writes the
// token's output o = S q^ at `orow` (the output row of this unit and token).
// `ub` is this wave's 32-float LDS area, through which u is broadcast to the
// lanes of its row group.  Cross-lane sums run on DPP and v_permlane16_swap.
// With NORM the output is normalised over the head's d rows, which needs
// every wave's part of the sum of squares: this wave's part goes to nb[wave]
// (nb: the unit's D/32-float LDS exchange area), the update runs, and the
// output is returned unwritten (lanes c >= d/8) for norm_output, which every
// wave of the workgroup must then call.  The wait for the other waves thus
// comes after the update (and whatever the caller puts in between).
template <int D, bool OUT_BF16, bool NORM = false>
__device__ __forceinline__ float decode_token(float4 (&sr)[D / 8], const float (&kin)[4], const float (&qin)[4],
                                              float vin, float alpha, float bin, void* out, size_t orow, int l2norm,
                                              float scale, float* ub, int wave, int lane, float* nb = nullptr) {
    constexpr int LPR = D / 4, RPI = WAVE / LPR, NL = LPR / 2;
    const int c = lane % LPR, sub = lane / LPR;
    // Every multiply-add below is an explicit fmaf: the rounding then does not
    // depend on how the compiler contracts in each kernel that inlines this.
    float ssk = 0.f, ssq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { ssk = fmaf(kin[e], kin[e], ssk); ssq = fmaf(qin[e], qin[e], ssq); }
    ssk = lane_group_sum<LPR>(ssk);
    ssq = lane_group_sum<LPR>(ssq);
    const float rk = l2norm ? 1.0f / sqrtf(ssk + 1e-6f) : 1.0f;
    const float rq = (l2norm ? 1.0f / sqrtf(ssq + 1e-6f) : 1.0f) * scale;
    float kx[4], qx[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) { kx[e] = kin[e] * rk; qx[e] = qin[e] * rq; }
    const float kq = lane_group_sum<LPR>(fmaf(kx[3], qx[3], fmaf(kx[2], qx[2], fmaf(kx[1], qx[1], kx[0] * qx[0]))));

    // partial row sums: x[m] = (S k^) part, x[NL + m] = (S q^) part
    float x[LPR];
#pragma unroll
    for (int m = 0; m < NL; ++m) {
        const float4 sm = sr[m];
        x[m] = fmaf(sm.w, kx[3], fmaf(sm.z, kx[2], fmaf(sm.y, kx[1], sm.x * kx[0])));
        x[NL + m] = fmaf(sm.w, qx[3], fmaf(sm.z, qx[2], fmaf(sm.y, qx[1], sm.x * qx[0])));
    }
    // afterwards lane c holds x[c] summed over its row group
    const float red = reduce_scatter<LPR>(x, c);
    // lanes c < NL: row (c) has p = S k^ ; lanes c >= NL: row (c - NL) has S q^
    const int mrow = (c < NL) ? c : c - NL;
    const int row = wave * 32 + mrow * RPI + sub;
    float u = 0.f;
    if (c < NL) u = bin * fmaf(-alpha, red, vin);
    // lane c >= NL takes u from lane c - NL
    float u_pair;
    if constexpr (NL == 16) u_pair = permlane16_swap(u, u).x;
    else u_pair = row_partner<8>(u);
    const float ov = fmaf(alpha, red, u_pair * kq);  // lanes c >= NL: the output of `row`
    if constexpr (NORM) {
        // sum of squares: this wave's 32 rows (the halves of the wave are its two
        // 32-lane sums), then the waves' sums through LDS
        const float o2 = lane_group_sum<32>(c >= NL ? ov * ov : 0.f);
        const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(o2), 0)) +
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(o2), 32));
        if (lane == 0) nb[wave] = ws;
    } else {
        if (c >= NL) store1<OUT_BF16>(out, orow * D + row, ov);
    }

    // rank-1 update; u of row m of this row group, broadcast through LDS
    // (one wave's LDS operations complete in order)
    if (c < NL) ub[sub * NL + c] = u;
    float um[NL];
#pragma unroll
    for (int j = 0; j < NL / 4; ++j) {
        const float4 t = *reinterpret_cast<const float4*>(ub + sub * NL + 4 * j);
        um[4 * j] = t.x; um[4 * j + 1] = t.y; um[4 * j + 2] = t.z; um[4 * j + 3] = t.w;
    }
#pragma unroll
    for (int m = 0; m < NL; ++m) {
        float4 sm = sr[m];
        sm.x = fmaf(um[m], kx[0], alpha * sm.x);
        sm.y = fmaf(um[m], kx[1], alpha * sm.y);
        sm.z = fmaf(um[m], kx[2], alpha * sm.z);
        sm.w = fmaf(um[m], kx[3], alpha * sm.w);
        sr[m] = sm;
    }
    return ov;
}

// Writes the output that decode_token<..., NORM = true> returned for row group
// `wave`: waits for every wave's sum of squares in nb, then stores
// o / sqrt(mean(o^2) + eps) * wrow (wrow: the weight of this lane's row).
template <int D, bool OUT_BF16>
__device__ __forceinline__ void norm_output(float ov, void* out, size_t orow, int wave, int lane, float wrow,
                                            float eps, const float* nb) {
    constexpr int LPR = D / 4, RPI = WAVE / LPR, NL = LPR / 2;
    const int c = lane % LPR, sub = lane / LPR;
    lds_barrier();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < D / 32; ++w) tot += nb[w];
    const float r = 1.0f / sqrtf(tot * (1.0f / D) + eps);
    if (c >= NL) store1<OUT_BF16>(out, orow * D + wave * 32 + (c - NL) * RPI + sub, ov * r * wrow);
}

// This lane's state slices of one (sequence, v-head) unit, in or out.
template <int D, bool NT = false>
__device__ __forceinline__ void state_store(const float4 (&sr)[D / 8], float* __restrict__ S, int wave, int lane) {
    constexpr int LPR = D / 4, RPI = WAVE / LPR, NL = LPR / 2;
    const int c = lane % LPR, sub = lane / LPR;
#pragma unroll
    for (int m = 0; m < NL; ++m) state_st<NT>(S + (size_t)(wave * 32 + m * RPI + sub) * D + 4 * c, sr[m]);
}

// raw_gates: in.g and in.b are the raw gate inputs (see the header).
template <int D, bool OUT_BF16, bool NORM, bool NT>
__device__ __forceinline__ void decode_compute(DecodeIn<D>& in, float* __restrict__ state, void* out, int unit,
                                               int h_v, int l2norm, float scale, float* ub, int wave, int lane,
                                               bool raw_gates, float eps, float* nb) {
    if (in.slot < 0) {  // skipped (every wave of the unit's workgroup): zero outputs, state untouched
        constexpr int LPR = D / 4, RPI = WAVE / LPR, NL = LPR / 2;
        const int c = lane % LPR, sub = lane / LPR;
        if (c >= NL) store1<OUT_BF16>(out, (size_t)unit * D + wave * 32 + (c - NL) * RPI + sub, 0.f);
        return;
    }
    const int h = unit % h_v;
    float alpha, bta;
    token_gates(in.g, in.b, raw_gates, alpha, bta);
    const float ov = decode_token<D, OUT_BF16, NORM>(in.s, in.kx, in.qx, in.v, alpha, bta, out, (size_t)unit,
                                                     l2norm, scale, ub, wave, lane, nb);
    state_store<D, NT>(in.s, state + ((size_t)in.slot * h_v + h) * D * D, wave, lane);
    if constexpr (NORM) norm_output<D, OUT_BF16>(ov, out, (size_t)unit, wave, lane, in.w, eps, nb);
}

template <int D, bool IN_BF16, bool OUT_BF16, bool NORM, bool NT>
__device__ __forceinline__ void decode_unit(const void* __restrict__ q, const void* __restrict__ k,
                                            const void* __restrict__ v, const float* __restrict__ g,
                                            const float* __restrict__ beta, float* __restrict__ state,
                                            const int32_t* __restrict__ slots, int num_slots, void* __restrict__ out,
                                            int h_k, int h_v, int l2norm, float scale, bool raw_gates,
                                            const float* __restrict__ norm_w, float eps, float* ub, float* nsum,
                                            int wave, int u) {
    const int lane = threadIdx.x % WAVE;
    DecodeIn<D> in;
    decode_load<D, IN_BF16, NT>(in, state, slots, num_slots, q, k, v, g, beta, norm_w, u, h_k, h_v, wave, lane);
    decode_compute<D, OUT_BF16, NORM, NT>(in, state, out, u, h_v, l2norm, scale, ub, wave, lane, raw_gates, eps,
                                          nsum);
}

// fuse: bit 0 raw gate inputs, bit 1 output norm (weights norm_w, NULL for ones),
// bit 2 the nontemporal state accesses.  The grid has one workgroup per unit:
// a workgroup of D/32 waves owns unit blockIdx.x (wave w: rows 32w..32w+31).  With
// one-wave workgroups (no output norm: the rows of a unit are independent) the
// D/32 row groups of a unit are D/32 workgroups, so a few units still spread
// over many compute units: workgroup b takes row group b % (D/32) of unit
// b / (D/32) (gridDim.x is a multiple of D/32).
template <int D, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(2 * D) void decode_step_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    const int32_t* __restrict__ slots, int num_slots, void* __restrict__ out, int units, int h_k, int h_v,
    int l2norm, float scale, int fuse, const float* __restrict__ norm_w, float norm_eps) {
    __shared__ __align__(16) float ubuf[(D / 32) * 32];
    __shared__ __align__(16) float nsum[D / 32];
    constexpr int NW = D / 32;
    const bool split = blockDim.x == WAVE;  // one-wave workgroups (launched only without the norm)
    const int wave = split ? (int)(blockIdx.x % NW) : (int)(threadIdx.x / WAVE);
    const int u = split ? (int)(blockIdx.x / NW) : (int)blockIdx.x;
    if (u >= units) return;  // the whole workgroup
    float* ub = ubuf + wave * 32;
    const bool raw_gates = (fuse & 1) != 0;
#define GDN_UNIT(NORM, NT)                                                                                      \
    decode_unit<D, IN_BF16, OUT_BF16, NORM, NT>(q, k, v, g, beta, state, slots, num_slots, out, h_k, h_v, l2norm, \
                                                scale, raw_gates, NORM ? norm_w : nullptr, NORM ? norm_eps : 0.f,  \
                                                ub, nsum, wave, u)
    if (fuse & 2) {
        if (fuse & 4) GDN_UNIT(true, true);
        else GDN_UNIT(true, false);
    } else {
        if (fuse & 4) GDN_UNIT(false, true);
        else GDN_UNIT(false, false);
    }
#undef GDN_UNIT
}

// ---- direct scan: the token recurrence with the state in registers ---------------------
// "Optimizing on-device inference for Apple Silicon", section "Qwen creates
// three distinct workload shapes", runs prefill either as this direct scan or
// in blocks; which is faster depends on the shape.  One workgroup per
// (sequence, v-head) unit loads its state once, walks the sequence's tokens
// with the inputs of the next DIRECT_PREFETCH tokens in flight while one
// computes, and writes the state once.  Sequence n spans tokens [cu[n], cu[n+1]), both
// clamped into [0, T] (an empty or inverted range has no tokens).
constexpr int DIRECT_PREFETCH = 4;  // tokens whose inputs are loaded ahead

template <int D, bool IN_BF16>
struct TokIn {
    float kx[4], qx[4];
    float v, g, b;
};

template <int D, bool IN_BF16>
__device__ __forceinline__ void token_load(TokIn<D, IN_BF16>& in, const void* q, const void* k, const void* v,
                                           const float* g, const float* beta, size_t tok, int h, int hk, int h_k,
                                           int h_v, int wave, int lane) {
    constexpr int LPR = D / 4, RPI = WAVE / LPR, NL = LPR / 2;
    const int c = lane % LPR, sub = lane / LPR;
    load4<IN_BF16>(k, (tok * h_k + hk) * D + 4 * c, in.kx);
    load4<IN_BF16>(q, (tok * h_k + hk) * D + 4 * c, in.qx);
    const int mrow = (c < NL) ? c : c - NL;
    in.v = load1<IN_BF16>(v, (tok * h_v + h) * D + wave * 32 + mrow * RPI + sub);
    in.g = g[tok * h_v + h];
    in.b = beta[tok * h_v + h];
}

// The scan of one workgroup's unit; with NORM each token's output is normalised
// over the head's d rows (the decode step's exchange, the two LDS areas
// alternating by token).  raw_gates: g and beta hold raw gate inputs.
template <int D, bool IN_BF16, bool OUT_BF16, bool NORM>
__device__ __forceinline__ void direct_unit(const void* __restrict__ q, const void* __restrict__ k,
                                            const void* __restrict__ v, const float* __restrict__ g,
                                            const float* __restrict__ beta, const int32_t* __restrict__ cu,
                                            const float* __restrict__ state_in, float* __restrict__ state_out,
                                            void* __restrict__ out, int T, int h_k, int h_v, int l2norm, float scale,
                                            bool raw_gates, const float* __restrict__ norm_w, float eps, float* ub,
                                            float* nsum) {
    constexpr int LPR = D / 4, RPI = WAVE / LPR, NL = LPR / 2;
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    const int c = lane % LPR, sub = lane / LPR;
    const int unit = blockIdx.x, n = unit / h_v, h = unit - n * h_v, hk = h / (h_v / h_k);
    int b0 = 0, e0 = T;
    if (cu) {
        b0 = min(max(cu[n], 0), T);
        e0 = min(max(cu[n + 1], b0), T);
    }
    const int mrow = (c < NL) ? c : c - NL;
    const float wrow = (NORM && norm_w) ? norm_w[wave * 32 + mrow * RPI + sub] : 1.f;
    float4 sr[D / 8];
    const size_t sbase = (size_t)unit * D * D;
#pragma unroll
    for (int m = 0; m < NL; ++m) {
        const size_t off = sbase + (size_t)(wave * 32 + m * RPI + sub) * D + 4 * c;
        sr[m] = state_in ? *reinterpret_cast<const float4*>(state_in + off) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (e0 > b0) {
        // the inputs of the next P tokens are in flight while a token computes
        // (past the end the last token is read again, unused)
        TokIn<D, IN_BF16> buf[DIRECT_PREFETCH];
#pragma unroll
        for (int i = 0; i < DIRECT_PREFETCH; ++i)
            token_load<D, IN_BF16>(buf[i], q, k, v, g, beta, (size_t)min(b0 + i, e0 - 1), h, hk, h_k, h_v, wave, lane);
        for (int t = b0; t < e0; t += DIRECT_PREFETCH) {
#pragma unroll
            for (int i = 0; i < DIRECT_PREFETCH; ++i) {
                if (t + i < e0) {
                    const TokIn<D, IN_BF16> cur = buf[i];
                    token_load<D, IN_BF16>(buf[i], q, k, v, g, beta, (size_t)min(t + i + DIRECT_PREFETCH, e0 - 1), h,
                                           hk, h_k, h_v, wave, lane);
                    float alpha, bta;
                    token_gates(cur.g, cur.b, raw_gates, alpha, bta);
                    float* nb = nsum + ((t + i - b0) & 1) * (D / 32);
                    const size_t orow = (size_t)(t + i) * h_v + h;
                    const float ov = decode_token<D, OUT_BF16, NORM>(sr, cur.kx, cur.qx, cur.v, alpha, bta, out,
                                                                     orow, l2norm, scale, ub, wave, lane, nb);
                    if constexpr (NORM) norm_output<D, OUT_BF16>(ov, out, orow, wave, lane, wrow, eps, nb);
                }
            }
        }
    }
    if (state_out) state_store<D>(sr, state_out + sbase, wave, lane);
}

// fuse: bit 0 raw gate inputs, bit 1 output norm (weights norm_w, NULL for ones).
template <int D, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(2 * D) void direct_scan_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    const float* __restrict__ state_in, float* __restrict__ state_out, void* __restrict__ out, int T, int h_k,
    int h_v, int l2norm, float scale, int fuse, const float* __restrict__ norm_w, float norm_eps) {
    __shared__ __align__(16) float ubuf[(D / 32) * 32];
    __shared__ __align__(16) float nsum[2 * (D / 32)];
    float* ub = ubuf + (threadIdx.x / WAVE) * 32;
    const bool raw_gates = (fuse & 1) != 0;
    if (fuse & 2)
        direct_unit<D, IN_BF16, OUT_BF16, true>(q, k, v, g, beta, cu, state_in, state_out, out, T, h_k, h_v, l2norm,
                                                scale, raw_gates, norm_w, norm_eps, ub, nsum);
    else
        direct_unit<D, IN_BF16, OUT_BF16, false>(q, k, v, g, beta, cu, state_in, state_out, out, T, h_k, h_v,
                                                 l2norm, scale, raw_gates, nullptr, 0.f, ub, nsum);
}

int compute_units();  // of the current device (prefill.hip)

template <int D, bool IB, bool OB>
static hipError_t launch_direct_t(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                  const int32_t* cu, const float* s_in, float* s_out, void* out, int units, int T,
                                  int h_k, int h_v, int l2norm, float scale, int fuse, const float* norm_w,
                                  float norm_eps, hipStream_t stream) {
    hipLaunchKernelGGL((direct_scan_kernel<D, IB, OB>), dim3(units), dim3(2 * D), 0, stream, q, k, v, g, beta, cu,
                       s_in, s_out, out, T, h_k, h_v, l2norm, scale, fuse, norm_w, norm_eps);
    return hipGetLastError();
}

hipError_t launch_direct(int d, bool in_bf16, bool out_bf16, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const int32_t* cu, const float* s_in, float* s_out,
                         void* out, int units, int T, int h_k, int h_v, int l2norm, float scale, int fuse,
                         const float* norm_w, float norm_eps, hipStream_t stream) {
#define GDN_DIR(D, IB, OB)                                                                                 \
    if (d == D && in_bf16 == IB && out_bf16 == OB)                                                         \
        return launch_direct_t<D, IB, OB>(q, k, v, g, beta, cu, s_in, s_out, out, units, T, h_k, h_v, l2norm, \
                                          scale, fuse, norm_w, norm_eps, stream);
    GDN_DIR(128, true, true) GDN_DIR(128, true, false) GDN_DIR(128, false, true)
    GDN_DIR(128, false, false) GDN_DIR(64, true, true) GDN_DIR(64, true, false)
    GDN_DIR(64, false, true) GDN_DIR(64, false, false)
#undef GDN_DIR
    return hipErrorInvalidValue;
}

// Most units one launch takes, one workgroup of 2 d threads each: the grid
// stays below 2^32 work-items.  The state of that many units (512 GiB at
// d = 64) exceeds the 288 GB of device memory.
template <int D>
constexpr int decode_max_units() { return (int)((1LL << 31) / D) - 1; }
// Dynamic LDS, unused, that the d = 128 whole-unit launch reserves so that two
// workgroups share a compute unit (the registers would allow four).  Measured
// on MI355X with states beyond the last-level cache, two move the state 3-7%
// faster than four, with either cache policy (256 and 1024 sequences x 32
// heads); a state that stays in the cache steps ~1% slower.  At d = 64, whose
// workgroups have two waves, the same cap measured slower at small batches.
constexpr size_t kDecodeResidencyLds = 60 * 1024;

template <int D, bool IB, bool OB>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, float* state, const int32_t* slots, int num_slots,
                                  void* out, int units, int h_k, int h_v, int l2norm, float scale, int fuse,
                                  const float* norm_w, float norm_eps, hipStream_t stream) {
    // Too few units to fill the chip (and no output norm): one-wave workgroups, one per
    // row group of a unit, so each unit's rows spread over D/32 compute units.
    const bool split = !(fuse & 2) && (long long)units * (D / 32) <= 2LL * compute_units();
    if (split) {
        hipLaunchKernelGGL((decode_step_kernel<D, IB, OB>), dim3(units * (D / 32)), dim3(WAVE), 0, stream, q, k, v,
                           g, beta, state, slots, num_slots, out, units, h_k, h_v, l2norm, scale, fuse, norm_w,
                           norm_eps);
        return hipGetLastError();
    }
    if (units > decode_max_units<D>()) return hipErrorInvalidValue;
    const size_t lds = D == 128 ? kDecodeResidencyLds : 0;
    hipLaunchKernelGGL((decode_step_kernel<D, IB, OB>), dim3(units), dim3(2 * D), lds, stream, q, k, v,
                       g, beta, state, slots, num_slots, out, units, h_k, h_v, l2norm, scale, fuse, norm_w,
                       norm_eps);
    return hipGetLastError();
}

hipError_t launch_decode(int d, bool in_bf16, bool out_bf16, const void* q, const void* k,
                         const void* v, const float* g, const float* beta, float* state, const int32_t* slots,
                         int num_slots, void* out, int units, int h_k, int h_v, int l2norm, float scale,
                         int fuse, const float* norm_w, float norm_eps, hipStream_t stream) {
#define GDN_DEC(D, IB, OB)                                                                        \
    if (d == D && in_bf16 == IB && out_bf16 == OB)                                                \
        return launch_decode_t<D, IB, OB>(q, k, v, g, beta, state, slots, num_slots, out, units, h_k, h_v, \
                                          l2norm, scale, fuse, norm_w, norm_eps, stream);
    GDN_DEC(128, true, true) GDN_DEC(128, true, false) GDN_DEC(128, false, true)
    GDN_DEC(128, false, false) GDN_DEC(64, true, true) GDN_DEC(64, true, false)
    GDN_DEC(64, false, true) GDN_DEC(64, false, false)
#undef GDN_DEC
    return hipErrorInvalidValue;
}

}  // namespace gdn

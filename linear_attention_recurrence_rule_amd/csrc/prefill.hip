// Blocked ("chunked") prefill of the gated delta rule on gfx950.
//
// "Optimizing on-device inference for Apple Silicon", section "Qwen creates
// three distinct workload shapes", says the recurrence can be regrouped into
// blocks of tokens that expose matrix work.  Section "Keep the recurrent state
// on chip" keeps the state on chip for the whole scan and writes it back once,
// in fp32.  This file implements that blocked form with matrix-core tiles.
//
// Per block of n <= 64 tokens (chunk) and v-head, with block-initial state S
// (d_v x d_k), cumulative log-decay G_i = g_1 + ... + g_i, effective keys k_i
// and queries q_i (normalised, query scaled):
//   A_ij = beta_i exp(G_i - G_j) k_i.k_j (i > j),  T = (I + A)^{-1} diag(beta)
//   W = T diag(exp G) K,  Ut = T V,  P_ij = exp(G_i - G_j) q_i.k_j (i >= j)
//   U = Ut - W S^T,  O = diag(exp G) Q S^T + P U,
//   S' = exp(G_n) S + U^T diag(exp(G_n - G)) K.
// Splitting O = Ot + Qt S^T with Ot = P Ut and Qt = diag(exp G) Q - P W gives
// two phases:
//   chunk_prep  (parallel over blocks x v-heads): everything not involving S,
//               written to a workspace record per (block, v-head);
//   chunk_scan  (sequential over the blocks of a sequence, parallel over
//               sequences x v-heads x row slices of S): S lives in registers
//               for the whole sequence and is read and written once.
// S's rows evolve independently, so a v-head's state can be split by rows
// over several workgroups.
//
// Precision.  q/k are scaled per token by a power of two (exact) and fed raw
// to the matrix cores.  Their L2 norms become fp32 row factors c_t.  Values
// enter as fp16 (exact for bf16 in range).  fp32 intermediates that feed the
// matrix cores are rounded to fp16 (bf16 inputs) or stay fp32 (fp32 inputs).
// Ut and Ot are stored in the operand type too; they only seed the scan's
// fp32 accumulators.
#include "gdn_device.h"

#include <stdlib.h>

namespace gdn {

struct SeqInfo {
    int32_t begin, len, slot_base, pad;
};

// ---- varlen plan: per-sequence token range and block-slot base, slot -> sequence ----
// One workgroup.  cu_seqlens is clamped into a non-decreasing sequence inside
// [0, T] so that every index stays in bounds whatever the caller passed.
__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu, int N, int T,
                                                   int max_slots, SeqInfo* __restrict__ info,
                                                   int32_t* __restrict__ slot_seq) {
    __shared__ int s_carry_tok, s_carry_slot;
    __shared__ int s_scan[256];
    const int tid = threadIdx.x;
    if (tid == 0) { s_carry_tok = 0; s_carry_slot = 0; }
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int n = base + tid;
        // running max of clamped ends (prefix max over this block, seeded by the carry)
        int end = 0;
        if (n < N) {
            end = cu[n + 1];
            end = end < 0 ? 0 : (end > T ? T : end);
        }
        s_scan[tid] = end;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            int o = (tid >= off) ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] = max(s_scan[tid], o);
            __syncthreads();
        }
        const int carry_tok = s_carry_tok;
        const int my_end = max(s_scan[tid], carry_tok);
        const int my_begin = (tid == 0) ? carry_tok : max(s_scan[tid - 1], carry_tok);
        const int len = (n < N) ? my_end - my_begin : 0;
        const int nch = (len + CHUNK - 1) / CHUNK;
        __syncthreads();
        s_scan[tid] = nch;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            int o = (tid >= off) ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += o;
            __syncthreads();
        }
        const int slot_base = s_carry_slot + s_scan[tid] - nch;
        if (n < N) {
            info[n] = SeqInfo{my_begin, len, slot_base, 0};
            for (int j = 0; j < nch; ++j)
                if (slot_base + j < max_slots) slot_seq[slot_base + j] = n;
        }
        __syncthreads();
        if (tid == 255) { s_carry_tok = my_end; s_carry_slot = slot_base + nch; }
        __syncthreads();
    }
    const int used = s_carry_slot;
    for (int s = used + tid; s < max_slots; s += 256) slot_seq[s] = -1;
}

// ---- workspace record of one (block slot, v-head) ----------------------------------------
template <int D, typename OP>
struct Rec {
    // Per (block, v-head), in the matrix-core operand type OP.  -W and Qt are
    // fragment-major (64 lanes x 8 elements per fragment); Ut and Ot are 16x16
    // accumulator tiles (64 lanes x 4 elements), ordered by row block of d_v,
    // then token block, so the tiles of a row slice are contiguous.
    static constexpr size_t W = 0;                                   // -W : (C/16) x (D/32) frags
    static constexpr size_t Q = W + (size_t)CHUNK * D * sizeof(OP);  // Qt : same
    static constexpr size_t U = Q + (size_t)CHUNK * D * sizeof(OP);  // Ut : (D/16) x (C/16) tiles
    static constexpr size_t O = U + (size_t)CHUNK * D * sizeof(OP);  // Ot : same
    static constexpr size_t S = O + (size_t)CHUNK * D * sizeof(OP);  // s_t = exp(G_n - G_t) c_t, fp32[C]
    static constexpr size_t M = S + CHUNK * 4;                       // gamma_n (fp32), pad
    static constexpr size_t BYTES = M + 256;
    static constexpr size_t TILE = 16 * 16 * sizeof(OP);             // one Ut / Ot tile
};

// Per (block, k-head): K^T fragments, (D/16) x (C/32), shared by the v-heads
// that read this k-head.
template <int D, typename OP>
struct KeyRec {
    static constexpr size_t BYTES = (size_t)CHUNK * D * sizeof(OP);
};

template <int D, typename OP>
constexpr int ldsk() { return D + 16 / (int)sizeof(OP); }  // row stride of [token][d] tiles
constexpr int LDF = CHUNK + 4;                                  // fp32 64x64 tiles

// LDS of chunk_prep (about 68 KiB at d = 128, so two workgroups share a
// compute unit).  q and k are kept row-major ([token][d]).  Operands that
// contract over tokens are read from them as column fragments.  T and P are
// only ever read as matrix-core fragments, so they are stored fragment-major
// (64 lanes x 8 elements per fragment, one contiguous 16-byte read per lane).
// Region b holds, by phase: A (strictly lower) with X^T = ((I + A)^{-1})^T in
// its upper triangle, then the values V, then -W.
// The in-block cumulative log-decay G.  Decay ratios are exp(G_i - G_j); after
// a run of strong decay both G_i and G_j are large and their fp32 difference
// carries ~1e-7 |G| of cancellation error.  fp16 operands absorb that; the
// fp32 path (a 1e-5 budget) keeps G in fp64 and takes the differences there.
template <typename OP> struct GType { using T = float; };
template <> struct GType<float> { using T = double; };

template <int D, typename OP>
struct PrepLds {
    static constexpr int LK = ldsk<D, OP>();
    OP k[CHUNK * LK];  // keys scaled per token by a power of two (exact)
    OP q[CHUNK * LK];  // queries, likewise
    union B {
        float ax[CHUNK * LDF];  // A_ij (i > j) at [i][j]; X_ij (i >= j) at [j][i]
        OP v[CHUNK * LK];       // values [token][d]
        OP w[CHUNK * LK];       // -W [token][d]
    } b;
    OP t[CHUNK * CHUNK];  // T = X diag(beta), fragment-major: (row block, 32-column block) fragments
    OP p[CHUNK * CHUNK];  // P = lower_incl(D o Q K^T), likewise
    typename GType<OP>::T G[CHUNK];
    float ck[CHUNK], cq[CHUNK], bt[CHUNK], gck[CHUNK], gcq[CHUNK];
    int zero;  // holds 0 (see chunk_prep_kernel)
};

template <int D, typename OP>
constexpr size_t prep_lds_bytes() { return sizeof(PrepLds<D, OP>); }

// Norm factor c of one (token, head) vector whose elements were scaled by
// 2^-e (exactly): the effective vector is c * scaled.  With the L2 norm,
// c = 1 / sqrt(sum scaled^2 + 1e-6 * 2^-2e); the epsilon term underflows to 0
// or overflows to +inf (c = 0) only where it is negligible or dominant.
__device__ __forceinline__ float norm_factor(float ss_scaled, int e, int l2norm, float mul) {
    if (!l2norm) return ldexpf(mul, e);
    return mul * rsqrtf(ss_scaled + ldexpf(1e-6f, -2 * e));
}

template <bool IN_BF16>
__device__ __forceinline__ void unpack8(const uint4* src, float x[8]) {
    if constexpr (IN_BF16) {
        const uint32_t w[4] = {src[0].x, src[0].y, src[0].z, src[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            x[4 * i + 0] = __uint_as_float(src[i].x); x[4 * i + 1] = __uint_as_float(src[i].y);
            x[4 * i + 2] = __uint_as_float(src[i].z); x[4 * i + 3] = __uint_as_float(src[i].w);
        }
    }
}

template <typename OP>
__device__ __forceinline__ void store8(OP* dst, const float x[8]) {
    if constexpr (sizeof(OP) == 2) {
        h8_t h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (_Float16)x[e];
        *reinterpret_cast<h8_t*>(dst) = h;
    } else {
        *reinterpret_cast<f4_t*>(dst) = f4_t{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f4_t*>(dst + 4) = f4_t{x[4], x[5], x[6], x[7]};
    }
}

template <typename OP>
__device__ __forceinline__ void store4(OP* dst, const f4_t& x) {
    if constexpr (sizeof(OP) == 2) {
        typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
        *reinterpret_cast<h4_t*>(dst) = h4_t{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
    } else {
        *reinterpret_cast<f4_t*>(dst) = x;
    }
}

// Workgroup size of the block-form work (8 waves).
constexpr int PREP_THREADS = 512;
constexpr int PREP_WAVES = PREP_THREADS / WAVE;

// Six 16x16 fp32 matrices in accumulator layout, kept in the blocks of b.ax above the
// diagonal (unused once A is formed): slot s is block (0,1), (0,2), (0,3), (1,2), (1,3), (2,3).
// Lane (j, q) owns row j, columns 4q..4q+3 of its block (one 16-byte access).
__device__ __forceinline__ float* prep_xslot(float* ax, int s, int li, int lq) {
    const int r = (s >= 3) + (s >= 5), c = s < 3 ? s + 1 : s < 5 ? s - 1 : 3;
    return ax + (16 * r + li) * LDF + 16 * c + 4 * lq;
}

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

// Row fragment of a row-major matrix M (leading dimension ld) for products
// whose two operands are both read this way: lane (i, q) holds the eight
// consecutive elements M[16 rb + i][32 kb + 8q + e], one 16-byte read (two for
// fp32) per lane, so each quarter-wave reads distinct banks.  The contraction
// index of element e is 8q + e, not the accumulator order of frag_colmajor and
// frag_from_acc; a product must take both operands in the same order.
template <typename OP>
__device__ __forceinline__ Frag<OP> frag_row8(const OP* M, int ld, int rb, int kb, int lane) {
    const OP* p = M + (size_t)(16 * rb + (lane & 15)) * ld + 32 * kb + 8 * (lane >> 4);
    Frag<OP> f;
    if constexpr (sizeof(OP) == 2) {
        f.v = *reinterpret_cast<const h8_t*>(p);
    } else {
        f.lo = *reinterpret_cast<const f4_t*>(p);
        f.hi = *reinterpret_cast<const f4_t*>(p + 4);
    }
    return f;
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

// One thread's share of a block's raw inputs for one (k-head, v-head).
template <int D, bool IN_BF16>
struct PrepIn {
    static constexpr int PER_TOK = D / 8, NIT = CHUNK * PER_TOK / PREP_THREADS, W16 = IN_BF16 ? 1 : 2;
    static constexpr int ES = IN_BF16 ? 2 : 4;  // bytes per input element
    uint4 q[NIT][W16], k[NIT][W16], v[NIT][W16];
    float g, b;

    // Token indices are clamped into [0, T); data past a block's end is zeroed on use.
    __device__ __forceinline__ void load_qk(const void* qp, const void* kp, int tok0, int T, int h_k, int hk) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int idx = threadIdx.x + PREP_THREADS * it, t = idx / PER_TOK, pc = idx % PER_TOK;
            const size_t off = (((size_t)min(tok0 + t, T - 1) * h_k + hk) * D + 8 * pc) * ES;
#pragma unroll
            for (int w = 0; w < W16; ++w) {
                q[it][w] = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(qp) + off)[w];
                k[it][w] = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(kp) + off)[w];
            }
        }
    }
    __device__ __forceinline__ void load_v(const void* vp, int tok0, int T, int h_v, int h) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int idx = threadIdx.x + PREP_THREADS * it, t = idx / PER_TOK, pc = idx % PER_TOK;
            const size_t off = (((size_t)min(tok0 + t, T - 1) * h_v + h) * D + 8 * pc) * ES;
#pragma unroll
            for (int w = 0; w < W16; ++w)
                v[it][w] = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(vp) + off)[w];
        }
    }
    __device__ __forceinline__ void load_gb(const float* gp, const float* bp, int tok0, int T, int h_v, int h) {
        const size_t tg = (size_t)min(tok0 + (int)(threadIdx.x % WAVE), T - 1) * h_v + h;
        g = gp[tg];
        b = bp[tg];
    }
};

// The block-form work that does not depend on the carried state, for
// (block, v-head) tasks.  A workgroup of PREP_THREADS threads takes a run of
// (block slot, k-head) items and, per item, the k-head's v-heads in turn: the
// queries and keys are scaled once per item, the K^T fragments are written
// once per item, and each v-head's work is written as one record.  The next
// task's inputs are loaded into registers as soon as the current ones have
// been consumed, so their latency is hidden behind the current task.
// Waves per SIMD the LDS allows (two workgroups per CU when they fit), as a register budget.
template <int D, typename OP>
constexpr int prep_min_waves() { return 2 * prep_lds_bytes<D, OP>() <= 160 * 1024 ? 4 : 2; }

template <int D, typename OP, bool IN_BF16>
__global__ __launch_bounds__(PREP_THREADS, (prep_min_waves<D, OP>())) void chunk_prep_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const SeqInfo* __restrict__ info,
    const int32_t* __restrict__ slot_seq, int T, int h_k, int h_v, int l2norm, float scale,
    char* __restrict__ recs, char* __restrict__ krecs, int slots, int items_per_wg) {
    using RC = Rec<D, OP>;
    using In = PrepIn<D, IN_BF16>;
    constexpr int LK = PrepLds<D, OP>::LK;
    constexpr int PER_TOK = In::PER_TOK, NIT = In::NIT;
    extern __shared__ __align__(16) char smem_raw[];
    PrepLds<D, OP>& L = *reinterpret_cast<PrepLds<D, OP>*>(smem_raw);
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int li = lane & 15, lq = lane >> 4;
    const int ratio = h_v / h_k;
    const int items = slots * h_k;
    const int i0 = blockIdx.x * items_per_wg, i1 = min(items, i0 + items_per_wg);
    if (i0 >= i1) return;
    // token range of a block slot; false for an unused slot of packed sequences
    auto slot_range = [&](int slot, int& tok0, int& nt) {
        if (slot_seq) {
            const int n = slot_seq[slot];
            if (n < 0) { tok0 = 0; nt = 0; return false; }
            const SeqInfo si = info[n];
            const int j = slot - si.slot_base;
            tok0 = si.begin + j * CHUNK;
            nt = min(CHUNK, si.len - j * CHUNK);
        } else {
            tok0 = slot * CHUNK;
            nt = min(CHUNK, T - tok0);
        }
        return true;
    };

    if (tid == 0) L.zero = 0;
    lds_barrier();
    In in;
    int tok0, nt;
    bool live = slot_range(i0 / h_k, tok0, nt);
    in.load_qk(q, k, tok0, T, h_k, i0 % h_k);
    in.load_v(v, tok0, T, h_v, (i0 % h_k) * ratio);
    in.load_gb(g, beta, tok0, T, h_v, (i0 % h_k) * ratio);
    for (int item = i0; item < i1; ++item) {
        const int slot = item / h_k, hk = item % h_k;
        const int ctok0 = tok0, cnt = nt;
        const bool clive = live;
        int ntok0 = 0, nnt = 0;
        const bool more = item + 1 < i1;
        const bool nlive = more && slot_range((item + 1) / h_k, ntok0, nnt);

        // ---- 1. per-token power-of-two scaling and norms; q, k to LDS (row-major) -----------
        if (clive) {
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int idx = tid + PREP_THREADS * it, t = idx / PER_TOK, pc = idx % PER_TOK;
                const bool tl = t < cnt;
                float kx[8], qx[8];
                unpack8<IN_BF16>(in.k[it], kx);
                unpack8<IN_BF16>(in.q[it], qx);
                float mk = 0.f, mq = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (!tl) { kx[e] = 0.f; qx[e] = 0.f; }
                    mk = fmaxf(mk, fabsf(kx[e]));
                    mq = fmaxf(mq, fabsf(qx[e]));
                }
                mk = group_max<PER_TOK>(mk);  // the PER_TOK lanes of a token are adjacent
                mq = group_max<PER_TOK>(mq);
                int ek = 0, eq = 0;
                frexpf(mk, &ek);
                frexpf(mq, &eq);
                float ssk = 0.f, ssq = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    kx[e] = ldexpf(kx[e], -ek);  // exact; representable in OP for bf16 inputs
                    qx[e] = ldexpf(qx[e], -eq);
                    ssk += kx[e] * kx[e];
                    ssq += qx[e] * qx[e];
                }
                ssk = group_sum<PER_TOK>(ssk);
                ssq = group_sum<PER_TOK>(ssq);
                store8<OP>(L.k + t * LK + 8 * pc, kx);
                store8<OP>(L.q + t * LK + 8 * pc, qx);
                if (pc == 0) {
                    L.ck[t] = tl ? norm_factor(ssk, ek, l2norm, 1.0f) : 0.f;
                    L.cq[t] = tl ? norm_factor(ssq, eq, l2norm, scale) : 0.f;
                }
            }
        }
        if (more) in.load_qk(q, k, ntok0, T, h_k, (item + 1) % h_k);

        for (int jv = 0; jv < ratio; ++jv) {
            // Lane indices re-derived through a volatile LDS read of 0.  Otherwise the
            // compiler hoists the task's per-lane LDS address arithmetic out of the
            // loops and keeps ~90 more registers live (wave stays uniform).
            const int tid = threadIdx.x + *reinterpret_cast<volatile int*>(&L.zero);
            const int lane = tid % WAVE, li = lane & 15, lq = lane >> 4;
            const int h = hk * ratio + jv;
            // the next task: this item's next v-head, or the next item's first
            const bool nxt = jv + 1 < ratio || more;
            const int nx_tok0 = jv + 1 < ratio ? ctok0 : ntok0;
            const int nx_h = jv + 1 < ratio ? h + 1 : ((item + 1) % h_k) * ratio;
            if (!clive) {
                if (nxt) {
                    in.load_gb(g, beta, nx_tok0, T, h_v, nx_h);
                    in.load_v(v, nx_tok0, T, h_v, nx_h);
                }
                continue;
            }
            char* rec = recs + ((size_t)slot * h_v + h) * RC::BYTES;
            // the first v-head of each k-head writes the k-head's key record
            OP* krec = jv == 0 ? reinterpret_cast<OP*>(krecs + ((size_t)slot * h_k + hk) * KeyRec<D, OP>::BYTES)
                               : nullptr;

            // ---- 1b. cumulative log-decay G, gamma = exp(G), beta ---------------------------
            using GT = typename GType<OP>::T;
            float gam = 0.f;
            if (wave == 0) {
                const bool tl = lane < cnt;
                if constexpr (sizeof(GT) == 4) {
                    const float gx = wave_inclusive_sum(tl ? in.g : 0.f);
                    L.G[lane] = gx;
                    L.bt[lane] = tl ? in.b : 0.f;
                    gam = __expf(gx);
                } else {
                    const GT gx = wave_inclusive_sum(tl ? (GT)in.g : (GT)0);
                    L.G[lane] = gx;
                    L.bt[lane] = tl ? in.b : 0.f;
                    gam = __expf((float)gx);
                }
            }
            if (nxt && wave == 0) in.load_gb(g, beta, nx_tok0, T, h_v, nx_h);  // only wave 0 reads them
            lds_barrier();
            if (wave == 0) {
                L.gck[lane] = gam * L.ck[lane];
                L.gcq[lane] = gam * L.cq[lane];
            }

            // ---- 2. decay-masked Gram products: A (fp32, strictly lower) and P ----------------------
            // 20 tile-products (10 lower 16x16 tiles of K K^T and of Q K^T) over the waves.
            for (int tp = wave; tp < 20; tp += PREP_WAVES) {
                const int tl = tp >> 1, isq = tp & 1;
                const int mb = (tl >= 6) ? 3 : (tl >= 3) ? 2 : (tl >= 1) ? 1 : 0;
                const int nb = tl - mb * (mb + 1) / 2;
                f4_t acc = {0, 0, 0, 0};
                if (!isq) {
#pragma unroll
                    for (int kb = 0; kb < D / 32; ++kb)
                        mma(acc, frag_row8<OP>(L.k, LK, mb, kb, lane), frag_row8<OP>(L.k, LK, nb, kb, lane));
                    const int j = 16 * nb + li, i0 = 16 * mb + 4 * lq;
                    if constexpr (sizeof(GT) == 4) {
                        const float Gj = L.G[j], ckj = L.ck[j];
                        const f4_t Gi = *reinterpret_cast<const f4_t*>(&L.G[i0]);
                        const f4_t cki = *reinterpret_cast<const f4_t*>(&L.ck[i0]);
                        const f4_t bti = *reinterpret_cast<const f4_t*>(&L.bt[i0]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int i = i0 + r;
                            if (j < i) L.b.ax[i * LDF + j] = bti[r] * __expf(Gi[r] - Gj) * acc[r] * cki[r] * ckj;
                        }
                    } else {
                        const GT Gj = L.G[j];
                        const float ckj = L.ck[j];
                        const f4_t cki = *reinterpret_cast<const f4_t*>(&L.ck[i0]);
                        const f4_t bti = *reinterpret_cast<const f4_t*>(&L.bt[i0]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int i = i0 + r;
                            if (j < i)
                                L.b.ax[i * LDF + j] = bti[r] * __expf((float)(L.G[i] - Gj)) * acc[r] * cki[r] * ckj;
                        }
                    }
                } else {
                    // The transposed tile K Q^T: lane (j, q) gets (Q K^T)[16mb + j][16nb + 4q + r],
                    // which is this lane's half of P's fragment (mb, nb / 2).
#pragma unroll
                    for (int kb = 0; kb < D / 32; ++kb)
                        mma(acc, frag_row8<OP>(L.k, LK, nb, kb, lane), frag_row8<OP>(L.q, LK, mb, kb, lane));
                    const int i = 16 * mb + li, c0 = 16 * nb + 4 * lq;
                    f4_t pv;
                    if constexpr (sizeof(GT) == 4) {
                        const float Gi = L.G[i], cqi = L.cq[i];
                        const f4_t Gc = *reinterpret_cast<const f4_t*>(&L.G[c0]);
                        const f4_t ckc = *reinterpret_cast<const f4_t*>(&L.ck[c0]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float dec = (c0 + r <= i) ? __expf(fminf(Gi - Gc[r], 0.f)) : 0.f;
                            pv[r] = dec * acc[r] * cqi * ckc[r];
                        }
                    } else {
                        const GT Gi = L.G[i];
                        const float cqi = L.cq[i];
                        const f4_t ckc = *reinterpret_cast<const f4_t*>(&L.ck[c0]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float dec = (c0 + r <= i) ? __expf(fminf((float)(Gi - L.G[c0 + r]), 0.f)) : 0.f;
                            pv[r] = dec * acc[r] * cqi * ckc[r];
                        }
                    }
                    store_part<OP>(L.p, mb * 2 + nb / 2, nb % 2, lane, pv);
                }
            }
            for (int tl = wave; tl < 6; tl += PREP_WAVES) {  // strictly-upper tiles of P are zero
                const int nb = (tl >= 3) ? 3 : (tl >= 1) ? 2 : 1;
                const int mb = tl - (nb - 1) * nb / 2;
                store_part<OP>(L.p, mb * 2 + nb / 2, nb % 2, lane, f4_t{0.f, 0.f, 0.f, 0.f});
            }
            lds_barrier();

            // ---- 3. T = (I + A)^{-1} diag(beta), written straight into T's fragments ---------------
            // X = (I + A)^{-1} by 16x16 blocks, in fp32 matrix-core products held in registers.
            // 3a (waves 0..3): wave bb inverts the diagonal block X_bb; waves 4..7 write the scan's
            //   K^T fragments meanwhile.
            // 3b (waves 0..5): one wave per block below the diagonal, from
            //   X_ij = -X_ii sum_{m=j}^{i-1} A_im X_mj; the waves that need X_10 or X_21 form it
            //   themselves rather than wait for another wave.
            // Matrices in accumulator layout, lane (j, q) holding M[4q + r][j] in element r; the
            // product C = X Y takes X^T and Y (mm16), and C^T = Y^T X^T the same two swapped.
            // T's fragment half (block row a, block column b) is X_ab^T in this layout scaled by
            // beta, so no pass re-reads X.
            if (wave >= 4) {
                for (int f = wave - 4; krec && f < (D / 16) * 2; f += PREP_WAVES - 4)
                    frag_store<OP>(krec, f, lane, frag_colmajor<OP>(L.k, LK, f / 2, f % 2, lane));
            } else {
                // X_bb = (I + N)^{-1} for the strictly lower 16x16 N, as the exact product
                // (I - N)(I + N^2)(I + N^4)(I + N^8) (N^16 = 0); each matrix is kept with its transpose.
                const int bb = wave;
                const float* blk = &L.b.ax[(16 * bb) * LDF + 16 * bb];
                const f4_t rowv = *reinterpret_cast<const f4_t*>(&blk[li * LDF + 4 * lq]);
                f4_t n, nt, eye;  // lane (j, q) element r: N[4q + r][j], N^T[4q + r][j], I
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * lq + r;
                    n[r] = row > li ? blk[row * LDF + li] : 0.f;  // entries on and above the diagonal are stale
                    nt[r] = li > row ? rowv[r] : 0.f;
                    eye[r] = row == li ? 1.f : 0.f;
                }
                const f4_t z = {0, 0, 0, 0};
                const f4_t n2 = mm16(nt, n, z), n2t = mm16(n, nt, z);
                const f4_t n4 = mm16(n2t, n2, z), n4t = mm16(n2, n2t, z);
                const f4_t n8 = mm16(n4t, n4, z);
                const f4_t m = eye - n, mt = eye - nt;
                const f4_t p1 = mm16(mt, n2, m), p1t = mm16(n2, mt, mt);
                const f4_t p2 = mm16(p1t, n4, p1), p2t = mm16(n4, p1t, p1t);
                const f4_t x = mm16(p2t, n8, p2), xt = mm16(n8, p2t, p2t);
                // 3b reads X_00, X_11, X_22 and X_11^T, X_22^T, X_33^T (slots 0..5 above the diagonal)
                if (bb < 3) *reinterpret_cast<f4_t*>(prep_xslot(L.b.ax, bb, li, lq)) = x;
                if (bb > 0) *reinterpret_cast<f4_t*>(prep_xslot(L.b.ax, bb + 2, li, lq)) = xt;
                f4_t tv = xt * *reinterpret_cast<const f4_t*>(&L.bt[16 * bb + 4 * lq]);
#pragma unroll
                for (int r = 0; r < 4; ++r) tv[r] = 4 * lq + r <= li ? tv[r] : 0.f;  // X_bb is lower triangular
                store_part<OP>(L.t, 2 * bb + (bb >> 1), bb & 1, lane, tv);
            }
            lds_barrier();
            if (wave < 6) {
                // A_ij^T in accumulator layout: A_ij row-major at [16 i + j'][16 j + 4q + r]
                auto at = [&](int i, int j) {
                    return *reinterpret_cast<const f4_t*>(&L.b.ax[(16 * i + li) * LDF + 16 * j + 4 * lq]);
                };
                auto xs = [&](int s) { return *reinterpret_cast<const f4_t*>(prep_xslot(L.b.ax, s, li, lq)); };
                const f4_t z = {0, 0, 0, 0};
                int a, b;  // the block this wave forms
                f4_t res;  // (X_aa sum)^T in accumulator layout, that is -X_ab^T
                if (wave == 0) {          // X_10 = -X_11 A_10 X_00
                    a = 1; b = 0;
                    res = mm16(mm16(at(1, 0), xs(0), z), xs(3), z);
                } else if (wave == 1) {   // X_21 = -X_22 A_21 X_11
                    a = 2; b = 1;
                    res = mm16(mm16(at(2, 1), xs(1), z), xs(4), z);
                } else if (wave == 2) {   // X_32 = -X_33 A_32 X_22
                    a = 3; b = 2;
                    res = mm16(mm16(at(3, 2), xs(2), z), xs(5), z);
                } else if (wave == 3) {   // X_20 = -X_22 (A_20 X_00 + A_21 X_10)
                    a = 2; b = 0;
                    const f4_t x00 = xs(0);
                    const f4_t x10 = -mm16(xs(3), mm16(at(1, 0), x00, z), z);
                    res = mm16(mm16(at(2, 1), x10, mm16(at(2, 0), x00, z)), xs(4), z);
                } else if (wave == 4) {   // X_31 = -X_33 (A_31 X_11 + A_32 X_21)
                    a = 3; b = 1;
                    const f4_t x11 = xs(1);
                    const f4_t x21 = -mm16(xs(4), mm16(at(2, 1), x11, z), z);
                    res = mm16(mm16(at(3, 2), x21, mm16(at(3, 1), x11, z)), xs(5), z);
                } else {                  // X_30 = -X_33 (A_30 X_00 + A_31 X_10 + A_32 X_20)
                    a = 3; b = 0;
                    const f4_t x00 = xs(0), x22t = xs(4);
                    const f4_t x10 = -mm16(xs(3), mm16(at(1, 0), x00, z), z);
                    const f4_t x20 = -mm16(x22t, mm16(at(2, 1), x10, mm16(at(2, 0), x00, z)), z);
                    res = mm16(mm16(at(3, 2), x20, mm16(at(3, 1), x10, mm16(at(3, 0), x00, z))), xs(5), z);
                }
                store_part<OP>(L.t, 2 * a + (b >> 1), b & 1, lane,
                               -res * *reinterpret_cast<const f4_t*>(&L.bt[16 * b + 4 * lq]));
            } else {
                // the halves of T above the diagonal: fragment 0 part 1, fragments 1 and 3, fragment 5 part 1
                for (int h = wave - 6; h < 6; h += 2) {
                    const int f = h == 0 ? 0 : h <= 2 ? 1 : h <= 4 ? 3 : 5;
                    const int part = (h == 0 || h == 2 || h == 4 || h == 5) ? 1 : 0;
                    store_part<OP>(L.t, f, part, lane, f4_t{0.f, 0.f, 0.f, 0.f});
                }
            }
            lds_barrier();

            // ---- 4. values to LDS (region b) ---------------------------------------------------
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int idx = tid + PREP_THREADS * it, t = idx / PER_TOK, pc = idx % PER_TOK;
                float vx[8];
                unpack8<IN_BF16>(in.v[it], vx);
                if (t >= cnt) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) vx[e] = 0.f;
                }
                store8<OP>(L.b.v + t * LK + 8 * pc, vx);
            }
            if (nxt) in.load_v(v, nx_tok0, T, h_v, nx_h);
            lds_barrier();

            // ---- 5. Ut = T V and Ot = P Ut (fp32 accumulator tiles) --------------------------------
            OP* urec = reinterpret_cast<OP*>(rec + RC::U);
            OP* orec = reinterpret_cast<OP*>(rec + RC::O);
            for (int nb = wave; nb < D / 16; nb += PREP_WAVES) {
                const Frag<OP> fv0 = frag_colmajor<OP>(L.b.v, LK, nb, 0, lane);
                const Frag<OP> fv1 = frag_colmajor<OP>(L.b.v, LK, nb, 1, lane);
                f4_t ut[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    ut[mb] = f4_t{0, 0, 0, 0};
                    mma(ut[mb], frag_stored<OP>(L.t, mb * 2 + 0, lane), fv0);
                    mma(ut[mb], frag_stored<OP>(L.t, mb * 2 + 1, lane), fv1);
                    store4<OP>(urec + ((size_t)(nb * 4 + mb) * WAVE + lane) * 4, ut[mb]);
                }
                const Frag<OP> fu0 = frag_from_acc<OP>(ut[0], ut[1]);
                const Frag<OP> fu1 = frag_from_acc<OP>(ut[2], ut[3]);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    f4_t ot = {0, 0, 0, 0};
                    mma(ot, frag_stored<OP>(L.p, mb * 2 + 0, lane), fu0);
                    mma(ot, frag_stored<OP>(L.p, mb * 2 + 1, lane), fu1);
                    store4<OP>(orec + ((size_t)(nb * 4 + mb) * WAVE + lane) * 4, ot);
                }
            }
            lds_barrier();  // the values are no longer read

            // ---- 6. W^T = (diag(gam c) K)^T T^T: the scan's -W fragments, and -W row-major in LDS -----
            // Units (kb, tb): d-blocks 2kb, 2kb+1 and token block tb; a wave's units share kb for d = 128.
            OP* wrec = reinterpret_cast<OP*>(rec + RC::W);
            OP* qrec = reinterpret_cast<OP*>(rec + RC::Q);
            constexpr int UPW = (D / 32) * 4 / PREP_WAVES;  // units per wave
            {
                int cur_kb = -1;
                Frag<OP> aw[2][2];
                for (int uu = 0; uu < UPW; ++uu) {
                    const int unit = wave * UPW + uu, kb = unit / 4, tb = unit % 4;
                    if (kb != cur_kb) {
                        cur_kb = kb;
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                            for (int kk = 0; kk < 2; ++kk) {
                                Frag<OP> f = frag_colmajor<OP>(L.k, LK, 2 * kb + s2, kk, lane);
#pragma unroll
                                for (int e = 0; e < 8; ++e)
                                    frag_set(f, e, frag_get(f, e) * L.gck[32 * kk + 4 * lq + (e & 3) + 16 * (e >> 2)]);
                                aw[s2][kk] = f;
                            }
                    }
                    f4_t acc[2];
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        acc[s2] = f4_t{0, 0, 0, 0};
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk) mma(acc[s2], aw[s2][kk], frag_stored<OP>(L.t, tb * 2 + kk, lane));
                    }
                    // lane (j, q): acc[s2][r] = W[token 16tb + j][d 16(2kb + s2) + 4q + r]
                    Frag<OP> fw;
#pragma unroll
                    for (int e = 0; e < 4; ++e) { frag_set(fw, e, -acc[0][e]); frag_set(fw, e + 4, -acc[1][e]); }
                    frag_store<OP>(wrec, tb * (D / 32) + kb, lane, fw);
                    const int tok = 16 * tb + li;
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) store4<OP>(L.b.w + tok * LK + 16 * (2 * kb + s2) + 4 * lq, -acc[s2]);
                }
            }
            lds_barrier();  // -W complete in LDS

            // ---- 7. Qt^T = (diag(gam cq) Q)^T + (-W)^T P^T: the scan's Qt fragments ----------------
            {
                int cur_kb = -1;
                Frag<OP> aw[2][2];
                for (int uu = 0; uu < UPW; ++uu) {
                    const int unit = wave * UPW + uu, kb = unit / 4, tb = unit % 4;
                    if (kb != cur_kb) {
                        cur_kb = kb;
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                            for (int kk = 0; kk < 2; ++kk) aw[s2][kk] = frag_colmajor<OP>(L.b.w, LK, 2 * kb + s2, kk, lane);
                    }
                    const int tok = 16 * tb + li;
                    const float gq = L.gcq[tok];
                    f4_t acc[2];
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const OP* qr = L.q + tok * LK + 16 * (2 * kb + s2) + 4 * lq;
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[s2][r] = (float)qr[r] * gq;
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk) mma(acc[s2], aw[s2][kk], frag_stored<OP>(L.p, tb * 2 + kk, lane));
                    }
                    Frag<OP> fq;
#pragma unroll
                    for (int e = 0; e < 4; ++e) { frag_set(fq, e, acc[0][e]); frag_set(fq, e + 4, acc[1][e]); }
                    frag_store<OP>(qrec, tb * (D / 32) + kb, lane, fq);
                }
            }

            // ---- 8. s_t = exp(G_n - G_t) c_t and gamma_n -------------------------------------------
            if (tid < CHUNK) {
                if constexpr (sizeof(GT) == 4) {
                    const float Gn = L.G[max(cnt - 1, 0)];
                    reinterpret_cast<float*>(rec + RC::S)[tid] = (tid < cnt) ? __expf(Gn - L.G[tid]) * L.ck[tid] : 0.f;
                    if (tid == 0) reinterpret_cast<float*>(rec + RC::M)[0] = __expf(Gn);
                } else {
                    const GT Gn = L.G[max(cnt - 1, 0)];
                    reinterpret_cast<float*>(rec + RC::S)[tid] =
                        (tid < cnt) ? __expf((float)(Gn - L.G[tid])) * L.ck[tid] : 0.f;
                    if (tid == 0) reinterpret_cast<float*>(rec + RC::M)[0] = __expf((float)Gn);
                }
            }

            lds_barrier();  // LDS is reused by the next task
        }
        tok0 = ntok0;
        nt = nnt;
        live = nlive;
    }
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---- block-form work for bf16 inputs: a k-head's v-heads in pairs -------------------------
// One workgroup per compute unit takes a run of items (block slot, k-head,
// pair of the k-head's v-heads) and computes both v-heads' records together,
// so that every phase has work for all eight compute waves and the raw Gram
// products K K^T and Q K^T are formed once per item (only the decay masks,
// beta and the norm factors differ between the two v-heads).
//
// Two loader waves copy each item's raw bf16 q, k, v tiles and its g, beta
// into LDS with direct global-to-LDS loads while the eight compute waves work
// on the previous item.  The compute waves issue no global loads, only
// record stores: the memory counter that a wave waits on covers its loads and
// its stores alike, so a wave that both loaded inputs and wrote records would
// wait for its record stores to drain before each item.
//   P2a waves 0, 1: the diagonal blocks of K K^T and Q Q^T (bf16 matrix cores
//       on the raw inputs), whose diagonals give the norm factors, then G
//       (cumulative log-decay) and the per-token exponent terms of v-head
//       `wave`; waves 2..5: the raw off-diagonal K K^T and the Q K^T tiles;
//       waves 6, 7: the raw diagonal K K^T tiles.
//   P2b decay masks: A_ij^T tiles (i > j blocks), P fragments, and the diagonal
//       blocks N_bb of A, which waves 6, 7 invert by forward substitution on
//       the vector unit (one lane per column of a block).
//   P4  the six blocks of X = (I + A)^{-1} below the diagonal (fp32 matrix
//       cores), written as T = X diag(beta) fragments.
//   P5  Ut = T V and Ot = P Ut; -W = -T diag(gamma c) K; the key record
//       (normalised keys, fp16) from the same key fragments.
//   P6  Qt = diag(gamma c_q) Q - P W (q is double-buffered).
// Decay ratios are exp2(r_i - c_j) with r_i = G_i log2(e) + log2(beta_i c_i)
// and c_j = G_j log2(e) - log2(c_j); only entries with i >= j are kept, so
// the exponent carries exp(G_i - G_j) <= 1.
// Raw tiles are stored unpadded, rows of D bf16, with the 16-byte units of
// row r permuted by XOR with (r mod units per row), so that the reads of a
// column or of 16 rows at one column spread over the LDS banks.
constexpr float LOG2E_F = 1.4426950408889634f;
constexpr int PAIR_COMPUTE_WAVES = 8, PAIR_LOADER_WAVES = 2;
constexpr int PAIR_THREADS = (PAIR_COMPUTE_WAVES + PAIR_LOADER_WAVES) * WAVE;

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef short s4v_t __attribute__((ext_vector_type(4)));
typedef _Float16 h4v_t __attribute__((ext_vector_type(4)));

struct PairMeta {
    int32_t tok0, nt, live, pad;
};

template <int D, int NH>
struct PairLds {
    static constexpr int LK = D + 8;    // row stride of the fp16 -W tile
    static constexpr int XS = 20;       // row stride of 16 x 16 fp32 blocks
    uint16_t kraw[CHUNK * D];           // raw bf16 keys (swizzled rows)
    uint16_t vraw[NH][CHUNK * D];       // raw bf16 values
    uint16_t qraw[2][CHUNK * D];        // raw bf16 queries, by item parity
    float gb[2][NH][2][CHUNK];          // g and beta of the v-heads, by item parity
    union {
        struct {
            float a[NH][6][WAVE * 4];   // A_ij^T (block i > j) in accumulator layout
            float nb[NH][4][16 * XS];   // diagonal blocks N_bb of A, row-major
            float xd[NH][4][16 * XS];   // X_bb = (I + N_bb)^{-1}, column-major [col][row]
        } s;
        _Float16 w[NH][CHUNK * LK];     // -W [token][d]
    } aw;
    _Float16 t[NH][CHUNK * CHUNK];      // T = X diag(beta), fragment-major
    _Float16 p[NH][CHUNK * CHUNK];      // P, fragment-major
    float cn[2][2 * CHUNK];             // norm factors c_k, c_q (one copy per wave 0, 1)
    float ra[NH][CHUNK], rq[NH][CHUNK], cb[NH][CHUNK];  // exponent terms (above)
    float gck[NH][CHUNK], gcq[NH][CHUNK], bt[NH][CHUNK];
    PairMeta meta[2];
    int zero;  // holds 0 (see chunk_prep_pair_kernel)
};

template <int D, int NH>
constexpr size_t pair_lds_bytes() { return sizeof(PairLds<D, NH>); }

// Slot of the off-diagonal block (i, j), i > j: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
__device__ __forceinline__ constexpr int aslot(int i, int j) { return i * (i - 1) / 2 + j; }

// Byte offset of the 16-byte unit u of row r in a swizzled raw tile of D bf16 per row.
template <int D>
__device__ __forceinline__ int raw_unit(int r, int u) {
    constexpr int UPR = D / 8;
    return r * (D * 2) + ((u ^ (r & (UPR - 1))) << 4);
}

// Row fragment (8 consecutive d of one token) of a raw tile, for products whose two
// operands are both read this way (the Gram products): lane (i, q) holds
// M[16 rb + i][32 kb + 8 q + e].
template <int D>
__device__ __forceinline__ bf8_t raw_row8(const uint16_t* M, int rb, int kb, int lane) {
    const int r = 16 * rb + (lane & 15), u = 4 * kb + (lane >> 4);
    return *reinterpret_cast<const bf8_t*>(reinterpret_cast<const char*>(M) + raw_unit<D>(r, u));
}

__device__ __forceinline__ void mma_bf16(f4_t& acc, const bf8_t& a, const bf8_t& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// Column fragment of a raw tile as fp32 (the layout of frag_colmajor): the
// contraction runs down the rows 32 kb + (4q + e) for e < 4 and
// 32 kb + 16 + 4q + (e - 4) for e >= 4, at column 16 cb + (lane % 16).  Two
// transposing reads (ds_read_b64_tr_b16) of the swizzled rows.
template <int D>
__device__ __forceinline__ void raw_col(const uint16_t* M, int cb, int kb, int lane, float x[8]) {
    typedef __attribute__((address_space(3))) s4v_t* lds_s4;
    const int s = lane & 15, q = lane >> 4;
    const int r = 32 * kb + 4 * q + (s >> 2), col = 16 * cb + 4 * (s & 3);
    const char* base = reinterpret_cast<const char*>(M);
    const int o0 = raw_unit<D>(r, col >> 3) + ((col & 7) << 1);
    const int o1 = raw_unit<D>(r + 16, col >> 3) + ((col & 7) << 1);
    const s4v_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(base + o0));
    const s4v_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(base + o1));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = __uint_as_float((uint32_t)(uint16_t)a[e] << 16);
        x[e + 4] = __uint_as_float((uint32_t)(uint16_t)b[e] << 16);
    }
}

template <int D, int NH>
__global__ __launch_bounds__(PAIR_THREADS, 1) void chunk_prep_pair_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const SeqInfo* __restrict__ info,
    const int32_t* __restrict__ slot_seq, int T, int h_k, int h_v, int l2norm, float scale,
    char* __restrict__ recs, char* __restrict__ krecs, int slots, int items_per_wg) {
    using OP = _Float16;
    using RC = Rec<D, OP>;
    using LT = PairLds<D, NH>;
    constexpr int LK = LT::LK, XS = LT::XS;
    constexpr int NKB = D / 32;       // contraction blocks over d
    extern __shared__ __align__(16) char smem_raw[];
    LT& L = *reinterpret_cast<LT*>(smem_raw);
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int li = lane & 15, lq = lane >> 4;
    const int ratio = h_v / h_k, pairs = ratio / NH;
    const int per_slot = h_k * pairs;
    const int items = slots * per_slot;
    const int i0 = blockIdx.x * items_per_wg, i1 = min(items, i0 + items_per_wg);
    if (i0 >= i1) return;
    auto heads_of = [&](int item, int& hk, int& pr) {
        hk = (item / pairs) % h_k;
        pr = item % pairs;
        return hk * ratio + pr * NH;
    };

    if (wave >= PAIR_COMPUTE_WAVES) {
        // ------------------------------ loader waves ------------------------------
        // Item i + 1's copies go out while item i is computed, each into a buffer that
        // is free by then: q, g and beta (double-buffered) after B1; k (read up to P5)
        // and the first half of v after B5; the second half of v after B6.  k, q, g and
        // beta must have landed by the next B1, v by the next B4.  Every item issues the
        // same number of loads (a dead item loads token 0), so the explicit vmcnt counts
        // below hold: loads complete in issue order.
        typedef __attribute__((address_space(3))) void* lds_ptr;
        const int lw = wave - PAIR_COMPUTE_WAVES;
        constexpr int RPI = 1024 / (2 * D);           // rows per direct load
        constexpr int UPR = D / 8;                    // 16-byte units per row
        constexpr int NL = CHUNK / RPI;               // loads per tile
        constexpr int PER = NL / PAIR_LOADER_WAVES;   // loads per tile and loader wave
        constexpr int GB = 2 * NH / PAIR_LOADER_WAVES > 0 ? 2 * NH / PAIR_LOADER_WAVES : 1;  // g/beta loads per wave
        constexpr int VH = NH * PER / 2 > 0 ? NH * PER / 2 : 1;  // loads per half of v, per wave
        static_assert(NL % PAIR_LOADER_WAVES == 0 && (NH * PER) % 2 == 0, "copy split");
        auto meta_of = [&](int item) {
            PairMeta m{0, 0, 0, 0};
            const int slot = item / per_slot;
            if (slot_seq) {
                const int n = slot_seq[slot];
                if (n >= 0) {
                    const SeqInfo si = info[n];
                    const int j = slot - si.slot_base;
                    m.tok0 = si.begin + j * CHUNK;
                    m.nt = min(CHUNK, si.len - j * CHUNK);
                    m.live = 1;
                }
            } else {
                m.tok0 = slot * CHUNK;
                m.nt = min(CHUNK, T - slot * CHUNK);
                m.live = 1;
            }
            return m;
        };
        // one direct load (64 lanes x 16 bytes = RPI rows) of row group m4 of a tile:
        // the LDS slot of unit p in row r holds the global unit p ^ (r mod UPR)
        auto tile_load = [&](const uint16_t* base, size_t row_stride, int tok0, uint16_t* dst, int m4) {
            const int r = m4 * RPI + lane / UPR, p = lane % UPR;
            const int u = p ^ (r & (UPR - 1));
            const size_t tt = (size_t)min(tok0 + r, T - 1);
            __builtin_amdgcn_global_load_lds(base + tt * row_stride + 8 * u, (lds_ptr)(dst + m4 * 512), 16, 0, 0);
        };
        auto issue_qgb = [&](int item, int tok0, int par) {  // PER + GB loads
            int hk, pr;
            const int h0 = heads_of(item, hk, pr);
            for (int i = 0; i < PER; ++i)
                tile_load(reinterpret_cast<const uint16_t*>(q) + (size_t)hk * D, (size_t)h_k * D, tok0, L.qraw[par],
                          lw + PAIR_LOADER_WAVES * i);
            for (int i = 0; i < GB; ++i) {
                const int x = lw + PAIR_LOADER_WAVES * i;  // (head, g or beta)
                const int j = min(x >> 1, NH - 1);
                const size_t tg = (size_t)min(tok0 + lane, T - 1) * h_v + h0 + j;
                const float* src = (x & 1) ? beta + tg : g + tg;
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)&L.gb[par][j][x & 1][0], 4, 0, 0);
            }
        };
        auto issue_k = [&](int item, int tok0) {  // PER loads
            int hk, pr;
            heads_of(item, hk, pr);
            for (int i = 0; i < PER; ++i)
                tile_load(reinterpret_cast<const uint16_t*>(k) + (size_t)hk * D, (size_t)h_k * D, tok0, L.kraw,
                          lw + PAIR_LOADER_WAVES * i);
        };
        auto issue_v = [&](int item, int tok0, int half) {  // VH loads
            int hk, pr;
            const int h0 = heads_of(item, hk, pr);
            for (int i = 0; i < VH; ++i) {
                const int x = half * VH + i;  // (head, row group) pairs of this wave
                const int j = x / PER, m4 = lw + PAIR_LOADER_WAVES * (x % PER);
                tile_load(reinterpret_cast<const uint16_t*>(v) + (size_t)(h0 + j) * D, (size_t)h_v * D, tok0,
                          L.vraw[j], m4);
            }
        };
        int par = 0;
        PairMeta m = meta_of(i0);
        if (lw == 0 && lane == 0) L.meta[0] = m;
        issue_qgb(i0, m.live ? m.tok0 : 0, 0);
        issue_k(i0, m.live ? m.tok0 : 0);
        issue_v(i0, m.live ? m.tok0 : 0, 0);
        issue_v(i0, m.live ? m.tok0 : 0, 1);
        wait_vmcnt<0>();
        for (int item = i0; item < i1; ++item, par ^= 1) {
            const bool more = item + 1 < i1;
            const PairMeta mn = more ? meta_of(item + 1) : PairMeta{0, 0, 0, 0};
            const int ntok0 = mn.live ? mn.tok0 : 0;
            lds_barrier();  // B1
            if (more) {
                if (lw == 0 && lane == 0) L.meta[par ^ 1] = mn;
                issue_qgb(item + 1, ntok0, par ^ 1);
            }
            lds_barrier();  // B2
            lds_barrier();  // B3
            if (item > i0) {  // this item's v has landed (issued before the next item's q, g, beta)
                if (more) wait_vmcnt<PER + GB>();
                else wait_vmcnt<0>();
            }
            lds_barrier();  // B4
            lds_barrier();  // B5: k and v are no longer read
            if (more) {
                issue_k(item + 1, ntok0);
                issue_v(item + 1, ntok0, 0);
            }
            lds_barrier();  // B6
            if (more) {
                issue_v(item + 1, ntok0, 1);
                wait_vmcnt<2 * VH>();  // the next item's q, g, beta and k have landed
            }
        }
        return;
    }

    // ------------------------------ compute waves ------------------------------
    if (tid == 0) L.zero = 0;
    int par = 0;
    for (int item = i0; item < i1; ++item, par ^= 1) {
        const int slot = item / per_slot;
        int hk, pr;
        const int h0 = heads_of(item, hk, pr);
        lds_barrier();  // B1: this item's raw inputs and meta are in LDS
        // Lane indices re-derived through a volatile LDS read of 0: left loop-invariant,
        // the compiler hoists the per-lane LDS address arithmetic of every phase out of
        // the item loop and runs out of registers (the value is uniform over the wave).
        const int lane = (threadIdx.x + *(volatile __attribute__((address_space(3))) int*)(&L.zero)) % WAVE;
        const int li = lane & 15, lq = lane >> 4;
        const PairMeta meta = L.meta[par];
        const bool live = meta.live != 0;
        const int cnt = meta.nt;
        const uint16_t* qr = L.qraw[par];

        // ---- P2a ------------------------------------------------------------------------------
        f4_t acc[4];
        if (live) {
            if (wave < 2) {
                // diagonal blocks of K K^T (b = 0..3) and Q Q^T (b = 4..7); the diagonal of
                // each is the squared norm of its 16 tokens
                float* cn = L.cn[wave];
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const uint16_t* M = b < 4 ? L.kraw : qr;
                    f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        const bf8_t x = raw_row8<D>(M, b & 3, kb, lane);
                        mma_bf16(d, x, x);
                    }
                    // lane (j, q) holds rows 4q + r of column j: the diagonal is r = j - 4q
                    if ((li >> 2) == lq) {
                        const float ss = d[li & 3];
                        const float mul = b < 4 ? 1.0f : scale;
                        cn[16 * b + li] = l2norm ? mul * rsqrtf(ss + 1e-6f) : mul;
                    }
                }
                if (wave < NH) {
                    const int hh = wave;
                    const bool tl = lane < cnt;
                    const float ckv = tl ? cn[lane] : 0.f, cqv = tl ? cn[CHUNK + lane] : 0.f;
                    const float gl = wave_inclusive_sum(tl ? L.gb[par][hh][0][lane] : 0.f) * LOG2E_F;
                    const float bv = tl ? L.gb[par][hh][1][lane] : 0.f;
                    L.ra[hh][lane] = gl + __builtin_amdgcn_logf(bv * ckv);
                    L.rq[hh][lane] = gl + __builtin_amdgcn_logf(cqv);
                    L.cb[hh][lane] = gl - __builtin_amdgcn_logf(ckv);
                    L.bt[hh][lane] = bv;
                    const float gam = __builtin_amdgcn_exp2f(gl);
                    L.gck[hh][lane] = gam * ckv;
                    L.gcq[hh][lane] = gam * cqv;
                    const float gln = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), max(cnt - 1, 0)));
                    char* rec = recs + ((size_t)slot * h_v + h0 + hh) * RC::BYTES;
                    reinterpret_cast<float*>(rec + RC::S)[lane] = tl ? __builtin_amdgcn_exp2f(gln - gl) : 0.f;
                    if (lane == 0) reinterpret_cast<float*>(rec + RC::M)[0] = __builtin_amdgcn_exp2f(gln);
                }
            } else if (wave < 6) {
                // tiles u = wave - 2 + 4m: u < 6 the off-diagonal K K^T block of slot u, computed
                // as K_j K_i^T so that lane (j', q) holds A_ij^T[4q + r][j']; u >= 6 the tile
                // K_nb Q_mb^T, which is this lane's half of P's fragment (mb, nb / 2).
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int u = wave - 2 + 4 * m;
                    acc[m] = f4_t{0.f, 0.f, 0.f, 0.f};
                    if (u < 6) {
                        const int bi = u >= 3 ? 3 : (u >= 1 ? 2 : 1), bj = u - bi * (bi - 1) / 2;
#pragma unroll
                        for (int kb = 0; kb < NKB; ++kb)
                            mma_bf16(acc[m], raw_row8<D>(L.kraw, bj, kb, lane), raw_row8<D>(L.kraw, bi, kb, lane));
                    } else {
                        const int tl = u - 6;
                        const int mb = (tl >= 6) ? 3 : (tl >= 3) ? 2 : (tl >= 1) ? 1 : 0, nb = tl - mb * (mb + 1) / 2;
#pragma unroll
                        for (int kb = 0; kb < NKB; ++kb)
                            mma_bf16(acc[m], raw_row8<D>(L.kraw, nb, kb, lane), raw_row8<D>(qr, mb, kb, lane));
                    }
                }
            } else if (wave - 6 < NH) {
                // the raw diagonal blocks K_b K_b^T (symmetric): lane (j', q) holds (K K^T)[16b + 4q + r][16b + j']
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    acc[b] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        const bf8_t x = raw_row8<D>(L.kraw, b, kb, lane);
                        mma_bf16(acc[b], x, x);
                    }
                }
            }
        }
        lds_barrier();  // B2

        // ---- P2b ------------------------------------------------------------------------------
        if (live) {
            if (wave < 2) {
                // zero halves: P above the diagonal (6 tiles), T above the diagonal (6 halves)
                for (int hh = 0; hh < NH; ++hh) {
                    for (int x = wave; x < 12; x += 2) {
                        const f4_t z = {0.f, 0.f, 0.f, 0.f};
                        if (x < 6) {
                            const int nb = (x >= 3) ? 3 : (x >= 1) ? 2 : 1, mb = x - (nb - 1) * nb / 2;
                            store_part<OP>(L.p[hh], mb * 2 + nb / 2, nb % 2, lane, z);
                        } else {
                            const int h = x - 6;
                            const int f = h == 0 ? 0 : h <= 2 ? 1 : h <= 4 ? 3 : 5;
                            const int part = (h == 0 || h == 2 || h == 4 || h == 5) ? 1 : 0;
                            store_part<OP>(L.t[hh], f, part, lane, z);
                        }
                    }
                }
            } else if (wave < 6) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int u = wave - 2 + 4 * m;
                    if (u < 6) {
                        const int bi = u >= 3 ? 3 : (u >= 1 ? 2 : 1), bj = u - bi * (bi - 1) / 2;
#pragma unroll
                        for (int hh = 0; hh < NH; ++hh) {
                            const float r = L.ra[hh][16 * bi + li];
                            const f4_t c = *reinterpret_cast<const f4_t*>(&L.cb[hh][16 * bj + 4 * lq]);
                            f4_t x;
#pragma unroll
                            for (int e = 0; e < 4; ++e) x[e] = acc[m][e] * __builtin_amdgcn_exp2f(r - c[e]);
                            *reinterpret_cast<f4_t*>(&L.aw.s.a[hh][u][lane * 4]) = x;
                        }
                    } else {
                        const int tl = u - 6;
                        const int mb = (tl >= 6) ? 3 : (tl >= 3) ? 2 : (tl >= 1) ? 1 : 0, nb = tl - mb * (mb + 1) / 2;
                        const int i = 16 * mb + li, c0 = 16 * nb + 4 * lq;
#pragma unroll
                        for (int hh = 0; hh < NH; ++hh) {
                            const float r = L.rq[hh][i];
                            const f4_t c = *reinterpret_cast<const f4_t*>(&L.cb[hh][c0]);
                            f4_t x;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                x[e] = (mb > nb || c0 + e <= i) ? acc[m][e] * __builtin_amdgcn_exp2f(r - c[e]) : 0.f;
                            store_part<OP>(L.p[hh], mb * 2 + nb / 2, nb % 2, lane, x);
                        }
                    }
                }
            } else if (wave - 6 < NH) {
                const int hh = wave - 6;
                // N_bb[j'][4q + r] (strictly lower) from the symmetric raw block, row-major
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float r = L.ra[hh][16 * b + li];
                    const f4_t c = *reinterpret_cast<const f4_t*>(&L.cb[hh][16 * b + 4 * lq]);
                    f4_t x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (4 * lq + e < li) ? acc[b][e] * __builtin_amdgcn_exp2f(r - c[e]) : 0.f;
                    *reinterpret_cast<f4_t*>(&L.aw.s.nb[hh][b][li * XS + 4 * lq]) = x;
                }
                // Forward substitution (I + N) X = I: lane (b, j) computes column j of X_bb,
                // X[i][j] = [i == j] - sum_{m < i} N[i][m] X[m][j].  N's rows are read as
                // broadcasts (the 16 lanes of a block read the same address).
                const int b = lq, j = li;
                const float* Nb = L.aw.s.nb[hh][b];
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float s = (i == j) ? 1.f : 0.f;
#pragma unroll
                    for (int m4 = 0; m4 < i; m4 += 4) {
                        const f4_t nr = *reinterpret_cast<const f4_t*>(&Nb[i * XS + m4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (m4 + e < i) s = fmaf(-nr[e], x[m4 + e], s);
                    }
                    x[i] = s;
                }
                float* xd = L.aw.s.xd[hh][b];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<f4_t*>(&xd[j * XS + 4 * c]) = f4_t{x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]};
                // T's diagonal block: T[16b + i][16b + j] = X[i][j] beta_{16b + j}, element
                // (j % 4) + 4 (b % 2) of lane ((j / 4), i) of fragment (b, b / 2)
                const float bj = L.bt[hh][16 * b + j];
                OP* tf = L.t[hh] + ((size_t)(2 * b + (b >> 1)) * WAVE + (j >> 2) * 16) * 8 + (j & 3) + 4 * (b & 1);
#pragma unroll
                for (int i = 0; i < 16; ++i) tf[i * 8] = (OP)(x[i] * bj);
            }
        }
        lds_barrier();  // B3

        // ---- P4: blocks of X below the diagonal, as T = X diag(beta) fragment halves ----------
        // Matrices in accumulator layout (lane (j, q) holds M[4q + r][j]); mm16(xt, y, c) =
        // c + X Y takes X^T and Y.  T's fragment half (block row a, block column b) is
        // X_ab^T in this layout, times beta of the column.
        if (live) {
            const int hh = wave >> 2;
            if (hh < NH) {
                // roles by wave: head 0 waves 0..3 take roles 3, 2, 0, 1 and head 1 roles 2, 3, 1, 0,
                // so the two waves that share a SIMD (w, w + 4) carry about equal matrix work
                const int role = ((hh ? 0x0132 : 0x1023) >> (4 * (wave & 3))) & 0xf;
                const f4_t z = {0.f, 0.f, 0.f, 0.f};
                auto at = [&](int i, int j) { return *reinterpret_cast<const f4_t*>(&L.aw.s.a[hh][aslot(i, j)][lane * 4]); };
                auto xa = [&](int b) { return *reinterpret_cast<const f4_t*>(&L.aw.s.xd[hh][b][li * XS + 4 * lq]); };
                auto xt = [&](int b) {
                    const float* x = L.aw.s.xd[hh][b];
                    return f4_t{x[(4 * lq) * XS + li], x[(4 * lq + 1) * XS + li], x[(4 * lq + 2) * XS + li],
                                x[(4 * lq + 3) * XS + li]};
                };
                auto put = [&](int a, int b, const f4_t& negxt) {  // negxt = -X_ab^T
                    store_part<OP>(L.t[hh], 2 * a + (b >> 1), b & 1, lane,
                                   -negxt * *reinterpret_cast<const f4_t*>(&L.bt[hh][16 * b + 4 * lq]));
                };
                if (role == 0) {  // X_10 = -X_11 A_10 X_00; X_20 = -X_22 (A_20 X_00 + A_21 X_10)
                    const f4_t x00 = xa(0), x11t = xt(1);
                    const f4_t r = mm16(at(1, 0), x00, z);
                    put(1, 0, mm16(r, x11t, z));
                    const f4_t x10 = -mm16(x11t, r, z);
                    const f4_t y = mm16(at(2, 1), x10, mm16(at(2, 0), x00, z));
                    put(2, 0, mm16(y, xt(2), z));
                } else if (role == 1) {  // X_21 = -X_22 A_21 X_11; X_31 = -X_33 (A_31 X_11 + A_32 X_21)
                    const f4_t x11 = xa(1), x22t = xt(2);
                    const f4_t r = mm16(at(2, 1), x11, z);
                    put(2, 1, mm16(r, x22t, z));
                    const f4_t x21 = -mm16(x22t, r, z);
                    const f4_t y = mm16(at(3, 2), x21, mm16(at(3, 1), x11, z));
                    put(3, 1, mm16(y, xt(3), z));
                } else if (role == 2) {  // X_32 = -X_33 A_32 X_22
                    put(3, 2, mm16(mm16(at(3, 2), xa(2), z), xt(3), z));
                } else {
                    // X_30 = -(X_32 Y_00 + X_33 Y_10), Y_00 = A_20 X_00 + A_21 X_10,
                    // Y_10 = A_30 X_00 + A_31 X_10 (the lower-left 32 x 32 block of X is
                    // -X_lower-right (A_lower-left X_upper-left))
                    const f4_t x00 = xa(0), x33t = xt(3);
                    const f4_t x10 = -mm16(xt(1), mm16(at(1, 0), x00, z), z);
                    const f4_t y00 = mm16(at(2, 1), x10, mm16(at(2, 0), x00, z));
                    const f4_t y10 = mm16(at(3, 1), x10, mm16(at(3, 0), x00, z));
                    const f4_t x32t = -mm16(mm16(at(3, 2), xa(2), z), x33t, z);
                    put(3, 0, mm16(y10, x33t, mm16(y00, x32t, z)));
                }
            }
        }
        lds_barrier();  // B4: T complete; A, N and X no longer read

        // ---- P5: Ut = T V and Ot = P Ut; -W ----------------------------------------------------
        constexpr int WUNITS = NH * NKB * 4, UPW = WUNITS / PAIR_COMPUTE_WAVES > 0 ? WUNITS / PAIR_COMPUTE_WAVES : 1;
        if (live) {
            for (int u = wave; u < NH * (D / 16); u += PAIR_COMPUTE_WAVES) {
                const int hh = u / (D / 16), nb = u % (D / 16);
                char* rec = recs + ((size_t)slot * h_v + h0 + hh) * RC::BYTES;
                OP* urec = reinterpret_cast<OP*>(rec + RC::U);
                OP* orec = reinterpret_cast<OP*>(rec + RC::O);
                Frag<OP> fv[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    float x[8];
                    raw_col<D>(L.vraw[hh], nb, kk, lane, x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) frag_set(fv[kk], e, x[e]);
                }
                f4_t ut[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    ut[mb] = f4_t{0, 0, 0, 0};
                    mma(ut[mb], frag_stored<OP>(L.t[hh], mb * 2 + 0, lane), fv[0]);
                    mma(ut[mb], frag_stored<OP>(L.t[hh], mb * 2 + 1, lane), fv[1]);
                    store4<OP>(urec + ((size_t)(nb * 4 + mb) * WAVE + lane) * 4, ut[mb]);
                }
                const Frag<OP> fu0 = frag_from_acc<OP>(ut[0], ut[1]);
                const Frag<OP> fu1 = frag_from_acc<OP>(ut[2], ut[3]);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    f4_t ot = {0, 0, 0, 0};
                    mma(ot, frag_stored<OP>(L.p[hh], mb * 2 + 0, lane), fu0);
                    mma(ot, frag_stored<OP>(L.p[hh], mb * 2 + 1, lane), fu1);
                    store4<OP>(orec + ((size_t)(nb * 4 + mb) * WAVE + lane) * 4, ot);
                }
            }
            // W^T = (diag(gamma c) K)^T T^T: units (head, kb, tb) with d-blocks 2kb, 2kb + 1 and
            // token block tb; a wave's units share (head, kb)
            int cur = -1;
            Frag<OP> aw[2][2];
            for (int uu = 0; uu < UPW; ++uu) {
                const int unit = wave * UPW + uu;
                if (unit >= WUNITS) break;
                const int hh = unit / (NKB * 4), kb = (unit / 4) % NKB, tb = unit % 4;
                if (unit / 4 != cur) {
                    cur = unit / 4;
                    // the key record (normalised keys, fp16) is written once per k-head, by
                    // the waves that hold the first v-head's (kb, token block 0) units
                    const bool krec_w = pr == 0 && hh == 0 && unit % 4 == 0;
                    OP* krec = reinterpret_cast<OP*>(krecs + ((size_t)slot * h_k + hk) * KeyRec<D, OP>::BYTES);
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk) {
                            float x[8];
                            raw_col<D>(L.kraw, 2 * kb + s2, kk, lane, x);
                            const f4_t s0 = *reinterpret_cast<const f4_t*>(&L.gck[hh][32 * kk + 4 * lq]);
                            const f4_t s1 = *reinterpret_cast<const f4_t*>(&L.gck[hh][32 * kk + 16 + 4 * lq]);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                frag_set(aw[s2][kk], e, x[e] * s0[e]);
                                frag_set(aw[s2][kk], e + 4, x[e + 4] * s1[e]);
                            }
                            if (krec_w) {
                                const f4_t c0 = *reinterpret_cast<const f4_t*>(&L.cn[0][32 * kk + 4 * lq]);
                                const f4_t c1 = *reinterpret_cast<const f4_t*>(&L.cn[0][32 * kk + 16 + 4 * lq]);
                                Frag<OP> fr;
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const int t0 = 32 * kk + 4 * lq + e, t1 = t0 + 16;
                                    frag_set(fr, e, t0 < cnt ? x[e] * c0[e] : 0.f);
                                    frag_set(fr, e + 4, t1 < cnt ? x[e + 4] * c1[e] : 0.f);
                                }
                                frag_store<OP>(krec, (2 * kb + s2) * 2 + kk, lane, fr);
                            }
                        }
                }
                char* rec = recs + ((size_t)slot * h_v + h0 + hh) * RC::BYTES;
                OP* wrec = reinterpret_cast<OP*>(rec + RC::W);
                f4_t a2[2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    a2[s2] = f4_t{0, 0, 0, 0};
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) mma(a2[s2], aw[s2][kk], frag_stored<OP>(L.t[hh], tb * 2 + kk, lane));
                }
                // lane (j, q): a2[s2][r] = W[token 16tb + j][d 16(2kb + s2) + 4q + r]
                Frag<OP> fw;
#pragma unroll
                for (int e = 0; e < 4; ++e) { frag_set(fw, e, -a2[0][e]); frag_set(fw, e + 4, -a2[1][e]); }
                frag_store<OP>(wrec, tb * NKB + kb, lane, fw);
                const int tok = 16 * tb + li;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) store4<OP>(L.aw.w[hh] + tok * LK + 16 * (2 * kb + s2) + 4 * lq, -a2[s2]);
            }
        }
        lds_barrier();  // B5: -W complete in LDS; k and v no longer read

        // ---- P6: Qt^T = (diag(gamma c_q) Q)^T + (-W)^T P^T --------------------------------------
        if (live) {
            int cur = -1;
            Frag<OP> aw[2][2];
            for (int uu = 0; uu < UPW; ++uu) {
                const int unit = wave * UPW + uu;
                if (unit >= WUNITS) break;
                const int hh = unit / (NKB * 4), kb = (unit / 4) % NKB, tb = unit % 4;
                if (unit / 4 != cur) {
                    cur = unit / 4;
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk) aw[s2][kk] = frag_colmajor<OP>(L.aw.w[hh], LK, 2 * kb + s2, kk, lane);
                }
                char* rec = recs + ((size_t)slot * h_v + h0 + hh) * RC::BYTES;
                OP* qrec = reinterpret_cast<OP*>(rec + RC::Q);
                const int tok = 16 * tb + li;
                const float gq = L.gcq[hh][tok];
                f4_t a2[2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    // the raw queries of token tok at d = 16 (2kb + s2) + 4q .. + 3 (8 bytes)
                    const int col = 16 * (2 * kb + s2) + 4 * lq;
                    const uint2 w2 = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(qr) +
                                                                     raw_unit<D>(tok, col >> 3) + ((col & 7) << 1));
                    a2[s2][0] = __uint_as_float(w2.x << 16) * gq;
                    a2[s2][1] = __uint_as_float(w2.x & 0xffff0000u) * gq;
                    a2[s2][2] = __uint_as_float(w2.y << 16) * gq;
                    a2[s2][3] = __uint_as_float(w2.y & 0xffff0000u) * gq;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) mma(a2[s2], aw[s2][kk], frag_stored<OP>(L.p[hh], tb * 2 + kk, lane));
                }
                Frag<OP> fq;
#pragma unroll
                for (int e = 0; e < 4; ++e) { frag_set(fq, e, a2[0][e]); frag_set(fq, e + 4, a2[1][e]); }
                frag_store<OP>(qrec, tb * NKB + kb, lane, fq);
            }
        }
        lds_barrier();  // B6: LDS is reused by the next item
    }
}

// ---- sequential phase -------------------------------------------------------------------
// One workgroup owns RS rows (16 or 32) of one (sequence, v-head) state, so a
// d-wide head has d/RS workgroups.  The rows of S evolve independently.  A
// workgroup has 12 waves.  Waves 0..7 compute; per 64-token block:
//   phase A (contraction over d_k): wave w forms, for token block w % 4, the
//     16 x RS tile of U = Ut - W S^T (w < 4) or of O = Ot + Qt S^T (w >= 4),
//     reading S (as matrix-core operands) from LDS;
//   phase B (contraction over tokens): each wave updates the S^T tiles it
//     owns, S^T <- gamma_n S^T + K^T diag(s) U, reading diag(s) U from LDS.
// The fp32 state stays in registers for the whole sequence, and the compute
// waves issue no global memory operation inside the block loop.
//
// Waves 8..11 copy the block records into a two-slot LDS ring with direct
// global-to-LDS loads and write the outputs.  A wave that issues a vector
// memory operation stalls while the compute unit's memory pipeline is full,
// so only these waves touch global memory, and each barrier interval gives
// them a bounded share of it: the copy of block c + 2 goes out in two halves
// (after the second barrier of block c, and after the first barrier of block
// c + 1) and must have landed by the first barrier of block c + 2.  The
// pipeline therefore always has copies queued while the compute waves work.
constexpr int SCAN_COMPUTE_WAVES = 8, SCAN_LOADER_WAVES = 4;
constexpr int SCAN_THREADS = (SCAN_COMPUTE_WAVES + SCAN_LOADER_WAVES) * WAVE;

template <int D, typename OP, int RS>
struct ScanShape {
    static constexpr int NB = RS / 16;                       // 16-row blocks of the slice
    static constexpr int FRAG_ELEMS = 3 * CHUNK * D;         // -W, Qt, K^T fragments
    static constexpr int UO_ELEMS = 2 * NB * 4 * WAVE * 4;   // Ut, Ot tiles: [Ut|Ot][row block][token block][lane][4]
    static constexpr int SG_FLOATS = CHUNK + 4;              // s_t, then gamma_n
    // direct loads of 1 KiB (64 lanes x 16 bytes), per loader wave
    static constexpr int FRAG_LOADS = FRAG_ELEMS * (int)sizeof(OP) / 1024 / SCAN_LOADER_WAVES;
    static constexpr int UO_LOADS = UO_ELEMS * (int)sizeof(OP) / 1024 / SCAN_LOADER_WAVES;
    static constexpr int PER_WAVE = FRAG_LOADS + UO_LOADS + 1;  // + s_t / gamma_n
    static constexpr int FIRST = PER_WAVE / 2;                  // loads in the first half of a copy
    static constexpr int NTB = (D / 16) * NB;                   // S^T tiles of the slice
    static constexpr int TPW = NTB >= SCAN_COMPUTE_WAVES ? NTB / SCAN_COMPUTE_WAVES : 1;
    static_assert(FRAG_ELEMS * (int)sizeof(OP) % (1024 * SCAN_LOADER_WAVES) == 0, "fragment split");
    static_assert(UO_ELEMS * (int)sizeof(OP) % (1024 * SCAN_LOADER_WAVES) == 0, "tile split");
    static_assert(NTB % SCAN_COMPUTE_WAVES == 0 || NTB < SCAN_COMPUTE_WAVES, "S^T tile split");
};

template <int D, typename OP, int RS>
struct ScanSlot {
    using Sh = ScanShape<D, OP, RS>;
    OP frag[Sh::FRAG_ELEMS];
    OP uo[Sh::UO_ELEMS];
    float sg[Sh::SG_FLOATS];
};

template <int D, typename OP, bool OUT_BF16, int RS>
constexpr size_t scan_lds_bytes() {
    return 2 * sizeof(ScanSlot<D, OP, RS>) + ((D / 32) + 2) * (RS / 16) * WAVE * 8 * sizeof(OP) +
           (size_t)CHUNK * RS * (OUT_BF16 ? 2 : 4);
}



// Loads I0..I1-1 of one loader wave's share of copying a block into a ring
// slot.  In order: the -W and Qt fragments (v-head record) and the K^T
// fragments (k-head record), contiguous in the slot; the slice's Ut and Ot
// tiles (contiguous in the record); s_t / gamma_n.
template <int D, typename OP, int RS, int I0, int I1>
__device__ __forceinline__ void scan_copy(const char* rec, const char* krec, ScanSlot<D, OP, RS>* s, int lw,
                                          int lane, int cb0) {
    using Sh = ScanShape<D, OP, RS>;
    using R = Rec<D, OP>;
    typedef __attribute__((address_space(3))) void* lds_ptr;
    constexpr int WQ = 2 * CHUNK * D * (int)sizeof(OP);         // bytes of -W and Qt
    constexpr int UO_HALF = Sh::NB * 4 * (int)R::TILE;          // bytes of the slice's Ut (or Ot) tiles
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        if (i < Sh::FRAG_LOADS) {
            const int j0 = (lw * Sh::FRAG_LOADS + i) * 1024;  // byte offset of this load in the slot
            const char* src = (j0 < WQ ? rec + j0 : krec + (j0 - WQ)) + lane * 16;
            __builtin_amdgcn_global_load_lds(src, (lds_ptr)(reinterpret_cast<char*>(s->frag) + j0), 16, 0, 0);
        } else if (i < Sh::FRAG_LOADS + Sh::UO_LOADS) {
            const int j0 = (lw * Sh::UO_LOADS + (i - Sh::FRAG_LOADS)) * 1024;  // byte offset in uo
            const char* src = (j0 < UO_HALF ? rec + R::U + j0 : rec + R::O + (j0 - UO_HALF)) +
                              (size_t)cb0 * 4 * R::TILE + lane * 16;
            __builtin_amdgcn_global_load_lds(src, (lds_ptr)(reinterpret_cast<char*>(s->uo) + j0), 16, 0, 0);
        } else if (lane < CHUNK / 4 + 1) {
            // s_t and gamma_n: 17 pieces.  A direct load writes lane l's 16
            // bytes at base + 16 l, so only lanes 0..16 take part.
            const char* src = rec + R::S + (size_t)lane * 16;
            __builtin_amdgcn_global_load_lds(src, (lds_ptr)reinterpret_cast<char*>(s->sg), 16, 0, 0);
        }
    }
}

// MODE 0: the scan.  MODE 1: both parts of a segment's state map, no outputs:
// the first half of the units runs from zero (the affine part B), the second
// half from the identity without Ut (the transition R), so that
// S_end = S_start R + B.  Both halves write state_out at their unit.
template <int D, typename OP, bool OUT_BF16, int RS, int MODE = 0>
__global__ __launch_bounds__(SCAN_THREADS) void chunk_scan_kernel(
    const char* __restrict__ recs, const char* __restrict__ krecs, const SeqInfo* __restrict__ info,
    const float* __restrict__ state_in, float* __restrict__ state_out, void* __restrict__ out,
    char* __restrict__ sink, int units, int T, int h_k, int h_v) {
    using R = Rec<D, OP>;
    using Sh = ScanShape<D, OP, RS>;
    using Slot = ScanSlot<D, OP, RS>;
    constexpr int NB = Sh::NB, SLICES = D / RS, TPW = Sh::TPW;
    constexpr int OB = OUT_BF16 ? 2 : 4;  // bytes per output element
    // Separate arrays: the direct loads target only `ring`, so the loader
    // waves' reads of `sO` need not wait for the loads in flight.
    __shared__ __align__(16) Slot ring[2];
    __shared__ __align__(16) OP sS[(D / 32) * NB * WAVE * 8];  // S^T as B fragments (kb, row block)
    __shared__ __align__(16) OP sU[2 * NB * WAVE * 8];         // diag(s) U as B fragments (kk, row block)
    __shared__ __align__(16) char sO[CHUNK * RS * OB];         // the block's 64 x RS outputs, row-major
    // Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8).
    // The SLICES workgroups of one (sequence, v-head) unit are placed on the
    // same XCD, so they share each block record through that XCD's L2.
    const int xcd = blockIdx.x % 8, m = blockIdx.x / 8;
    const int slice = m % SLICES;
    const int unit = (m / SLICES) * 8 + xcd;  // sequence * h_v + v-head
    if (unit >= units) return;
    // MODE 1: units [units/2, units) are the transition runs of the same segments
    const bool lin = MODE == 1 && unit >= units / 2;
    const int su = lin ? unit - units / 2 : unit;
    const int n = su / h_v, h = su - n * h_v;
    const int tid = threadIdx.x, w = tid / WAVE, lane = tid % WAVE;
    const int j16 = lane & 15, q4 = lane >> 4;
    const int r0 = slice * RS, cb0 = r0 / 16;
    int begin, len, slot0;
    if (info) {
        const SeqInfo si = info[n];
        begin = si.begin; len = si.len; slot0 = si.slot_base;
    } else {
        begin = 0; len = T; slot0 = 0;
    }
    const int nchunks = (len + CHUNK - 1) / CHUNK;
    const int hk = h / (h_v / h_k);
    auto rec_of = [&](int c) { return recs + ((size_t)(slot0 + c) * h_v + h) * R::BYTES; };
    auto krec_of = [&](int c) { return krecs + ((size_t)(slot0 + c) * h_k + hk) * KeyRec<D, OP>::BYTES; };

    if (w >= SCAN_COMPUTE_WAVES) {
        // ------------------------------ loader waves ------------------------------
        constexpr int F = Sh::PER_WAVE, H = Sh::FIRST;
        constexpr int LPR = RS * OB / 16;  // 16-byte pieces per output row
        constexpr int PIECES = CHUNK * LPR;
        constexpr int LT = SCAN_LOADER_WAVES * WAVE;
        const int lw = w - SCAN_COMPUTE_WAVES;
        if (nchunks == 0) return;
        scan_copy<D, OP, RS, 0, F>(rec_of(0), krec_of(0), &ring[0], lw, lane, cb0);
        if (nchunks > 1) {
            scan_copy<D, OP, RS, 0, F>(rec_of(1), krec_of(1), &ring[1], lw, lane, cb0);
            wait_vmcnt<F>();
        } else {
            wait_vmcnt<0>();
        }
        for (int c = 0; c < nchunks; ++c) {
            lds_barrier();  // B1: block c is in slot c % 2
            if (c >= 1 && c + 1 < nchunks) scan_copy<D, OP, RS, H, F>(rec_of(c + 1), krec_of(c + 1), &ring[(c + 1) & 1], lw, lane, cb0);
            lds_barrier();  // B2: slot c % 2 is free; the outputs of block c are in sO
            // outputs: 16 bytes per lane, rows past the block's end go to the sink
            const int tok0 = begin + c * CHUNK, nt = min(CHUNK, len - c * CHUNK);
#pragma unroll
            for (int i = 0; i < (MODE == 0 ? (PIECES + LT - 1) / LT : 0); ++i) {
                const int p = i * LT + lw * WAVE + lane;
                if (PIECES % LT == 0 || p < PIECES) {
                    const int row = p / LPR, col16 = p % LPR;
                    const uint4 val = *reinterpret_cast<const uint4*>(sO + row * RS * OB + col16 * 16);
                    char* dst = row < nt ? reinterpret_cast<char*>(out) +
                                               (((size_t)(tok0 + row) * h_v + h) * D + r0) * OB + col16 * 16
                                         : sink + lane * 16;
                    *reinterpret_cast<uint4*>(dst) = val;
                }
            }
            // Loads complete in issue order, so once no more than H operations
            // are outstanding, every load issued before the last H has landed:
            // all of block c + 1.
            if (c + 2 < nchunks) {
                scan_copy<D, OP, RS, 0, H>(rec_of(c + 2), krec_of(c + 2), &ring[c & 1], lw, lane, cb0);
                wait_vmcnt<H>();
            } else if (c + 1 < nchunks) {
                wait_vmcnt<0>();
            }
        }
        return;
    }

    // ------------------------------ compute waves ------------------------------
    const int which = w >> 2, tb = w & 3;  // phase A: U (which 0) or O (which 1), token block tb
    // S^T tiles owned in phase B: number w*TPW + i -> (mb, nb) = (number / NB, number % NB);
    // lane (j, q) holds S[r0 + 16nb + j][16 mb + 4q + 0..3]
    f4_t St[TPW];
    const size_t sbase = (size_t)unit * D * D;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = w * TPW + i, mb = t / NB, nb = t % NB;
        if (t >= Sh::NTB) break;
        if (lin) {  // identity: S[r][c] = (r == c)
            const int row = r0 + 16 * nb + j16, col = 16 * mb + 4 * q4;
            St[i] = f4_t{row == col ? 1.f : 0.f, row == col + 1 ? 1.f : 0.f, row == col + 2 ? 1.f : 0.f,
                         row == col + 3 ? 1.f : 0.f};
        } else if (state_in) {
            const float4 x = *reinterpret_cast<const float4*>(
                state_in + sbase + (size_t)(r0 + 16 * nb + j16) * D + 16 * mb + 4 * q4);
            St[i] = f4_t{x.x, x.y, x.z, x.w};
        } else {
            St[i] = f4_t{0, 0, 0, 0};
        }
        store_part<OP>(sS, (mb / 2) * NB + nb, mb % 2, lane, St[i]);
    }
    for (int c = 0; c < nchunks; ++c) {
        __syncthreads();  // B1: block c in its slot; S^T fragments complete; sU and sO free
        const Slot& B = ring[c & 1];
        const OP* Ab = B.frag + which * CHUNK * D;  // -W or Qt
        const OP* Kb = B.frag + 2 * CHUNK * D;
        f4_t acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const OP* u = &B.uo[(((which * NB + nb) * 4 + tb) * WAVE + lane) * 4];
            if (lin) {
                acc[nb] = f4_t{0.f, 0.f, 0.f, 0.f};
            } else if constexpr (sizeof(OP) == 2) {
                typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
                const h4_t x = *reinterpret_cast<const h4_t*>(u);
                acc[nb] = f4_t{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
            } else {
                acc[nb] = *reinterpret_cast<const f4_t*>(u);
            }
        }
        if (MODE == 0 || which == 0) {  // O is needed only by the scan itself
#pragma unroll
            for (int kb = 0; kb < D / 32; ++kb) {
                const Frag<OP> a = frag_stored<OP>(Ab, tb * (D / 32) + kb, lane);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) mma(acc[nb], a, frag_stored<OP>(sS, kb * NB + nb, lane));
            }
        }
        Frag<OP> kf[TPW][2];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int mb = (w * TPW + i) / NB;
            if (w * TPW + i >= Sh::NTB) break;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) kf[i][kk] = frag_stored<OP>(Kb, mb * 2 + kk, lane);
        }
        const float gn = B.sg[CHUNK];
        if (which == 0) {
            const f4_t sv = *reinterpret_cast<const f4_t*>(&B.sg[16 * tb + 4 * q4]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) store_part<OP>(sU, (tb / 2) * NB + nb, tb % 2, lane, acc[nb] * sv);
        } else if (MODE == 0) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = (16 * tb + 4 * q4 + r) * RS + 16 * nb + j16;
                    if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(sO)[e] = f32_to_bf16(acc[nb][r]);
                    else reinterpret_cast<float*>(sO)[e] = acc[nb][r];
                }
        }
        __syncthreads();  // B2: diag(s) U and the outputs complete; S^T fragments and slot c % 2 no longer read
        // phase B: S^T <- gamma_n S^T + K^T diag(s) U
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = w * TPW + i, mb = t / NB, nb = t % NB;
            if (t >= Sh::NTB) break;
            St[i] *= gn;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) mma(St[i], kf[i][kk], frag_stored<OP>(sU, kk * NB + nb, lane));
            store_part<OP>(sS, (mb / 2) * NB + nb, mb % 2, lane, St[i]);
        }
    }

    if (state_out) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = w * TPW + i, mb = t / NB, nb = t % NB;
            if (t >= Sh::NTB) break;
            *reinterpret_cast<float4*>(state_out + sbase + (size_t)(r0 + 16 * nb + j16) * D + 16 * mb + 4 * q4) =
                make_float4(St[i][0], St[i][1], St[i][2], St[i][3]);
        }
    }
}

// ---- host launchers ----------------------------------------------------------------------
size_t prefill_record_bytes(int d, bool in_bf16) {
    if (d == 128) return in_bf16 ? Rec<128, _Float16>::BYTES : Rec<128, float>::BYTES;
    return in_bf16 ? Rec<64, _Float16>::BYTES : Rec<64, float>::BYTES;
}

size_t prefill_key_record_bytes(int d, bool in_bf16) {
    if (d == 128) return in_bf16 ? KeyRec<128, _Float16>::BYTES : KeyRec<128, float>::BYTES;
    return in_bf16 ? KeyRec<64, _Float16>::BYTES : KeyRec<64, float>::BYTES;
}

hipError_t launch_plan(const int32_t* cu, int N, int T, int max_slots, void* info, int32_t* slot_seq,
                       hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu, N, T, max_slots,
                       reinterpret_cast<SeqInfo*>(info), slot_seq);
    return hipGetLastError();
}

// Compute units of the current device (cached per device).
int compute_units() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int D, int NH>
static hipError_t launch_prep_pair_t(const void* q, const void* k, const void* v, const float* g,
                                     const float* beta, const void* info, const int32_t* slot_seq,
                                     int slots, int T, int h_k, int h_v, int l2norm, float scale,
                                     char* recs, char* krecs, hipStream_t stream) {
    constexpr size_t lds = pair_lds_bytes<D, NH>();
    static_assert(lds <= 160 * 1024, "chunk_prep_pair LDS budget");
    auto kern = chunk_prep_pair_kernel<D, NH>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // one workgroup per compute unit, each a contiguous run of items
    const int items = slots * h_k * (h_v / h_k / NH), resident = compute_units();
    const int per = (items + resident - 1) / resident;
    const int grid = (items + per - 1) / per;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(PAIR_THREADS), lds, stream, q, k, v, g, beta,
                       reinterpret_cast<const SeqInfo*>(info), slot_seq, T, h_k, h_v, l2norm, scale, recs, krecs,
                       slots, per);
    return hipGetLastError();
}

template <int D, typename OP, bool IB>
static hipError_t launch_prep_t(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const void* info, const int32_t* slot_seq,
                                int slots, int T, int h_k, int h_v, int l2norm, float scale,
                                char* recs, char* krecs, hipStream_t stream) {
    constexpr size_t lds = prep_lds_bytes<D, OP>();
    static_assert(lds <= 160 * 1024, "chunk_prep LDS budget");
    auto kern = chunk_prep_kernel<D, OP, IB>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // One run of (block slot, k-head) items per resident workgroup.
    constexpr int per_cu = 2 * lds <= 160 * 1024 ? 2 : 1;
    const int items = slots * h_k, resident = per_cu * compute_units();
    const int per = (items + resident - 1) / resident;
    const int grid = (items + per - 1) / per;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(PREP_THREADS), lds, stream, q, k, v, g, beta,
                       reinterpret_cast<const SeqInfo*>(info), slot_seq, T, h_k, h_v, l2norm, scale, recs, krecs,
                       slots, per);
    return hipGetLastError();
}

hipError_t launch_prep(int d, bool in_bf16, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const void* info, const int32_t* slot_seq,
                       int slots, int T, int h_k, int h_v, int l2norm, float scale, void* recs,
                       void* krecs, hipStream_t stream) {
    char* r = reinterpret_cast<char*>(recs);
    char* kr = reinterpret_cast<char*>(krecs);
    const bool pair = (h_v / h_k) % 2 == 0;
    if (d == 128 && in_bf16)
        return pair ? launch_prep_pair_t<128, 2>(q, k, v, g, beta, info, slot_seq, slots, T, h_k, h_v, l2norm, scale, r, kr, stream)
                    : launch_prep_pair_t<128, 1>(q, k, v, g, beta, info, slot_seq, slots, T, h_k, h_v, l2norm, scale, r, kr, stream);
    if (d == 64 && in_bf16)
        return pair ? launch_prep_pair_t<64, 2>(q, k, v, g, beta, info, slot_seq, slots, T, h_k, h_v, l2norm, scale, r, kr, stream)
                    : launch_prep_pair_t<64, 1>(q, k, v, g, beta, info, slot_seq, slots, T, h_k, h_v, l2norm, scale, r, kr, stream);
    if (d == 64 && !in_bf16)
        return launch_prep_t<64, float, false>(q, k, v, g, beta, info, slot_seq, slots, T, h_k, h_v, l2norm, scale, r, kr, stream);
    return hipErrorInvalidValue;
}

template <int D, typename OP, bool OB, int RS, int MODE = 0>
static hipError_t launch_scan_t(const void* recs, const void* krecs, const void* info, const float* s_in,
                                float* s_out, void* out, void* sink, int units, int T, int h_k, int h_v,
                                hipStream_t stream) {
    static_assert(scan_lds_bytes<D, OP, OB, RS>() <= 160 * 1024, "chunk_scan LDS budget");
    const int groups = (units + 7) / 8;  // see the XCD placement in chunk_scan_kernel
    hipLaunchKernelGGL((chunk_scan_kernel<D, OP, OB, RS, MODE>), dim3(groups * 8 * (D / RS)), dim3(SCAN_THREADS), 0,
                       stream, reinterpret_cast<const char*>(recs), reinterpret_cast<const char*>(krecs),
                       reinterpret_cast<const SeqInfo*>(info), s_in, s_out, out, reinterpret_cast<char*>(sink), units,
                       T, h_k, h_v);
    return hipGetLastError();
}

int scan_rows_per_workgroup(int d, int units) {
    // GDN_SCAN_ROWS=16 or 32 fixes the choice (tuning and tests).
    if (const char* e = getenv("GDN_SCAN_ROWS")) {
        const int v = atoi(e);
        if (v == 16 || v == 32) return v;
    }
    // 16-row slices double the workgroups (each still copies the whole -W,
    // Qt, K^T record part), which pays while 32-row slices leave compute
    // units idle.
    return (long long)units * (d / 32) < compute_units() ? 16 : 32;
}

hipError_t launch_scan(int d, bool in_bf16, bool out_bf16, const void* recs, const void* krecs, const void* info,
                       const float* s_in, float* s_out, void* out, void* sink, int units, int T, int h_k, int h_v,
                       hipStream_t stream) {
    const int rs = scan_rows_per_workgroup(d, units);
#define GDN_SCAN(D, OP, IB, OB)                                                                          \
    if (d == D && in_bf16 == IB && out_bf16 == OB)                                                       \
        return rs == 16 ? launch_scan_t<D, OP, OB, 16>(recs, krecs, info, s_in, s_out, out, sink, units, T, h_k, h_v, stream) \
                        : launch_scan_t<D, OP, OB, 32>(recs, krecs, info, s_in, s_out, out, sink, units, T, h_k, h_v, stream);
    GDN_SCAN(128, _Float16, true, true) GDN_SCAN(128, _Float16, true, false)
    GDN_SCAN(64, _Float16, true, true) GDN_SCAN(64, _Float16, true, false)
    GDN_SCAN(64, float, false, true) GDN_SCAN(64, float, false, false)
#undef GDN_SCAN
    return hipErrorInvalidValue;
}

// ---- two-level scan of one long sequence -------------------------------------------------
// The state map of a run of blocks is affine, S_end = S_start R + B (section
// "Keep the recurrent state on chip" carries S across pieces of a prompt the
// same way).  Split into P segments, each segment's R and B come from two
// state-carrying passes run in parallel (MODE 2 from the identity, MODE 1 from
// zero), the segments' start states from a short sequential composition, and
// the outputs from the scan rerun on all segments in parallel.

__global__ void segment_info_kernel(SeqInfo* __restrict__ info, int P, int sb, int T) {
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s < P) {
        const int b = s * sb * CHUNK;
        info[s] = SeqInfo{b, min(sb * CHUNK, T - b), s * sb, 0};
    }
}

// Segment start states: S_0 = state_in (or zero), S_{s+1} = S_s R_s + B_s.
// One workgroup per (v-head, 16 rows): rows evolve independently.  R_s is
// staged through LDS with coalesced loads.  fp32.
template <int D>
__global__ __launch_bounds__(512) void compose_kernel(const float* __restrict__ state_in,
                                                      const float* __restrict__ R, const float* __restrict__ B,
                                                      float* __restrict__ starts, int P, int h_v) {
    constexpr int ROWS = 16, CPT = D * ROWS / 512, GROUPS = D / CPT;  // columns per thread, column groups
    __shared__ float Rl[D * D];
    __shared__ float cur[ROWS][D];
    const int h = blockIdx.x / (D / ROWS), r0 = (blockIdx.x % (D / ROWS)) * ROWS;
    const int lr = threadIdx.x / GROUPS, c0 = (threadIdx.x % GROUPS) * CPT;
    const size_t hd = (size_t)h * D * D, row = (size_t)(r0 + lr) * D;
    float s[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        s[j] = state_in ? state_in[hd + row + c0 + j] : 0.f;
        starts[hd + row + c0 + j] = s[j];
    }
    for (int st = 0; st + 1 < P; ++st) {
        const size_t m = (size_t)(st * h_v) * D * D + hd;
        __syncthreads();  // the previous step's reads of Rl and cur are done
#pragma unroll
        for (int j = 0; j < CPT; ++j) cur[lr][c0 + j] = s[j];
#pragma unroll
        for (int i = 0; i < D * D / 4 / 512; ++i) {
            const int e = (i * 512 + threadIdx.x) * 4;
            *reinterpret_cast<float4*>(&Rl[e]) = *reinterpret_cast<const float4*>(R + m + e);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPT; ++j) s[j] = B[m + row + c0 + j];
#pragma unroll 8
        for (int k = 0; k < D; ++k) {
            const float a = cur[lr][k];
#pragma unroll
            for (int j = 0; j < CPT; ++j) s[j] = fmaf(a, Rl[k * D + c0 + j], s[j]);
        }
        const size_t o = (size_t)((st + 1) * h_v) * D * D + hd;
#pragma unroll
        for (int j = 0; j < CPT; ++j) starts[o + row + c0 + j] = s[j];
    }
}

hipError_t launch_segment_info(void* info, int P, int sb, int T, hipStream_t stream) {
    hipLaunchKernelGGL(segment_info_kernel, dim3((P + 255) / 256), dim3(256), 0, stream,
                       reinterpret_cast<SeqInfo*>(info), P, sb, T);
    return hipGetLastError();
}

hipError_t launch_compose(int d, const float* state_in, const float* R, const float* B, float* starts, int P,
                          int h_v, hipStream_t stream) {
    if (d == 128)
        hipLaunchKernelGGL(compose_kernel<128>, dim3(h_v * 8), dim3(512), 0, stream, state_in, R, B, starts, P, h_v);
    else if (d == 64)
        hipLaunchKernelGGL(compose_kernel<64>, dim3(h_v * 4), dim3(512), 0, stream, state_in, R, B, starts, P, h_v);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// Both state-map parts of every segment in `info` (MODE 1): units = 2 x
// (segments x v-heads); state_out receives B for the first half, R for the second.
hipError_t launch_scan_transition(int d, bool in_bf16, const void* recs, const void* krecs, const void* info,
                                  float* s_out, void* sink, int units, int T, int h_k, int h_v, hipStream_t stream) {
    const int rs = scan_rows_per_workgroup(d, units);
#define GDN_TR(D, OP, IB)                                                                                        \
    if (d == D && in_bf16 == IB)                                                                                 \
        return rs == 16 ? launch_scan_t<D, OP, false, 16, 1>(recs, krecs, info, nullptr, s_out, nullptr, sink,    \
                                                              units, T, h_k, h_v, stream)                        \
                        : launch_scan_t<D, OP, false, 32, 1>(recs, krecs, info, nullptr, s_out, nullptr, sink,    \
                                                              units, T, h_k, h_v, stream);
    GDN_TR(128, _Float16, true) GDN_TR(64, _Float16, true) GDN_TR(64, float, false)
#undef GDN_TR
    return hipErrorInvalidValue;
}

}  // namespace gdn

// Blocked ("chunked") prefill of the gated delta rule on gfx950: the fp32-input
// kernels, the varlen plan, the two-level scan's segment kernels and the host
// launchers of both input types (the bf16-input kernels are in prefill_bf16.hip).
//
// "Optimizing on-device inference for Apple Silicon", section "Qwen creates
// three distinct workload shapes", says the recurrence can be regrouped into
// blocks of tokens that expose matrix work.  Section "Keep the recurrent state
// on chip" keeps the state on chip for the whole scan and writes it back once,
// in fp32.
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
// Precision (fp32 inputs).  q/k are scaled per token by a power of two (exact)
// and their L2 norms become fp32 row factors c_t; every matrix product runs on
// the fp32 matrix cores, with fp32 intermediates and records.
#include "prefill_shared.h"


namespace gdn {

// ---- varlen plan: per-sequence token range and block-slot base, slot -> sequence ----
// One workgroup.  cu_seqlens is clamped into a non-decreasing sequence inside
// [0, T] so that every index stays in bounds whatever the caller passed.  The
// plan also resets the prefill status word, setting the clamped bit when the
// array broke its contract (first entry not 0, a decrease, an entry outside
// [0, T], last entry not T).
__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu, int N, int T,
                                                   int max_slots, SeqInfo* __restrict__ info,
                                                   int32_t* __restrict__ slot_seq, unsigned* __restrict__ status) {
    __shared__ int s_carry_tok, s_carry_slot, s_bad;
    __shared__ int s_scan[256];
    const int tid = threadIdx.x;
    if (tid == 0) { s_carry_tok = 0; s_carry_slot = 0; s_bad = 0; }
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int n = base + tid;
        // running max of clamped ends (prefix max over this block, seeded by the carry)
        int end = 0;
        if (n < N) {
            const int raw_begin = cu[n], raw_end = cu[n + 1];
            if (raw_end < raw_begin || raw_end < 0 || raw_end > T || (n == 0 && raw_begin != 0) ||
                (n == N - 1 && raw_end != T))
                atomicOr(&s_bad, 1);
            end = raw_end < 0 ? 0 : (raw_end > T ? T : raw_end);
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
    if (tid == 0 && status) *status = s_bad ? (unsigned)GDN_PREFILL_STATUS_CU_SEQLENS_CLAMPED : 0u;
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
    char* __restrict__ recs, char* __restrict__ krecs, int slots, int items_per_wg,
    unsigned* __restrict__ clear_status) {
    using RC = Rec<D, OP>;
    if (clear_status && blockIdx.x == 0 && threadIdx.x == 0) *clear_status = 0u;  // a new call's status word
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
    char* __restrict__ sink, int units, int T, int h_k, int h_v, unsigned* __restrict__ status) {
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
    bool bad = false;  // a non-finite output or final state in this lane
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
            for (int nb = 0; nb < NB; ++nb) {
                bad |= any_nonfinite(acc[nb]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = (16 * tb + 4 * q4 + r) * RS + 16 * nb + j16;
                    if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(sO)[e] = f32_to_bf16(acc[nb][r]);
                    else reinterpret_cast<float*>(sO)[e] = acc[nb][r];
                }
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
    if (MODE == 0) {
#pragma unroll
        for (int i = 0; i < TPW; ++i)
            if (w * TPW + i < Sh::NTB) bad |= any_nonfinite(St[i]);
        report_status(status, bad, GDN_PREFILL_STATUS_NONFINITE);
    }
}

// ---- host launchers ----------------------------------------------------------------------
size_t tp_record_bytes();
size_t key16_record_bytes(int d);
hipError_t launch_prep_bf16(int d, const void* q, const void* k, const float* g, const float* beta,
                            const void* info, const int32_t* slot_seq, int slots, int T, int h_k, int h_v,
                            int l2norm, float scale, void* recs, void* krecs, unsigned* clear_status,
                            hipStream_t stream);
hipError_t launch_scan_bf16(int d, bool out_bf16, int rows, int mode, const void* q, const void* k, const void* v,
                            const void* recs, const void* krecs, const void* info, const float* s_in, float* s_out, void* out, void* sink,
                            int units, int T, int h_k, int h_v, unsigned* status, hipStream_t stream);

// Workspace record sizes: bf16 inputs use one record per (block slot, v-head)
// (prefill_bf16.hip); fp32 inputs one per (block slot, v-head) plus a key
// record per (block slot, k-head).
size_t prefill_record_bytes(int d, bool in_bf16) {
    if (in_bf16) return tp_record_bytes();
    return d == 128 ? Rec<128, float>::BYTES : Rec<64, float>::BYTES;
}

size_t prefill_key_record_bytes(int d, bool in_bf16) {
    if (in_bf16) return key16_record_bytes(d);
    return d == 128 ? KeyRec<128, float>::BYTES : KeyRec<64, float>::BYTES;
}

hipError_t launch_plan(const int32_t* cu, int N, int T, int max_slots, void* info, int32_t* slot_seq,
                       unsigned* status, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu, N, T, max_slots,
                       reinterpret_cast<SeqInfo*>(info), slot_seq, status);
    return hipGetLastError();
}

__global__ void status_reset_kernel(unsigned* __restrict__ status) { *status = 0u; }

hipError_t launch_status_reset(unsigned* status, hipStream_t stream) {
    hipLaunchKernelGGL(status_reset_kernel, dim3(1), dim3(1), 0, stream, status);
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

template <int D, typename OP, bool IB>
static hipError_t launch_prep_t(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const void* info, const int32_t* slot_seq,
                                int slots, int T, int h_k, int h_v, int l2norm, float scale,
                                char* recs, char* krecs, unsigned* clear_status, hipStream_t stream) {
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
                       slots, per, clear_status);
    return hipGetLastError();
}

hipError_t launch_prep(int d, bool in_bf16, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const void* info, const int32_t* slot_seq,
                       int slots, int T, int h_k, int h_v, int l2norm, float scale, void* recs,
                       void* krecs, unsigned* clear_status, hipStream_t stream) {
    if (in_bf16)
        return launch_prep_bf16(d, q, k, g, beta, info, slot_seq, slots, T, h_k, h_v, l2norm, scale, recs, krecs,
                                clear_status, stream);
    if (d == 64)
        return launch_prep_t<64, float, false>(q, k, v, g, beta, info, slot_seq, slots, T, h_k, h_v, l2norm, scale,
                                               reinterpret_cast<char*>(recs), reinterpret_cast<char*>(krecs),
                                               clear_status, stream);
    return hipErrorInvalidValue;
}

template <int D, typename OP, bool OB, int RS, int MODE = 0>
static hipError_t launch_scan_t(const void* recs, const void* krecs, const void* info, const float* s_in,
                                float* s_out, void* out, void* sink, int units, int T, int h_k, int h_v,
                                unsigned* status, hipStream_t stream) {
    static_assert(scan_lds_bytes<D, OP, OB, RS>() <= 160 * 1024, "chunk_scan LDS budget");
    const int groups = (units + 7) / 8;  // see the XCD placement in chunk_scan_kernel
    hipLaunchKernelGGL((chunk_scan_kernel<D, OP, OB, RS, MODE>), dim3(groups * 8 * (D / RS)), dim3(SCAN_THREADS), 0,
                       stream, reinterpret_cast<const char*>(recs), reinterpret_cast<const char*>(krecs),
                       reinterpret_cast<const SeqInfo*>(info), s_in, s_out, out, reinterpret_cast<char*>(sink), units,
                       T, h_k, h_v, status);
    return hipGetLastError();
}

// Rows of a state per scan workgroup: `requested` (16 or 32), or for 0 the
// default.  bf16 inputs: 16 rows, whose layout gives every SIMD one chain wave
// and keeps q in LDS (32-row workgroups measured about twice as slow per
// block at any occupancy).  fp32 inputs: 16-row slices double the workgroups
// (each still copies the whole shared part of a block), which pays while
// 32-row slices leave compute units idle.
int scan_rows_per_workgroup(int d, bool in_bf16, int units, int requested) {
    if (requested == 16 || requested == 32) return requested;
    if (in_bf16) return 16;
    return (long long)units * (d / 32) < compute_units() ? 16 : 32;
}

hipError_t launch_scan(int d, bool in_bf16, bool out_bf16, int rows, const void* q, const void* k, const void* v,
                       const void* recs, const void* krecs, const void* info, const float* s_in, float* s_out,
                       void* out, void* sink, int units, int T, int h_k, int h_v, unsigned* status,
                       hipStream_t stream) {
    const int rs = scan_rows_per_workgroup(d, in_bf16, units, rows);
    if (in_bf16)
        return launch_scan_bf16(d, out_bf16, rs, 0, q, k, v, recs, krecs, info, s_in, s_out, out, sink, units, T, h_k, h_v,
                                status, stream);
#define GDN_SCAN(D, OP, IB, OB)                                                                                \
    if (d == D && in_bf16 == IB && out_bf16 == OB)                                                             \
        return rs == 16 ? launch_scan_t<D, OP, OB, 16>(recs, krecs, info, s_in, s_out, out, sink, units, T, h_k, \
                                                       h_v, status, stream)                                    \
                        : launch_scan_t<D, OP, OB, 32>(recs, krecs, info, s_in, s_out, out, sink, units, T, h_k, \
                                                       h_v, status, stream);
    GDN_SCAN(64, float, false, true) GDN_SCAN(64, float, false, false)
#undef GDN_SCAN
    return hipErrorInvalidValue;
}

// ---- two-level scan of one long sequence -------------------------------------------------
// The state map of a run of blocks is affine, S_end = S_start R + B (section
// "Keep the recurrent state on chip" carries S across pieces of a prompt the
// same way).  Split into P segments, each segment's R and B come from one
// state-carrying pass over all segments in parallel (the transition scan: half
// of its units start from the identity without the value term and give R, the
// other half start from zero and give B), the segments' start states from a
// short sequential composition, and the outputs from the scan rerun on all
// segments in parallel.

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
hipError_t launch_scan_transition(int d, bool in_bf16, int rows, const void* q, const void* k, const void* v,
                                  const void* recs, const void* krecs, const void* info, float* s_out, void* sink,
                                  int units, int T, int h_k, int h_v, hipStream_t stream) {
    const int rs = scan_rows_per_workgroup(d, in_bf16, units, rows);
    if (in_bf16)
        return launch_scan_bf16(d, false, rs, 1, q, k, v, recs, krecs, info, nullptr, s_out, nullptr, sink, units, T, h_k,
                                h_v, nullptr, stream);
    if (d == 64)
        return rs == 16 ? launch_scan_t<64, float, false, 16, 1>(recs, krecs, info, nullptr, s_out, nullptr, sink,
                                                                 units, T, h_k, h_v, nullptr, stream)
                        : launch_scan_t<64, float, false, 32, 1>(recs, krecs, info, nullptr, s_out, nullptr, sink,
                                                                 units, T, h_k, h_v, nullptr, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn

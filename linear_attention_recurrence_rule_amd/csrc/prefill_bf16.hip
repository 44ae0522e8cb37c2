// Blocked ("chunked") prefill of the gated delta rule for bf16 inputs on gfx950.
//
// "Optimizing on-device inference for Apple Silicon", section "Qwen creates
// three distinct workload shapes", says the recurrence can be regrouped into
// blocks of tokens that expose matrix work; section "Keep the recurrent state
// on chip" keeps the state on chip for the whole scan and writes it once.
//
// Per block of n <= 64 tokens and v-head, with block-initial state S
// (d_v x d_k), cumulative log-decay G_i = g_1 + ... + g_i, normalised keys
// and queries k_i = c_i k_i^raw, q_i = c^q_i q_i^raw (c the L2 norm factor,
// c^q also the query scale):
//   A_ij = beta_i exp(G_i - G_j) k_i.k_j (i > j),  T = (I + A)^{-1} diag(beta),
//   P_ij = exp(G_i - G_j) q_i.k_j (i >= j),
//   U = T (V - diag(gamma c) K^raw S^T),  gamma = exp(G),
//   O = diag(gamma c^q) Q^raw S^T + P U,
//   S' = exp(G_n) S + U^T diag(exp(G_n - G) c) K^raw.
// Kernels:
//   chunk_prep_pair (parallel over blocks x k-heads): T, P and the per-token
//     factors of each (block, v-head), about 13 KiB per record, and a key
//     record per (block, k-head): the keys and queries as fp16, each token's
//     row scaled by a power of two;
//   chunk_scan_tpf (sequential over the blocks of a sequence, parallel over
//     sequences x v-heads x 16-row slices of S): reads each block's key
//     record, v slice and record, keeps S in registers in fp32 and writes it
//     once.  Its state-side products (K S^T, Q S^T and the update) run on
//     fp16 matrix cores, S^T's operand copy scaled per key block and row by a
//     power of two;
//   chunk_scan_tp (32-row slices, and the segment maps of the two-level scan):
//     the same recurrence from the raw bf16 q and k tiles, with S (and
//     diag(s) U) split into a bf16 high and low part, about 16 significant bits.
// In both scans T, P, R = V - ... and U enter the token contractions U = T R
// and P U as fp16.
#include "prefill_shared.h"

namespace gdn {

constexpr float LOG2E_F = 1.4426950408889634f;

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf4_t __attribute__((ext_vector_type(4)));
typedef short s4v_t __attribute__((ext_vector_type(4)));

// ---- record of one (block slot, v-head) ---------------------------------------------------
// T and P are lower triangular 64 x 64; as fragment-major fp16 matrices
// (fragment (row block mb, 32-column block kb)) only six of the eight
// fragments can be non-zero: (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
struct TpRec {
    static constexpr int NF = 6;
    static constexpr size_t T = 0;                  // T fragments, NF x 1 KiB
    static constexpr size_t P = T + NF * 1024;      // P fragments
    static constexpr size_t F = P + NF * 1024;      // gck[64], gcq[64], sck[64], gamma_n (fp32)
    static constexpr size_t BYTES = F + 1024;
    static constexpr int GCK = 0, GCQ = 64, SCK = 128, GN = 192;  // float offsets in F
};
__device__ __forceinline__ int tri_frag(int mb, int kb) { return mb < 2 ? mb : 2 * mb - 2 + kb; }

// ---- key record of one (block slot, k-head) -----------------------------------------------
// The block's keys and queries as fp16, each token's row scaled by 2^-E with E
// the exponent of the row's largest magnitude (so every element is below 1 and
// the conversion from bf16 is exact down to 2^-14 of that magnitude), then the
// factors 2^E per token (keys, then queries).  The keys are rows in a swizzled
// layout (key_unit): the scan reads them as rows and as columns from LDS.  The
// queries are stored as the A fragments of their 16-token blocks (fragment
// tb * (D / 32) + kb, 64 lanes x 16 bytes, the permuted key order of h16_row8),
// which the scan loads straight into registers.  Both v-heads of a k-head read
// the same record.
template <int D>
struct KeyRec16 {
    static constexpr size_t K = 0;
    static constexpr size_t Q = (size_t)CHUNK * D * 2;
    static constexpr size_t E = 2 * (size_t)CHUNK * D * 2;
    static constexpr size_t BYTES = E + 1024;
    static constexpr int EK = 0, EQ = 64;  // float offsets in E
};

// Byte offset of the 16-byte unit u of row r in a swizzled raw tile of D bf16 per row:
// the units of row r are permuted by XOR with (r mod units per row), so that a
// column read or a read of 16 rows at one column spreads over the LDS banks.
template <int D>
__device__ __forceinline__ int raw_unit(int r, int u) {
    constexpr int UPR = D / 8;
    return r * (D * 2) + ((u ^ (r & (UPR - 1))) << 4);
}

// Row fragment (8 consecutive d of one token) of a raw tile, for the Gram
// products whose two operands are both read this way: lane (i, q) holds
// M[16 rb + i][32 kb + 8 q + e].
template <int D>
__device__ __forceinline__ bf8_t raw_row8(const uint16_t* M, int rb, int kb, int lane) {
    const int r = 16 * rb + (lane & 15), u = 4 * kb + (lane >> 4);
    return *reinterpret_cast<const bf8_t*>(reinterpret_cast<const char*>(M) + raw_unit<D>(r, u));
}

// Row fragment in the accumulator-chaining order of gdn_device.h: lane (i, q)
// holds M[16 rb + i][32 kb + 4q + e] for e < 4 and M[16 rb + i][32 kb + 16 + 4q + e - 4]
// for e >= 4 (the order of the state fragments it meets).
template <int D>
__device__ __forceinline__ bf8_t raw_rowfrag(const uint16_t* M, int rb, int kb, int lane) {
    const int r = 16 * rb + (lane & 15), q = lane >> 4;
    const char* base = reinterpret_cast<const char*>(M);
    const uint2 a = *reinterpret_cast<const uint2*>(base + raw_unit<D>(r, 4 * kb + (q >> 1)) + 8 * (q & 1));
    const uint2 b = *reinterpret_cast<const uint2*>(base + raw_unit<D>(r, 4 * kb + 2 + (q >> 1)) + 8 * (q & 1));
    return __builtin_bit_cast(bf8_t, uint4{a.x, a.y, b.x, b.y});
}

// Column fragment of a raw tile (the layout of frag_colmajor): the contraction
// runs down the rows 32 kb + (4q + e) for e < 4 and 32 kb + 16 + 4q + (e - 4)
// for e >= 4, at column 16 cb + (lane % 16).  Two transposing reads
// (ds_read_b64_tr_b16) of the swizzled rows.
template <int D>
__device__ __forceinline__ bf8_t raw_colfrag(const uint16_t* M, int cb, int kb, int lane) {
    typedef __attribute__((address_space(3))) s4v_t* lds_s4;
    const int s = lane & 15, q = lane >> 4;
    const int r = 32 * kb + 4 * q + (s >> 2), col = 16 * cb + 4 * (s & 3);
    const char* base = reinterpret_cast<const char*>(M);
    const int o0 = raw_unit<D>(r, col >> 3) + ((col & 7) << 1);
    const int o1 = raw_unit<D>(r + 16, col >> 3) + ((col & 7) << 1);
    const s4v_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(base + o0));
    const s4v_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(base + o1));
    return __builtin_bit_cast(bf8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ void mma_bf16(f4_t& acc, const bf8_t& a, const bf8_t& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_f16(f4_t& acc, const h8_t& a, const h8_t& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
// Fragments of an fp16 tile in the swizzled row layout, for products with S^T
// fragments built from accumulator tiles.  Key index x of such a product (x the
// position in the accumulator order: 32 kb + 4 q + e for e < 4, 32 kb + 16 + 4 q + e - 4
// for e >= 4) stands for the key 32 kb + 8 q + e, a permutation inside each block of
// 32 keys.  The state's tiles hold the keys in that order, so a row fragment is 16
// contiguous bytes (raw_row8), and a column fragment of tile m holds, for lane i, the
// column 32 (m / 2) + 8 (i / 4) + 4 (m mod 2) + (i mod 4).
//
// The key tile of the key record (and of the scan's LDS) has a swizzle of its own:
// the 16-byte units of row r are XOR-permuted by ((r mod 4) << 2) | ((r / 4) mod 4).
// A row fragment reads one unit of 16 consecutive rows and a column fragment four
// units of 4 consecutive rows; both land on 16 distinct units (with the row-only
// permutation of raw_unit the column reads met only 4).
template <int D>
__device__ __forceinline__ int key_unit(int r, int u) {
    constexpr int UPR = D / 8;
    return r * (D * 2) + ((u ^ ((((r & 3) << 2) | ((r >> 2) & 3)) & (UPR - 1))) << 4);
}
template <int D>
__device__ __forceinline__ h8_t h16_row8(const _Float16* M, int rb, int kb, int lane) {
    const int r = 16 * rb + (lane & 15), u = 4 * kb + (lane >> 4);
    return *reinterpret_cast<const h8_t*>(reinterpret_cast<const char*>(M) + key_unit<D>(r, u));
}
// Column fragment (A of the update: rows = the keys of tile m, contraction = the tokens
// of the 32-token block kb): two transposing reads (ds_read_b64_tr_b16) of the swizzled
// rows.  Lane s of group q addresses token row 32 kb + 4 q + (s >> 2) at the four
// columns of column group s & 3; lane i then receives its column's four rows.
template <int D>
__device__ __forceinline__ h8_t h16_colfrag_p(const _Float16* M, int m, int kb, int lane) {
    typedef __attribute__((address_space(3))) s4v_t* lds_s4;
    const int s = lane & 15, q = lane >> 4;
    const int r = 32 * kb + 4 * q + (s >> 2), col = 32 * (m >> 1) + 8 * (s & 3) + 4 * (m & 1);
    const char* base = reinterpret_cast<const char*>(M);
    const int o0 = key_unit<D>(r, col >> 3) + ((col & 7) << 1);
    const int o1 = key_unit<D>(r + 16, col >> 3) + ((col & 7) << 1);
    const s4v_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(base + o0));
    const s4v_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(base + o1));
    return __builtin_bit_cast(h8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ float bf16_lo_bits(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_bits(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ============================================================================================
// chunk_prep_pair: T, P and the per-token factors, a k-head's v-heads in pairs
// ============================================================================================
// One workgroup per compute unit takes a run of items (block slot, k-head,
// pair of the k-head's v-heads).  The raw Gram products K K^T and Q K^T are
// formed once per item; only the decay masks, beta and the norm factors differ
// between the two v-heads.  Two loader waves copy the next item's raw q, k, g
// and beta into LDS with direct global-to-LDS loads while the eight compute
// waves work, so the compute waves issue no global loads: the memory counter
// a wave waits on covers its loads and its stores alike, and a wave that
// loaded inputs and wrote records would wait for its record stores to drain.
//   P2a waves 0, 1: the diagonal blocks of K K^T and Q Q^T (bf16 matrix cores
//       on the raw inputs), whose diagonals give the norm factors, then G and
//       the per-token terms of v-head `wave`; waves 2..5: the raw off-diagonal
//       K K^T and the Q K^T tiles; waves 6, 7: the raw diagonal K K^T tiles.
//   P2b decay masks: A_ij^T tiles (i > j blocks), P fragment halves (to the
//       records), and the diagonal blocks N_bb of A, which waves 6, 7 invert by
//       forward substitution on the vector unit (one lane per column of a block);
//       waves 0, 1 write the zero halves of the records' fragments.
//   P4  the six blocks of X = (I + A)^{-1} below the diagonal (fp32 matrix
//       cores), written with the four diagonal ones as T = X diag(beta)
//       fragment halves to the records.
// The records' fragments go out half by half, straight from the registers.
// Decay ratios are exp2(r_i - c_j) with r_i = G_i log2(e) + log2(beta_i c_i)
// and c_j = G_j log2(e) - log2(c_j); only entries with i >= j are kept, so
// the exponent carries exp(G_i - G_j) <= 1.
constexpr int PAIR_COMPUTE_WAVES = 8, PAIR_LOADER_WAVES = 2;
constexpr int PAIR_THREADS = (PAIR_COMPUTE_WAVES + PAIR_LOADER_WAVES) * WAVE;

struct PairMeta {
    int32_t tok0, nt, live, pad;
};

template <int D, int NH>
struct PairLds {
    static constexpr int XS = 20;       // row stride of 16 x 16 fp32 blocks
    uint16_t kraw[CHUNK * D];           // raw bf16 keys (swizzled rows)
    uint16_t qraw[CHUNK * D];           // raw bf16 queries
    float gb[NH][2][CHUNK];             // g and beta of the v-heads
    float a[NH][6][WAVE * 4];           // A_ij^T (block i > j) in accumulator layout
    float nb[NH][4][16 * XS];           // diagonal blocks N_bb of A, transposed (row j = column j of N)
    float xd[NH][4][16 * XS];           // X_bb = (I + N_bb)^{-1}, column-major [col][row]
    float ra[NH][CHUNK], rq[NH][CHUNK], cb[NH][CHUNK], bt[NH][CHUNK];
    PairMeta meta[2];
    int zero;                           // holds 0 (see the compute waves)
};

template <int D, int NH>
constexpr size_t pair_lds_bytes() { return sizeof(PairLds<D, NH>); }

// Slot of the off-diagonal block (i, j), i > j: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
__device__ __forceinline__ constexpr int aslot(int i, int j) { return i * (i - 1) / 2 + j; }

template <int D, int NH>
__global__ __launch_bounds__(PAIR_THREADS, 1) void chunk_prep_pair_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, const SeqInfo* __restrict__ info, const int32_t* __restrict__ slot_seq,
    int T, int h_k, int h_v, int l2norm, float scale, char* __restrict__ recs, char* __restrict__ krecs, int slots,
    int items_per_wg, unsigned* __restrict__ clear_status) {
    using OP = _Float16;
    using LT = PairLds<D, NH>;
    if (clear_status && blockIdx.x == 0 && threadIdx.x == 0) *clear_status = 0u;  // a new call's status word
    constexpr int XS = LT::XS;
    constexpr int NKB = D / 32;  // contraction blocks over d
    extern __shared__ __align__(16) char smem_raw[];
    LT& L = *reinterpret_cast<LT*>(smem_raw);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);  // wave-uniform: role branches stay scalar
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
        // Item i + 1's copies go out while item i is in P2b and P4 (q, k, g and beta are
        // read in P2a only) and must have landed by the next B1: the raw k tile and half
        // the q tile after B2 (part 0), the rest of q, g and beta after B3 (part 1).
        // Issued all after B2, the loads queue behind the compute waves' record stores
        // long enough to make the loaders the last waves at B3.
        typedef __attribute__((address_space(3))) void* lds_ptr;
        const int lw = wave - PAIR_COMPUTE_WAVES, lane = tid % WAVE;
        constexpr int RPI = 1024 / (2 * D);  // rows per direct load
        constexpr int UPR = D / 8;           // 16-byte units per row
        constexpr int NL = CHUNK / RPI;      // loads per tile
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
        // token indices clamped into [0, T); rows past the block end are masked on use
        constexpr int EARLY = (3 * NL / 2) / PAIR_LOADER_WAVES;  // part 0's tile loads per loader
        auto issue = [&](int item, int tok0, int part) __attribute__((always_inline)) {
            int hk, pr;
            const int h0 = heads_of(item, hk, pr);
            static_assert((2 * NL) % PAIR_LOADER_WAVES == 0 && (2 * NH) % PAIR_LOADER_WAVES == 0,
                          "loads in multiples of the loader count");
#pragma unroll
            for (int mm = 0; mm < 2 * NL / PAIR_LOADER_WAVES; ++mm) {
                if ((mm < EARLY) != (part == 0)) continue;
                const int i = mm * PAIR_LOADER_WAVES + lw;
                const int m4 = i % NL;
                const int r = m4 * RPI + lane / UPR, p = lane % UPR;
                const int u = p ^ (r & (UPR - 1));  // the global unit this lane's LDS slot holds
                const size_t tt = (size_t)min(tok0 + r, T - 1);
                const uint16_t* src = reinterpret_cast<const uint16_t*>(i < NL ? k : q) + (tt * h_k + hk) * D;
                uint16_t* dst = i < NL ? L.kraw : L.qraw;
                __builtin_amdgcn_global_load_lds(src + 8 * u, (lds_ptr)(dst + m4 * 512), 16, 0, 0);
            }
#pragma unroll
            for (int mm = 0; mm < 2 * NH / PAIR_LOADER_WAVES; ++mm) {  // g and beta, one fp32 per lane
                if (part == 0) break;
                const int i = mm * PAIR_LOADER_WAVES + lw;
                const int j = i >> 1;
                const size_t tg = (size_t)min(tok0 + lane, T - 1) * h_v + h0 + j;
                const float* src = (i & 1) ? beta + tg : g + tg;
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)&L.gb[j][i & 1][0], 4, 0, 0);
            }
        };
        int par = 0;
        {
            const PairMeta m = meta_of(i0);
            if (lw == 0 && lane == 0) L.meta[0] = m;
            issue(i0, m.live ? m.tok0 : 0, 0);
            issue(i0, m.live ? m.tok0 : 0, 1);
            wait_vmcnt<0>();
        }
        for (int item = i0; item < i1; ++item, par ^= 1) {
            lds_barrier();  // B1
            lds_barrier();  // B2: q, k, g and beta are no longer read
            PairMeta mn{0, 0, 0, 0};
            if (item + 1 < i1) {
                mn = meta_of(item + 1);
                if (lw == 0 && lane == 0) L.meta[par ^ 1] = mn;
                issue(item + 1, mn.live ? mn.tok0 : 0, 0);
            }
            lds_barrier();  // B3
            if (item + 1 < i1) issue(item + 1, mn.live ? mn.tok0 : 0, 1);
            wait_vmcnt<0>();
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

        // ---- P2a ------------------------------------------------------------------------------
        // The 16 off-diagonal tiles u (u < 6 the K K^T block of slot u, u >= 6 the Q K^T tile
        // u - 6) go to waves 0..5: three each to waves 0, 1, 4 and 5, two each to waves 2, 3
        // (waves 4 and 5, whose tiles' P halves go to the records in P2b, bound that phase).
        const int u0 = wave < 2 ? 3 * wave : wave < 4 ? 6 + 2 * (wave - 2) : 10 + 3 * (wave - 4);
        const int nt = wave < 2 ? 3 : wave < 4 ? 2 : wave < 6 ? 3 : 0;
        f4_t acc[4];
        if (live) {
            if (wave < 4) {
                // block wave b: the squared norms of tokens 16b .. 16b + 15 (lane (i, q) sums the
                // squares of its 32 elements of row 16b + i, then the four rows of 16 lanes add
                // up), then those tokens' per-token terms for each v-head
                const int b = wave;
                float sk = 0.f, sq = 0.f;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
                    const bf8_t xk = raw_row8<D>(L.kraw, b, kb, lane), xq = raw_row8<D>(L.qraw, b, kb, lane);
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {  // bf16 pair dot products, fp32 sums
                        const bf2_t pk = {xk[e], xk[e + 1]}, pq = {xq[e], xq[e + 1]};
                        sk = __builtin_amdgcn_fdot2_f32_bf16(pk, pk, sk, false);
                        sq = __builtin_amdgcn_fdot2_f32_bf16(pq, pq, sq, false);
                    }
                }
                F2 t = permlane16_swap(sk, sk);
                sk = t.x + t.y;
                t = permlane32_swap(sk, sk);
                sk = t.x + t.y;
                t = permlane16_swap(sq, sq);
                sq = t.x + t.y;
                t = permlane32_swap(sq, sq);
                sq = t.x + t.y;
                const bool tl = lane < cnt;
                const float ckv = tl ? (l2norm ? rsqrtf(sk + 1e-6f) : 1.0f) : 0.f;
                const float cqv = tl ? (l2norm ? scale * rsqrtf(sq + 1e-6f) : scale) : 0.f;
                float gv[NH], bv[NH];
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    gv[hh] = tl ? L.gb[hh][0][lane] : 0.f;
                    bv[hh] = tl ? L.gb[hh][1][lane] : 0.f;
                }
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    const float gl = wave_inclusive_sum(gv[hh]) * LOG2E_F;
                    const float gln = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), max(cnt - 1, 0)));
                    float* f = reinterpret_cast<float*>(recs + ((size_t)slot * h_v + h0 + hh) * TpRec::BYTES + TpRec::F);
                    if (lq == b) {  // tokens 16b .. 16b + 15
                        L.ra[hh][lane] = gl + __builtin_amdgcn_logf(bv[hh] * ckv);
                        L.rq[hh][lane] = gl + __builtin_amdgcn_logf(cqv);
                        L.cb[hh][lane] = gl - __builtin_amdgcn_logf(ckv);
                        L.bt[hh][lane] = bv[hh];
                        const float gam = __builtin_amdgcn_exp2f(gl);
                        f[TpRec::GCK + lane] = gam * ckv;
                        f[TpRec::GCQ + lane] = gam * cqv;
                        f[TpRec::SCK + lane] = tl ? __builtin_amdgcn_exp2f(gln - gl) * ckv : 0.f;
                    }
                    if (b == 0 && lane == 0) f[TpRec::GN] = __builtin_amdgcn_exp2f(gln);
                }
            }
            if (wave < 6) {
                // tile u < 6: the off-diagonal K K^T block of slot u, computed as K_j K_i^T so that
                // lane (j', q) holds A_ij^T[4q + r][j']; u >= 6: the tile K_nb Q_mb^T, which is this
                // lane's half of P's fragment (mb, nb / 2)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if (m >= nt) break;
                    const int u = u0 + m;
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
                            mma_bf16(acc[m], raw_row8<D>(L.kraw, nb, kb, lane), raw_row8<D>(L.qraw, mb, kb, lane));
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
        if (live && pr == 0) {
            // The key record of (block slot, k-head), written once per k-head: every
            // compute wave takes 8 rows of the key and the query tile.  A row's UPR
            // 16-byte units sit in UPR consecutive lanes, which find the row's largest
            // magnitude together; the row is scaled by 2^-E and rounded to fp16.
            constexpr int UPR = D / 8, RPR = WAVE / UPR, ROUNDS = 8 / RPR;
            const int u = lane % UPR;
            char* kr = krecs + ((size_t)slot * h_k + hk) * KeyRec16<D>::BYTES;
#pragma unroll
            for (int op = 0; op < 2; ++op) {
                const uint16_t* tile = op ? L.qraw : L.kraw;
#pragma unroll
                for (int rr = 0; rr < ROUNDS; ++rr) {
                    const int r = 8 * wave + RPR * rr + lane / UPR;
                    const uint4 w4 = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(tile) + raw_unit<D>(r, u));
                    const uint32_t wd[4] = {w4.x, w4.y, w4.z, w4.w};
                    float x[8], m = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[2 * e] = bf16_lo_bits(wd[e]);
                        x[2 * e + 1] = bf16_hi_bits(wd[e]);
                        m = fmaxf(m, fmaxf(fabsf(x[2 * e]), fabsf(x[2 * e + 1])));
                    }
                    m = group_max<UPR>(m);
                    const int E = min(__builtin_amdgcn_frexp_expf(m), 127);
                    h8_t hx;
#pragma unroll
                    for (int e = 0; e < 8; ++e) hx[e] = (_Float16)__builtin_amdgcn_ldexpf(x[e], -E);
                    if (op == 0) {
                        *reinterpret_cast<h8_t*>(kr + KeyRec16<D>::K + key_unit<D>(r, u)) = hx;
                    } else {
                        // queries as A fragments in the permuted key order (h16_row8): unit u of
                        // row 16 tb + i is lane i + 16 (u mod 4) of fragment tb * (D / 32) + u / 4
                        *reinterpret_cast<h8_t*>(kr + KeyRec16<D>::Q +
                                                 ((size_t)(((r >> 4) * (D / 32) + (u >> 2)) * WAVE) + (r & 15) +
                                                  16 * (u & 3)) * 16) = hx;
                    }
                    if (u == 0)
                        reinterpret_cast<float*>(kr + KeyRec16<D>::E)[(op ? KeyRec16<D>::EQ : KeyRec16<D>::EK) + r] =
                            __builtin_amdgcn_ldexpf(1.f, E);
                }
            }
        }
        lds_barrier();  // B2: the raw inputs are no longer read; the per-token terms in LDS

        // ---- P2b ------------------------------------------------------------------------------
        if (live) {
            if (wave < 2) {
                // the halves above the diagonal in the stored fragments, blocks (0, 1) and (2, 3)
                // of T (wave 0) and of P (wave 1)
                const f4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    OP* rec = reinterpret_cast<OP*>(recs + ((size_t)slot * h_v + h0 + hh) * TpRec::BYTES +
                                                    (wave ? TpRec::P : TpRec::T));
                    store_part<OP>(rec, tri_frag(0, 0), 1, lane, z);
                    store_part<OP>(rec, tri_frag(2, 1), 1, lane, z);
                }
            }
            if (wave < 6) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if (m >= nt) break;
                    const int u = u0 + m;
                    if (u < 6) {
                        const int bi = u >= 3 ? 3 : (u >= 1 ? 2 : 1), bj = u - bi * (bi - 1) / 2;
#pragma unroll
                        for (int hh = 0; hh < NH; ++hh) {
                            const float r = L.ra[hh][16 * bi + li];
                            const f4_t c = *reinterpret_cast<const f4_t*>(&L.cb[hh][16 * bj + 4 * lq]);
                            f4_t x;
#pragma unroll
                            for (int e = 0; e < 4; ++e) x[e] = acc[m][e] * __builtin_amdgcn_exp2f(r - c[e]);
                            *reinterpret_cast<f4_t*>(&L.a[hh][u][lane * 4]) = x;
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
                            store_part<OP>(reinterpret_cast<OP*>(recs + ((size_t)slot * h_v + h0 + hh) * TpRec::BYTES +
                                                                 TpRec::P),
                                           tri_frag(mb, nb / 2), nb % 2, lane, x);
                        }
                    }
                }
            } else if (wave - 6 < NH) {
                const int hh = wave - 6;
                // N_bb (strictly lower) transposed, from the symmetric raw block: lane (j', q)
                // holds N[4q + r][j'] = raw[4q + r][j'] exp2(r_{4q+r} - c_j'), stored at row j'
                // of N^T
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const f4_t r = *reinterpret_cast<const f4_t*>(&L.ra[hh][16 * b + 4 * lq]);
                    const float c = L.cb[hh][16 * b + li];
                    f4_t x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (4 * lq + e > li) ? acc[b][e] * __builtin_amdgcn_exp2f(r[e] - c) : 0.f;
                    *reinterpret_cast<f4_t*>(&L.nb[hh][b][li * XS + 4 * lq]) = x;
                }
                // Forward substitution (I + N) X = I, column by column of N: lane (b, j)
                // computes column j of X_bb.  Once x_m = X[m][j] is final, it is taken out of
                // every later row, s_i -= N[i][m] x_m, so each step's updates are independent.
                // The rows of N^T are read as broadcasts (the 16 lanes of a block read the
                // same address).
                const int b = lq, j = li;
                const float* Nt = L.nb[hh][b];
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
                // Each step's row of N^T is read one step ahead (left to the compiler,
                // every step waited for its own reads; further ahead the registers
                // would no longer allow two workgroups per CU).
                f4_t nr[15][4];
                constexpr int AHEAD = 1;
                auto fetch = [&](int m) __attribute__((always_inline)) {
#pragma unroll
                    for (int i4 = ((m + 1) / 4) * 4; i4 < 16; i4 += 4)
                        nr[m][i4 / 4] = *reinterpret_cast<const f4_t*>(&Nt[m * XS + i4]);
                };
#pragma unroll
                for (int m = 0; m < AHEAD; ++m) fetch(m);
#pragma unroll
                for (int m = 0; m < 15; ++m) {
                    if (m + AHEAD < 15) fetch(m + AHEAD);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i4 = ((m + 1) / 4) * 4; i4 < 16; i4 += 4) {
                        const f4_t nc = nr[m][i4 / 4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (i4 + e > m) x[i4 + e] = fmaf(-nc[e], x[m], x[i4 + e]);
                    }
                }
                float* xd = L.xd[hh][b];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<f4_t*>(&xd[j * XS + 4 * c]) = f4_t{x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]};
            }
        }
        lds_barrier();  // B3: P complete

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
                auto at = [&](int i, int j) { return *reinterpret_cast<const f4_t*>(&L.a[hh][aslot(i, j)][lane * 4]); };
                auto xa = [&](int b) { return *reinterpret_cast<const f4_t*>(&L.xd[hh][b][li * XS + 4 * lq]); };
                auto xt = [&](int b) {
                    const float* x = L.xd[hh][b];
                    return f4_t{x[(4 * lq) * XS + li], x[(4 * lq + 1) * XS + li], x[(4 * lq + 2) * XS + li],
                                x[(4 * lq + 3) * XS + li]};
                };
                auto put = [&](int a, int b, const f4_t& negxt) {  // negxt = -X_ab^T
                    store_part<OP>(reinterpret_cast<OP*>(recs + ((size_t)slot * h_v + h0 + hh) * TpRec::BYTES + TpRec::T),
                                   tri_frag(a, b >> 1), b & 1, lane,
                                   -negxt * *reinterpret_cast<const f4_t*>(&L.bt[hh][16 * b + 4 * lq]));
                };
                put(role, role, -xt(role));  // T's diagonal block role
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
    }
}

// ============================================================================================
// chunk_scan_tp: the state-dependent part, sequential over blocks
// ============================================================================================
// One workgroup owns NB row blocks of 16 rows of one (sequence, v-head) state;
// the rows of S evolve independently.  Three kinds of waves:
//   chain waves (two per row block, one per half of the key dimension) hold
//     their half of S^T as fp32 accumulator tiles (lane (j, q) of tile mb holds
//     S[row j][16 mb + 4q + r]) and run the two products that carry the state:
//     Y_h = K^raw_h S^T_h over their half, and the update
//     S^T_h <- gamma_n S^T_h + K^raw_h^T diag(s c) U;
//   token waves (one per token block of 16) do the rest, off the products:
//     Z = Q^raw S^T (queries loaded straight into registers two blocks ahead),
//     R = V - diag(gamma c) (Y_0 + Y_1), U = T R, the bf16 high and low parts of
//     diag(s c) U, and O = diag(gamma c_q) Z + P U;
//   copier waves fill a ring of three LDS slots (raw k, the v slice, T, P and
//     the factors) with direct global-to-LDS loads, block c + 2's copy going
//     out as block c starts.
// Four barriers per block:
//   B1  block c in its slot, S^T in LDS     -> chain: Y_h;  token: Z
//   BX  partial products in LDS             -> token: R;  chain: block c - 1's outputs to HBM
//   BR  R in LDS                            -> token: U, its parts
//   BU  U and its parts in LDS              -> chain: update, S^T to LDS;  token: O
// Waves that load inside the block loop never store there (a wave's memory
// counter covers both, so a load wait would also wait for its stores).
template <int D, int NB>
struct TpsRoles {
    // chain waves per row block: one per 32-wide key block with one row block (so
    // that every SIMD holds one chain wave), one per half with two
    static constexpr int CPB = NB == 1 ? D / 32 : 2;
    static constexpr int KPW = D / 32 / CPB;  // 32-wide key blocks per chain wave
    static constexpr int CHAIN = CPB * NB, OUTW = 4, LOAD = 4;
    static constexpr int WAVES = CHAIN + OUTW + LOAD;
    static constexpr int THREADS = WAVES * WAVE;
};
constexpr int TPS_MAX_THREADS = 12 * WAVE;  // launch bound shared by all shapes
static_assert(TpsRoles<128, 1>::THREADS <= TPS_MAX_THREADS && TpsRoles<128, 2>::THREADS <= TPS_MAX_THREADS,
              "scan workgroup size");

template <int D, int NB>
struct TpSlot {
    static constexpr int RS = 16 * NB;
    uint16_t k[CHUNK * D];                  // raw keys (swizzled rows)
    uint16_t vs[CHUNK * RS];                // the row blocks' raw values [token][RS]
    _Float16 tp[2][TpRec::NF * WAVE * 8];   // T and P fragments, as in the record
    float fac[256];                         // gck, gcq, sck, gamma_n
};

template <int D, int NB>
struct TpShape {
    static constexpr int RS = 16 * NB;
    static constexpr int RING = 3;
    static constexpr int NK = CHUNK * D * 2 / 1024;        // 1 KiB loads of the raw k tile
    static constexpr int NV = CHUNK * RS * 2 / 256;        // 256-byte loads (4 bytes a lane) of the v slice
    static constexpr int N = NK + NV + 2 * TpRec::NF + 4;  // a block's loads: k, v, T and P, factors
    static constexpr int L = N / TpsRoles<D, NB>::LOAD;    // per copier wave
    static_assert(N % TpsRoles<D, NB>::LOAD == 0, "copy split");
    static constexpr int NKB = D / 32;                     // 32-wide key blocks
};

// B fragment from two accumulator tiles stacked along the contraction (as
// frag_from_acc), split into bf16 high (round to nearest) and low (x - high) parts.
__device__ __forceinline__ void split_from_acc(const f4_t& top, const f4_t& bot, bf8_t& hi, bf8_t& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hi[e] = (__bf16)top[e];
        lo[e] = (__bf16)(top[e] - (float)hi[e]);
        hi[e + 4] = (__bf16)bot[e];
        lo[e + 4] = (__bf16)(bot[e] - (float)hi[e + 4]);
    }
}

// Four accumulator values as half (part 0: elements 0..3, part 1: 4..7) of a
// stored bf16 fragment, split into high and low parts.
__device__ __forceinline__ void store_split(uint16_t* hi, uint16_t* lo, int frag, int part, int lane, const f4_t& x) {
    const int off = (frag * WAVE + lane) * 8 + 4 * part;
    bf4_t h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = (__bf16)x[e];
        l[e] = (__bf16)(x[e] - (float)h[e]);
    }
    *reinterpret_cast<bf4_t*>(hi + off) = h;
    *reinterpret_cast<bf4_t*>(lo + off) = l;
}

__device__ __forceinline__ bf8_t bfrag(const uint16_t* base, int frag, int lane) {
    return *reinterpret_cast<const bf8_t*>(base + ((size_t)frag * WAVE + lane) * 8);
}
__device__ __forceinline__ void bfrag_store(uint16_t* base, int frag, int lane, const bf8_t& x) {
    *reinterpret_cast<bf8_t*>(base + ((size_t)frag * WAVE + lane) * 8) = x;
}

// Partial Y tiles (live from phase Y to phase R) share their LDS with U and the
// parts of diag(s c) U (live from phase U to phase S).
template <int D, int NB>
struct TpsXchg {
    static constexpr int Y_FLOATS = NB * TpsRoles<D, NB>::CPB * 4 * WAVE * 4;
    static constexpr int U_HALVES = 3 * NB * 2 * WAVE * 8;  // U, high, low
    static constexpr size_t BYTES = Y_FLOATS * 4 > U_HALVES * 2 ? Y_FLOATS * 4 : U_HALVES * 2;
};

template <int D, int NB>
constexpr size_t tp_scan_lds_bytes(bool out_bf16) {
    return TpShape<D, NB>::RING * sizeof(TpSlot<D, NB>)  // ring
           + 2 * (D / 32) * NB * WAVE * 8 * 2            // S^T high / low
           + TpsXchg<D, NB>::BYTES                       // partial Y, or U and its parts
           + NB * 2 * WAVE * 8 * 2                       // R
           + (size_t)CHUNK * 16 * NB * (out_bf16 ? 2 : 4);  // outputs
}

// MODE 0: the scan.  MODE 1: both parts of a segment's state map, no outputs:
// the first half of the units runs from zero (the affine part B), the second
// half from the identity without the value term (the transition R), so that
// S_end = S_start R + B.  Both halves write state_out at their unit.
template <int D, bool OUT_BF16, int NB, int MODE = 0>
__global__ __launch_bounds__(TPS_MAX_THREADS) void chunk_scan_tp_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const char* __restrict__ recs, const SeqInfo* __restrict__ info, const float* __restrict__ state_in,
    float* __restrict__ state_out, void* __restrict__ out, char* __restrict__ sink, int units, int T, int h_k,
    int h_v, unsigned* __restrict__ status) {
    using Sh = TpShape<D, NB>;
    using Ro = TpsRoles<D, NB>;
    using Slot = TpSlot<D, NB>;
    constexpr int RS = Sh::RS, SLICES = D / RS, NKB = Sh::NKB, RING = Sh::RING, CPB = Ro::CPB, KPW = Ro::KPW;
    constexpr int OB = OUT_BF16 ? 2 : 4;  // bytes per output element
    __shared__ __align__(16) Slot ring[RING];
    __shared__ __align__(16) uint16_t sShi[NKB * NB * WAVE * 8];  // S^T high / low B fragments (kb, row block)
    __shared__ __align__(16) uint16_t sSlo[NKB * NB * WAVE * 8];
    __shared__ __align__(16) char sX[TpsXchg<D, NB>::BYTES];
    float* sY = reinterpret_cast<float*>(sX);                    // partial Y tiles (row block, chain wave, token block)
    _Float16* sU = reinterpret_cast<_Float16*>(sX);              // U as fp16 B fragments (kb, row block)
    uint16_t* sUh = reinterpret_cast<uint16_t*>(sX) + NB * 2 * WAVE * 8;  // diag(s c) U high / low B fragments
    uint16_t* sUl = sUh + NB * 2 * WAVE * 8;
    __shared__ __align__(16) _Float16 sR[NB * 2 * WAVE * 8];     // R as fp16 B fragments (kb, row block)
    __shared__ __align__(16) char sO[CHUNK * RS * OB];           // one block's 64 x RS outputs, row-major
    // Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8).
    // The SLICES workgroups of one (sequence, v-head) unit are placed on the
    // same XCD, so they share each block's inputs through that XCD's L2.
    const int xcd = blockIdx.x % 8, m = blockIdx.x / 8;
    const int slice = m % SLICES;
    const int unit = (m / SLICES) * 8 + xcd;  // sequence * h_v + v-head
    if (unit >= units) return;
    const bool lin = MODE == 1 && unit >= units / 2;
    const int su = lin ? unit - units / 2 : unit;
    const int n = su / h_v, h = su - n * h_v;
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);  // wave-uniform: role branches stay scalar
    const int j16 = lane & 15, q4 = lane >> 4;
    const int r0 = slice * RS;
    int begin, len, slot0;
    if (info) {
        const SeqInfo si = info[n];
        begin = si.begin; len = si.len; slot0 = si.slot_base;
    } else {
        begin = 0; len = T; slot0 = 0;
    }
    const int nchunks = (len + CHUNK - 1) / CHUNK;
    const int hk = h / (h_v / h_k);
    auto rec_of = [&](int c) __attribute__((always_inline)) {
        return recs + ((size_t)(slot0 + c) * h_v + h) * TpRec::BYTES;
    };

    bool bad = false;  // a non-finite output or final state in this lane (token and chain waves)

    if (w >= Ro::CHAIN + Ro::OUTW) {
        // ------------------------------ copier waves ------------------------------
        typedef __attribute__((address_space(3))) void* lds_ptr;
        const int lw = w - Ro::CHAIN - Ro::OUTW;
        constexpr int RPI = 1024 / (2 * D), UPR = D / 8;   // rows per 1 KiB load, 16-byte units per row
        constexpr int HPT = RS / 2, TPI = 256 / (2 * RS);  // 4-byte pieces per token of the v slice, tokens per load
        // Load i = 4 mm + lw of a block's copy (token indices clamped into [0, T)).  Every
        // kind of load (k, v, T and P, factors) comes in a multiple of four, so the
        // kind depends on mm alone and is fixed when the loop over mm is unrolled.
        static_assert(Sh::NK % Ro::LOAD == 0 && Sh::NV % Ro::LOAD == 0 && (2 * TpRec::NF) % Ro::LOAD == 0 &&
                          4 % Ro::LOAD == 0, "load kinds in multiples of the copier count");
        // 1 KiB piece i of a raw q or k tile (RPI whole rows), XOR-swizzled as raw_unit
        auto tile_load = [&](const void* base, int tok0, uint16_t* dst, int i) __attribute__((always_inline)) {
            const int r = i * RPI + lane / UPR, p = lane % UPR;
            const int u = p ^ (r & (UPR - 1));  // the global unit this lane's LDS slot holds
            const size_t tt = (size_t)min(tok0 + r, T - 1);
            const uint16_t* src = reinterpret_cast<const uint16_t*>(base) + (tt * h_k + hk) * D + 8 * u;
            __builtin_amdgcn_global_load_lds(src, (lds_ptr)(dst + i * 512), 16, 0, 0);
        };
        auto load = [&](int c, int mm) __attribute__((always_inline)) {
            Slot* sl = &ring[c % RING];
            const int tok0 = begin + c * CHUNK;
            const int i = Ro::LOAD * mm + lw;
            if (Ro::LOAD * mm < Sh::NK) {
                tile_load(k, tok0, sl->k, i);
            } else if (Ro::LOAD * mm < Sh::NK + Sh::NV) {
                const int jv = i - Sh::NK, r = jv * TPI + lane / HPT, e2 = lane % HPT;
                const size_t tt = (size_t)min(tok0 + r, T - 1);
                const uint16_t* src = reinterpret_cast<const uint16_t*>(v) + (tt * h_v + h) * D + r0 + 2 * e2;
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)(sl->vs + jv * 128), 4, 0, 0);
            } else if (Ro::LOAD * mm < Sh::NK + Sh::NV + 2 * TpRec::NF) {
                const int j = i - Sh::NK - Sh::NV;
                const char* rec = rec_of(c);
                __builtin_amdgcn_global_load_lds(rec + (size_t)j * 1024 + lane * 16,
                                                 (lds_ptr)(reinterpret_cast<char*>(sl->tp) + j * 1024), 16, 0, 0);
            } else {
                const int j = i - Sh::NK - Sh::NV - 2 * TpRec::NF;
                const char* rec = rec_of(c);
                __builtin_amdgcn_global_load_lds(rec + TpRec::F + (size_t)j * 256 + lane * 4,
                                                 (lds_ptr)(reinterpret_cast<char*>(sl->fac) + j * 256), 4, 0, 0);
            }
        };
        auto copy = [&](int c) __attribute__((always_inline)) {
#pragma unroll
            for (int mm = 0; mm < Sh::L; ++mm) load(c, mm);
        };
        if (nchunks > 0) copy(0);
        if (nchunks > 1) {
            copy(1);
            wait_vmcnt<Sh::L>();
        } else {
            wait_vmcnt<0>();
        }
        // (block 1 is waited for at BR of block 0 like any other)
        for (int c = 0; c < nchunks; ++c) {
            lds_barrier();  // B1: the slot of block c - 1 is free
            if (c + 2 < nchunks) copy(c + 2);
            lds_barrier();  // BX
            // Loads complete in issue order: once no more than block c + 2's slot loads are
            // outstanding, block c + 1 (slot and q) has landed, and BR publishes it.
            if (c + 1 < nchunks) {
                if (c + 2 < nchunks) wait_vmcnt<Sh::L>();
                else wait_vmcnt<0>();
            }
            lds_barrier();  // BR: block c + 1 has landed
            lds_barrier();  // BU
        }
        lds_barrier();  // B1 after the last block
        lds_barrier();  // BF
        return;
    }

    // Block c's outputs from sO to out, by thread t of NT: 16-byte pieces, rows past
    // the sequence's end to the sink.
    constexpr int LPR = RS * OB / 16;  // 16-byte pieces per output row
    constexpr int PIECES = CHUNK * LPR;
    auto store_out = [&](int c, int t, int NT) __attribute__((always_inline)) {
        const int nt = min(CHUNK, len - c * CHUNK);
        for (int p = t; p < PIECES; p += NT) {
            const int row = p / LPR, col16 = p % LPR;
            const uint4 val = *reinterpret_cast<const uint4*>(sO + row * RS * OB + col16 * 16);
            char* dst = row < nt ? reinterpret_cast<char*>(out) +
                                       (((size_t)(begin + c * CHUNK + row) * h_v + h) * D + r0) * OB + col16 * 16
                                 : sink + (t % WAVE) * 16;
            *reinterpret_cast<uint4*>(dst) = val;
        }
    };

    if (w >= Ro::CHAIN) {
        // ------------------------------ token waves ------------------------------
        const int tb = w - Ro::CHAIN;
        const int kbt = tb >> 1, part = tb & 1;  // this token block's 32-token block and half
        // A fragments of Q^raw (token block tb, in the order of the S^T fragments), two
        // blocks deep: block c's are loaded during block c - 2, after the barrier BU.
        bf8_t qa[2][NKB];
        auto load_q = [&](int c, bf8_t(&dst)[NKB]) __attribute__((always_inline)) {
            const size_t tt = (size_t)min(begin + c * CHUNK + 16 * tb + j16, T - 1);
            const char* row = reinterpret_cast<const char*>(q) + ((tt * h_k + hk) * D) * 2;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const uint2 x0 = *reinterpret_cast<const uint2*>(row + (32 * kb + 4 * q4) * 2);
                const uint2 x1 = *reinterpret_cast<const uint2*>(row + (32 * kb + 16 + 4 * q4) * 2);
                dst[kb] = __builtin_bit_cast(bf8_t, uint4{x0.x, x0.y, x1.x, x1.y});
            }
        };
        auto step = [&](int c, bf8_t(&cur)[NKB]) __attribute__((always_inline)) {
            const Slot& B = ring[c % RING];
            typedef __attribute__((address_space(3))) s4v_t* lds_s4;
            f4_t zc[NB];
            lds_barrier();  // B1: block c in its slot, S^T of block c in LDS
            // Everything of block c's slot that the later phases read, read now (one LDS round
            // trip less in each of them): factors, v, and the T and P fragments of token block
            // tb (for tb < 2 the second fragment repeats the first and goes unused).
            const f4_t gck = *reinterpret_cast<const f4_t*>(&B.fac[TpRec::GCK + 16 * tb + 4 * q4]);
            const f4_t sc = *reinterpret_cast<const f4_t*>(&B.fac[TpRec::SCK + 16 * tb + 4 * q4]);
            const f4_t gcq = *reinterpret_cast<const f4_t*>(&B.fac[TpRec::GCQ + 16 * tb + 4 * q4]);
            s4v_t vv[NB];
            if (!lin) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)  // v[token 16tb + 4q + e][row 16nb + j], e = 0..3
                    vv[nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s4)(B.vs + (16 * tb + 4 * q4 + (j16 >> 2)) * RS + 16 * nb + 4 * (j16 & 3)));
            }
            Frag<_Float16> tf[2], pf[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                tf[kb] = frag_stored<_Float16>(B.tp[0], tri_frag(tb, kb), lane);
                if (MODE == 0) pf[kb] = frag_stored<_Float16>(B.tp[1], tri_frag(tb, kb), lane);
            }
            if (MODE == 0) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {  // Z = Q^raw S^T, high and low parts into one accumulator
                    f4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        mma_bf16(acc, cur[kb], bfrag(sShi, kb * NB + nb, lane));
                        mma_bf16(acc, cur[kb], bfrag(sSlo, kb * NB + nb, lane));
                    }
                    zc[nb] = acc;
                }
            }
            lds_barrier();  // BX: partial products in LDS
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {  // R = V - diag(gamma c) Y, token block tb
                f4_t yy = *reinterpret_cast<const f4_t*>(sY + (((nb * CPB) * 4 + tb) * WAVE + lane) * 4);
#pragma unroll
                for (int cq = 1; cq < CPB; ++cq)
                    yy += *reinterpret_cast<const f4_t*>(sY + (((nb * CPB + cq) * 4 + tb) * WAVE + lane) * 4);
                f4_t r;
                if (lin) {
                    r = -(gck * yy);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        r[e] = __uint_as_float((uint32_t)(uint16_t)vv[nb][e] << 16) - gck[e] * yy[e];
                }
                store_part<_Float16>(sR, kbt * NB + nb, part, lane, r);
            }
            lds_barrier();  // BR: R in LDS
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {  // U = T R (T is zero right of its diagonal block), its parts
                f4_t u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    if (kb <= kbt) mma(u, tf[kb], frag_stored<_Float16>(sR, kb * NB + nb, lane));
                if (MODE == 0) store_part<_Float16>(sU, kbt * NB + nb, part, lane, u);
                store_split(sUh, sUl, kbt * NB + nb, part, lane, u * sc);
            }
            lds_barrier();  // BU: U and its parts in LDS
            if (MODE == 0) {  // O = diag(gamma c_q) Z + P U, token block tb
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    f4_t o = gcq * zc[nb];
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
                        if (kb <= kbt) mma(o, pf[kb], frag_stored<_Float16>(sU, kb * NB + nb, lane));
                    bad |= any_nonfinite(o);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = (16 * tb + 4 * q4 + r) * RS + 16 * nb + j16;
                        if constexpr (OUT_BF16) reinterpret_cast<__bf16*>(sO)[e] = (__bf16)o[r];
                        else reinterpret_cast<float*>(sO)[e] = o[r];
                    }
                }
                if (c + 2 < nchunks) load_q(c + 2, cur);
            }
        };
        if (MODE == 0 && nchunks > 0) load_q(0, qa[0]);
        if (MODE == 0 && nchunks > 1) load_q(1, qa[1]);
        for (int c = 0; c < nchunks; c += 2) {
            step(c, qa[0]);
            if (c + 1 < nchunks) step(c + 1, qa[1]);
        }
        lds_barrier();  // B1 after the last block
        lds_barrier();  // BF
        if (MODE == 0) report_status(status, bad, GDN_PREFILL_STATUS_NONFINITE);
        return;
    }

    // ------------------------------ chain waves ------------------------------
    const int s = w / CPB, cq = w % CPB;  // row block, share of the key dimension
    const int mb0 = 2 * KPW * cq;         // first S^T tile of this share
    f4_t St[2 * KPW];
    bf8_t shi[KPW], slo[KPW];
    const size_t sbase = (size_t)unit * D * D;
    const int srow = r0 + 16 * s + j16;
#pragma unroll
    for (int i = 0; i < 2 * KPW; ++i) {
        const int col = 16 * (mb0 + i) + 4 * q4;
        if (lin) {  // identity: S[r][c] = (r == c)
            St[i] = f4_t{srow == col ? 1.f : 0.f, srow == col + 1 ? 1.f : 0.f, srow == col + 2 ? 1.f : 0.f,
                         srow == col + 3 ? 1.f : 0.f};
        } else if (state_in) {
            const float4 x = *reinterpret_cast<const float4*>(state_in + sbase + (size_t)srow * D + col);
            St[i] = f4_t{x.x, x.y, x.z, x.w};
        } else {
            St[i] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    auto publish = [&]() __attribute__((always_inline)) {  // this share's high / low B fragments, registers and LDS
#pragma unroll
        for (int kk = 0; kk < KPW; ++kk) {
            split_from_acc(St[2 * kk], St[2 * kk + 1], shi[kk], slo[kk]);
            const int kb = KPW * cq + kk;
            bfrag_store(sShi, kb * NB + s, lane, shi[kk]);
            bfrag_store(sSlo, kb * NB + s, lane, slo[kk]);
        }
    };
    publish();
    float* yown = sY + (size_t)(s * CPB + cq) * 4 * WAVE * 4;
    bf8_t ka[4][KPW];  // K^raw row fragments of this share for the next Y, read one phase early
    auto read_ka = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int kk = 0; kk < KPW; ++kk) ka[tb][kk] = raw_rowfrag<D>(ring[c % RING].k, tb, KPW * cq + kk, lane);
    };
    for (int c = 0; c < nchunks; ++c) {
        const Slot& B = ring[c % RING];
        lds_barrier();  // B1: block c in its slot
        if (c == 0) read_ka(0);
        {   // ---- partial Y = K^raw S^T over this share (high and low parts into one accumulator) ----
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                f4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KPW; ++kk) {
                    mma_bf16(acc, ka[tb][kk], shi[kk]);
                    mma_bf16(acc, ka[tb][kk], slo[kk]);
                }
                *reinterpret_cast<f4_t*>(yown + (tb * WAVE + lane) * 4) = acc;
            }
        }
        lds_barrier();  // BX: partial products in LDS; the outputs of block c - 1 in sO
        if (MODE == 0 && c >= 1) store_out(c - 1, w * WAVE + lane, Ro::CHAIN * WAVE);
        bf8_t kt[2 * KPW][2];  // K^raw^T column fragments of this share, read while R and U form
#pragma unroll
        for (int i = 0; i < 2 * KPW; ++i)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) kt[i][kk] = raw_colfrag<D>(B.k, mb0 + i, kk, lane);
        lds_barrier();  // BR: block c + 1 has landed
        if (c + 1 < nchunks) read_ka(c + 1);
        const float gn = B.fac[TpRec::GN];
        lds_barrier();  // BU: diag(s c) U high / low parts in LDS
        {   // ---- this share of S^T <- gamma_n S^T + K^raw^T diag(s c) U ----
            bf8_t uh[2], ul[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uh[kk] = bfrag(sUh, kk * NB + s, lane);
                ul[kk] = bfrag(sUl, kk * NB + s, lane);
            }
#pragma unroll
            for (int i = 0; i < 2 * KPW; ++i) {
                St[i] *= gn;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    mma_bf16(St[i], kt[i][kk], uh[kk]);
                    mma_bf16(St[i], kt[i][kk], ul[kk]);
                }
            }
        }
        publish();
    }
    lds_barrier();  // B1 after the last block
    lds_barrier();  // BF: the last block's outputs are in sO
    if (MODE == 0 && nchunks > 0) store_out(nchunks - 1, w * WAVE + lane, Ro::CHAIN * WAVE);
    if (state_out) {
#pragma unroll
        for (int i = 0; i < 2 * KPW; ++i)
            *reinterpret_cast<float4*>(state_out + sbase + (size_t)srow * D + 16 * (mb0 + i) + 4 * q4) =
                make_float4(St[i][0], St[i][1], St[i][2], St[i][3]);
    }
    if (MODE == 0) {
#pragma unroll
        for (int i = 0; i < 2 * KPW; ++i) bad |= any_nonfinite(St[i]);
        report_status(status, bad, GDN_PREFILL_STATUS_NONFINITE);
    }
}

// ============================================================================================
// chunk_scan_tpf: the scan for 16-row slices, two waves per token block
// ============================================================================================
// The arithmetic of chunk_scan_tp (MODE 0, one 16-row slice per workgroup) on
// fp16 matrix cores with power-of-two scaling instead of bf16 high / low parts:
//   * keys and queries come from the key records, each token's row scaled by
//     2^-E and rounded to fp16; the factors 2^E join gamma c, s c and gamma c_q;
//   * S^T is published as one fp16 fragment per 32-wide key block kb, each of
//     its 16 columns (rows of S) scaled by 2^-F(kb, column), F the exponent of
//     that column's largest magnitude in the block, so every element is below 1
//     and the fp32 range of S is kept.  A product with S^T keeps one
//     accumulator per kb and sums them with the factors 2^F;
//   * diag(s c 2^E) U, the operand of the update, is one fp16 fragment like U.
// The roles are arranged so that no partial product crosses waves; per-wave LDS
// reads are the scarce resource, so the work of token block tb is split over
// two waves:
//   Y-wave tb (w = tb):     Y and R, U = T R and diag(s c 2^E) U, and the output
//                           stores; the Y-waves w < D / 32 also hold the fp32 S^T
//                           tiles of key block w and update and publish them;
//   Z-wave tb (w = 4 + tb): Z = Q S^T (the query fragments loaded straight into
//                           registers) and O = diag(gamma c_q 2^E) Z + P U;
//   copier waves (w = 8..11) stream the keys, v, T, P and the factors into LDS.
// Three barriers per block:
//   B1  block c in its slot, S^T published  -> Y-waves: Y, R;  Z-waves: Z
//   BR  R in LDS                            -> Y-waves: U, diag(s c 2^E) U, block c - 1's outputs to HBM;
//                                              Z-waves: the queries of block c + 2
//   BU  U and diag(s c 2^E) U in LDS        -> Y-waves: S^T update, published;  Z-waves: O, to LDS
// Reads that phase B1 does not need (T, P and their factors) wait until after BR:
// phase B1 is the one bound by the workgroup's LDS read bandwidth, and for the same
// reason a Y-wave takes its own key block of S^T from registers.
// Inside the block loop the Y-waves store but never load and the Z-waves load but
// never store: a wave's memory counter covers both, so a Z-wave's wait for its
// queries never waits for output stores.

constexpr int TPF_YW = 4, TPF_ZW = 4, TPF_LOAD = 4;
constexpr int TPF_COMPUTE = TPF_YW + TPF_ZW;
constexpr int TPF_THREADS = (TPF_COMPUTE + TPF_LOAD) * WAVE;

template <int D>
struct TpfSlot {
    _Float16 k[CHUNK * D];                  // scaled fp16 keys (swizzled rows), from the key record
    uint16_t vs[CHUNK * 16];                // the slice's raw values [token][16]
    _Float16 tp[2][TpRec::NF * WAVE * 8];   // T and P fragments, as in the record
    float fac[256];                         // gck, gcq, sck, gamma_n
    float es[256];                          // 2^E of the keys and of the queries
};

template <int D, bool OUT_BF16>
constexpr size_t tpf_scan_lds_bytes() {
    return 3 * sizeof(TpfSlot<D>)             // ring
           + (D / 32) * WAVE * 8 * 2          // S^T fragments
           + 16 * 4 * 4                       // their column factors
           + 3 * 2 * WAVE * 8 * 2             // R, U, diag(s c 2^E) U
           + (size_t)CHUNK * 16 * (OUT_BF16 ? 2 : 4);  // outputs
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(TPF_THREADS) void chunk_scan_tpf_kernel(
    const void* __restrict__ v, const char* __restrict__ recs, const char* __restrict__ krecs,
    const SeqInfo* __restrict__ info, const float* __restrict__ state_in, float* __restrict__ state_out,
    void* __restrict__ out, char* __restrict__ sink, int units, int T, int h_k, int h_v,
    unsigned* __restrict__ status) {
    using Slot = TpfSlot<D>;
    using KR = KeyRec16<D>;
    constexpr int RS = 16, SLICES = D / RS, NKB = D / 32, RING = 3;
    constexpr int NK = CHUNK * D * 2 / 1024;   // 1 KiB loads of a key or query tile
    constexpr int NV = CHUNK * RS * 2 / 1024;  // 1 KiB loads of the v slice
    constexpr int KL = NK / TPF_LOAD;          // key (or query) loads per copier wave
    constexpr int TPL = 2 * TpRec::NF / TPF_LOAD;  // T and P loads per copier wave
    static_assert(NK % TPF_LOAD == 0 && (2 * TpRec::NF) % TPF_LOAD == 0 && NV + 2 == TPF_LOAD,
                  "copy split over the copier waves");
    static_assert(NKB <= TPF_YW && NKB <= 4, "one key block of S^T per holding Y-wave");
    constexpr int OB = OUT_BF16 ? 2 : 4;  // bytes per output element
    __shared__ __align__(16) Slot ring[RING];
    __shared__ __align__(16) _Float16 sS[NKB * WAVE * 8];         // S^T fragments (kb), scaled
    __shared__ __align__(16) float sScl[16 * 4];                  // 2^F of column j, key block kb at [4 j + kb]
    __shared__ __align__(16) _Float16 sR[2 * WAVE * 8];           // R, fp16 B fragments (32-token block)
    __shared__ __align__(16) _Float16 sU[2 * WAVE * 8];           // U
    __shared__ __align__(16) _Float16 sUs[2 * WAVE * 8];          // diag(s c 2^E) U
    __shared__ __align__(16) char sO[CHUNK * RS * OB];            // one block's 64 x 16 outputs, row-major
    // XCD placement as in chunk_scan_tp: a unit's SLICES workgroups share an XCD.
    const int xcd = blockIdx.x % 8, m = blockIdx.x / 8;
    const int slice = m % SLICES;
    const int unit = (m / SLICES) * 8 + xcd;  // sequence * h_v + v-head
    if (unit >= units) return;
    const int n = unit / h_v, h = unit - n * h_v;
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int j16 = lane & 15, q4 = lane >> 4;
    const int r0 = slice * RS;
    int begin, len, slot0;
    if (info) {
        const SeqInfo si = info[n];
        begin = si.begin; len = si.len; slot0 = si.slot_base;
    } else {
        begin = 0; len = T; slot0 = 0;
    }
    const int nchunks = (len + CHUNK - 1) / CHUNK;
    const int hk = h / (h_v / h_k);

    if (w >= TPF_COMPUTE) {
        // ------------------------------ copier waves ------------------------------
        // Block c + 2 is copied during block c: its keys after B1 (the slot of block
        // c - 1 is free), T, P, the v slice and the factors after BU.  Every load moves
        // 16 bytes a lane; copiers 0 .. NV - 1 also take a 1 KiB piece of the v slice,
        // copier NV the record's factors and copier NV + 1 the key record's.  Before B1
        // of block c + 1 a copier waits until only block c + 2's loads are in flight.
        typedef __attribute__((address_space(3))) void* lds_ptr;
        const int lw = w - TPF_COMPUTE;
        auto krec = [&](int c) __attribute__((always_inline)) {
            return krecs + ((size_t)(slot0 + c) * h_k + hk) * KR::BYTES;
        };
        auto copy_k = [&](int c) __attribute__((always_inline)) {
            const char* src = krec(c) + KR::K;
            char* dst = reinterpret_cast<char*>(ring[c % RING].k);
#pragma unroll
            for (int mm = 0; mm < KL; ++mm) {
                const int j = TPF_LOAD * mm + lw;
                __builtin_amdgcn_global_load_lds(src + j * 1024 + lane * 16, (lds_ptr)(dst + j * 1024), 16, 0, 0);
            }
        };
        auto copy_rest = [&](int c) __attribute__((always_inline)) {
            Slot* sl = &ring[c % RING];
            const char* rec = recs + ((size_t)(slot0 + c) * h_v + h) * TpRec::BYTES;
#pragma unroll
            for (int mm = 0; mm < TPL; ++mm) {
                const int j = TPF_LOAD * mm + lw;
                __builtin_amdgcn_global_load_lds(rec + (size_t)j * 1024 + lane * 16,
                                                 (lds_ptr)(reinterpret_cast<char*>(sl->tp) + j * 1024), 16, 0, 0);
            }
            if (lw < NV) {  // tokens 32 lw .. + 31 of the v slice, half a token's 16 values a lane
                const int r = lw * (CHUNK / NV) + lane / 2;
                const size_t tt = (size_t)min(begin + c * CHUNK + r, T - 1);
                const uint16_t* src = reinterpret_cast<const uint16_t*>(v) + (tt * h_v + h) * D + r0 + 8 * (lane & 1);
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)(sl->vs + lw * 512), 16, 0, 0);
            } else if (lw == NV) {
                __builtin_amdgcn_global_load_lds(rec + TpRec::F + lane * 16, (lds_ptr)(sl->fac), 16, 0, 0);
            } else {
                const char* src = krec(c) + KR::E + lane * 16;
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)(sl->es), 16, 0, 0);
            }
        };
        constexpr int LB = KL + TPL + 1;  // loads per block of every copier
        if (nchunks > 0) { copy_k(0); copy_rest(0); }
        if (nchunks > 1) {
            copy_k(1); copy_rest(1);
            wait_vmcnt<LB>();
        } else {
            wait_vmcnt<0>();
        }
        for (int c = 0; c < nchunks; ++c) {
            lds_barrier();  // B1
            if (c + 2 < nchunks) copy_k(c + 2);
            lds_barrier();  // BR
            lds_barrier();  // BU
            if (c + 2 < nchunks) copy_rest(c + 2);
            if (c + 1 < nchunks) {
                if (c + 2 < nchunks) wait_vmcnt<LB>();
                else wait_vmcnt<0>();
            }
        }
        lds_barrier();  // B1 after the last block
        return;
    }

    bool bad = false;  // a non-finite output or final state in this lane
    typedef __attribute__((address_space(3))) s4v_t* lds_s4;
    const f4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    // Sum over the key blocks of a product with S^T: acc[i] times scl[i], the factor
    // 2^F of acc[i]'s key block and column j16.  Arrays are indexed by loop position
    // only (a runtime index into a register array would compile to indexed register
    // moves); a rotation of the key blocks goes into the LDS addresses of the reads.
    auto combine = [&](const f4_t (&acc)[NKB], const float (&scl)[NKB]) __attribute__((always_inline)) {
        f4_t s = acc[0] * scl[0];
#pragma unroll
        for (int i = 1; i < NKB; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] = fmaf(acc[i][e], scl[i], s[e]);
        return s;
    };
    // Each phase first issues the LDS reads that its products need, then a scheduling
    // barrier: left alone the compiler puts every read just before its use and waits
    // for it there, one read latency per product.
    constexpr int LPR = RS * OB / 16;  // 16-byte pieces per output row
    constexpr int PIECES = CHUNK * LPR;
    // Block c's outputs, sO to HBM, by the Y-waves (they issue no loads, so no load
    // wait ever covers these stores).
    auto store_out = [&](int c, int yw) __attribute__((always_inline)) {
        const int nt = min(CHUNK, len - c * CHUNK), t = yw * WAVE + lane;
        for (int p = t; p < PIECES; p += TPF_YW * WAVE) {
            const int row = p / LPR, col16 = p % LPR;
            const uint4 val = *reinterpret_cast<const uint4*>(sO + row * RS * OB + col16 * 16);
            char* dst = row < nt ? reinterpret_cast<char*>(out) +
                                       (((size_t)(begin + c * CHUNK + row) * h_v + h) * D + r0) * OB + col16 * 16
                                 : sink + (t % WAVE) * 16;
            *reinterpret_cast<uint4*>(dst) = val;
        }
    };
    if (w >= TPF_YW) {
        // ------------------------------ Z-waves ------------------------------
        // The query fragments of token block tb go straight from the key record into
        // registers, two blocks ahead: block c + 2's after BR of block c, into the set
        // block c has just used.  The loop is unrolled by two so that the sets are
        // fixed registers.  These waves issue no stores, so each wait covers loads only.
        const int tb = w - TPF_YW, kbt = tb >> 1;
        auto load_q = [&](h8_t (&qs)[NKB], int c) __attribute__((always_inline)) {
            const char* src = krecs + ((size_t)(slot0 + c) * h_k + hk) * KR::BYTES + KR::Q;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                qs[kb] = *reinterpret_cast<const h8_t*>(src + ((size_t)(tb * NKB + kb) * WAVE + lane) * 16);
        };
        auto block = [&](int c, h8_t (&qs)[NKB]) __attribute__((always_inline)) {
            const Slot& B = ring[c % RING];
            lds_barrier();  // B1: block c in its slot, S^T published
            // ---- Z = Q S^T for token block tb, one accumulator per key block ----
            h8_t sf[NKB];
            float scl[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                sf[kb] = *reinterpret_cast<const h8_t*>(&sS[(kb * WAVE + lane) * 8]);
                scl[kb] = sScl[4 * j16 + kb];
            }
            __builtin_amdgcn_sched_barrier(0);
            f4_t za[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                za[kb] = zero4;
                mma_f16(za[kb], qs[kb], sf[kb]);
            }
            f4_t z = combine(za, scl);
            // Z is complete in this phase: keeps the compiler from sinking its products
            // into phase BU, where they would contend with the Y-wave's update on this SIMD.
            asm volatile("" : "+v"(z));
            lds_barrier();  // BR
            // (the last two blocks reload the last block: an unconditional load keeps the
            // compiler's wait for a set at "all but the other set's four loads")
            load_q(qs, min(c + 2, nchunks - 1));
            const f4_t gcq = *reinterpret_cast<const f4_t*>(&B.fac[TpRec::GCQ + 16 * tb + 4 * q4]) *
                             *reinterpret_cast<const f4_t*>(&B.es[KR::EQ + 16 * tb + 4 * q4]);
            Frag<_Float16> pf[2];  // (for tb < 2 the second fragment repeats the first and goes unused)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) pf[kb] = frag_stored<_Float16>(B.tp[1], tri_frag(tb, kb), lane);
            lds_barrier();  // BU: U in LDS; sO is no longer read
            {   // ---- O = diag(gamma c_q 2^E) Z + P U ----
                f4_t o = gcq * z;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    if (kb <= kbt) mma(o, pf[kb], frag_stored<_Float16>(sU, kb, lane));
                bad |= any_nonfinite(o);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = (16 * tb + 4 * q4 + r) * RS + j16;
                    if constexpr (OUT_BF16) reinterpret_cast<__bf16*>(sO)[e] = (__bf16)o[r];
                    else reinterpret_cast<float*>(sO)[e] = o[r];
                }
            }
        };
        if (nchunks > 0) {
            h8_t qa[NKB], qb[NKB];
            load_q(qa, 0);
            load_q(qb, min(1, nchunks - 1));
            // whole pairs, so that no path skips a set's loads (the compiler's waits then
            // hold a set's loads only)
            int c = 0;
            for (; c + 1 < nchunks; c += 2) {
                block(c, qa);
                block(c + 1, qb);
            }
            if (c < nchunks) block(c, qa);
        }
        lds_barrier();  // B1 after the last block
        report_status(status, bad, GDN_PREFILL_STATUS_NONFINITE);
        return;
    }

    // ------------------------------ Y-waves ------------------------------
    const int tb = w, kbt = tb >> 1, part = tb & 1;  // token block, its 32-token block and half
    const bool holder = w < NKB;  // holds S^T tiles 32 w .. 32 w + 31 of the keys
    f4_t St[2];  // the two 16-key accumulator tiles of key block w x this slice's 16 rows
    const size_t sbase = (size_t)unit * D * D;
    const int srow = r0 + j16;
    if (holder) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int col = 32 * w + 8 * q4 + 4 * i;  // the permuted key order (h16_row8)
            if (state_in) {
                const float4 x = *reinterpret_cast<const float4*>(state_in + sbase + (size_t)srow * D + col);
                St[i] = f4_t{x.x, x.y, x.z, x.w};
            } else {
                St[i] = zero4;
            }
        }
    }
    h8_t own;  // this holder's published fragment
    auto publish = [&]() __attribute__((always_inline)) {
        // the column's largest magnitude over key block w: each lane holds 8 of its 32
        // entries, the lanes j16 + 16 q of the four rows of lanes the rest
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(St[i][e]));
        // (magnitudes: their bit patterns order as unsigned integers, and an integer
        // maximum needs no canonicalising of its inputs)
        auto umax = [](float a, float b) { return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b))); };
        F2 t = permlane16_swap(mx, mx);
        mx = umax(t.x, t.y);
        t = permlane32_swap(mx, mx);
        mx = umax(t.x, t.y);
        const int F = __builtin_amdgcn_frexp_expf(mx);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            own[e] = (_Float16)__builtin_amdgcn_ldexpf(St[0][e], -F);
            own[e + 4] = (_Float16)__builtin_amdgcn_ldexpf(St[1][e], -F);
        }
        *reinterpret_cast<h8_t*>(&sS[(w * WAVE + lane) * 8]) = own;
        if (q4 == 0) sScl[4 * j16 + w] = __builtin_amdgcn_ldexpf(1.f, F);
    };
    if (holder) publish();
    for (int c = 0; c < nchunks; ++c) {
        const Slot& B = ring[c % RING];
        lds_barrier();  // B1: block c in its slot, S^T published
        // ---- Y = K S^T and R = V - diag(gamma c 2^E) Y for token block tb ----
        const s4v_t vv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(  // v[token 16tb + 4q + e][row j]
            (lds_s4)(B.vs + (16 * tb + 4 * q4 + (j16 >> 2)) * RS + 4 * (j16 & 3)));
        const f4_t gck = *reinterpret_cast<const f4_t*>(&B.fac[TpRec::GCK + 16 * tb + 4 * q4]) *
                         *reinterpret_cast<const f4_t*>(&B.es[KR::EK + 16 * tb + 4 * q4]);
        // key blocks from this wave's own on (its fragment is in registers)
        const int rot = holder ? w : 0;
        h8_t ka[NKB], sf[NKB];
        float scl[NKB];
#pragma unroll
        for (int kr = 0; kr < NKB; ++kr) {
            const int kb = (kr + rot) & (NKB - 1);
            ka[kr] = h16_row8<D>(B.k, tb, kb, lane);
            sf[kr] = (holder && kr == 0) ? own : *reinterpret_cast<const h8_t*>(&sS[(kb * WAVE + lane) * 8]);
            scl[kr] = sScl[4 * j16 + kb];
        }
        __builtin_amdgcn_sched_barrier(0);
        f4_t ya[NKB];
#pragma unroll
        for (int kr = 0; kr < NKB; ++kr) {
            ya[kr] = zero4;
            mma_f16(ya[kr], ka[kr], sf[kr]);
        }
        {
            const f4_t yy = combine(ya, scl);
            f4_t r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = fmaf(-gck[e], yy[e], __uint_as_float((uint32_t)(uint16_t)vv[e] << 16));
            store_part<_Float16>(sR, kbt, part, lane, r);
        }
        lds_barrier();  // BR: R in LDS; S^T is no longer read
        const f4_t sc = *reinterpret_cast<const f4_t*>(&B.fac[TpRec::SCK + 16 * tb + 4 * q4]) *
                        *reinterpret_cast<const f4_t*>(&B.es[KR::EK + 16 * tb + 4 * q4]);
        Frag<_Float16> tf[2], rr[2];  // (for tb < 2 the second fragments go unused)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            tf[kb] = frag_stored<_Float16>(B.tp[0], tri_frag(tb, kb), lane);
            rr[kb] = frag_stored<_Float16>(sR, kb, lane);
        }
        h8_t kt[2][2];  // K^T column fragments of this holder's key tiles
        if (holder) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) kt[i][kk] = h16_colfrag_p<D>(B.k, 2 * w + i, kk, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- U = T R and diag(s c 2^E) U ----
        {
            f4_t u = zero4;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (kb <= kbt) mma(u, tf[kb], rr[kb]);
            store_part<_Float16>(sU, kbt, part, lane, u);
            store_part<_Float16>(sUs, kbt, part, lane, u * sc);
        }
        if (c >= 1) store_out(c - 1, w);
        lds_barrier();  // BU: U and diag(s c 2^E) U in LDS
        // ---- S^T <- gamma_n S^T + K^T diag(s c 2^E) U on this holder's tiles ----
        if (holder) {
            const float gn = B.fac[TpRec::GN];
            h8_t us[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) us[kk] = *reinterpret_cast<const h8_t*>(&sUs[(kk * WAVE + lane) * 8]);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                St[i] *= gn;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) mma_f16(St[i], kt[i][kk], us[kk]);
            }
            publish();
        }
    }
    lds_barrier();  // B1 after the last block: its outputs are in sO
    if (nchunks > 0) store_out(nchunks - 1, w);
    if (holder) {
        if (state_out) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                *reinterpret_cast<float4*>(state_out + sbase + (size_t)srow * D + 32 * w + 8 * q4 + 4 * i) =
                    make_float4(St[i][0], St[i][1], St[i][2], St[i][3]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) bad |= any_nonfinite(St[i]);
    }
    report_status(status, bad, GDN_PREFILL_STATUS_NONFINITE);
}

// ============================================================================================
// host launchers
// ============================================================================================
int compute_units();

size_t tp_record_bytes() { return TpRec::BYTES; }
size_t key16_record_bytes(int d) { return d == 128 ? KeyRec16<128>::BYTES : KeyRec16<64>::BYTES; }

template <int D, int NH>
static hipError_t launch_prep_pair_t(const void* q, const void* k, const float* g, const float* beta,
                                     const void* info, const int32_t* slot_seq, int slots, int T, int h_k, int h_v,
                                     int l2norm, float scale, char* recs, char* krecs, unsigned* clear_status,
                                     hipStream_t stream) {
    constexpr size_t lds = pair_lds_bytes<D, NH>();
    static_assert(lds <= 160 * 1024, "chunk_prep_pair LDS budget");
    auto kern = chunk_prep_pair_kernel<D, NH>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // two workgroups per compute unit (one's memory waits overlap the other's work), each a
    // contiguous run of items
    static_assert(2 * lds <= 160 * 1024, "two chunk_prep_pair workgroups per compute unit");
    const int items = slots * h_k * (h_v / h_k / NH), resident = 2 * compute_units();
    const int per = (items + resident - 1) / resident;
    const int grid = (items + per - 1) / per;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(PAIR_THREADS), lds, stream, q, k, g, beta,
                       reinterpret_cast<const SeqInfo*>(info), slot_seq, T, h_k, h_v, l2norm, scale, recs, krecs, slots,
                       per, clear_status);
    return hipGetLastError();
}

hipError_t launch_prep_bf16(int d, const void* q, const void* k, const float* g, const float* beta,
                            const void* info, const int32_t* slot_seq, int slots, int T, int h_k, int h_v,
                            int l2norm, float scale, void* recs, void* krecs, unsigned* clear_status,
                            hipStream_t stream) {
    char* r = reinterpret_cast<char*>(recs);
    char* kr = reinterpret_cast<char*>(krecs);
    unsigned* cs = clear_status;
    const bool pair = (h_v / h_k) % 2 == 0;
#define GDN_PREP(D, NH) \
    launch_prep_pair_t<D, NH>(q, k, g, beta, info, slot_seq, slots, T, h_k, h_v, l2norm, scale, r, kr, cs, stream)
    if (d == 128) return pair ? GDN_PREP(128, 2) : GDN_PREP(128, 1);
    if (d == 64) return pair ? GDN_PREP(64, 2) : GDN_PREP(64, 1);
#undef GDN_PREP
    return hipErrorInvalidValue;
}

template <int D, bool OB, int NB, int MODE>
static hipError_t launch_scan_tp_t(const void* q, const void* k, const void* v, const void* recs, const void* info,
                                   const float* s_in, float* s_out, void* out, void* sink, int units, int T, int h_k,
                                   int h_v, unsigned* status, hipStream_t stream) {
    static_assert(tp_scan_lds_bytes<D, NB>(OB) <= 160 * 1024, "chunk_scan_tp LDS budget");
    const int groups = (units + 7) / 8;  // see the XCD placement in chunk_scan_tp_kernel
    hipLaunchKernelGGL((chunk_scan_tp_kernel<D, OB, NB, MODE>), dim3(groups * 8 * (D / (16 * NB))), dim3(TpsRoles<D, NB>::THREADS),
                       0, stream, q, k, v, reinterpret_cast<const char*>(recs), reinterpret_cast<const SeqInfo*>(info),
                       s_in, s_out, out, reinterpret_cast<char*>(sink), units, T, h_k, h_v, status);
    return hipGetLastError();
}

template <int D, bool OB>
static hipError_t launch_scan_tpf_t(const void* v, const void* recs, const void* krecs, const void* info,
                                    const float* s_in, float* s_out, void* out, void* sink, int units, int T, int h_k,
                                    int h_v, unsigned* status, hipStream_t stream) {
    static_assert(tpf_scan_lds_bytes<D, OB>() <= 160 * 1024, "chunk_scan_tpf LDS budget");
    const int groups = (units + 7) / 8;  // see the XCD placement in chunk_scan_tp_kernel
    hipLaunchKernelGGL((chunk_scan_tpf_kernel<D, OB>), dim3(groups * 8 * (D / 16)), dim3(TPF_THREADS), 0, stream, v,
                       reinterpret_cast<const char*>(recs), reinterpret_cast<const char*>(krecs),
                       reinterpret_cast<const SeqInfo*>(info), s_in, s_out, out, reinterpret_cast<char*>(sink), units,
                       T, h_k, h_v, status);
    return hipGetLastError();
}

hipError_t launch_scan_bf16(int d, bool out_bf16, int rows, int mode, const void* q, const void* k, const void* v,
                            const void* recs, const void* krecs, const void* info, const float* s_in, float* s_out, void* out, void* sink,
                            int units, int T, int h_k, int h_v, unsigned* status, hipStream_t stream) {
    // The scan proper on 16-row slices runs on chunk_scan_tpf; chunk_scan_tp takes
    // 32-row slices and the segment maps (MODE 1).
#define GDN_TPF(D, OB)                                                                                         \
    if (d == D && out_bf16 == OB && rows == 16 && mode == 0)                                                  \
        return launch_scan_tpf_t<D, OB>(v, recs, krecs, info, s_in, s_out, out, sink, units, T, h_k, h_v, status, \
                                        stream);
    GDN_TPF(128, true) GDN_TPF(128, false) GDN_TPF(64, true) GDN_TPF(64, false)
#undef GDN_TPF
#define GDN_TPS(D, OB, NB, MODE)                                                                              \
    if (d == D && out_bf16 == OB && rows == 16 * NB && mode == MODE)                                          \
        return launch_scan_tp_t<D, OB, NB, MODE>(q, k, v, recs, info, s_in, s_out, out, sink, units, T, h_k, h_v, \
                                                 status, stream);
    GDN_TPS(128, true, 2, 0) GDN_TPS(128, false, 2, 0) GDN_TPS(64, true, 2, 0) GDN_TPS(64, false, 2, 0)
    GDN_TPS(128, false, 1, 1) GDN_TPS(128, false, 2, 1) GDN_TPS(64, false, 1, 1) GDN_TPS(64, false, 2, 1)
#undef GDN_TPS
    return hipErrorInvalidValue;
}

}  // namespace gdn

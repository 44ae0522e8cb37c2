/*
 * gdn.h -- C ABI of the Gated DeltaNet gated-delta-rule library for MI355X
 * (gfx950).
 *
 * The operation.  "Optimizing on-device inference for Apple Silicon"
 * (Perplexity blog), section "Qwen creates three distinct workload shapes",
 * describes the Gated DeltaNet layer.  It keeps a fixed-size recurrent state
 * per head.  A learned gate sets how much of that state survives each token,
 * and a delta update writes the current token in.  Per (sequence, v-head),
 * with S a d_v x d_k fp32 matrix:
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,          alpha_t = exp(g_t).
 *
 * The same section gives two ways to evaluate it.  One scans tokens directly
 * (gdn_decode_step for one token per sequence, gdn_prefill_direct for short
 * runs of tokens).  The other regroups the updates into blocks of tokens that
 * expose matrix work (gdn_prefill, blocks of `chunk` tokens).  Section "Keep the recurrent state on chip" keeps the state
 * and its gate in fp32 and the query/key activations in bf16.  This library
 * does the same, and reads and writes each state exactly once per call.
 *
 * Choosing a prefill entry point (measured on MI355X, 32 v-heads over 16 k-heads,
 * d = 128, bf16):
 *   - up to about 16 tokens per sequence (multi-token decode, verify steps):
 *     gdn_prefill_direct; at 64 sequences x 16 tokens it takes 142 us against
 *     212 us for gdn_prefill;
 *   - longer sequences: gdn_prefill, up to 40x faster than the direct scan;
 *   - one long sequence with few heads, so that (v-heads x d/16) is well below
 *     the compute-unit count: gdn_prefill_two_level with 4-16 segments (2.0x at
 *     2 or 4 v-heads, 1.7x at 8; no gain at 32 v-heads);
 *   - a prompt whose workspace must stay bounded: gdn_prefill_segmented.
 *
 * Conventions shared by every call:
 *   - All tensors are contiguous, in device memory, and owned by the caller.
 *     The library never allocates, frees or synchronises.  Every call is
 *     enqueued on `stream` (a hipStream_t; NULL = the null stream) and returns
 *     once it is enqueued.
 *   - q, k   [tokens, h_k, d_k]  in io_dtype (bf16 or fp32)
 *     v      [tokens, h_v, d_v]  in io_dtype
 *     g      [tokens, h_v]       fp32, the log of the decay (alpha = exp(g), g <= 0)
 *     beta   [tokens, h_v]       fp32 in [0, 1], used as given (no sigmoid inside)
 *     out    [tokens, h_v, d_v]  in out_dtype (bf16 or fp32)
 *     state  [num_seqs, h_v, d_v, d_k] fp32, row-major: row i holds the d_k
 *            key-side entries of value index i.
 *   - v-head h reads q/k head h / (h_v / h_k): consecutive v-heads share one
 *     q/k head.
 *   - qk_l2norm = 1 normalises q and k per (token, k-head) inside the kernel,
 *     x / sqrt(sum x^2 + 1e-6).  The query is then multiplied by `scale`.
 *   - Supported shapes: d_k = d_v in {64, 128}; h_v % h_k == 0; chunk = 64.
 *   - Numerics: bf16-input prefill runs the state-side products (K S^T, Q S^T
 *     and the state update) on bf16 matrix cores with the state and the
 *     update's operand split into bf16 high and low parts (fp32 range, about
 *     16 significant bits).  The two token-by-token contractions (U = T R and
 *     P U, with R = v - decayed (S k)) take fp16 operands: |v - S k| and |U|
 *     must stay below 65504.  Beyond that the results become infinite or NaN
 *     and the prefill status word reports GDN_PREFILL_STATUS_NONFINITE.
 *     fp32 inputs use fp32 matrix-core operands throughout.
 *   - Errors: every scalar and pointer check runs on the host before anything
 *     is enqueued.  A failed check returns GDN_ERR_INVALID_ARGUMENT or
 *     GDN_ERR_UNSUPPORTED, and the call then has no effect.  A failed launch
 *     returns GDN_ERR_HIP.  gdn_last_error() gives a detail string for the
 *     calling thread.
 *   - The library holds no state between calls.  Calls on different streams
 *     may overlap.  They must not share output or workspace buffers.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARGUMENT = 1,
    GDN_ERR_UNSUPPORTED = 2,
    GDN_ERR_WORKSPACE = 3,
    GDN_ERR_HIP = 4
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Problem description.  Plain data.  The integer fields hold gdn_dtype values. */
typedef struct {
    int32_t num_seqs;      /* N >= 1 */
    int64_t total_tokens;  /* prefill: packed token count T >= 0.  decode: ignored (N tokens) */
    int32_t h_k;           /* q/k heads >= 1 */
    int32_t h_v;           /* v-heads, a multiple of h_k */
    int32_t d_k;           /* key width: 64 or 128 */
    int32_t d_v;           /* value width: must equal d_k */
    int32_t io_dtype;      /* dtype of q, k, v */
    int32_t out_dtype;     /* dtype of out */
    int32_t qk_l2norm;     /* 1: L2-normalise q and k per token inside the kernel */
    float   scale;         /* multiplies the (normalised) query; 1.0 = plain rule */
} gdn_desc;

/*
 * Bytes of device workspace gdn_prefill needs for this problem.  It depends
 * only on the descriptor and chunk (whether or not cu_seqlens is passed).
 * Returns 0 and sets gdn_last_error() for an invalid descriptor.
 */
size_t gdn_prefill_workspace_bytes(const gdn_desc *desc, int32_t chunk);

/*
 * Blocked ("chunked") prefill over packed sequences.  This is the block form
 * of the rule from the workload-shapes section.
 *
 *   cu_seqlens  device int32 [num_seqs + 1].  Sequence n covers packed tokens
 *               [cu[n], cu[n+1]).  The array must start at 0, never decrease,
 *               and end at total_tokens.  The kernels clamp values that break
 *               this, so memory stays in bounds, but the results are then
 *               unspecified.  NULL is allowed only when num_seqs == 1.  A
 *               zero-length sequence passes its state through unchanged.
 *               Blocks restart at every sequence start.
 *   state_in    initial states, or NULL for zeros.
 *   state_out   final states, or NULL to skip them.  May equal state_in
 *               (in place).  No other argument may alias another.
 *   chunk       block length in tokens: 64.
 *   workspace   device scratch of at least gdn_prefill_workspace_bytes().
 *               Contents on entry do not matter.
 *
 * A single sequence (num_seqs == 1, no cu_seqlens) whose block records would
 * not stay in the last-level cache between the two kernels is run as
 * consecutive segments of whole blocks (as gdn_prefill_segmented, within the
 * same workspace).  The results are bit-identical to one pass.
 * gdn_prefill_ex chooses the segment length (or one pass) explicitly.
 *
 * Status word.  Every prefill call leaves a 32-bit word of
 * gdn_prefill_status_flag bits in the workspace, at byte offset
 * gdn_prefill_status_offset().  The call's first kernel resets it, and the
 * last one to finish has set its bits when the stream reaches the end of the
 * call; the caller reads it after that (the library does not synchronise).
 */
gdn_status gdn_prefill(const gdn_desc *desc,
                       const void *q, const void *k, const void *v,
                       const float *g, const float *beta,
                       const float *state_in,
                       void *out, float *state_out,
                       const int32_t *cu_seqlens, int32_t chunk,
                       void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * gdn_prefill with explicit tuning choices.  options == NULL is gdn_prefill.
 *
 *   scan_rows       rows of a state per scan workgroup: 0 for the default, or
 *                   16 or 32 (the results are bit-identical: rows evolve
 *                   independently and each row's arithmetic is the same).
 *   reserved        must be 0.
 *   segment_tokens  a single sequence (num_seqs == 1, no cu_seqlens) only:
 *                   0 chooses as gdn_prefill does, -1 runs one pass, and a
 *                   positive multiple of chunk runs segments of that length
 *                   within the same workspace (bit-identical to one pass).
 *                   Other callers must pass 0 or -1.
 *
 * Errors: those of gdn_prefill, plus GDN_ERR_INVALID_ARGUMENT for a
 * scan_rows other than 0, 16 or 32, a non-zero reserved field, or a negative
 * segment length other than -1; GDN_ERR_UNSUPPORTED for a positive segment
 * length that is not a multiple of chunk or is given with packed sequences;
 * GDN_ERR_WORKSPACE when the segments need more workspace than was given.
 */
typedef struct {
    int32_t scan_rows;
    int32_t reserved;
    int64_t segment_tokens;
} gdn_prefill_options;

gdn_status gdn_prefill_ex(const gdn_desc *desc,
                          const void *q, const void *k, const void *v,
                          const float *g, const float *beta,
                          const float *state_in,
                          void *out, float *state_out,
                          const int32_t *cu_seqlens, int32_t chunk,
                          const gdn_prefill_options *options,
                          void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Bits of the prefill status word.
 *   GDN_PREFILL_STATUS_CU_SEQLENS_CLAMPED  cu_seqlens broke its contract (did
 *       not start at 0, decreased, left [0, total_tokens] or did not end at
 *       total_tokens) and was clamped; the results are then unspecified.
 *   GDN_PREFILL_STATUS_NONFINITE  an output or a final state came out
 *       infinite or NaN: an input was, or a bf16-input call went beyond the
 *       fp16 range of its matrix-core operands (see Numerics above).
 */
typedef enum {
    GDN_PREFILL_STATUS_CU_SEQLENS_CLAMPED = 1,
    GDN_PREFILL_STATUS_NONFINITE = 2
} gdn_prefill_status_flag;

/*
 * Byte offset of the status word inside the workspace of gdn_prefill,
 * gdn_prefill_ex, gdn_prefill_prepare/gdn_prefill_scan, gdn_prefill_segmented
 * and gdn_prefill_two_level (the same offset for all; 4-byte aligned).
 * gdn_prefill_prepare resets the word and gdn_prefill_scan adds to it; each
 * of the other calls resets it once and then adds the bits of all its
 * kernels.  Returns 0 (never a valid offset) and sets gdn_last_error() for an
 * invalid descriptor or chunk.
 */
size_t gdn_prefill_status_offset(const gdn_desc *desc, int32_t chunk);

/*
 * The two phases of gdn_prefill, for callers that schedule or time them
 * separately.  gdn_prefill_prepare followed by gdn_prefill_scan on the same
 * stream, with the same workspace, is gdn_prefill in one pass (bit-identical
 * to gdn_prefill also where it runs segments).
 *
 * gdn_prefill_prepare: the state-free work of every block at once (parallel
 *   over blocks and heads).  Reads q, k, v, g, beta and cu_seqlens.  Writes
 *   only the workspace.
 * gdn_prefill_scan: walks each sequence's blocks in order with the state held
 *   on chip.  Reads q, k, v (the same tensors), the prepared workspace and
 *   state_in, and writes out and state_out.  Pass the same desc, cu_seqlens
 *   (as a layout flag: NULL or not) and workspace as the prepare call.  The
 *   workspace and the inputs must not change in between.
 * Arguments, validation and errors are those of gdn_prefill.
 */
gdn_status gdn_prefill_prepare(const gdn_desc *desc,
                               const void *q, const void *k, const void *v,
                               const float *g, const float *beta,
                               const int32_t *cu_seqlens, int32_t chunk,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

gdn_status gdn_prefill_scan(const gdn_desc *desc,
                            const void *q, const void *k, const void *v,
                            const float *state_in, void *out, float *state_out,
                            const int32_t *cu_seqlens, int32_t chunk,
                            void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * One decode step: one new token for each of num_seqs sequences.  This is the
 * direct token scan of the workload-shapes section, fused with the q/k
 * normalisation and the exponential gate ("Reduce intermediate traffic and
 * state traffic": the recurrent update is fused with its normalisation).
 * Shapes are those above with tokens = num_seqs.  `state` is read and written
 * in place, once each.  GDN_ERR_UNSUPPORTED if num_seqs * h_v * 2 * d_k
 * reaches 2^32 (one launch; the state would exceed 512 GiB).
 */
gdn_status gdn_decode_step(const gdn_desc *desc,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           float *state, void *out, void *stream);

/*
 * One decode step over a pool of states, for a serving loop that keeps one
 * state per live request and steps any subset of them together.  It is
 * gdn_decode_step with one indirection: sequence n reads and updates, in
 * place, slot state_slots[n] of
 *
 *   state_pool   fp32 [num_slots, h_v, d_v, d_k] (device; caller-owned),
 *   state_slots  int32 [num_seqs] (device; caller-owned).
 *
 * The section "Decode: minimise bytes moved per token" counts each state
 * read and written once per token; the indirection adds none.  Each slot
 * index is read on the device.  A slot outside [0, num_slots) skips its
 * sequence: that state is not touched and the sequence's output rows are
 * written as zeros.  Two sequences naming the same slot race (the result is
 * undefined; nothing faults).  Other arguments, shapes and errors are those of
 * gdn_decode_step, plus GDN_ERR_INVALID_ARGUMENT for num_slots < 1 or a NULL
 * state_pool or state_slots.
 */
gdn_status gdn_decode_step_slots(const gdn_desc *desc,
                                 const void *q, const void *k, const void *v,
                                 const float *g, const float *beta,
                                 float *state_pool, int32_t num_slots,
                                 const int32_t *state_slots,
                                 void *out, void *stream);

/*
 * One decode step with the per-token operations beside the recurrent update
 * folded into the same kernel.  The section "Reduce intermediate traffic and
 * state traffic" fuses the recurrent update with its normalisation, so that
 * temporaries stay in registers instead of passing through memory.  `fuse` is
 * a bitwise OR of:
 *
 *   GDN_FUSE_GATE_ACTIVATIONS  g and beta hold raw gate inputs x_g, x_beta
 *                              (fp32 [num_seqs, h_v]); the step uses
 *                              alpha = exp(-softplus(x_g)) = 1 / (1 + e^x_g)
 *                              and beta = 1 / (1 + e^-x_beta).
 *   GDN_FUSE_OUTPUT_NORM       each (sequence, v-head) output o (d_v values)
 *                              is written as o / sqrt(mean(o^2) + norm_eps),
 *                              times norm_weight channel-wise.  norm_weight
 *                              is fp32 [d_v] on the device, shared by all
 *                              heads, or NULL for ones; norm_eps is finite
 *                              and > 0.  The state update is not affected.
 *   GDN_STREAM_STATE           a cache policy, not an operation: the state is
 *                              read and written with nontemporal accesses,
 *                              which do not keep it in the GPU's caches.
 *                              Results are bit-identical either way.  Set it
 *                              when other work runs through the caches before
 *                              this state is stepped again, as a model's
 *                              layers each step their own state (section
 *                              "Decode: minimise bytes moved per token"):
 *                              there the step runs ~8% faster.  Leave it off
 *                              when the same states are stepped back to back
 *                              and fit in the 256 MiB last-level cache, which
 *                              then serves part of each step.
 *
 * Without flags this is gdn_decode_step (bit-identical results); norm_weight
 * and norm_eps are read only with GDN_FUSE_OUTPUT_NORM.  The state is still
 * read and written once.  Other arguments, shapes and errors are those of
 * gdn_decode_step, plus GDN_ERR_INVALID_ARGUMENT for unknown flags, a
 * norm_eps that is not finite and positive, or a norm_weight that overlaps
 * another buffer.
 */
typedef enum { GDN_FUSE_GATE_ACTIVATIONS = 1, GDN_FUSE_OUTPUT_NORM = 2, GDN_STREAM_STATE = 4 } gdn_fuse_flag;

gdn_status gdn_decode_step_ex(const gdn_desc *desc,
                              const void *q, const void *k, const void *v,
                              const float *g, const float *beta,
                              float *state, void *out,
                              int32_t fuse, const float *norm_weight, float norm_eps,
                              void *stream);

/*
 * Bounded-memory prefill of one long sequence (num_seqs == 1, no
 * cu_seqlens): the tokens run through gdn_prefill in consecutive segments of
 * `segment_tokens` (a positive multiple of chunk), each starting from the
 * state the previous one left.  Section "Keep the recurrent state on chip"
 * splits long prompts into pieces the same way and carries the state between
 * them.  Because segments start on block boundaries, the result is bit for
 * bit that of one gdn_prefill call, while the workspace needs room for one
 * segment only (plus a state buffer when state_out is NULL):
 * gdn_prefill_segmented_workspace_bytes().  The segments are enqueued from
 * the host one after another on `stream`.
 *
 * Other arguments are those of gdn_prefill.  Errors: as gdn_prefill, and
 * GDN_ERR_UNSUPPORTED for num_seqs != 1, a non-NULL cu_seqlens, or a segment
 * length that is not a positive multiple of chunk.
 */
size_t gdn_prefill_segmented_workspace_bytes(const gdn_desc *desc, int32_t chunk, int64_t segment_tokens);

gdn_status gdn_prefill_segmented(const gdn_desc *desc,
                                 const void *q, const void *k, const void *v,
                                 const float *g, const float *beta,
                                 const float *state_in,
                                 void *out, float *state_out,
                                 int32_t chunk, int64_t segment_tokens,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * Two-level prefill of one long sequence (num_seqs == 1, no cu_seqlens), for
 * shapes whose (v-head x row-slice) units leave compute units idle, such as a
 * long prompt with few heads.  The block chain of the scan is cut into
 * `segments` segments of whole blocks.  A run of blocks maps the state
 * affinely, S_end = S_start R + B (the section "Keep the recurrent state on
 * chip" carries the state across pieces of a prompt the same way), so:
 * (1) one state-carrying pass over all segments at once yields each segment's
 * B (run from zero) and R (run from the identity without the value term);
 * (2) a short sequential pass composes the segments' start states in fp32;
 * (3) the scan reruns every segment from its start state, in parallel, and
 * writes the outputs.  This does about three times the state-dependent
 * work of gdn_prefill on `segments`-fold more parallel units.  The result
 * matches gdn_prefill within the same tolerance; the rounding order differs.
 * segments == 1 (or a sequence of one block) is gdn_prefill.
 *
 * Workspace: gdn_prefill_two_level_workspace_bytes().  Other arguments and
 * errors are those of gdn_prefill, plus GDN_ERR_UNSUPPORTED for
 * num_seqs != 1 and GDN_ERR_INVALID_ARGUMENT for segments < 1.
 */
size_t gdn_prefill_two_level_workspace_bytes(const gdn_desc *desc, int32_t chunk, int32_t segments);

gdn_status gdn_prefill_two_level(const gdn_desc *desc,
                                 const void *q, const void *k, const void *v,
                                 const float *g, const float *beta,
                                 const float *state_in,
                                 void *out, float *state_out,
                                 int32_t chunk, int32_t segments,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * Direct (token-by-token) prefill over packed sequences: the other evaluation
 * of the workload-shapes section, which says the faster of the two depends on
 * the shape.  Each (sequence, v-head) state is loaded once, kept in registers
 * while the sequence's tokens stream through one by one, and written once, so
 * no workspace is needed.  It suits short sequences: multi-token decode and
 * verify steps of a few tokens per sequence (state_in == state_out, in place).
 * The arithmetic is fp32 throughout, as in gdn_decode_step.
 *
 * Arguments and layouts are those of gdn_prefill without chunk and workspace.
 * cu_seqlens has the same contract; here each range [cu[n], cu[n+1]) is
 * clamped into [0, total_tokens] on its own (an inverted range has no tokens).
 * With one token per sequence and state_in == state_out this is
 * gdn_decode_step.
 */
gdn_status gdn_prefill_direct(const gdn_desc *desc,
                              const void *q, const void *k, const void *v,
                              const float *g, const float *beta,
                              const float *state_in,
                              void *out, float *state_out,
                              const int32_t *cu_seqlens,
                              void *stream);

/*
 * gdn_prefill_direct with the per-token operations of gdn_decode_step_ex
 * folded in, token by token: raw gate inputs (GDN_FUSE_GATE_ACTIVATIONS) and
 * each (token, v-head) output normalised over d_v (GDN_FUSE_OUTPUT_NORM, with
 * norm_weight and norm_eps as there), for multi-token decode and verify steps.
 * Without flags this is gdn_prefill_direct.  GDN_STREAM_STATE is a decode-step
 * flag only and is rejected here.  Errors: those of gdn_prefill_direct and the
 * flag, eps and weight checks of gdn_decode_step_ex.
 */
gdn_status gdn_prefill_direct_ex(const gdn_desc *desc,
                                 const void *q, const void *k, const void *v,
                                 const float *g, const float *beta,
                                 const float *state_in,
                                 void *out, float *state_out,
                                 const int32_t *cu_seqlens,
                                 int32_t fuse, const float *norm_weight, float norm_eps,
                                 void *stream);

/*
 * gdn_prefill for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid hipMalloc.
 * The workspace is the library's own: a static device array of
 * GDN_PREFILL_NOALLOC_WORKSPACE_BYTES (64 MiB) on each GPU it runs on, held
 * until the process ends.  The call allocates nothing.  Its first call on a
 * device looks up that device's copy of the array (no allocation either).
 *
 * Problems whose gdn_prefill_workspace_bytes() exceeds the array are
 * rejected with GDN_ERR_WORKSPACE before anything is enqueued (at 32 v-heads
 * and d = 128 the array holds about 4400 tokens).  All calls on one GPU share
 * the array, so calls that overlap on one GPU (on different streams, or
 * from different host threads without ordering) race; serialise them.  The
 * contents left by an earlier call do not matter.  The status word of the
 * call lands in the shared array and is not exposed.  Other arguments,
 * results and errors are those of gdn_prefill, whose result this is bit for
 * bit.
 */
#define GDN_PREFILL_NOALLOC_WORKSPACE_BYTES (64u << 20)

gdn_status gdn_prefill_noalloc(const gdn_desc *desc,
                               const void *q, const void *k, const void *v,
                               const float *g, const float *beta,
                               const float *state_in,
                               void *out, float *state_out,
                               const int32_t *cu_seqlens, int32_t chunk,
                               void *stream);

/* Static, English name of a status code. */
const char *gdn_status_str(gdn_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char *gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */

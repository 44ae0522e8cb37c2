// Host side of the C ABI declared in include/gdn.h.  It validates every
// argument before anything is enqueued, sizes the prefill workspace, picks
// launch shapes, and launches the kernels in decode.hip and prefill.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "gdn.h"

namespace gdn {
hipError_t launch_decode(int d, bool in_bf16, bool out_bf16, const void* q, const void* k,
                         const void* v, const float* g, const float* beta, float* state, const int32_t* slots,
                         int num_slots, void* out, int units, int h_k, int h_v, int l2norm, float scale,
                         int fuse, const float* norm_w, float norm_eps, hipStream_t stream);
size_t prefill_record_bytes(int d, bool in_bf16);
size_t prefill_key_record_bytes(int d, bool in_bf16);
hipError_t launch_segment_info(void* info, int P, int sb, int T, hipStream_t stream);
hipError_t launch_compose(int d, const float* state_in, const float* R, const float* B, float* starts, int P,
                          int h_v, hipStream_t stream);
hipError_t launch_scan_transition(int d, bool in_bf16, int rows, const void* q, const void* k, const void* v,
                                  const void* recs, const void* krecs, const void* info, float* s_out, void* sink,
                                  int units, int T, int h_k, int h_v, hipStream_t stream);
hipError_t launch_direct(int d, bool in_bf16, bool out_bf16, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const int32_t* cu, const float* s_in, float* s_out,
                         void* out, int units, int T, int h_k, int h_v, int l2norm, float scale, int fuse, const float* norm_w,
                         float norm_eps, hipStream_t stream);
hipError_t launch_plan(const int32_t* cu, int N, int T, int max_slots, void* info, int32_t* slot_seq,
                       unsigned* status, hipStream_t stream);
hipError_t launch_status_reset(unsigned* status, hipStream_t stream);
hipError_t launch_prep(int d, bool in_bf16, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const void* info, const int32_t* slot_seq,
                       int slots, int T, int h_k, int h_v, int l2norm, float scale, void* recs,
                       void* krecs, unsigned* clear_status, hipStream_t stream);
hipError_t launch_scan(int d, bool in_bf16, bool out_bf16, int rows, const void* q, const void* k, const void* v,
                       const void* recs, const void* krecs, const void* info, const float* s_in, float* s_out,
                       void* out, void* sink, int units, int T, int h_k, int h_v, unsigned* status,
                       hipStream_t stream);
}  // namespace gdn

namespace {

constexpr int kChunk = 64;
constexpr int64_t kMaxTokens = (int64_t)1 << 30;

thread_local char g_err[512] = "";

gdn_status fail(gdn_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

size_t dtype_size(int32_t dt) { return dt == GDN_BF16 ? 2 : 4; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Common descriptor checks for both calls.
gdn_status check_desc(const gdn_desc* d, bool prefill) {
    if (!d) return fail(GDN_ERR_INVALID_ARGUMENT, "desc is NULL");
    if (d->num_seqs < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "num_seqs must be >= 1 (got %d)", d->num_seqs);
    if (d->h_k < 1 || d->h_v < 1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "h_k and h_v must be >= 1 (got %d, %d)", d->h_k, d->h_v);
    if (d->h_v % d->h_k != 0)
        return fail(GDN_ERR_INVALID_ARGUMENT, "h_v (%d) must be a multiple of h_k (%d)", d->h_v, d->h_k);
    if (d->d_k < 1 || d->d_v < 1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "d_k and d_v must be >= 1 (got %d, %d)", d->d_k, d->d_v);
    if (d->d_k != d->d_v)
        return fail(GDN_ERR_UNSUPPORTED, "d_k (%d) must equal d_v (%d)", d->d_k, d->d_v);
    if (d->d_k != 64 && d->d_k != 128)
        return fail(GDN_ERR_UNSUPPORTED, "head width %d not supported (64 or 128)", d->d_k);
    if ((d->io_dtype != GDN_F32 && d->io_dtype != GDN_BF16) ||
        (d->out_dtype != GDN_F32 && d->out_dtype != GDN_BF16))
        return fail(GDN_ERR_INVALID_ARGUMENT, "io_dtype/out_dtype must be GDN_F32 or GDN_BF16");
    if (d->qk_l2norm != 0 && d->qk_l2norm != 1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "qk_l2norm must be 0 or 1");
    if (!std::isfinite(d->scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (d->h_v > 65535) return fail(GDN_ERR_UNSUPPORTED, "h_v above 65535 not supported");
    if ((int64_t)d->num_seqs * d->h_v * 4 > INT32_MAX)
        return fail(GDN_ERR_UNSUPPORTED, "num_seqs * h_v too large");
    if (prefill) {
        if (d->total_tokens < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "total_tokens must be >= 0");
        if (d->total_tokens > kMaxTokens)
            return fail(GDN_ERR_UNSUPPORTED, "total_tokens above 2^30 not supported");
        if (d->io_dtype == GDN_F32 && d->d_k == 128)
            return fail(GDN_ERR_UNSUPPORTED, "fp32-input prefill supports head width 64 only");
    }
    return GDN_OK;
}

int64_t max_slots(const gdn_desc* d, bool varlen) {
    const int64_t T = d->total_tokens;
    if (!varlen) return (T + kChunk - 1) / kChunk;
    return (T + (int64_t)d->num_seqs * (kChunk - 1)) / kChunk;
}

// Workspace: [sink 1 KiB][status word, 256 B][plan: per-sequence info, slot -> sequence]
//            [records per (block slot, v-head)][key records per (block slot, k-head)]
// The sink absorbs the chunk scan's stores for rows past the end of a block.
constexpr size_t kSinkBytes = 1024;
constexpr size_t kStatusOff = kSinkBytes, kStatusBytes = 256;

struct WsLayout {
    size_t sink_off, info_off, slot_off, rec_off, key_off, total;
    int64_t slots;
};

WsLayout ws_layout(const gdn_desc* d, bool varlen) {
    WsLayout w{};
    w.slots = max_slots(d, varlen);
    w.sink_off = 0;
    size_t plan = kStatusOff + kStatusBytes;
    if (varlen) {
        w.info_off = plan;
        w.slot_off = plan + (size_t)d->num_seqs * 16;
        plan = align_up(w.slot_off + (size_t)w.slots * 4, 256);
    }
    const bool bf16 = d->io_dtype == GDN_BF16;
    w.rec_off = plan;
    w.key_off = w.rec_off + (size_t)w.slots * d->h_v * gdn::prefill_record_bytes(d->d_k, bf16);
    w.total = w.key_off + (size_t)w.slots * d->h_k * gdn::prefill_key_record_bytes(d->d_k, bf16);
    return w;
}

struct Span {
    const char* p;
    size_t n;
    const char* name;
};

// Vector loads and stores need 16-byte aligned tensors (4 bytes for g, beta, cu_seqlens).
gdn_status check_align(const Span* s, int count) {
    for (int i = 0; i < count; ++i) {
        if (!s[i].p || !s[i].n) continue;
        const bool small = !strcmp(s[i].name, "g") || !strcmp(s[i].name, "beta") ||
                           !strcmp(s[i].name, "cu_seqlens") || !strcmp(s[i].name, "norm_weight");
        const uintptr_t a = small ? 4 : (!strcmp(s[i].name, "workspace") ? 256 : 16);
        if (reinterpret_cast<uintptr_t>(s[i].p) % a)
            return fail(GDN_ERR_INVALID_ARGUMENT, "%s must be %zu-byte aligned", s[i].name, (size_t)a);
    }
    return GDN_OK;
}

// Any two non-empty ranges that overlap (other than the allowed in-place state pair) are rejected.
gdn_status check_overlaps(const Span* s, int count, const void* allow_a, const void* allow_b) {
    for (int i = 0; i < count; ++i)
        for (int j = i + 1; j < count; ++j) {
            if (!s[i].p || !s[j].p || !s[i].n || !s[j].n) continue;
            // in place: the allowed pair at exactly the same address and size
            if (allow_a && allow_a == allow_b && s[i].p == allow_a && s[j].p == allow_a && s[i].n == s[j].n)
                continue;
            if (s[i].p < s[j].p + s[j].n && s[j].p < s[i].p + s[i].n)
                return fail(GDN_ERR_INVALID_ARGUMENT, "buffers %s and %s overlap", s[i].name, s[j].name);
        }
    return GDN_OK;
}

// Workspace of gdn_prefill_noalloc: a file-scope device array (each GPU the
// library runs on holds its own copy until the process ends).  In host code
// `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
constexpr size_t kNoallocBytes = (size_t)GDN_PREFILL_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
gdn_status scratch_address(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(GDN_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return GDN_OK;
}

// Shared by gdn_prefill_direct and gdn_prefill_direct_ex (fuse flags, norm weight and eps).
gdn_status direct_call(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* state_in, void* out, float* state_out,
                       const int32_t* cu_seqlens, void* stream, int fuse, const float* norm_w, float norm_eps) {
    gdn_status st = check_desc(desc, false);  // every head width and dtype the direct kernels build
    if (st != GDN_OK) return st;
    if (desc->total_tokens < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "total_tokens must be >= 0");
    if (desc->total_tokens > kMaxTokens) return fail(GDN_ERR_UNSUPPORTED, "total_tokens above 2^30 not supported");
    const int64_t T = desc->total_tokens;
    const int N = desc->num_seqs, hk = desc->h_k, hv = desc->h_v, d = desc->d_k;
    if (!cu_seqlens && N != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL but num_seqs = %d", N);
    if (T > 0 && (!q || !k || !v || !g || !beta || !out))
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, g, beta and out must be non-NULL");
    const size_t io = dtype_size(desc->io_dtype), os = dtype_size(desc->out_dtype);
    const size_t sbytes = (size_t)N * hv * d * d * 4;
    const Span spans[] = {
        {(const char*)q, (size_t)T * hk * d * io, "q"},
        {(const char*)k, (size_t)T * hk * d * io, "k"},
        {(const char*)v, (size_t)T * hv * d * io, "v"},
        {(const char*)g, (size_t)T * hv * 4, "g"},
        {(const char*)beta, (size_t)T * hv * 4, "beta"},
        {(const char*)out, (size_t)T * hv * d * os, "out"},
        {(const char*)state_in, state_in ? sbytes : 0, "state_in"},
        {(const char*)state_out, state_out ? sbytes : 0, "state_out"},
        {(const char*)cu_seqlens, cu_seqlens ? (size_t)(N + 1) * 4 : 0, "cu_seqlens"},
        {(const char*)norm_w, norm_w ? (size_t)d * 4 : 0, "norm_weight"},
    };
    st = check_align(spans, sizeof(spans) / sizeof(spans[0]));
    if (st != GDN_OK) return st;
    st = check_overlaps(spans, sizeof(spans) / sizeof(spans[0]), state_in, state_out);
    if (st != GDN_OK) return st;
    if (!state_out && T == 0) return GDN_OK;  // nothing to compute or write
    hipError_t e = gdn::launch_direct(d, desc->io_dtype == GDN_BF16, desc->out_dtype == GDN_BF16, q, k, v, g, beta,
                                      cu_seqlens, state_in, state_out, out, N * hv, (int)T, hk, hv, desc->qk_l2norm,
                                      desc->scale, fuse, norm_w, norm_eps, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "direct prefill launch: %s", hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_str(gdn_status s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_INVALID_ARGUMENT: return "GDN_ERR_INVALID_ARGUMENT";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
        case GDN_ERR_HIP: return "GDN_ERR_HIP";
    }
    return "GDN_UNKNOWN_STATUS";
}

const char* gdn_last_error(void) { return g_err; }

size_t gdn_prefill_workspace_bytes(const gdn_desc* desc, int32_t chunk) {
    g_err[0] = 0;
    if (check_desc(desc, true) != GDN_OK) return 0;
    if (chunk != kChunk) { fail(GDN_ERR_UNSUPPORTED, "chunk must be 64 (got %d)", chunk); return 0; }
    // the packed-sequence layout is a superset; size for it so one query covers both uses
    return ws_layout(desc, true).total;
}

}  // extern "C"

namespace {

enum Phase { kPrepare = 1, kScan = 2, kBoth = 3 };

// Validation shared by gdn_prefill and its two phases.  Pointers that a phase
// does not use are passed as NULL and not checked.
// clear_status: the prepare phase resets the status word (false for the
// segments after the first of a segmented call, which add to it).
gdn_status prefill_call(Phase phase, const gdn_desc* desc, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const float* state_in, void* out,
                        float* state_out, const int32_t* cu_seqlens, int32_t chunk, void* workspace,
                        size_t workspace_bytes, void* stream, int scan_rows = 0, bool clear_status = true) {
    g_err[0] = 0;
    gdn_status st = check_desc(desc, true);
    if (st != GDN_OK) return st;
    if (chunk != kChunk) return fail(GDN_ERR_UNSUPPORTED, "chunk must be 64 (got %d)", chunk);
    const int64_t T = desc->total_tokens;
    const int N = desc->num_seqs, hk = desc->h_k, hv = desc->h_v, d = desc->d_k;
    if (!cu_seqlens && N != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL but num_seqs = %d", N);
    if (T > 0 && (phase & kPrepare) && (!q || !k || !v || !g || !beta))
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, g and beta must be non-NULL");
    if (T > 0 && (phase & kScan) && (!q || !k || !v || !out))
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v and out must be non-NULL");
    const bool varlen = cu_seqlens != nullptr;
    const WsLayout ws = ws_layout(desc, varlen);
    // the requirement is what gdn_prefill_workspace_bytes reports, whichever layout is used
    const size_t need = ws_layout(desc, true).total;
    if (need > 0 && !workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
    const size_t io = dtype_size(desc->io_dtype), os = dtype_size(desc->out_dtype);
    const size_t sbytes = (size_t)N * hv * d * d * 4;
    const Span spans[] = {
        {(const char*)q, (size_t)T * hk * d * io, "q"},
        {(const char*)k, (size_t)T * hk * d * io, "k"},
        {(const char*)v, (size_t)T * hv * d * io, "v"},
        {(const char*)g, (size_t)T * hv * 4, "g"},
        {(const char*)beta, (size_t)T * hv * 4, "beta"},
        {(const char*)out, (size_t)T * hv * d * os, "out"},
        {(const char*)state_in, state_in ? sbytes : 0, "state_in"},
        {(const char*)state_out, state_out ? sbytes : 0, "state_out"},
        {(const char*)cu_seqlens, cu_seqlens ? (size_t)(N + 1) * 4 : 0, "cu_seqlens"},
        {(const char*)workspace, need, "workspace"},
    };
    st = check_align(spans, sizeof(spans) / sizeof(spans[0]));
    if (st != GDN_OK) return st;
    st = check_overlaps(spans, sizeof(spans) / sizeof(spans[0]), state_in, state_out);
    if (st != GDN_OK) return st;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool in_bf16 = desc->io_dtype == GDN_BF16, out_bf16 = desc->out_dtype == GDN_BF16;
    char* wsb = reinterpret_cast<char*>(workspace);
    void* info = varlen ? wsb + ws.info_off : nullptr;
    int32_t* slot_seq = varlen ? reinterpret_cast<int32_t*>(wsb + ws.slot_off) : nullptr;
    unsigned* status = reinterpret_cast<unsigned*>(wsb + kStatusOff);
    hipError_t e = hipSuccess;
    if (phase & kPrepare) {
        // the status word is reset by the plan (which may set the clamped bit) or else by chunk_prep
        bool reset = !clear_status;
        if (varlen) {
            e = gdn::launch_plan(cu_seqlens, N, (int)T, (int)ws.slots, info, slot_seq, clear_status ? status : nullptr,
                                 s);
            if (e != hipSuccess) return fail(GDN_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
            reset = true;
        }
        if (ws.slots > 0 && T > 0) {  // chunk_prep clamps token indices into [0, T)
            e = gdn::launch_prep(d, in_bf16, q, k, v, g, beta, info, slot_seq, (int)ws.slots, (int)T, hk, hv,
                                 desc->qk_l2norm, desc->scale, wsb + ws.rec_off, wsb + ws.key_off,
                                 reset ? nullptr : status, s);
            if (e != hipSuccess) return fail(GDN_ERR_HIP, "chunk_prep launch: %s", hipGetErrorString(e));
            reset = true;
        }
        if (!reset) {  // no kernel to reset it: an empty problem (a kernel, not a memset node, so capturable)
            e = gdn::launch_status_reset(status, s);
            if (e != hipSuccess) return fail(GDN_ERR_HIP, "status reset: %s", hipGetErrorString(e));
        }
    }
    if ((phase & kScan) && (state_out || T > 0)) {
        e = gdn::launch_scan(d, in_bf16, out_bf16, scan_rows, q, k, v, wsb + ws.rec_off, wsb + ws.key_off, info,
                             state_in, state_out, out, wsb + ws.sink_off, N * hv, (int)T, hk, hv, status, s);
        if (e != hipSuccess) return fail(GDN_ERR_HIP, "chunk_scan launch: %s", hipGetErrorString(e));
    }
    return GDN_OK;
}

// Two-level plan of one sequence: P segments of sb blocks each (the last may
// be shorter), and the workspace after the single-sequence prefill layout:
// segment table, per-segment affine parts B and transitions R (segments
// 0..P-2, adjacent), and start and end states of every segment.
struct TwoLevel {
    int64_t nblocks;
    int P, sb;
    size_t info_off, b_off, r_off, start_off, end_off, total;
};

gdn_status two_level_plan(const gdn_desc* desc, int32_t chunk, int32_t segments, TwoLevel* tl) {
    gdn_status st = check_desc(desc, true);
    if (st != GDN_OK) return st;
    if (chunk != kChunk) return fail(GDN_ERR_UNSUPPORTED, "chunk must be 64 (got %d)", chunk);
    if (desc->num_seqs != 1)
        return fail(GDN_ERR_UNSUPPORTED, "two-level prefill takes one sequence (num_seqs = %d)", desc->num_seqs);
    if (segments < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "segments must be >= 1 (got %d)", segments);
    const int64_t T = desc->total_tokens;
    tl->nblocks = (T + kChunk - 1) / kChunk;
    const int64_t want = segments < tl->nblocks ? segments : (tl->nblocks > 0 ? tl->nblocks : 1);
    tl->sb = (int)(tl->nblocks > 0 ? (tl->nblocks + want - 1) / want : 1);
    tl->P = (int)(tl->nblocks > 0 ? (tl->nblocks + tl->sb - 1) / tl->sb : 1);
    if (tl->P == 1) {  // the plain prefill
        tl->total = ws_layout(desc, true).total;
        return GDN_OK;
    }
    const size_t st_bytes = (size_t)desc->h_v * desc->d_k * desc->d_k * 4;
    tl->info_off = align_up(ws_layout(desc, false).total, 256);
    tl->b_off = align_up(tl->info_off + (size_t)tl->P * 16, 256);
    tl->r_off = tl->b_off + (size_t)(tl->P - 1) * st_bytes;
    tl->start_off = tl->r_off + (size_t)(tl->P - 1) * st_bytes;
    tl->end_off = tl->start_off + (size_t)tl->P * st_bytes;
    tl->total = tl->end_off + (size_t)tl->P * st_bytes;
    return GDN_OK;
}

// Segment descriptor and state buffer of the segmented prefill.
// gdn_prefill runs a long single sequence as consecutive segments of whole
// blocks, so that each segment's block records (written by chunk_prep, read
// by chunk_scan) stay in the last-level cache (256 MiB on MI355X) between the
// two kernels instead of going out to HBM and back.  Results are bit-identical
// to a single call: the block grid is the same, and the fp32 state passes
// between segments unrounded.  Returns the segment length in tokens, or 0 to
// run one call.
constexpr size_t kSegmentRecordBudget = (size_t)146 << 20;

int64_t auto_segment_tokens(const gdn_desc* d) {
    if (d->num_seqs != 1 || d->total_tokens <= 0) return 0;
    const bool bf16 = d->io_dtype == GDN_BF16;
    const size_t per_block = (size_t)d->h_v * gdn::prefill_record_bytes(d->d_k, bf16) +
                             (size_t)d->h_k * gdn::prefill_key_record_bytes(d->d_k, bf16);
    const int64_t blocks = (d->total_tokens + kChunk - 1) / kChunk;
    if ((size_t)blocks * per_block <= kSegmentRecordBudget) return 0;
    const int64_t seg_blocks = std::max<int64_t>(1, (int64_t)(kSegmentRecordBudget / per_block));
    const int64_t nseg = (blocks + seg_blocks - 1) / seg_blocks;
    return (blocks + nseg - 1) / nseg * kChunk;  // equal segments
}

gdn_status segment_plan(const gdn_desc* desc, int32_t chunk, int64_t seg, gdn_desc* sub, size_t* need,
                               size_t* state_off) {
    gdn_status st = check_desc(desc, true);
    if (st != GDN_OK) return st;
    if (chunk != kChunk) return fail(GDN_ERR_UNSUPPORTED, "chunk must be 64 (got %d)", chunk);
    if (desc->num_seqs != 1) return fail(GDN_ERR_UNSUPPORTED, "segmented prefill takes one sequence (num_seqs = %d)",
                                         desc->num_seqs);
    if (seg <= 0 || seg % kChunk != 0)
        return fail(GDN_ERR_UNSUPPORTED, "segment_tokens must be a positive multiple of %d (got %lld)", kChunk,
                    (long long)seg);
    *sub = *desc;
    sub->total_tokens = desc->total_tokens < seg ? desc->total_tokens : seg;
    const size_t seg_ws = ws_layout(sub, true).total;
    *state_off = align_up(seg_ws, 256);
    *need = *state_off + (size_t)desc->h_v * desc->d_k * desc->d_k * 4;
    return GDN_OK;
}

// The segmented prefill (defined with gdn_prefill_segmented), shared with gdn_prefill_ex.
gdn_status segmented_call(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* state_in, void* out, float* state_out, int32_t chunk,
                          int64_t segment_tokens, void* workspace, size_t workspace_bytes, void* stream,
                          int scan_rows);

// Shared by gdn_decode_step (slots == NULL: sequence n uses state n),
// gdn_decode_step_slots and gdn_decode_step_ex (fuse flags, norm weight and eps).
gdn_status decode_call(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                       const float* beta, float* state, int32_t num_slots, const int32_t* slots, void* out,
                       void* stream, int fuse = 0, const float* norm_w = nullptr, float norm_eps = 0.f) {
    const int N = desc->num_seqs, hk = desc->h_k, hv = desc->h_v, d = desc->d_k;
    // one workgroup of 2 d threads per (sequence, v-head): the grid stays below 2^32 work-items
    if ((int64_t)N * hv * 2 * d >= ((int64_t)1 << 32))
        return fail(GDN_ERR_UNSUPPORTED, "num_seqs * h_v = %lld units exceed one decode launch",
                    (long long)N * hv);
    const size_t io = dtype_size(desc->io_dtype), os = dtype_size(desc->out_dtype);
    const Span spans[] = {
        {(const char*)q, (size_t)N * hk * d * io, "q"},
        {(const char*)k, (size_t)N * hk * d * io, "k"},
        {(const char*)v, (size_t)N * hv * d * io, "v"},
        {(const char*)g, (size_t)N * hv * 4, "g"},
        {(const char*)beta, (size_t)N * hv * 4, "beta"},
        {(const char*)out, (size_t)N * hv * d * os, "out"},
        {(const char*)state, (size_t)num_slots * hv * d * d * 4, "state"},
        {(const char*)slots, slots ? (size_t)N * 4 : 0, "state_slots"},
        {(const char*)norm_w, norm_w ? (size_t)d * 4 : 0, "norm_weight"},
    };
    gdn_status st = check_align(spans, sizeof(spans) / sizeof(spans[0]));
    if (st != GDN_OK) return st;
    st = check_overlaps(spans, sizeof(spans) / sizeof(spans[0]), nullptr, nullptr);
    if (st != GDN_OK) return st;
    hipError_t e = gdn::launch_decode(d, desc->io_dtype == GDN_BF16, desc->out_dtype == GDN_BF16, q, k, v, g,
                                      beta, state, slots, num_slots, out, N * hv, hk, hv, desc->qk_l2norm,
                                      desc->scale, fuse, norm_w, norm_eps,
                                      reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_ex(const gdn_desc* desc, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, const float* state_in, void* out,
                          float* state_out, const int32_t* cu_seqlens, int32_t chunk,
                          const gdn_prefill_options* options, void* workspace, size_t workspace_bytes,
                          void* stream) {
    g_err[0] = 0;
    gdn_prefill_options opt = {0, 0, 0};
    if (options) opt = *options;
    if (opt.scan_rows != 0 && opt.scan_rows != 16 && opt.scan_rows != 32)
        return fail(GDN_ERR_INVALID_ARGUMENT, "scan_rows must be 0, 16 or 32 (got %d)", opt.scan_rows);
    if (opt.reserved != 0) return fail(GDN_ERR_INVALID_ARGUMENT, "options.reserved must be 0");
    if (opt.segment_tokens < -1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "segment_tokens must be -1, 0 or positive (got %lld)",
                    (long long)opt.segment_tokens);
    const bool single = !cu_seqlens && desc && desc->num_seqs == 1;
    if (opt.segment_tokens > 0 && !single)
        return fail(GDN_ERR_UNSUPPORTED, "segment_tokens needs one sequence without cu_seqlens");
    if (opt.segment_tokens > 0 && opt.segment_tokens % kChunk != 0)
        return fail(GDN_ERR_UNSUPPORTED, "segment_tokens must be a multiple of %d (got %lld)", kChunk,
                    (long long)opt.segment_tokens);
    // A long single sequence runs as consecutive segments (same results, see
    // auto_segment_tokens), after the checks of the one-call contract.
    if (single && opt.segment_tokens != -1 && check_desc(desc, true) == GDN_OK && chunk == kChunk) {
        const int64_t seg = opt.segment_tokens > 0 ? opt.segment_tokens : auto_segment_tokens(desc);
        if (seg > 0 && seg < desc->total_tokens) {
            const size_t need = ws_layout(desc, true).total;
            if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
            if (workspace_bytes < need)
                return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                            need);
            gdn_desc sub;
            size_t seg_need = 0, soff = 0;
            gdn_status st = segment_plan(desc, chunk, seg, &sub, &seg_need, &soff);
            if (st != GDN_OK) return st;
            if (seg_need > workspace_bytes)
                return fail(GDN_ERR_WORKSPACE, "segments of %lld tokens need %zu workspace bytes, %zu given",
                            (long long)seg, seg_need, workspace_bytes);
            return segmented_call(desc, q, k, v, g, beta, state_in, out, state_out, chunk, seg, workspace,
                                  workspace_bytes, stream, opt.scan_rows);
        }
    }
    return prefill_call(kBoth, desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, chunk,
                        workspace, workspace_bytes, stream, opt.scan_rows);
}

gdn_status gdn_prefill(const gdn_desc* desc, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const float* state_in, void* out,
                       float* state_out, const int32_t* cu_seqlens, int32_t chunk, void* workspace,
                       size_t workspace_bytes, void* stream) {
    return gdn_prefill_ex(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, chunk, nullptr, workspace,
                          workspace_bytes, stream);
}

size_t gdn_prefill_status_offset(const gdn_desc* desc, int32_t chunk) {
    g_err[0] = 0;
    if (check_desc(desc, true) != GDN_OK) return 0;
    if (chunk != kChunk) { fail(GDN_ERR_UNSUPPORTED, "chunk must be 64 (got %d)", chunk); return 0; }
    return kStatusOff;
}

gdn_status gdn_prefill_prepare(const gdn_desc* desc, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const int32_t* cu_seqlens,
                               int32_t chunk, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_call(kPrepare, desc, q, k, v, g, beta, nullptr, nullptr, nullptr, cu_seqlens, chunk,
                        workspace, workspace_bytes, stream);
}

gdn_status gdn_prefill_scan(const gdn_desc* desc, const void* q, const void* k, const void* v,
                            const float* state_in, void* out, float* state_out,
                            const int32_t* cu_seqlens, int32_t chunk, void* workspace,
                            size_t workspace_bytes, void* stream) {
    return prefill_call(kScan, desc, q, k, v, nullptr, nullptr, state_in, out, state_out,
                        cu_seqlens, chunk, workspace, workspace_bytes, stream);
}


size_t gdn_prefill_segmented_workspace_bytes(const gdn_desc* desc, int32_t chunk, int64_t segment_tokens) {
    g_err[0] = 0;
    gdn_desc sub;
    size_t need = 0, soff = 0;
    if (segment_plan(desc, chunk, segment_tokens, &sub, &need, &soff) != GDN_OK) return 0;
    return need;
}

}  // extern "C"

namespace {

gdn_status segmented_call(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* state_in, void* out, float* state_out, int32_t chunk,
                          int64_t segment_tokens, void* workspace, size_t workspace_bytes, void* stream,
                          int scan_rows) {
    gdn_desc sub;
    size_t need = 0, soff = 0;
    gdn_status st = segment_plan(desc, chunk, segment_tokens, &sub, &need, &soff);
    if (st != GDN_OK) return st;
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
    const int64_t T = desc->total_tokens;
    const int hk = desc->h_k, hv = desc->h_v, d = desc->d_k;
    if (T > 0 && (!q || !k || !v || !g || !beta || !out))
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, g, beta and out must be non-NULL");
    const size_t io = dtype_size(desc->io_dtype), os = dtype_size(desc->out_dtype);
    const size_t sbytes = (size_t)hv * d * d * 4;
    const Span spans[] = {
        {(const char*)q, (size_t)T * hk * d * io, "q"},
        {(const char*)k, (size_t)T * hk * d * io, "k"},
        {(const char*)v, (size_t)T * hv * d * io, "v"},
        {(const char*)g, (size_t)T * hv * 4, "g"},
        {(const char*)beta, (size_t)T * hv * 4, "beta"},
        {(const char*)out, (size_t)T * hv * d * os, "out"},
        {(const char*)state_in, state_in ? sbytes : 0, "state_in"},
        {(const char*)state_out, state_out ? sbytes : 0, "state_out"},
        {(const char*)workspace, need, "workspace"},
    };
    st = check_align(spans, sizeof(spans) / sizeof(spans[0]));
    if (st != GDN_OK) return st;
    st = check_overlaps(spans, sizeof(spans) / sizeof(spans[0]), state_in, state_out);
    if (st != GDN_OK) return st;
    // the carried state: state_out, or a workspace buffer when the caller wants none
    float* carry = state_out ? state_out : reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + soff);
    const size_t seg_ws = soff;
    const int64_t nseg = T == 0 ? 1 : (T + segment_tokens - 1) / segment_tokens;
    for (int64_t i = 0; i < nseg; ++i) {
        const int64_t t0 = i * segment_tokens;
        gdn_desc part = *desc;
        part.total_tokens = (T - t0) < segment_tokens ? (T - t0) : segment_tokens;
        const char* qc = reinterpret_cast<const char*>(q) + (size_t)t0 * hk * d * io;
        const char* kc = reinterpret_cast<const char*>(k) + (size_t)t0 * hk * d * io;
        const char* vc = reinterpret_cast<const char*>(v) + (size_t)t0 * hv * d * io;
        const float* gc = g + (size_t)t0 * hv;
        const float* bc = beta + (size_t)t0 * hv;
        char* oc = reinterpret_cast<char*>(out) + (size_t)t0 * hv * d * os;
        const float* sin = (i == 0) ? state_in : carry;
        // the last segment writes state_out (or nothing when it is NULL)
        float* sout = (i + 1 == nseg) ? state_out : carry;
        st = prefill_call(kBoth, &part, T > 0 ? qc : q, T > 0 ? kc : k, T > 0 ? vc : v, T > 0 ? gc : g,
                          T > 0 ? bc : beta, sin, T > 0 ? oc : out, sout, nullptr, chunk, workspace, seg_ws, stream,
                          scan_rows, i == 0);
        if (st != GDN_OK) return st;
    }
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_segmented(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* state_in, void* out,
                                 float* state_out, int32_t chunk, int64_t segment_tokens, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    return segmented_call(desc, q, k, v, g, beta, state_in, out, state_out, chunk, segment_tokens, workspace,
                          workspace_bytes, stream, 0);
}


gdn_status gdn_decode_step(const gdn_desc* desc, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* state, void* out, void* stream) {
    g_err[0] = 0;
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if (!q || !k || !v || !g || !beta || !state || !out)
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, g, beta, state and out must be non-NULL");
    return decode_call(desc, q, k, v, g, beta, state, desc->num_seqs, nullptr, out, stream);
}

gdn_status gdn_prefill_direct(const gdn_desc* desc, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* state_in, void* out,
                              float* state_out, const int32_t* cu_seqlens, void* stream) {
    g_err[0] = 0;
    return direct_call(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, stream, 0, nullptr, 0.f);
}

gdn_status gdn_prefill_direct_ex(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* state_in, void* out,
                                 float* state_out, const int32_t* cu_seqlens, int32_t fuse,
                                 const float* norm_weight, float norm_eps, void* stream) {
    g_err[0] = 0;
    if (fuse & ~(GDN_FUSE_GATE_ACTIVATIONS | GDN_FUSE_OUTPUT_NORM))
        return fail(GDN_ERR_INVALID_ARGUMENT, "unknown fuse flags 0x%x", (unsigned)fuse);
    const bool norm = (fuse & GDN_FUSE_OUTPUT_NORM) != 0;
    if (norm && !(std::isfinite(norm_eps) && norm_eps > 0.f))
        return fail(GDN_ERR_INVALID_ARGUMENT, "norm_eps must be finite and > 0 (got %g)", (double)norm_eps);
    return direct_call(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, stream, fuse,
                       norm ? norm_weight : nullptr, norm ? norm_eps : 0.f);
}

gdn_status gdn_decode_step_ex(const gdn_desc* desc, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, float* state, void* out, int32_t fuse,
                              const float* norm_weight, float norm_eps, void* stream) {
    g_err[0] = 0;
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if (!q || !k || !v || !g || !beta || !state || !out)
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, g, beta, state and out must be non-NULL");
    if (fuse & ~(GDN_FUSE_GATE_ACTIVATIONS | GDN_FUSE_OUTPUT_NORM | GDN_STREAM_STATE))
        return fail(GDN_ERR_INVALID_ARGUMENT, "unknown fuse flags 0x%x", (unsigned)fuse);
    const bool norm = (fuse & GDN_FUSE_OUTPUT_NORM) != 0;
    if (norm && !(std::isfinite(norm_eps) && norm_eps > 0.f))
        return fail(GDN_ERR_INVALID_ARGUMENT, "norm_eps must be finite and > 0 (got %g)", (double)norm_eps);
    return decode_call(desc, q, k, v, g, beta, state, desc->num_seqs, nullptr, out, stream, fuse,
                       norm ? norm_weight : nullptr, norm ? norm_eps : 0.f);
}

gdn_status gdn_decode_step_slots(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, float* state_pool, int32_t num_slots,
                                 const int32_t* state_slots, void* out, void* stream) {
    g_err[0] = 0;
    gdn_status st = check_desc(desc, false);
    if (st != GDN_OK) return st;
    if (!q || !k || !v || !g || !beta || !state_pool || !state_slots || !out)
        return fail(GDN_ERR_INVALID_ARGUMENT,
                    "q, k, v, g, beta, state_pool, state_slots and out must be non-NULL");
    if (num_slots < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "num_slots must be >= 1 (got %d)", num_slots);
    return decode_call(desc, q, k, v, g, beta, state_pool, num_slots, state_slots, out, stream);
}


size_t gdn_prefill_two_level_workspace_bytes(const gdn_desc* desc, int32_t chunk, int32_t segments) {
    g_err[0] = 0;
    TwoLevel tl;
    return two_level_plan(desc, chunk, segments, &tl) == GDN_OK ? tl.total : 0;
}

gdn_status gdn_prefill_two_level(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* state_in, void* out,
                                 float* state_out, int32_t chunk, int32_t segments, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    TwoLevel tl;
    gdn_status st = two_level_plan(desc, chunk, segments, &tl);
    if (st != GDN_OK) return st;
    if (tl.P == 1)
        return prefill_call(kBoth, desc, q, k, v, g, beta, state_in, out, state_out, nullptr, chunk, workspace,
                            workspace_bytes, stream);
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", tl.total);
    if (workspace_bytes < tl.total)
        return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, tl.total);
    const int64_t T = desc->total_tokens;
    const int hk = desc->h_k, hv = desc->h_v, d = desc->d_k;
    if (!q || !k || !v || !g || !beta || !out)
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, g, beta and out must be non-NULL");
    const size_t io = dtype_size(desc->io_dtype), os = dtype_size(desc->out_dtype);
    const size_t sbytes = (size_t)hv * d * d * 4;
    const Span spans[] = {
        {(const char*)q, (size_t)T * hk * d * io, "q"},
        {(const char*)k, (size_t)T * hk * d * io, "k"},
        {(const char*)v, (size_t)T * hv * d * io, "v"},
        {(const char*)g, (size_t)T * hv * 4, "g"},
        {(const char*)beta, (size_t)T * hv * 4, "beta"},
        {(const char*)out, (size_t)T * hv * d * os, "out"},
        {(const char*)state_in, state_in ? sbytes : 0, "state_in"},
        {(const char*)state_out, state_out ? sbytes : 0, "state_out"},
        {(const char*)workspace, tl.total, "workspace"},
    };
    st = check_align(spans, sizeof(spans) / sizeof(spans[0]));
    if (st != GDN_OK) return st;
    st = check_overlaps(spans, sizeof(spans) / sizeof(spans[0]), state_in, state_out);
    if (st != GDN_OK) return st;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool in_bf16 = desc->io_dtype == GDN_BF16, out_bf16 = desc->out_dtype == GDN_BF16;
    const WsLayout ws = ws_layout(desc, false);
    char* wsb = reinterpret_cast<char*>(workspace);
    char* recs = wsb + ws.rec_off;
    char* krecs = wsb + ws.key_off;
    void* info = wsb + tl.info_off;
    float* R = reinterpret_cast<float*>(wsb + tl.r_off);
    float* B = reinterpret_cast<float*>(wsb + tl.b_off);
    float* starts = reinterpret_cast<float*>(wsb + tl.start_off);
    float* ends = reinterpret_cast<float*>(wsb + tl.end_off);
    const int P = tl.P;
    unsigned* status = reinterpret_cast<unsigned*>(wsb + kStatusOff);
    hipError_t e = gdn::launch_prep(d, in_bf16, q, k, v, g, beta, nullptr, nullptr, (int)tl.nblocks, (int)T, hk, hv,
                                    desc->qk_l2norm, desc->scale, recs, krecs, status, s);
    if (e == hipSuccess) e = gdn::launch_segment_info(info, P, tl.sb, (int)T, s);
    // segments 0..P-2 in one pass: affine parts B from zero, transitions R from the identity
    // (B and R are adjacent, so one state_out array holds both halves)
    if (e == hipSuccess)
        e = gdn::launch_scan_transition(d, in_bf16, 0, q, k, v, recs, krecs, info, B, wsb + ws.sink_off,
                                        2 * (P - 1) * hv, (int)T, hk, hv, s);
    if (e == hipSuccess) e = gdn::launch_compose(d, state_in, R, B, starts, P, hv, s);
    if (e == hipSuccess)
        e = gdn::launch_scan(d, in_bf16, out_bf16, 0, q, k, v, recs, krecs, info, starts, ends, out,
                             wsb + ws.sink_off, P * hv, (int)T, hk, hv, status, s);
    if (e == hipSuccess && state_out)
        e = hipMemcpyAsync(state_out, ends + (size_t)(P - 1) * hv * d * d, sbytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "two-level prefill launch: %s", hipGetErrorString(e));
    return GDN_OK;
}

gdn_status gdn_prefill_noalloc(const gdn_desc* desc, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const float* state_in, void* out,
                               float* state_out, const int32_t* cu_seqlens, int32_t chunk, void* stream) {
    g_err[0] = 0;
    gdn_status st = check_desc(desc, true);
    if (st != GDN_OK) return st;
    if (chunk != kChunk) return fail(GDN_ERR_UNSUPPORTED, "chunk must be 64 (got %d)", chunk);
    const size_t need = ws_layout(desc, true).total;
    if (need > kNoallocBytes)
        return fail(GDN_ERR_WORKSPACE, "this problem needs %zu workspace bytes; gdn_prefill_noalloc has %zu", need,
                    kNoallocBytes);
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != GDN_OK) return st;
    return gdn_prefill_ex(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, chunk, nullptr, ws,
                          kNoallocBytes, stream);
}

}  // extern "C"

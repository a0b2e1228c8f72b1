// Host side of libgdn: argument validation, dispatch and HIP error capture
// for the C ABI declared in include/gdn.h.
//
// Validation is fail-closed, in the spirit of the dispatch the
// jax-linear-attention page describes under "How it works" (a kernel runs
// only for the shapes it is tested on), except that there is no fallback: a
// call the kernels do not cover returns GDN_ERR_UNSUPPORTED.  Every check
// runs before any HIP call, so a rejected call touches no device state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

// Scratch of gdn_chunk_fwd_noalloc: the piece scan's end and start states,
// for callers that cannot allocate.  A device global, so every GPU the
// library runs on holds its own copy (at its own address) until the process
// ends.  In host code `scratch` names a host-side stand-in, never the device
// memory: kernels get the address hipGetSymbolAddress returns for the
// current device (static_scratch below).
static constexpr size_t kStaticScratchBytes = GDN_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

thread_local hipError_t g_last_hip_error = hipSuccess;

// The device address of `scratch` on each device, looked up once per device
// (with that device current) on its first gdn_chunk_fwd_noalloc call.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t static_scratch(void *&ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

bool aligned16(const void *p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// The forward's shapes: both dtypes take dk, dv in {64, 128, 256}.
bool supported(gdn_dtype dtype, int32_t dk, int32_t dv) {
    if (dtype != GDN_BF16 && dtype != GDN_F32)
        return false;
    return (dk == 64 || dk == 128 || dk == 256) && (dv == 64 || dv == 128 || dv == 256);
}

// Pieces per row for the piece-parallel scan of long rows (1: one pass over
// whole rows), for batch-mode bf16 calls.  With P pieces the first pass runs
// (P - 1) pieces x (value tiles + dk / 64 transition tiles) workgroups and
// the output pass P pieces x value tiles, each workgroup walking about
// chunks / P chunks; one workgroup per CU is resident.  The cost, in units of
// one whole-row chunk step, is rounds x chunks per piece for each pass (a
// first-pass chunk costs about what an output-pass chunk does), plus P - 1
// serial steps of the scan over start states (kScanStep, by dk) and a fixed
// cost for the two extra launches.  These were fitted to forced piece counts
// on rows of 1,024 to 16,384 tokens with 8 to 128 rows; a plan is used only
// when it beats whole rows by a twentieth.  Pieces hold at least
// kMinPieceChunks chunks.
constexpr int64_t kCUs = 256;
constexpr int64_t kMinPieceChunks = 4;
constexpr double kPieceFixed = 2.0;

double scan_step_cost(int32_t dk) { return dk == 64 ? 1.9 : dk == 128 ? 3.9 : 8.3; }

struct PiecePlan {
    int32_t pieces;
    int64_t piece_len;  // tokens, a multiple of 64
};

PiecePlan plan_pieces(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_v, int32_t dk, int32_t dv,
                      bool packed) {
    PiecePlan best{1, T};
    if (packed || dtype != GDN_BF16 || dv % 64 != 0)
        return best;
    const int64_t rows = B * H_v;
    const int64_t items = rows * (dv / 64);
    const int64_t items_ends = rows * (dv / 64 + dk / 64);
    const int64_t chunks = (T + 63) / 64;
    const auto rounds = [](int64_t wgs) { return (double)((wgs + kCUs - 1) / kCUs); };
    const double whole = rounds(items) * (double)chunks;
    double best_cost = 0.95 * whole;
    const int64_t max_p = chunks / kMinPieceChunks < 256 ? chunks / kMinPieceChunks : 256;
    for (int64_t n = 2; n <= max_p; ++n) {
        const int64_t per = (chunks + n - 1) / n;
        const int64_t pieces = (chunks + per - 1) / per;
        const double cost = (rounds((pieces - 1) * items_ends) + rounds(pieces * items)) *
                                (double)per +
                            scan_step_cost(dk) * (double)(pieces - 1) + kPieceFixed;
        if (cost < best_cost) {
            best_cost = cost;
            best = PiecePlan{(int32_t)pieces, per * 64};
        }
    }
    return best;
}

// Pieces of packed documents, planned from the host copy of cu_seqlens.
// Whole documents are scheduled longest first (doc_order), so their cost is
// about max(longest document, total chunk steps over the CUs); with pieces of
// piece_len tokens the two passes run every piece but each document's last
// (with the transition tiles), then all pieces, each pass in rounds of one
// workgroup per CU times the piece length (pieces are near-equal, so they do
// not spread below whole rounds: 16 documents x 8 heads measured 162 us in
// pieces against 123 us whole when the second pass was costed as spread
// work), plus the scan's serial steps over the most pieces a document has,
// in the same units as plan_pieces.
// Pieces may use at most `max_slots` slots, the capacity the size-only
// workspace query promises (the single-row plan of T tokens).
struct PackedPlan {
    int64_t piece_len = 0;   // 0: whole documents
    int64_t slots = 0;       // sum over documents of (pieces - 1)
    int64_t items_ends = 0;  // pieces of the first pass
    int64_t items_all = 0;   // all pieces
};

PackedPlan plan_packed(gdn_dtype dtype, int32_t H_v, int32_t dk, int32_t dv, const int32_t *cu,
                       int32_t N, int64_t max_slots) {
    PackedPlan best;
    if (dtype != GDN_BF16 || dv % 64 != 0 || max_slots <= 0)
        return best;
    const int64_t tiles = dv / 64, ends_tiles = dv / 64 + dk / 64;
    int64_t total = 0, maxc = 0;
    for (int32_t n = 0; n < N; ++n) {
        const int64_t c = ((int64_t)cu[n + 1] - cu[n] + 63) / 64;
        total += c;
        maxc = c > maxc ? c : maxc;
    }
    const auto rounds = [](int64_t wgs) { return (double)((wgs + kCUs - 1) / kCUs); };
    const double spread = (double)((total * H_v * tiles + kCUs - 1) / kCUs);
    const double whole = (double)maxc > spread ? (double)maxc : spread;
    double best_cost = 0.95 * whole;
    for (int64_t pc = kMinPieceChunks; pc < maxc; pc = pc + 1 + pc / 8) {
        int64_t slots = 0, np_max = 1;
        for (int32_t n = 0; n < N; ++n) {
            const int64_t c = ((int64_t)cu[n + 1] - cu[n] + 63) / 64;
            const int64_t np = c > pc ? (c + pc - 1) / pc : 1;
            slots += np - 1;
            np_max = np > np_max ? np : np_max;
        }
        if (slots == 0 || slots > max_slots)
            continue;
        const double cost = (rounds(slots * H_v * ends_tiles) +
                             rounds((slots + N) * H_v * tiles)) * (double)pc +
                            scan_step_cost(dk) * (double)(np_max - 1) + kPieceFixed;
        if (cost < best_cost) {
            best_cost = cost;
            best.piece_len = pc * 64;
            best.slots = slots;
        }
    }
    if (best.piece_len > 0) {
        best.items_ends = best.slots;
        best.items_all = best.slots + N;
    }
    return best;
}

// Bytes of the document order array of a packed call (0 when not used).
size_t order_bytes(int32_t N) {
    return N > 1 && N <= gdn::kMaxOrderedDocs ? ((size_t)N * 4 + 255) / 256 * 256 : 0;
}

}  // namespace

extern "C" {

size_t gdn_chunk_fwd_workspace_size(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk,
                                    int32_t H_v, int32_t dk, int32_t dv, int32_t n_seqs) {
    (void)n_seqs;
    if (B < 1 || T < 1 || H_qk < 1 || H_v < 1 || H_v % H_qk != 0 || B > INT32_MAX ||
        !supported(dtype, dk, dv))
        return 0;
    // The piece scan stages the end states and start states of its pieces;
    // a packed call (B = 1) may also rank its documents.  A packed call's
    // pieces use at most the slots of the single-row plan of T tokens.
    const PiecePlan p = plan_pieces(dtype, B, T, H_v, dk, dv, false);
    return gdn::fwd_piece_bytes(B * (p.pieces - 1), H_v, dk, dv) +
           (B == 1 && dtype == GDN_BF16 ? order_bytes(n_seqs) : 0);
}

// Checks a forward call before anything touches the GPU; on success N is
// the number of sequences.
static gdn_status fwd_validate(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk, int32_t H_v,
                               int32_t dk, int32_t dv, const void *q, const void *k,
                               const void *v, const float *g, const float *beta, uint32_t flags,
                               const float *h0, const int32_t *cu_seqlens,
                               const int32_t *cu_seqlens_host, int32_t n_seqs, const void *o,
                               const float *ht, int32_t &N) {
    if (B < 1 || T < 1 || H_qk < 1 || H_v < 1 || dk < 1 || dv < 1)
        return GDN_ERR_INVALID_ARG;
    if (!q || !k || !v || !g || !beta || !o)
        return GDN_ERR_INVALID_ARG;
    if ((flags & ~(GDN_QK_L2NORM | GDN_GATE_ACT)) != 0)
        return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_F32 && dtype != GDN_BF16)
        return GDN_ERR_UNSUPPORTED;
    if (H_v % H_qk != 0 || !supported(dtype, dk, dv))
        return GDN_ERR_UNSUPPORTED;
    // Sizes must index without overflow: B * T * H * d elements in int64.
    const int64_t hmax = H_v > H_qk ? H_v : H_qk;
    const int64_t dmax = dk > dv ? dk : dv;
    if (B > INT64_MAX / T || B * T > INT64_MAX / (hmax * dmax))
        return GDN_ERR_INVALID_ARG;
    N = (int32_t)B;
    if (cu_seqlens) {
        if (B != 1 || n_seqs < 1)
            return GDN_ERR_INVALID_ARG;
        N = n_seqs;
        if (cu_seqlens_host) {
            if (cu_seqlens_host[0] != 0 || (int64_t)cu_seqlens_host[N] != T)
                return GDN_ERR_INVALID_ARG;
            for (int32_t i = 0; i < N; ++i)
                if (cu_seqlens_host[i + 1] < cu_seqlens_host[i])
                    return GDN_ERR_INVALID_ARG;
        }
    } else if (cu_seqlens_host) {
        return GDN_ERR_INVALID_ARG;
    } else if (B > INT32_MAX) {
        return GDN_ERR_INVALID_ARG;
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(o) || !aligned16(h0) || !aligned16(ht) || !aligned16(cu_seqlens))
        return GDN_ERR_MISALIGNED;
    return GDN_OK;
}

// The plan of one forward call: the piece scan (pieces > 1) over batch rows
// or packed documents, and the schedule of packed documents.
struct FwdPlan {
    int32_t pieces = 1;         // batch rows: pieces per row; packed: 2 when split
    int64_t piece_len = 0;
    int64_t slots = 0;
    int64_t items_ends = 0, items_all = 0;
    bool order = false;         // packed: rank the documents, longest first
};

// Bytes of the workspace a plan uses: the order array, then the piece arrays.
static size_t plan_bytes(const FwdPlan &p, int32_t N, int32_t H_v, int32_t dk, int32_t dv) {
    return (p.order ? order_bytes(N) : 0) + gdn::fwd_piece_bytes(p.slots, H_v, dk, dv);
}

// The plan of a validated call given `ws_bytes` of workspace (0: none).
static FwdPlan plan_call(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_v, int32_t dk,
                         int32_t dv, const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                         int32_t N, bool have_ws) {
    FwdPlan f;
    if (!have_ws)
        return f;
    if (!cu_seqlens) {
        const PiecePlan p = plan_pieces(dtype, B, T, H_v, dk, dv, false);
        f.pieces = p.pieces;
        f.piece_len = p.piece_len;
        f.slots = (int64_t)N * (p.pieces - 1);
        return f;
    }
    // Ranking the documents pays only when their workgroups do not all fit
    // on the CUs at once (then the longest start first); otherwise its launch
    // is pure cost (about 3 us measured on 16 documents x 8 heads).
    f.order = dtype == GDN_BF16 && order_bytes(N) > 0 && (int64_t)N * H_v * (dv / 64) > kCUs;
    if (cu_seqlens_host) {
        const PiecePlan single = plan_pieces(dtype, 1, T, H_v, dk, dv, false);
        const PackedPlan pp = plan_packed(dtype, H_v, dk, dv, cu_seqlens_host, N,
                                          single.pieces - 1);
        if (pp.piece_len > 0) {
            f.pieces = 2;
            f.piece_len = pp.piece_len;
            f.slots = pp.slots;
            f.items_ends = pp.items_ends;
            f.items_all = pp.items_all;
        }
    }
    return f;
}

// Launches a validated forward call with `plan`, whose arrays (if any) live
// at `scratch`.
static gdn_status fwd_launch(gdn_dtype dtype, int64_t T, int32_t H_qk, int32_t H_v, int32_t dk,
                             int32_t dv, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, float scale, uint32_t flags,
                             const float *h0, const int32_t *cu_seqlens, int32_t N, void *o,
                             float *ht, const FwdPlan &plan, void *scratch,
                             hipStream_t stream) {
    gdn::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.h0 = h0;
    a.cu = cu_seqlens;
    a.o = o;
    a.ht = ht;
    a.T = T;
    a.Hqk = H_qk;
    a.Hv = H_v;
    a.dk = dk;
    a.dv = dv;
    a.n_seqs = N;
    a.scale = scale;
    a.flags = flags;
    a.pieces = plan.pieces;
    a.piece_len = plan.piece_len;
    a.n_slots = plan.slots;
    a.items_ends = plan.items_ends;
    a.items_all = plan.items_all;
    a.piece_ends = nullptr;
    a.piece_starts = nullptr;
    a.order = nullptr;
    a.chunk_states = nullptr;
    char *ws = static_cast<char *>(scratch);
    if (plan.order) {
        a.order = reinterpret_cast<const int32_t *>(ws);
        ws += order_bytes(N);
    }
    if (plan.pieces > 1) {
        a.piece_ends = reinterpret_cast<float *>(ws);
        a.piece_starts =
            reinterpret_cast<float *>(ws + gdn::fwd_piece_starts_offset(plan.slots, H_v, dk, dv));
    }
    hipError_t e = hipSuccess;
    if (plan.order)
        e = gdn::launch_doc_order(cu_seqlens, N, reinterpret_cast<int32_t *>(scratch), stream);
    if (e == hipSuccess)
        e = dtype == GDN_BF16 ? gdn::launch_fwd_bf16(a, stream) : gdn::launch_fwd_f32(a, stream);
    if (e != hipSuccess) {
        g_last_hip_error = e;
        return GDN_ERR_HIP;
    }
    return GDN_OK;
}

gdn_status gdn_chunk_fwd_plan(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk, int32_t H_v,
                              int32_t dk, int32_t dv, const int32_t *cu_seqlens_host,
                              int32_t n_seqs, int64_t *piece_len, int64_t *slots,
                              int32_t *ordered) {
    if (!piece_len || !slots || !ordered)
        return GDN_ERR_INVALID_ARG;
    // Validated as a call; fake aligned addresses stand in for the tensors.
    const void *fake = reinterpret_cast<const void *>(uintptr_t{0x10000});
    const float *ff = static_cast<const float *>(fake);
    const int32_t *cu = cu_seqlens_host ? static_cast<const int32_t *>(fake) : nullptr;
    int32_t N = 0;
    const gdn_status st = fwd_validate(dtype, B, T, H_qk, H_v, dk, dv, fake, fake, fake, ff, ff,
                                       0u, nullptr, cu, cu_seqlens_host, n_seqs, fake, nullptr,
                                       N);
    if (st != GDN_OK)
        return st;
    const FwdPlan plan = plan_call(dtype, B, T, H_v, dk, dv, cu, cu_seqlens_host, N, true);
    *piece_len = plan.pieces > 1 ? plan.piece_len : 0;
    *slots = plan.slots;
    *ordered = plan.order ? 1 : 0;
    return GDN_OK;
}

gdn_status gdn_chunk_fwd(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk, int32_t H_v,
                         int32_t dk, int32_t dv, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, float scale, uint32_t flags,
                         const float *h0,
                         const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                         int32_t n_seqs, void *o, float *ht, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    int32_t N = 0;
    const gdn_status st = fwd_validate(dtype, B, T, H_qk, H_v, dk, dv, q, k, v, g, beta, flags,
                                       h0, cu_seqlens, cu_seqlens_host, n_seqs, o, ht, N);
    if (st != GDN_OK)
        return st;
    // The piece scan and the document order run when a workspace is given;
    // without one, whole rows (documents in index order).
    const FwdPlan plan = plan_call(dtype, B, T, H_v, dk, dv, cu_seqlens, cu_seqlens_host, N,
                                   workspace != nullptr);
    const size_t need = plan_bytes(plan, N, H_v, dk, dv);
    if (need > 0) {
        if (workspace_bytes < need)
            return GDN_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return GDN_ERR_MISALIGNED;
    }
    return fwd_launch(dtype, T, H_qk, H_v, dk, dv, q, k, v, g, beta, scale, flags, h0,
                      cu_seqlens, N, o, ht, plan, workspace, stream);
}

gdn_status gdn_chunk_fwd_noalloc(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk,
                                 int32_t H_v, int32_t dk, int32_t dv, const void *q,
                                 const void *k, const void *v, const float *g,
                                 const float *beta, float scale, uint32_t flags,
                                 const float *h0, const int32_t *cu_seqlens,
                                 const int32_t *cu_seqlens_host, int32_t n_seqs, void *o,
                                 float *ht, hipStream_t stream) {
    int32_t N = 0;
    const gdn_status st = fwd_validate(dtype, B, T, H_qk, H_v, dk, dv, q, k, v, g, beta, flags,
                                       h0, cu_seqlens, cu_seqlens_host, n_seqs, o, ht, N);
    if (st != GDN_OK)
        return st;
    // The same plan gdn_chunk_fwd makes with a workspace; its arrays go to
    // this device's static scratch, which bounds what it may need.
    const FwdPlan plan = plan_call(dtype, B, T, H_v, dk, dv, cu_seqlens, cu_seqlens_host, N,
                                   true);
    if (plan_bytes(plan, N, H_v, dk, dv) > kStaticScratchBytes)
        return GDN_ERR_SCRATCH_LIMIT;
    void *scratch_ptr = nullptr;
    const hipError_t e = static_scratch(scratch_ptr);
    if (e != hipSuccess) {
        g_last_hip_error = e;
        return GDN_ERR_HIP;
    }
    return fwd_launch(dtype, T, H_qk, H_v, dk, dv, q, k, v, g, beta, scale, flags, h0,
                      cu_seqlens, N, o, ht, plan, scratch_ptr, stream);
}

// The backward's shapes: bf16, dk in {64, 128, 256}, dv in {64, 128, 256}.
static bool bwd_supported(gdn_dtype dtype, int32_t dk, int32_t dv) {
    return dtype == GDN_BF16 && (dk == 64 || dk == 128 || dk == 256) &&
           (dv == 64 || dv == 128 || dv == 256);
}

// Chunks over all sequences (64 tokens, 32 at dk = 256): exact for batch
// rows; with cu_seqlens the bound ceil(T / C) + N covers any split into N
// documents.
static int64_t bwd_chunks(int64_t B, int64_t T, bool packed, int32_t N, int32_t dk) {
    const int64_t C = dk == 256 ? 32 : 64;
    const int64_t per_row = (T + C - 1) / C;
    return packed ? per_row + N : B * per_row;
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace bytes after the backward's own for the prepared copies of the
// inputs an option rewrites: q and k in bf16, g and beta in fp32.
static size_t bwd_prep_bytes(uint32_t flags, int64_t B, int64_t T, int32_t H_qk, int32_t H_v,
                             int32_t dk) {
    size_t n = 0;
    if (flags & GDN_QK_L2NORM)
        n += 2 * round256((size_t)B * (size_t)T * (size_t)H_qk * (size_t)dk * 2);
    if (flags & GDN_GATE_ACT)
        n += 2 * round256((size_t)B * (size_t)T * (size_t)H_v * 4);
    return n;
}

size_t gdn_chunk_bwd_workspace_size(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk,
                                    int32_t H_v, int32_t dk, int32_t dv, int32_t n_seqs,
                                    uint32_t flags) {
    if (!bwd_supported(dtype, dk, dv) || B < 1 || T < 1 || H_qk < 1 || H_v < 1 ||
        H_v % H_qk != 0 || n_seqs < 1 || (flags & ~(GDN_QK_L2NORM | GDN_GATE_ACT)) != 0)
        return 0;
    if (B > INT64_MAX / T || B * T > INT64_MAX / ((int64_t)(H_v > H_qk ? H_v : H_qk) * 256))
        return 0;
    // Packed documents need B == 1; the packed bound also covers one row.
    return gdn::bwd_workspace_bytes(bwd_chunks(B, T, B == 1, B == 1 ? n_seqs : (int32_t)B, dk),
                                    H_v, dk, dv) +
           bwd_prep_bytes(flags, B, T, H_qk, H_v, dk);
}

gdn_status gdn_chunk_bwd(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk, int32_t H_v,
                         int32_t dk, int32_t dv, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, float scale, uint32_t flags,
                         const float *h0, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, int32_t n_seqs, const void *dout,
                         const float *dht, void *dq, void *dk_, void *dv_, float *dg,
                         float *dbeta, float *dh0, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    if (B < 1 || T < 1 || H_qk < 1 || H_v < 1 || dk < 1 || dv < 1)
        return GDN_ERR_INVALID_ARG;
    if ((flags & ~(GDN_QK_L2NORM | GDN_GATE_ACT)) != 0)
        return GDN_ERR_INVALID_ARG;
    if (!q || !k || !v || !g || !beta || !dout || !dq || !dk_ || !dv_ || !dg || !dbeta)
        return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_F32 && dtype != GDN_BF16)
        return GDN_ERR_UNSUPPORTED;
    if (H_v % H_qk != 0 || !bwd_supported(dtype, dk, dv))
        return GDN_ERR_UNSUPPORTED;
    const int64_t hmax = H_v > H_qk ? H_v : H_qk;
    // the workspace states are 128 keys wide (256 at dk = 256)
    const int64_t dmax = dv > 128 || dk > 128 ? 256 : 128;
    if (B > INT64_MAX / T || B * T > INT64_MAX / (hmax * dmax))
        return GDN_ERR_INVALID_ARG;
    int32_t N = (int32_t)B;
    if (cu_seqlens) {
        if (B != 1 || n_seqs < 1)
            return GDN_ERR_INVALID_ARG;
        N = n_seqs;
        if (cu_seqlens_host) {
            if (cu_seqlens_host[0] != 0 || (int64_t)cu_seqlens_host[N] != T)
                return GDN_ERR_INVALID_ARG;
            for (int32_t i = 0; i < N; ++i)
                if (cu_seqlens_host[i + 1] < cu_seqlens_host[i])
                    return GDN_ERR_INVALID_ARG;
        }
    } else if (cu_seqlens_host) {
        return GDN_ERR_INVALID_ARG;
    } else if (B > INT32_MAX) {
        return GDN_ERR_INVALID_ARG;
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(h0) || !aligned16(cu_seqlens) || !aligned16(dout) || !aligned16(dht) ||
        !aligned16(dq) || !aligned16(dk_) || !aligned16(dv_) || !aligned16(dg) ||
        !aligned16(dbeta) || !aligned16(dh0))
        return GDN_ERR_MISALIGNED;
    const int64_t n_chunks = bwd_chunks(B, T, cu_seqlens != nullptr, N, dk);
    if (n_chunks > INT32_MAX)
        return GDN_ERR_INVALID_ARG;
    const size_t own = gdn::bwd_workspace_bytes(n_chunks, H_v, dk, dv);
    const size_t need = own + bwd_prep_bytes(flags, B, T, H_qk, H_v, dk);
    if (!workspace || workspace_bytes < need)
        return GDN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return GDN_ERR_MISALIGNED;

    // With an option set, the prepared inputs go to the end of the workspace,
    // the backward runs on them, and the chain through the preparation then
    // rewrites dq, dk, dg and dbeta in place.
    const bool l2 = flags & GDN_QK_L2NORM, gate = flags & GDN_GATE_ACT;
    const int64_t qk_rows = B * T * H_qk, gates = B * T * H_v;
    const void *qp = q, *kp = k;
    const float *gp = g, *bp = beta;
    if (flags) {
        unsigned char *w = static_cast<unsigned char *>(workspace) + own;
        gdn::PrepArgs p;
        p.q = q;
        p.k = k;
        p.g = g;
        p.beta = beta;
        p.q_out = p.k_out = nullptr;
        p.g_out = p.beta_out = nullptr;
        if (l2) {
            const size_t rows_bytes = round256((size_t)qk_rows * (size_t)dk * 2);
            p.q_out = w;
            p.k_out = w + rows_bytes;
            w += 2 * rows_bytes;
            qp = p.q_out;
            kp = p.k_out;
        }
        if (gate) {
            const size_t gate_bytes = round256((size_t)gates * 4);
            p.g_out = reinterpret_cast<float *>(w);
            p.beta_out = reinterpret_cast<float *>(w + gate_bytes);
            gp = p.g_out;
            bp = p.beta_out;
        }
        p.qk_rows = l2 ? qk_rows : 0;
        p.gate_n = gate ? gates : 0;
        p.dk = dk;
        p.flags = flags;
        p.bf16 = true;
        const hipError_t e = gdn::launch_preprocess(p, stream);
        if (e != hipSuccess) {
            g_last_hip_error = e;
            return GDN_ERR_HIP;
        }
    }

    gdn::BwdArgs a;
    a.q = qp;
    a.k = kp;
    a.v = v;
    a.g = gp;
    a.beta = bp;
    a.h0 = h0;
    a.cu = cu_seqlens;
    a.dout = dout;
    a.dht = dht;
    a.dq = dq;
    a.dk_ = dk_;
    a.dv_ = dv_;
    a.dg = dg;
    a.dbeta = dbeta;
    a.dh0 = dh0;
    a.T = T;
    a.n_chunks = n_chunks;
    a.Hqk = H_qk;
    a.Hv = H_v;
    a.dk = dk;
    a.dv = dv;
    a.n_seqs = N;
    a.scale = scale;
    gdn::bwd_carve(a, workspace);
    hipError_t e = gdn::launch_bwd_bf16(a, stream);
    if (e == hipSuccess && flags) {
        gdn::PrepBwdArgs c;
        c.q = q;
        c.k = k;
        c.dq = c.dq_out = dq;
        c.dk = c.dk_out = dk_;
        c.g = g;
        c.beta = beta;
        c.dg = c.dg_out = dg;
        c.dbeta = c.dbeta_out = dbeta;
        c.qk_rows = l2 ? qk_rows : 0;
        c.gate_n = gate ? gates : 0;
        c.dk_dim = dk;
        c.flags = flags;
        c.bf16 = true;
        e = gdn::launch_preprocess_bwd(c, stream);
    }
    if (e != hipSuccess) {
        g_last_hip_error = e;
        return GDN_ERR_HIP;
    }
    return GDN_OK;
}

gdn_status gdn_prepare_inputs(gdn_dtype dtype, int64_t n_qk_rows, int32_t dk, const void *q,
                              const void *k, void *q_out, void *k_out, int64_t n_gates,
                              const float *g, const float *beta, float *g_out,
                              float *beta_out, uint32_t flags, hipStream_t stream) {
    if ((flags & ~(GDN_QK_L2NORM | GDN_GATE_ACT)) != 0)
        return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_F32 && dtype != GDN_BF16)
        return GDN_ERR_UNSUPPORTED;
    const bool l2 = flags & GDN_QK_L2NORM, gate = flags & GDN_GATE_ACT;
    if (l2) {
        if (n_qk_rows < 0 || n_qk_rows > INT64_MAX / 256 || dk < 1)
            return GDN_ERR_INVALID_ARG;
        if (dk > 256)
            return GDN_ERR_UNSUPPORTED;
    }
    if (gate && (n_gates < 0 || n_gates > INT64_MAX / 2))
        return GDN_ERR_INVALID_ARG;
    // Pointers of an option with nothing to do are not read.
    if (l2 && n_qk_rows > 0) {
        if (!q || !k || !q_out || !k_out)
            return GDN_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(q_out) || !aligned16(k_out))
            return GDN_ERR_MISALIGNED;
    }
    if (gate && n_gates > 0) {
        if (!g || !beta || !g_out || !beta_out)
            return GDN_ERR_INVALID_ARG;
        if (!aligned16(g) || !aligned16(beta) || !aligned16(g_out) || !aligned16(beta_out))
            return GDN_ERR_MISALIGNED;
    }
    gdn::PrepArgs a;
    a.q = q;
    a.k = k;
    a.q_out = q_out;
    a.k_out = k_out;
    a.g = g;
    a.beta = beta;
    a.g_out = g_out;
    a.beta_out = beta_out;
    a.qk_rows = l2 ? n_qk_rows : 0;
    a.gate_n = gate ? n_gates : 0;
    a.dk = dk;
    a.flags = flags;
    a.bf16 = dtype == GDN_BF16;
    const hipError_t e = gdn::launch_preprocess(a, stream);
    if (e != hipSuccess) {
        g_last_hip_error = e;
        return GDN_ERR_HIP;
    }
    return GDN_OK;
}

gdn_status gdn_prepare_inputs_bwd(gdn_dtype dtype, int64_t n_qk_rows, int32_t dk,
                                  const void *q, const void *k, const void *dq_in,
                                  const void *dk_in, void *dq_out, void *dk_out,
                                  int64_t n_gates, const float *g, const float *beta,
                                  const float *dg_in, const float *dbeta_in, float *dg_out,
                                  float *dbeta_out, uint32_t flags, hipStream_t stream) {
    if ((flags & ~(GDN_QK_L2NORM | GDN_GATE_ACT)) != 0)
        return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_F32 && dtype != GDN_BF16)
        return GDN_ERR_UNSUPPORTED;
    const bool l2 = flags & GDN_QK_L2NORM, gate = flags & GDN_GATE_ACT;
    if (l2) {
        if (n_qk_rows < 0 || n_qk_rows > INT64_MAX / 256 || dk < 1)
            return GDN_ERR_INVALID_ARG;
        if (dk > 256)
            return GDN_ERR_UNSUPPORTED;
    }
    if (gate && (n_gates < 0 || n_gates > INT64_MAX / 2))
        return GDN_ERR_INVALID_ARG;
    if (l2 && n_qk_rows > 0) {
        if (!q || !k || !dq_in || !dk_in || !dq_out || !dk_out)
            return GDN_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(dq_in) || !aligned16(dk_in) ||
            !aligned16(dq_out) || !aligned16(dk_out))
            return GDN_ERR_MISALIGNED;
    }
    if (gate && n_gates > 0) {
        if (!g || !beta || !dg_in || !dbeta_in || !dg_out || !dbeta_out)
            return GDN_ERR_INVALID_ARG;
        if (!aligned16(g) || !aligned16(beta) || !aligned16(dg_in) || !aligned16(dbeta_in) ||
            !aligned16(dg_out) || !aligned16(dbeta_out))
            return GDN_ERR_MISALIGNED;
    }
    gdn::PrepBwdArgs a;
    a.q = q;
    a.k = k;
    a.dq = dq_in;
    a.dk = dk_in;
    a.dq_out = dq_out;
    a.dk_out = dk_out;
    a.g = g;
    a.beta = beta;
    a.dg = dg_in;
    a.dbeta = dbeta_in;
    a.dg_out = dg_out;
    a.dbeta_out = dbeta_out;
    a.qk_rows = l2 ? n_qk_rows : 0;
    a.gate_n = gate ? n_gates : 0;
    a.dk_dim = dk;
    a.flags = flags;
    a.bf16 = dtype == GDN_BF16;
    const hipError_t e = gdn::launch_preprocess_bwd(a, stream);
    if (e != hipSuccess) {
        g_last_hip_error = e;
        return GDN_ERR_HIP;
    }
    return GDN_OK;
}

gdn_status gdn_recurrent_step(gdn_dtype dtype, int64_t N, int32_t H_qk, int32_t H_v,
                              int32_t dk, int32_t dv, const void *q, const void *k,
                              const void *v, const float *g, const float *beta, float scale,
                              uint32_t flags, float *state, const int32_t *slots,
                              int64_t n_slots, void *o, hipStream_t stream) {
    if (N < 0 || H_qk < 1 || H_v < 1 || dk < 1 || dv < 1 || n_slots < 0)
        return GDN_ERR_INVALID_ARG;
    if ((flags & ~(GDN_QK_L2NORM | GDN_GATE_ACT)) != 0)
        return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_F32 && dtype != GDN_BF16)
        return GDN_ERR_UNSUPPORTED;
    const auto size_ok = [](int32_t d) { return d == 64 || d == 128 || d == 256; };
    if (H_v % H_qk != 0 || !size_ok(dk) || !size_ok(dv))
        return GDN_ERR_UNSUPPORTED;
    if (!slots && n_slots < N)
        return GDN_ERR_INVALID_ARG;
    const int64_t per_slot = (int64_t)H_v * dk * dv;
    if (n_slots > INT64_MAX / per_slot || N > INT32_MAX / ((int64_t)H_v * (dv / 64)))
        return GDN_ERR_INVALID_ARG;
    if (N == 0)
        return GDN_OK;  // nothing to do; the pointers are not read
    if (!q || !k || !v || !g || !beta || !state || !o)
        return GDN_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(state) || !aligned16(slots) || !aligned16(o))
        return GDN_ERR_MISALIGNED;
    gdn::StepArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.slots = slots;
    a.o = o;
    a.N = N;
    a.n_slots = n_slots;
    a.Hqk = H_qk;
    a.Hv = H_v;
    a.dk = dk;
    a.dv = dv;
    a.scale = scale;
    a.flags = flags;
    a.bf16 = dtype == GDN_BF16;
    const hipError_t e = gdn::launch_recurrent_step(a, stream);
    if (e != hipSuccess) {
        g_last_hip_error = e;
        return GDN_ERR_HIP;
    }
    return GDN_OK;
}

const char *gdn_status_string(gdn_status status) {
    switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG: invalid argument";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: no kernel for this shape or dtype";
    case GDN_ERR_MISALIGNED: return "GDN_ERR_MISALIGNED: pointer not 16-byte aligned";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: a HIP launch failed";
    case GDN_ERR_SCRATCH_LIMIT:
        return "GDN_ERR_SCRATCH_LIMIT: the call needs more scratch than the library's static "
               "maximum (GDN_STATIC_SCRATCH_BYTES)";
    }
    return "unknown gdn_status";
}

hipError_t gdn_last_hip_error(void) {
    return g_last_hip_error;
}

int32_t gdn_version(void) {
    return 100;  // 0.1.0
}

}  // extern "C"

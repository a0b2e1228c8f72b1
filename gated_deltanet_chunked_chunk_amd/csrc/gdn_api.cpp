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

#include "gdn.h"
#include "gdn_internal.h"

namespace {

thread_local hipError_t g_last_hip_error = hipSuccess;

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

}  // namespace

extern "C" {

size_t gdn_chunk_fwd_workspace_size(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk,
                                    int32_t H_v, int32_t dk, int32_t dv, int32_t n_seqs) {
    (void)n_seqs;
    if (B < 1 || T < 1 || H_qk < 1 || H_v < 1 || H_v % H_qk != 0 || B > INT32_MAX ||
        !supported(dtype, dk, dv))
        return 0;
    // Only the piece scan of long rows stages anything in HBM: the end states
    // and start states of its pieces.
    const PiecePlan p = plan_pieces(dtype, B, T, H_v, dk, dv, false);
    return gdn::fwd_piece_bytes((int32_t)B, p.pieces, H_v, dk, dv);
}

gdn_status gdn_chunk_fwd(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk, int32_t H_v,
                         int32_t dk, int32_t dv, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, float scale, uint32_t flags,
                         const float *h0,
                         const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                         int32_t n_seqs, void *o, float *ht, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
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
        !aligned16(o) || !aligned16(h0) || !aligned16(ht) || !aligned16(cu_seqlens))
        return GDN_ERR_MISALIGNED;
    // The piece scan runs when a workspace is given; without one, whole rows.
    PiecePlan plan = plan_pieces(dtype, B, T, H_v, dk, dv, cu_seqlens != nullptr);
    if (!workspace)
        plan = PiecePlan{1, T};
    const size_t need = gdn::fwd_piece_bytes(N, plan.pieces, H_v, dk, dv);
    if (need > 0) {
        if (workspace_bytes < need)
            return GDN_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return GDN_ERR_MISALIGNED;
    }

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
    a.piece_ends = nullptr;
    a.piece_starts = nullptr;
    a.chunk_states = nullptr;
    if (plan.pieces > 1) {
        const size_t per = (size_t)N * (plan.pieces - 1) * H_v * dk;
        a.piece_ends = static_cast<float *>(workspace);
        a.piece_starts = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                                   (per * (dv + dk) * 4 + 255) / 256 * 256);
    }

    const hipError_t e = dtype == GDN_BF16 ? gdn::launch_fwd_bf16(a, stream)
                                           : gdn::launch_fwd_f32(a, stream);
    if (e != hipSuccess) {
        g_last_hip_error = e;
        return GDN_ERR_HIP;
    }
    return GDN_OK;
}

// The backward's shapes: bf16, dk in {64, 128}, dv in {64, 128, 256}.
static bool bwd_supported(gdn_dtype dtype, int32_t dk, int32_t dv) {
    return dtype == GDN_BF16 && (dk == 64 || dk == 128) && (dv == 64 || dv == 128 || dv == 256);
}

// Chunks of 64 tokens over all sequences: exact for batch rows; with
// cu_seqlens the bound ceil(T / 64) + N covers any split into N documents.
static int64_t bwd_chunks(int64_t B, int64_t T, bool packed, int32_t N) {
    const int64_t per_row = (T + 63) / 64;
    return packed ? per_row + N : B * per_row;
}

size_t gdn_chunk_bwd_workspace_size(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk,
                                    int32_t H_v, int32_t dk, int32_t dv, int32_t n_seqs) {
    if (!bwd_supported(dtype, dk, dv) || B < 1 || T < 1 || H_qk < 1 || H_v < 1 ||
        H_v % H_qk != 0 || n_seqs < 1)
        return 0;
    // Packed documents need B == 1; the packed bound also covers one row.
    return gdn::bwd_workspace_bytes(bwd_chunks(B, T, B == 1, B == 1 ? n_seqs : (int32_t)B), H_v,
                                    dk, dv);
}

gdn_status gdn_chunk_bwd(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk, int32_t H_v,
                         int32_t dk, int32_t dv, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, float scale, const float *h0,
                         const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                         int32_t n_seqs, const void *dout, const float *dht, void *dq,
                         void *dk_, void *dv_, float *dg, float *dbeta, float *dh0,
                         void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B < 1 || T < 1 || H_qk < 1 || H_v < 1 || dk < 1 || dv < 1)
        return GDN_ERR_INVALID_ARG;
    if (!q || !k || !v || !g || !beta || !dout || !dq || !dk_ || !dv_ || !dg || !dbeta)
        return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_F32 && dtype != GDN_BF16)
        return GDN_ERR_UNSUPPORTED;
    if (H_v % H_qk != 0 || !bwd_supported(dtype, dk, dv))
        return GDN_ERR_UNSUPPORTED;
    const int64_t hmax = H_v > H_qk ? H_v : H_qk;
    const int64_t dmax = dv > 128 ? dv : 128;  // the workspace states are 128 keys wide
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
    const int64_t n_chunks = bwd_chunks(B, T, cu_seqlens != nullptr, N);
    if (n_chunks > INT32_MAX)
        return GDN_ERR_INVALID_ARG;
    const size_t need = gdn::bwd_workspace_bytes(n_chunks, H_v, dk, dv);
    if (!workspace || workspace_bytes < need)
        return GDN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return GDN_ERR_MISALIGNED;

    gdn::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
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
    const hipError_t e = gdn::launch_bwd_bf16(a, stream);
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

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

bool supported(gdn_dtype dtype, int32_t dk, int32_t dv) {
    if (dtype == GDN_BF16)
        return dk == 128 && (dv == 64 || dv == 128);
    if (dtype == GDN_F32)
        return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
    return false;
}

}  // namespace

extern "C" {

size_t gdn_chunk_fwd_workspace_size(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk,
                                    int32_t H_v, int32_t dk, int32_t dv, int32_t n_seqs) {
    (void)dtype; (void)B; (void)T; (void)H_qk; (void)H_v; (void)dk; (void)dv; (void)n_seqs;
    return 0;  // the forward kernels keep every intermediate on chip
}

gdn_status gdn_chunk_fwd(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk, int32_t H_v,
                         int32_t dk, int32_t dv, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, float scale, const float *h0,
                         const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                         int32_t n_seqs, void *o, float *ht, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    if (B < 1 || T < 1 || H_qk < 1 || H_v < 1 || dk < 1 || dv < 1)
        return GDN_ERR_INVALID_ARG;
    if (!q || !k || !v || !g || !beta || !o)
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
    const size_t need = gdn_chunk_fwd_workspace_size(dtype, B, T, H_qk, H_v, dk, dv, N);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return GDN_ERR_WORKSPACE;

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

    const hipError_t e = dtype == GDN_BF16 ? gdn::launch_fwd_bf16(a, stream)
                                           : gdn::launch_fwd_f32(a, stream);
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

// Internal interface between the host API (gdn_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Arguments of one forward call, after validation.  Sizes are as in
// gdn_chunk_fwd; `n_seqs` is the number of sequences (documents, or B).
struct FwdArgs {
    const void *q;
    const void *k;
    const void *v;
    const float *g;
    const float *beta;
    const float *h0;        // [n_seqs, Hv, dk, dv] or null
    const int32_t *cu;      // [n_seqs + 1] device offsets, or null (rows of T tokens)
    void *o;
    float *ht;              // [n_seqs, Hv, dk, dv] or null
    int64_t T;              // tokens per row (batch mode)
    int32_t Hqk, Hv, dk, dv;
    int32_t n_seqs;
    float scale;
};

// bf16 q/k/v/o, dk = 128, dv a multiple of 64: one workgroup per
// (sequence, value head, 64 value columns).
hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream);

// fp32 q/k/v/o, dk and dv in {64, 128}: one workgroup per (sequence, value
// head, 32 value columns).
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream);

}  // namespace gdn

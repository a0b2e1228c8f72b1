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

// Arguments of one backward call, after validation (bf16, dk = 128, dv a
// multiple of 64).  The workspace regions are described in gdn_bwd_bf16.hip.
struct BwdArgs {
    const void *q;
    const void *k;
    const void *v;
    const float *g;
    const float *beta;
    const float *h0;        // [n_seqs, Hv, dk, dv] or null
    const int32_t *cu;      // [n_seqs + 1] device offsets, or null
    const void *dout;       // [B, T, Hv, dv]
    const float *dht;       // [n_seqs, Hv, dk, dv] or null
    void *dq;               // [B, T, Hqk, dk]
    void *dk_;              // [B, T, Hqk, dk]
    void *dv_;              // [B, T, Hv, dv]
    float *dg;              // [B, T, Hv]
    float *dbeta;           // [B, T, Hv]
    float *dh0;             // [n_seqs, Hv, dk, dv] or null
    float *ws_T;            // [n_chunks, Hv, 64, 64]
    uint16_t *ws_P;         // [n_chunks, Hv, 64, 64]
    float *ws_gam;          // [n_chunks, Hv, 64]
    uint16_t *ws_hs;        // [n_chunks, Hv, dv, dk] bf16: the state entering each chunk
    uint16_t *ws_dhs;       // [n_chunks, Hv, dv, dk] bf16: the gradient of the state leaving it
    int64_t T;              // tokens per row (batch mode)
    int64_t n_chunks;       // chunks the workspace holds (an upper bound with cu)
    int32_t Hqk, Hv, dk, dv;
    int32_t n_seqs;
    float scale;
};

// Workspace bytes of the backward for `n_chunks` chunks (all sequences).
size_t bwd_workspace_bytes(int64_t n_chunks, int32_t Hv, int32_t dk, int32_t dv);

// Carves the workspace into the BwdArgs regions.
void bwd_carve(BwdArgs &a, void *workspace);

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t stream);

}  // namespace gdn

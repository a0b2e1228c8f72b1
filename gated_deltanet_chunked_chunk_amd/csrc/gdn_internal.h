// Internal interface between the host API (gdn_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Option bits of the forward, the preparation pass and the recurrent step
// (GDN_QK_L2NORM and GDN_GATE_ACT in gdn.h).
constexpr uint32_t kStepL2Norm = 1u;
constexpr uint32_t kStepGateAct = 2u;

// The gate activations, in fp32 with the accurate expf:
// logsigmoid(x) = min(x, 0) - log(1 + exp(-|x|)) and sigmoid(x), the latter
// as exp(x) / (1 + exp(x)) for x < 0 so neither form overflows.
__device__ __forceinline__ float logsigmoid_f32(float x) {
    return fminf(x, 0.0f) - log1pf(expf(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid_f32(float x) {
    const float e = expf(-fabsf(x));
    return x >= 0.0f ? 1.0f / (1.0f + e) : e / (1.0f + e);
}

// 1 / ||x|| from a row's sum of squares, with the hardware reciprocal square
// root (within 1 ulp; a correctly rounded 1 / sqrt costs the forward kernel's
// helper waves 8 us more at 8 x 2048 x 16 heads); a zero row stays zero.
__device__ __forceinline__ float inv_l2_norm(float sumsq) {
    return sumsq > 0.0f ? __builtin_amdgcn_rsqf(sumsq) : 0.0f;
}

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
    uint32_t flags;         // kStepL2Norm | kStepGateAct: in-op preparation
    // Piece-parallel scan (pieces <= 1: off).  Batch rows: row n is split
    // into `pieces` runs of piece_len tokens (a multiple of 64; the last
    // takes the rest).  Packed documents (cu set, pieces > 1): document n is
    // split into ceil(len / piece_len) runs (one for a shorter or empty
    // document).  Every piece but a sequence's last has a slot in the piece
    // arrays, the slots of sequence n following those of sequences < n;
    // n_slots is their number (the arrays' capacity).
    int32_t pieces;
    int64_t piece_len;
    int64_t n_slots;
    int64_t items_ends;     // packed pieces: pieces of the first pass (all but each document's last)
    int64_t items_all;      // packed pieces: all pieces
    float *piece_ends;      // [n_slots, Hv, dk, dv + dk]: F | Phi of each piece but the last
    float *piece_starts;    // [n_slots, Hv, dk, dv]: the state entering the piece after each slot's
    const int32_t *order;   // packed: [n_seqs] documents longest first (doc_order), or null
    // The backward's two state passes (launch_bwd_state_passes); chunks are
    // numbered over the sequences in order, 64 tokens each.
    uint16_t *chunk_states; // [n_chunks, Hv, dv, 128] bf16: the state entering each chunk
    uint16_t *chunk_deltas; // [n_chunks, Hv, 64, dv] bf16: each chunk's Delta rows
    uint16_t *chunk_dstates;// [n_chunks, Hv, dv, 128] bf16: the gradient of the state leaving each chunk
    uint16_t *chunk_drhs;   // [n_chunks, Hv, 64, dv] bf16: each chunk's drhs rows
    void *dv_out;           // [B, T, Hv, dv] bf16: the gradient of v
    const float *dht;       // [n_seqs, Hv, dk, dv] or null
    float *dh0;             // [n_seqs, Hv, dk, dv] or null
};

// The backward's state passes, on the forward kernel's helper/state
// pipeline (bf16, dk = 64 or 128; `a` as for the forward with pieces = 1,
// flags = 0):
//   forward pass (v = the input v): every chunk's entering state M0
//     (chunk_states, transposed, zeros past dk) and Delta rows (chunk_deltas);
//   reverse pass (v = dout): the state-gradient recurrence from dht, chunks in
//     reverse, storing the gradient of every chunk's leaving state
//     (chunk_dstates), its drhs rows (chunk_drhs), dV (dv_out) and dh0.
hipError_t launch_bwd_state_passes(const FwdArgs &fwd, const FwdArgs &rev, hipStream_t stream);

// Workspace bytes of the piece scan for `slots` slots (batch rows:
// n_seqs * (pieces - 1)); the start states follow the end states at
// fwd_piece_starts_offset().
size_t fwd_piece_bytes(int64_t slots, int32_t Hv, int32_t dk, int32_t dv);
size_t fwd_piece_starts_offset(int64_t slots, int32_t Hv, int32_t dk, int32_t dv);

// Ranks the n_seqs documents of cu by length, longest first (ties by index),
// into order[n_seqs]: the order in which the forward schedules them.
// n_seqs <= kMaxOrderedDocs.
constexpr int32_t kMaxOrderedDocs = 2048;
hipError_t launch_doc_order(const int32_t *cu, int32_t n_seqs, int32_t *order, hipStream_t stream);

// bf16 q/k/v/o, dk in {64, 128, 256}, dv a multiple of 64: one workgroup per
// (sequence, value head, 64 value columns).
hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream);

// fp32 q/k/v/o, dk and dv in {64, 128, 256}: one workgroup per (sequence,
// value head, 32 value columns).
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream);

// Arguments of one backward call, after validation (bf16, dk in {64, 128},
// dv a multiple of 64).  The workspace regions are described in gdn_bwd_bf16.hip.
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
    uint16_t *ws_hs;        // [n_chunks, Hv, dv, 128] bf16: the state entering each chunk
    uint16_t *ws_dhs;       // [n_chunks, Hv, dv, 128] bf16: the gradient of the state leaving it
    uint16_t *ws_delta;     // [n_chunks, Hv, 64, dv] bf16: each chunk's Delta rows
    uint16_t *ws_drhs;      // [n_chunks, Hv, 64, dv] bf16: each chunk's drhs rows
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

// One recurrent step for N sequences, the state updated in place in a cache
// of n_slots states.  Sizes: dk in {64, 128, 256}, dv a multiple of 64.
struct StepArgs {
    const void *q;          // [N, Hqk, dk]
    const void *k;          // [N, Hqk, dk]
    const void *v;          // [N, Hv, dv]
    const float *g;         // [N, Hv]
    const float *beta;      // [N, Hv]
    float *state;           // [n_slots, Hv, dk, dv]
    const int32_t *slots;   // [N] cache slot of each sequence, or null (slot n)
    void *o;                // [N, Hv, dv]
    int64_t N, n_slots;
    int32_t Hqk, Hv, dk, dv;
    float scale;
    uint32_t flags;
    bool bf16;
};

hipError_t launch_recurrent_step(const StepArgs &a, hipStream_t stream);

// Rows of q and k divided by their L2 norms and the gate activations, written
// to separate outputs (which may be the inputs).  dk <= 128.
struct PrepArgs {
    const void *q;
    const void *k;
    void *q_out;
    void *k_out;
    const float *g;
    const float *beta;
    float *g_out;
    float *beta_out;
    int64_t qk_rows;        // rows of dk elements in q (and in k)
    int64_t gate_n;         // elements of g (and of beta)
    int32_t dk;
    uint32_t flags;
    bool bf16;
};

hipError_t launch_preprocess(const PrepArgs &a, hipStream_t stream);

// The reverse of the preparation: gradients with respect to the raw q, k, g
// and beta from those with respect to the prepared values.  Outputs may be
// their gradient inputs (in place).
struct PrepBwdArgs {
    const void *q;          // raw rows
    const void *k;
    const void *dq;         // gradients with respect to the normalised rows
    const void *dk;
    void *dq_out;
    void *dk_out;
    const float *g;         // raw gates
    const float *beta;
    const float *dg;        // gradients with respect to the activated gates
    const float *dbeta;
    float *dg_out;
    float *dbeta_out;
    int64_t qk_rows;
    int64_t gate_n;
    int32_t dk_dim;
    uint32_t flags;
    bool bf16;
};

hipError_t launch_preprocess_bwd(const PrepBwdArgs &a, hipStream_t stream);

}  // namespace gdn

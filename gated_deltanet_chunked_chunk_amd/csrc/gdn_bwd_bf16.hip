// Chunkwise gated delta rule backward, bf16 inputs, dk = 128 (and dk = 64,
// staged into the 128-wide tiles with zero upper halves), for gfx950.
//
// Reverse mode of the forward in gdn_fwd_bf16.hip: the gradients of
// L = sum(do * o) + sum(dht * ht) with respect to q, k, v, g, beta and h0.
// The pages name the backward as the follow-on of the forward call and give
// no formulas for it; the chunk equations below are the chain rule applied to
// the forward's chunk equations (with gamma the in-chunk cumulative
// log-decay, e = exp(gamma), l = exp(gamma_L - gamma), D[r][s] =
// exp(gamma_r - gamma_s) for s <= r, M0 the state entering the chunk, dML the
// gradient of the state leaving it and dO = scale * do):
//
//   forward   A = beta_r D (K K^T) strictly below the diagonal, T = (I + A)^-1
//             X = K M0, rhs = diag(beta) (V - diag(e) X), Delta = T rhs
//             P = D * (Q K^T) on and below the diagonal
//             O = diag(e) Q M0 + P Delta,  M_L = exp(gamma_L) M0 + K^T diag(l) Delta
//   reverse   dDelta = diag(l) K dML + P^T dO,  drhs = T^T dDelta
//             dM0 = exp(gamma_L) dML + Q^T diag(e) dO - K^T diag(beta e) drhs
//             dV = diag(beta) drhs,  dA = -drhs Delta^T (strictly lower)
//             dQ = diag(e) dO M0^T + (dP * D) K,          dP = dO Delta^T
//             dK = -diag(beta e) drhs M0^T + diag(l) Delta dML^T + (dP * D)^T Q
//                  + (S + S^T) K,  S = diag(beta) (dA * D)
//             dbeta_r = sum_c drhs (V - diag(e) X) + sum_s (dA * D * K K^T)
//             dgamma from e, l, exp(gamma_L) and D; dg = the reverse
//             cumulative sum of dgamma over the chunk.
//
// Three passes:
//   forward state pass and reverse state pass (gdn_fwd_bf16.hip, the
//                forward kernel's helper/state pipeline, launch_bwd_state_passes):
//                the forward pass stores every chunk's entering state M0
//                (transposed, [dv][128]) and Delta rows; the reverse pass
//                walks the chunks backwards with dM in MFMA accumulators (the
//                helper waves rebuild A, the diagonal inverses and P for each
//                chunk exactly as in the forward), stores the gradient of every
//                chunk's leaving state and its drhs rows, writes dV and dh0.
//                Only these four bf16 arrays cross HBM between the passes.
//   bwd_grads    per (chunk, q/k head), all in parallel: the contractions
//                over the value columns (dP, dA, dQ, dK) and the gate
//                gradients, from M0, dML, Delta and drhs; the value heads
//                sharing the q/k head are summed in a fixed order.
//
// Precision: products accumulate in fp32 on bf16 MFMA.  The state passes
// carry fp32 states and split computed operands of their recurrences into
// hi + lo bf16 pairs (see gdn_fwd_bf16.hip).  bwd_grads uses single bf16
// roundings of M0, dML, Delta, drhs and of the row-scaled operands (e dO,
// beta e drhs, l Delta, dP * D, S + S^T); every result it forms is an output
// (relative tolerance 1e-2), not a recurrence.
//
// MFMA v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][8(l/16)+j] and
// B[8(l/16)+j][l%16] (j = 0..7), receives C[4(l/16)+r][l%16] (r = 0..3).
// ds_read_b64_tr_b16: within 16 lanes, lane 16g+i receives element i%4 of the
// 8-byte words addressed by lanes 16g + 4j + i/4, j = 0..3.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kC = 64;     // chunk length
constexpr int kDK = 128;   // key dimension
constexpr int kLK = 136;   // row stride (bf16) of K and Q tiles
constexpr int kL64 = 72;   // row stride (bf16) of 64-wide tiles
constexpr unsigned kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit elements
constexpr float kLog2e = 1.44269504088896341f;
constexpr int kGT = 512;   // bwd_grads threads
constexpr int64_t kGradGrid = 256;  // bwd_grads workgroups: one per CU

// Barrier for LDS hand-offs between the waves: waits for this wave's LDS
// operations only, so vector-memory loads in flight (the prefetched tiles)
// stay in flight across it.  Loads that write LDS directly are waited for
// explicitly (vmcnt) where their tiles are first read.
__device__ __forceinline__ void lds_barrier() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t f2bf(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ float bf2f(uint16_t x) {
    return __uint_as_float(static_cast<unsigned>(x) << 16);
}

__device__ __forceinline__ bf16x8 cat(u32x2 a, u32x2 b) {
    const u32x4 v = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ u32x2 ld8(const uint16_t *p) {
    return *reinterpret_cast<const u32x2 *>(p);
}

__device__ __forceinline__ u32x2 ld_tr(const uint16_t *p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ f32x4 ld4f(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}

__device__ __forceinline__ u32x2 pack4(f32x4 x) {
    return u32x2{f2bf(x[0]) | (unsigned)f2bf(x[1]) << 16, f2bf(x[2]) | (unsigned)f2bf(x[3]) << 16};
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi) (x - hi is exact in fp32).
__device__ __forceinline__ void split4(f32x4 x, u32x2 &hi, u32x2 &lo) {
    f32x4 r;
    uint16_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = f2bf(x[i]);
        r[i] = x[i] - bf2f(h[i]);
    }
    hi = u32x2{h[0] | (unsigned)h[1] << 16, h[2] | (unsigned)h[3] << 16};
    lo = pack4(r);
}

// Fragments from bf16 tiles in LDS (row stride ld elements).
// A operand rows [row0 + lr][k0 + 8 lg .. + 7] of a row-major tile; also the
// B operand of X^T for a row-major X[n][k].
__device__ __forceinline__ bf16x8 frag_rows(const uint16_t *t, int ld, int row0, int k0, int lr,
                                            int lg) {
    return __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const u32x4 *>(t + (row0 + lr) * ld + k0 + 8 * lg));
}

// The same rows in the permuted k order of a B operand assembled from two
// C-layout tiles: positions 8g..8g+3 hold k0 + 4g .., 8g+4..8g+7 hold
// k0 + 16 + 4g ...
__device__ __forceinline__ bf16x8 frag_rows_perm(const uint16_t *t, int ld, int row0, int k0,
                                                 int lr, int lg) {
    const uint16_t *p = t + (row0 + lr) * ld + k0 + 4 * lg;
    return cat(ld8(p), ld8(p + 16));
}

// From a row-major X[k][col]: lane (lr, lg) receives X[k0 + 8 lg + j][col0 + lr],
// j = 0..7: the B operand of X, or the A operand of X^T.
__device__ __forceinline__ bf16x8 frag_cols(const uint16_t *t, int ld, int k0, int col0, int lr,
                                            int lg) {
    const uint16_t *p = t + (k0 + 8 * lg + (lr >> 2)) * ld + col0 + 4 * (lr & 3);
    return cat(ld_tr(p), ld_tr(p + 4 * ld));
}

// The same in the permuted k order (rows k0 + 4g + j and k0 + 16 + 4g + j).
__device__ __forceinline__ bf16x8 frag_cols_perm(const uint16_t *t, int ld, int k0, int col0,
                                                 int lr, int lg) {
    const uint16_t *p = t + (k0 + 4 * lg + (lr >> 2)) * ld + col0 + 4 * (lr & 3);
    return cat(ld_tr(p), ld_tr(p + 16 * ld));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// The same for a base and size the caller knows to be equal on every lane
// (they depend only on the work item): taken from the first lane, so the
// descriptor sits in scalar registers and each load is issued once instead
// of in a loop over the distinct descriptors the compiler would otherwise
// have to allow for.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_uniform(const void *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
    return rsrc(reinterpret_cast<const void *>(static_cast<uint64_t>(hi) << 32 | lo),
                __builtin_amdgcn_readfirstlane(bytes));
}

template <int Ctrl, int RowMask>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl, RowMask, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp<0x111, 0xF>(x);
    x += dpp<0x112, 0xF>(x);
    x += dpp<0x114, 0xF>(x);
    x += dpp<0x118, 0xF>(x);
    x += dpp<0x142, 0xA>(x);
    x += dpp<0x143, 0xC>(x);
    return x;
}

// Sum over the 16 lanes of this lane's row, by DPP (no LDS round trips):
// swaps within quads (xor 1, xor 2), then the half-row and row mirrors.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1, 0xF>(x);
    x += dpp<0x4E, 0xF>(x);
    x += dpp<0x141, 0xF>(x);
    x += dpp<0x140, 0xF>(x);
    return x;
}

// Sum over the 64 lanes, the same on every lane.
__device__ __forceinline__ float wave_sum(float x) {
    const int r = __builtin_bit_cast(int, row16_sum(x));
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 48)));
}

// Where chunk gc of the whole call lies.
struct ChunkLoc {
    int n;          // sequence
    int c;          // chunk within the sequence
    int64_t p;      // first token
    int L;          // valid tokens
};

__device__ __forceinline__ int64_t seq_start(const BwdArgs &a, int n) {
    return a.cu ? (int64_t)a.cu[n] : (int64_t)n * a.T;
}

__device__ __forceinline__ int64_t seq_len(const BwdArgs &a, int n) {
    return a.cu ? (int64_t)a.cu[n + 1] - a.cu[n] : a.T;
}

// Where chunk gc (of CL tokens) of the whole call lies; false past the last.
template <int CL = kC>
__device__ __forceinline__ bool locate(const BwdArgs &a, int64_t gc, ChunkLoc &cl) {
    if (!a.cu) {
        const int64_t nch = (a.T + CL - 1) / CL;
        const int64_t n = gc / nch;
        if (n >= a.n_seqs)
            return false;
        cl.n = (int)n;
        cl.c = (int)(gc % nch);
    } else {
        int64_t b = 0;
        int n = 0;
        for (; n < a.n_seqs; ++n) {
            const int64_t nc = (seq_len(a, n) + CL - 1) / CL;
            if (gc < b + nc)
                break;
            b += nc;
        }
        if (n >= a.n_seqs)
            return false;
        cl.n = n;
        cl.c = (int)(gc - b);
    }
    cl.p = seq_start(a, cl.n) + (int64_t)CL * cl.c;
    cl.L = (int)min<int64_t>(CL, seq_len(a, cl.n) - (int64_t)CL * cl.c);
    return true;
}

__device__ __forceinline__ float dot8(u32x4 a, u32x4 b) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s += bf2f(a[i] & 0xffff) * bf2f(b[i] & 0xffff) + bf2f(a[i] >> 16) * bf2f(b[i] >> 16);
    return s;
}

// Rows [p, p + L) of a [*, H, dk] bf16 tensor (dk = 64 or 128) at head h,
// written straight into a [64][kLK] LDS tile by buffer loads that store to
// LDS (no registers): the tile's 64 x 17 slots of 16 bytes
// (16 of data and the pad per row) are 17 wave-wide loads, wave w issuing
// loads w, w + 8 and w + 16.  Lane i of load n fills slot 64 n + i.  The pad
// slots, the slots past dk and the rows past L read out of the buffer's
// range, which loads zeros.  The data lands after the wave's vmcnt drains.
__device__ __forceinline__ void rows_to_lds(uint16_t *tile, const void *src, int64_t p, int L,
                                            int H, int h, int dk, int w, int lane) {
    constexpr int kSlots = kLK / 8;  // 17 per row
    const uint32_t row_bytes = (uint32_t)H * dk * 2;
    const __amdgpu_buffer_rsrc_t r =
        rsrc_uniform(static_cast<const uint16_t *>(src) + (p * H + h) * (int64_t)dk,
                     (uint32_t)(L - 1) * row_bytes + dk * 2);
    for (int n = w; n < kSlots; n += kGT / 64) {
        const int s = 64 * n + lane, row = s / kSlots, pc = s - kSlots * row;
        const uint32_t off = pc < 16 && 8 * pc < dk ? row * row_bytes + 16 * pc : 0x40000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void *)(tile + 8 * 64 * n), 16, off, 0, 0, 0);
    }
}


// ---------------------------------------------------------------------------
// bwd_grads: per (chunk, q/k head), 512 threads, one persistent workgroup per
// CU walking the (chunk, q/k head) items.  Each item's K and Q rows are
// loaded into registers once the value steps of the item before it are done
// and stored to the other half of the K/Q tiles before that item's epilogue;
// its first value step is loaded during that item's last one.  The barriers
// wait for LDS operations only, so these loads stay in flight across them.
// Wave w works on the chunk's rows [16 rb, 16 rb + 16), rb = w % 4, and the
// half hd = w / 4 of every [64 x *] result: of a 64-column value step the columns 32 hd ..,
// of dq and dk the key tiles 4 hd .. 4 hd + 3, of the 64 x 64 products the
// column tiles 2 hd, 2 hd + 1.  The value heads of the q/k head are taken in
// turn, each in steps of 64 value columns whose tiles (v, do, Delta, drhs
// rows; M0^T, dML^T rows) are loaded into registers during the previous
// step and stored to LDS at the next.


struct alignas(16) GradSmem {
    // The small tables and the step tiles first, so that their addresses
    // fit the 16-bit immediate offsets of LDS instructions.  Every tile
    // starts 16-byte aligned (alignas): its 16-byte accesses need it.
    float gam[kC], e[kC], l[kC], bt[kC];  // gam: gamma log2(e), the decays are exp2 of differences
    float rowb[2][kC], rowg[2][kC];
    float colpart[4][kC];
    float red[kGT];
    float eL;
    alignas(16) union {
        struct {
            uint16_t V[kC * kL64];   // v rows, the step's 64 columns
            uint16_t dO[kC * kL64];  // do rows (unscaled)
            uint16_t Dl[kC * kL64];  // Delta rows
            uint16_t dR[kC * kL64];  // drhs rows
        } t;
        struct {
            uint16_t PD[kC * kL64];  // scale dP * D (diagonal included)
            uint16_t SS[kC * kL64];  // S + S^T, S = diag(beta) (-dA * D) strictly lower
        } d;
    } u;
    alignas(16) union {
        struct {
            uint16_t M0[kC * kLK];   // M0^T of the step's 64 value columns: [col][key]
            uint16_t dM[kC * kLK];   // dML^T
        } s;
        uint16_t out[2][kC * kLK];   // dq, dk rows at the end
    } m;
    alignas(16) uint16_t KQ[2][2][kC * kLK];  // [item parity][K, Q]: the next item's land in the other half
};
static_assert(offsetof(GradSmem, u) % 16 == 0 && offsetof(GradSmem, m) % 16 == 0 &&
                  offsetof(GradSmem, KQ) % 16 == 0 && (kC * kLK * 2) % 16 == 0 &&
                  (kC * kL64 * 2) % 16 == 0,
              "16-byte LDS accesses need 16-byte aligned tiles");

// One value step's tiles in flight: thread t holds pieces t and t + 512 of
// M0^T and dML^T (row i / 16, 16 bytes i % 16) and piece t of the v, do,
// Delta and drhs rows (row t / 8, 16 bytes t % 8); wave 0 the head's gates.
struct GradPre {
    u32x4 m[2], d[2], v, o, dl, dr;
    float g, b;
};

__device__ __forceinline__ void grads_issue(GradPre &pre, const BwdArgs &a, const ChunkLoc &cl,
                                            int64_t gc, int j, int step_col, bool gates, int tid) {
    const int64_t wi = gc * a.Hv + j;
    const uint16_t *m0 = a.ws_hs + (wi * a.dv + step_col) * (int64_t)kDK;
    const uint16_t *dm = a.ws_dhs + (wi * a.dv + step_col) * (int64_t)kDK;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + kGT * u;
        pre.m[u] = *reinterpret_cast<const u32x4 *>(m0 + (i >> 4) * kDK + 8 * (i & 15));
        pre.d[u] = *reinterpret_cast<const u32x4 *>(dm + (i >> 4) * kDK + 8 * (i & 15));
    }
    const int row = tid >> 3, pc = tid & 7;
    const uint32_t xrow = (uint32_t)a.Hv * a.dv * 2;
    const int64_t xofs = (cl.p * a.Hv + j) * (int64_t)a.dv + step_col;
    const uint32_t span = (uint32_t)(cl.L - 1) * xrow + 128;
    const __amdgpu_buffer_rsrc_t rv =
        rsrc_uniform(static_cast<const uint16_t *>(a.v) + xofs, span);
    const __amdgpu_buffer_rsrc_t ro =
        rsrc_uniform(static_cast<const uint16_t *>(a.dout) + xofs, span);
    pre.v = __builtin_amdgcn_raw_buffer_load_b128(rv, row * xrow + 16 * pc, 0, 0);
    pre.o = __builtin_amdgcn_raw_buffer_load_b128(ro, row * xrow + 16 * pc, 0, 0);
    const int64_t wofs = (wi * kC + row) * (int64_t)a.dv + step_col + 8 * pc;
    pre.dl = *reinterpret_cast<const u32x4 *>(a.ws_delta + wofs);
    pre.dr = *reinterpret_cast<const u32x4 *>(a.ws_drhs + wofs);
    // The head's gates (used by wave 0 on a head's first step), loaded by
    // every thread with no branch: rows past L, and threads past the chunk,
    // read out of the buffer's range, which loads zeros.  (A conditional
    // load here made the compiler drain every load in flight before the
    // step's work.)
    const uint32_t gspan = (uint32_t)(cl.L - 1) * a.Hv * 4 + 4;
    const __amdgpu_buffer_rsrc_t rg = rsrc_uniform(a.g + cl.p * a.Hv + j, gspan);
    const __amdgpu_buffer_rsrc_t rb = rsrc_uniform(a.beta + cl.p * a.Hv + j, gspan);
    const uint32_t goff = tid < kC ? (uint32_t)(tid * a.Hv * 4) : 0x40000000u;
    pre.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, goff, 0, 0));
    pre.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, goff, 0, 0));
    (void)gates;
}

__device__ __forceinline__ void grads_commit(GradSmem &S, const GradPre &pre, int tid) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + kGT * u;
        *reinterpret_cast<u32x4 *>(S.m.s.M0 + (i >> 4) * kLK + 8 * (i & 15)) = pre.m[u];
        *reinterpret_cast<u32x4 *>(S.m.s.dM + (i >> 4) * kLK + 8 * (i & 15)) = pre.d[u];
    }
    const int o = (tid >> 3) * kL64 + 8 * (tid & 7);
    *reinterpret_cast<u32x4 *>(S.u.t.V + o) = pre.v;
    *reinterpret_cast<u32x4 *>(S.u.t.dO + o) = pre.o;
    *reinterpret_cast<u32x4 *>(S.u.t.Dl + o) = pre.dl;
    *reinterpret_cast<u32x4 *>(S.u.t.dR + o) = pre.dr;
}

// The next item's K and Q rows in registers: thread t holds 16-byte pieces
// t + kGT u (row i / (dk / 8), piece i % (dk / 8)) of each; rows past L, and
// every piece when there is no next item (a buffer of no bytes), read as
// zeros.  Loaded when an item's value steps are done (behind the next item's
// first value step, so neither delays the loads of this item's steps),
// stored to the other K/Q half of LDS before the item's dq/dk epilogue.
template <int KX>
struct KQPre {
    u32x4 k[KX / 2], q[KX / 2];
};

template <int KX>
__device__ __forceinline__ void kq_issue(KQPre<KX> &pre, const BwdArgs &a, const ChunkLoc &cl,
                                         int hk, bool any, int tid) {
    constexpr int pieces = 4 * KX;  // per row
    const uint32_t row_bytes = (uint32_t)a.Hqk * a.dk * 2;
    const uint32_t span = any ? (uint32_t)(cl.L - 1) * row_bytes + a.dk * 2 : 0u;
    const int64_t base = (cl.p * a.Hqk + hk) * (int64_t)a.dk;
    const __amdgpu_buffer_rsrc_t rk = rsrc_uniform(static_cast<const uint16_t *>(a.k) + base, span);
    const __amdgpu_buffer_rsrc_t rq = rsrc_uniform(static_cast<const uint16_t *>(a.q) + base, span);
#pragma unroll
    for (int u = 0; u < KX / 2; ++u) {
        const int i = tid + kGT * u, row = i / pieces, pc = i % pieces;
        const uint32_t off = row * row_bytes + 16 * pc;
        pre.k[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        pre.q[u] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    }
}

template <int KX>
__device__ __forceinline__ void kq_commit(uint16_t *sK, uint16_t *sQ, const KQPre<KX> &pre, int tid) {
    constexpr int pieces = 4 * KX;
#pragma unroll
    for (int u = 0; u < KX / 2; ++u) {
        const int i = tid + kGT * u, row = i / pieces, pc = i % pieces;
        *reinterpret_cast<u32x4 *>(sK + row * kLK + 8 * pc) = pre.k[u];
        *reinterpret_cast<u32x4 *>(sQ + row * kLK + 8 * pc) = pre.q[u];
    }
}

// An A operand (rows row0 + lr, k0 + 8 lg .. + 7 of a row-major bf16 tile)
// multiplied by the row's factor f and rounded back to bf16.
__device__ __forceinline__ bf16x8 frag_rows_scaled(const uint16_t *t, int ld, int row0, int k0,
                                                   int lr, int lg, float f) {
    const u32x4 x = *reinterpret_cast<const u32x4 *>(t + (row0 + lr) * ld + k0 + 8 * lg);
    u32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned w = x[i];
        const float lo = bf2f(static_cast<uint16_t>(w & 0xffff)) * f;
        const float hi = bf2f(static_cast<uint16_t>(w >> 16)) * f;
        y[i] = f2bf(lo) | (unsigned)f2bf(hi) << 16;
    }
    return __builtin_bit_cast(bf16x8, y);
}

// Four rows (16 rb + 4 lg + r) of column c0 + lr of a row-major bf16 tile,
// the C layout of a 16 x 16 tile, by one transpose read.
__device__ __forceinline__ f32x4 tile_c(const uint16_t *t, int ld, int row0, int c0, int lr,
                                        int lg) {
    const u32x2 v = ld_tr(t + (row0 + 4 * lg + (lr >> 2)) * ld + c0 + 4 * (lr & 3));
    return f32x4{bf2f(static_cast<uint16_t>(v.x & 0xffff)), bf2f(static_cast<uint16_t>(v.x >> 16)),
                 bf2f(static_cast<uint16_t>(v.y & 0xffff)), bf2f(static_cast<uint16_t>(v.y >> 16))};
}

// KX: 32-wide key steps that carry data (dk / 32), a constant so that the
// key loops unroll and their LDS reads issue together.
template <int KX>
__global__ __launch_bounds__(kGT) void bwd_grads(BwdArgs a) {
    __shared__ GradSmem S;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rb = w & 3, hd = w >> 2;
    const int G = a.Hv / a.Hqk;
    const int nsteps = a.dv / 64;
    const int steps = G * nsteps;
    const float scale = a.scale;
    constexpr int kx_end = KX;
    // Persistent: workgroup b takes work items b, b + gridDim.x, ..., item i
    // being chunk i / Hqk and q/k head i % Hqk; chunks past the last
    // document's (the packed bound) are skipped.  The next item's first
    // value step is loaded during the current item's last step, its K and Q
    // rows once the current item's value steps are done.
    const int64_t total = a.n_chunks * a.Hqk;
    auto find = [&](int64_t from, ChunkLoc &c, int64_t &g, int &h) {
        for (int64_t i = from; i < total; i += gridDim.x) {
            g = i / a.Hqk;
            h = (int)(i % a.Hqk);
            if (locate(a, g, c))
                return i;
        }
        return total;
    };
    ChunkLoc cl;
    int64_t gc = 0;
    int hk = 0;
    int64_t item = find(blockIdx.x, cl, gc, hk);
    if (item >= total)
        return;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    rows_to_lds(S.KQ[0][0], a.k, cl.p, cl.L, a.Hqk, hk, a.dk, wu, lane);
    rows_to_lds(S.KQ[0][1], a.q, cl.p, cl.L, a.Hqk, hk, a.dk, wu, lane);
    GradPre pre;
    grads_issue(pre, a, cl, gc, hk * G, 0, true, tid);

    for (int par = 0;; par ^= 1) {
    ChunkLoc ncl;
    int64_t ngc = 0;
    int nhk = 0;
    const int64_t nitem = find(item + gridDim.x, ncl, ngc, nhk);
    // This item's K and Q tiles are in LDS (the first item's loaded straight
    // into LDS above, later ones stored from registers by every wave before
    // this barrier) and its first value step's loads, needed next, have
    // landed; every wave is past the previous item, whose tiles the other
    // half held, so the next item's K and Q can go to that half.
    // Vector memory operations complete in order, so waiting until at most
    // KX are outstanding (the previous item's dq and dk stores) suffices.
    __builtin_amdgcn_s_waitcnt(0x0f70 | KX);  // vmcnt(KX)
    lds_barrier();
    KQPre<KX> kqn;
    const uint16_t *sK = S.KQ[par][0], *sQ = S.KQ[par][1];

    f32x4 dQ[4], dK[4];   // key tiles 4 hd + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dQ[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        dK[i] = dQ[i];
    }

    for (int gi = 0; gi < G; ++gi) {
        const int j = hk * G + gi;
        f32x4 dP[2], dA[2];   // column tiles 2 hd + i
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            dP[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            dA[i] = dP[i];
        }
        float pb[4] = {0.f, 0.f, 0.f, 0.f};   // dbeta parts of rows 16 rb + 4 lg + r
        float pg[4] = {0.f, 0.f, 0.f, 0.f};   // dgamma parts
        float msum = 0.0f;                    // this thread's part of sum(M0 * dML)
        float lsum = 0.0f;                    // this thread's part of sum_r l_r Delta U
        for (int vs = 0; vs < nsteps; ++vs) {
            const int step = gi * nsteps + vs;
            lds_barrier();  // the previous step's (or head's) readers are done
            grads_commit(S, pre, tid);
#pragma unroll
            for (int u = 0; u < 2; ++u)
                msum += dot8(pre.m[u], pre.d[u]);
            if (vs == 0 && w == 0) {
                // The head's gate tables; padded rows carry g = 0, so
                // gamma_63 = gamma_{L-1}.
                const float x = wave_prefix_sum(pre.g);
                const float gL = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), kC - 1));
                S.gam[lane] = x * kLog2e;
                S.e[lane] = __expf(x);
                S.l[lane] = __expf(gL - x);
                S.bt[lane] = pre.b;
                if (lane == 0)
                    S.eL = __expf(gL);
            }
            lds_barrier();
            {
                // One issue site with no branch around it (two sites, or a
                // skipped issue, made the compiler copy the loaded registers
                // and wait for the loads right after issuing them): the next
                // step, else the next item's first, else this step again.
                const bool more = step + 1 < steps, next_item = !more && nitem < total;
                const int sn = more ? step + 1 : next_item ? 0 : step;
                const int gn = sn / nsteps, vn = sn % nsteps;
                grads_issue(pre, a, next_item ? ncl : cl, next_item ? ngc : gc,
                            (next_item ? nhk : hk) * G + gn, 64 * vn, vn == 0, tid);
            }
            // The lane indices pass through an empty asm so that the many
            // addresses formed from them are computed here, not hoisted out
            // of the loop and held across it.
            int lrv = lane & 15, lgv = lane >> 4;
            asm volatile("" : "+v"(lrv), "+v"(lgv));
            const int lr = lrv, lg = lgv;

            // X = K M0, Y = Q M0, U = K dML on this wave's 32 columns, one
            // 16-column tile at a time, and the row terms of dbeta and dgamma
            // from their elementwise products.
            const f32x4 b4 = ld4f(S.bt + 16 * rb + 4 * lg), e4 = ld4f(S.e + 16 * rb + 4 * lg);
            const f32x4 l4 = ld4f(S.l + 16 * rb + 4 * lg);
            // K and Q fragments are read once for both 16-column tiles.
            f32x4 Xt[2], Yt[2], Ut[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                Xt[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                Yt[t] = Xt[t];
                Ut[t] = Xt[t];
            }
#pragma unroll
            for (int kx = 0; kx < kx_end; ++kx) {
                const bf16x8 fk = frag_rows(sK, kLK, 16 * rb, 32 * kx, lr, lg);
                const bf16x8 fq = frag_rows(sQ, kLK, 16 * rb, 32 * kx, lr, lg);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int c0 = 32 * hd + 16 * t;
                    const bf16x8 bm = frag_rows(S.m.s.M0, kLK, c0, 32 * kx, lr, lg);
                    const bf16x8 bd = frag_rows(S.m.s.dM, kLK, c0, 32 * kx, lr, lg);
                    Xt[t] = mma(fk, bm, Xt[t]);
                    Yt[t] = mma(fq, bm, Yt[t]);
                    Ut[t] = mma(fk, bd, Ut[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int c0 = 32 * hd + 16 * t;
                const f32x4 X = Xt[t], Y = Yt[t], U = Ut[t];
                const f32x4 vv = tile_c(S.u.t.V, kL64, 16 * rb, c0, lr, lg);
                const f32x4 oo = tile_c(S.u.t.dO, kL64, 16 * rb, c0, lr, lg);
                const f32x4 dl = tile_c(S.u.t.Dl, kL64, 16 * rb, c0, lr, lg);
                const f32x4 dr = tile_c(S.u.t.dR, kL64, 16 * rb, c0, lr, lg);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pb[r] += dr[r] * (vv[r] - e4[r] * X[r]);
                    const float lu = l4[r] * dl[r] * U[r];
                    pg[r] += e4[r] * scale * oo[r] * Y[r] - b4[r] * e4[r] * dr[r] * X[r] - lu;
                    lsum += lu;
                }
            }
            // dQ += diag(e) dO M0^T, dK += -diag(beta e) drhs M0^T + diag(l) Delta dML^T
            // (rows 16 rb, key tiles 4 hd + i); dP += do Delta^T, dA += drhs Delta^T.
            const int rrow = 16 * rb + lr;
            const float fe = scale * S.e[rrow], fx = -S.bt[rrow] * S.e[rrow], fl = S.l[rrow];
#pragma unroll 1
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 ye = frag_rows_scaled(S.u.t.dO, kL64, 16 * rb, 32 * kk, lr, lg, fe);
                const bf16x8 xe = frag_rows_scaled(S.u.t.dR, kL64, 16 * rb, 32 * kk, lr, lg, fx);
                const bf16x8 wl = frag_rows_scaled(S.u.t.Dl, kL64, 16 * rb, 32 * kk, lr, lg, fl);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int nj = 4 * hd + i;
                    if (nj >= 2 * kx_end)
                        continue;  // key tiles past dk
                    const bf16x8 bm = frag_cols(S.m.s.M0, kLK, 32 * kk, 16 * nj, lr, lg);
                    const bf16x8 bd = frag_cols(S.m.s.dM, kLK, 32 * kk, 16 * nj, lr, lg);
                    dQ[i] = mma(ye, bm, dQ[i]);
                    dK[i] = mma(xe, bm, dK[i]);
                    dK[i] = mma(wl, bd, dK[i]);
                }
                const bf16x8 fo = frag_rows(S.u.t.dO, kL64, 16 * rb, 32 * kk, lr, lg);
                const bf16x8 fr = frag_rows(S.u.t.dR, kL64, 16 * rb, 32 * kk, lr, lg);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const bf16x8 bdl = frag_rows(S.u.t.Dl, kL64, 16 * (2 * hd + i), 32 * kk, lr, lg);
                    dP[i] = mma(fo, bdl, dP[i]);
                    dA[i] = mma(fr, bdl, dA[i]);
                }
            }
        }
        lds_barrier();  // every read of the step tiles is done: the D-phase tiles take their space
        if (gi + 1 == G)
            kq_issue<KX>(kqn, a, nitem < total ? ncl : cl, nitem < total ? nhk : hk, nitem < total, tid);

        // Through A and P: D, S = diag(beta) (-dA * D), dP * D, and their
        // dbeta and dgamma terms.
        int lrv = lane & 15, lgv = lane >> 4;
        asm volatile("" : "+v"(lrv), "+v"(lgv));
        const int lr = lrv, lg = lgv;
        // K K^T and Q K^T on this wave's tiles (rows 16 rb, column tiles 2 hd + i).
        f32x4 kk4[2], qk4[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            kk4[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            qk4[i] = kk4[i];
#pragma unroll
            for (int kx = 0; kx < kx_end; ++kx) {
                const bf16x8 b = frag_rows(sK, kLK, 16 * (2 * hd + i), 32 * kx, lr, lg);
                kk4[i] = mma(frag_rows(sK, kLK, 16 * rb, 32 * kx, lr, lg), b, kk4[i]);
                qk4[i] = mma(frag_rows(sQ, kLK, 16 * rb, 32 * kx, lr, lg), b, qk4[i]);
            }
        }
        float cp[2] = {0.f, 0.f};  // column parts of dgamma, columns 16 (2 hd + i) + lr
        // The tables of this lane's rows (16 rb + 4 lg + r) and columns
        // (16 (2 hd + i) + lr) are read once, and every element is formed in
        // registers before any is stored: with the stores in between, the
        // compiler re-read the tables for each element, one LDS round trip
        // after another.
        const f32x4 grow = ld4f(S.gam + 16 * rb + 4 * lg);
        const f32x4 brow = ld4f(S.bt + 16 * rb + 4 * lg);
        const float gcol[2] = {S.gam[32 * hd + lr], S.gam[32 * hd + 16 + lr]};
        float pdv[2][4], sfv[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * lg + r, sc = 16 * (2 * hd + i) + lr;
                const bool incl = sc <= row, strict = sc < row;
                // above the diagonal the exponent may overflow: selected away
                const float d = incl ? __builtin_amdgcn_exp2f(grow[r] - gcol[i]) : 0.0f;
                const float dpv = scale * dP[i][r];
                const float dav = -dA[i][r];
                pdv[i][r] = incl ? dpv * d : 0.0f;
                sfv[i][r] = strict ? brow[r] * dav * d : 0.0f;
                if (strict)
                    pb[r] += dav * d * kk4[i][r];
                const float dDv = (incl ? dpv * qk4[i][r] : 0.0f) +
                                  (strict ? brow[r] * dav * kk4[i][r] : 0.0f);
                const float dDD = incl ? dDv * d : 0.0f;
                pg[r] += dDD;
                cp[i] -= dDD;
            }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * lg + r, sc = 16 * (2 * hd + i) + lr;
                S.u.d.PD[row * kL64 + sc] = f2bf(pdv[i][r]);
                // S is strictly lower, so S + S^T holds S's element at (row,
                // sc) and at (sc, row) and zero on the diagonal: each wave
                // writes its own tile's nonzeros to both places.
                if (sc < row) {
                    const uint16_t sv = f2bf(sfv[i][r] + 0.0f);  // a -0 is stored as +0, the sum with S^T's zero
                    S.u.d.SS[row * kL64 + sc] = sv;
                    S.u.d.SS[sc * kL64 + row] = sv;
                } else if (sc == row) {
                    S.u.d.SS[row * kL64 + sc] = 0;
                }
            }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float x = cp[i];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            if (lg == 0)
                S.colpart[rb][16 * (2 * hd + i) + lr] = x;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float xb = row16_sum(pb[r]);
            const float xg = row16_sum(pg[r]);
            if (lr == 0) {
                const int row = 16 * rb + 4 * lg + r;
                S.rowb[hd][row] = xb;
                S.rowg[hd][row] = xg;
            }
        }
        // d gamma_L: exp(gamma_L) sum(M0 * dML) from the state term and
        // sum_r l_r Delta U from the l terms.
        S.red[tid] = S.eL * msum + lsum;
        lds_barrier();
        if (w == 0) {
            float tot = 0.0f;
#pragma unroll
            for (int i = 0; i < kGT / 64; ++i)
                tot += S.red[64 * i + lane];
            const float gl = wave_sum(tot);
            float dgm = S.rowg[0][lane] + S.rowg[1][lane] + S.colpart[0][lane] +
                        S.colpart[1][lane] + S.colpart[2][lane] + S.colpart[3][lane];
            if (lane == kC - 1)
                dgm += gl;
            // dg: the reverse cumulative sum of dgamma over the 64 rows
            // (padded rows carry gamma_{L-1}), as a prefix scan of the
            // lane-reversed values.
            const float rev = __shfl(dgm, kC - 1 - lane);
            const float dgs = __shfl(wave_prefix_sum(rev), kC - 1 - lane);
            // The row's address is formed here (through an empty asm), not
            // hoisted to the kernel's start and held in registers.
            int row = lane;
            asm volatile("" : "+v"(row));
            if (row < cl.L) {
                const int64_t o = (cl.p + row) * a.Hv + j;
                a.dbeta[o] = S.rowb[0][row] + S.rowb[1][row];
                a.dg[o] = dgs;
            }
        }
        // dQ += (dP * D) K; dK += (dP * D)^T Q + (S + S^T) K (wave 0's tables
        // above are not written again before the next head's barriers).
#pragma unroll 1
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 pr = frag_rows(S.u.d.PD, kL64, 16 * rb, 32 * kk, lr, lg);
            const bf16x8 pc = frag_cols(S.u.d.PD, kL64, 32 * kk, 16 * rb, lr, lg);
            const bf16x8 sr = frag_rows(S.u.d.SS, kL64, 16 * rb, 32 * kk, lr, lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int nj = 4 * hd + i;
                if (nj >= 2 * kx_end)
                    continue;
                const bf16x8 bk = frag_cols(sK, kLK, 32 * kk, 16 * nj, lr, lg);
                const bf16x8 bq = frag_cols(sQ, kLK, 32 * kk, 16 * nj, lr, lg);
                dQ[i] = mma(pr, bk, dQ[i]);
                dK[i] = mma(pc, bq, dK[i]);
                dK[i] = mma(sr, bk, dK[i]);
            }
        }
    }
    kq_commit<KX>(S.KQ[par ^ 1][0], S.KQ[par ^ 1][1], kqn, tid);
    lds_barrier();  // the last head's readers of the state tiles are done

    // dq and dk through LDS, then 16-byte stores of whole rows.
    {
        const int lr = lane & 15, lg = lane >> 4;
        uint16_t *dqs = S.m.out[0], *dks = S.m.out[1];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * lg + r, colk = 16 * (4 * hd + i) + lr;
                dqs[row * kLK + colk] = f2bf(dQ[i][r]);
                dks[row * kLK + colk] = f2bf(dK[i][r]);
            }
    }
    lds_barrier();
    // KX stores per thread, with no branch (rows past L fall outside the
    // buffer's range and are dropped): the next item waits for everything
    // but these last KX vector-memory operations.
    {
        constexpr int pieces = 4 * KX;  // 16-byte pieces per row (dk / 8)
        const uint32_t row_bytes = (uint32_t)a.Hqk * a.dk * 2;
        const uint32_t span = (uint32_t)(cl.L - 1) * row_bytes + a.dk * 2;
        const int64_t base = (cl.p * a.Hqk + hk) * (int64_t)a.dk;
        const __amdgpu_buffer_rsrc_t rq = rsrc_uniform(static_cast<uint16_t *>(a.dq) + base, span);
        const __amdgpu_buffer_rsrc_t rk = rsrc_uniform(static_cast<uint16_t *>(a.dk_) + base, span);
#pragma unroll
        for (int e0 = 0; e0 < kC * pieces; e0 += kGT) {
            const int e = e0 + tid, row = e / pieces, pc = e % pieces;
            const uint32_t off = row * row_bytes + 16 * pc;
            __builtin_amdgcn_raw_buffer_store_b128(
                *reinterpret_cast<const u32x4 *>(S.m.out[0] + row * kLK + 8 * pc), rq, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(
                *reinterpret_cast<const u32x4 *>(S.m.out[1] + row * kLK + 8 * pc), rk, off, 0, 0);
        }
    }
    if (nitem >= total)
        break;
    item = nitem;
    cl = ncl;
    gc = ngc;
    hk = nhk;
    }
}

// ---------------------------------------------------------------------------
// bwd_grads_k256: the same per (chunk, q/k head) at dk = 256, where a chunk
// is 32 tokens (as in the forward's dk = 256 instance), so the workspace
// holds 256-key states and 32 Delta and drhs rows per chunk.  512 threads,
// one persistent workgroup per CU.  Wave w works on the chunk's rows
// [16 rb, 16 rb + 16), rb = w % 2, and the quarter qd = w / 2 of each
// result: of a 64-column value step the columns 16 qd .. 16 qd + 15, of dq and
// dk the key tiles 4 qd .. 4 qd + 3; the 32 x 32 products (column tiles
// qd < 2) fall to the waves with qd < 2.

constexpr int kC2 = 32;    // tokens per chunk at dk = 256
constexpr int kLK2 = 264;  // row stride (bf16) of 256-wide tiles
constexpr int kL32 = 40;   // row stride (bf16) of 32-wide tiles

struct alignas(16) GradSmem256 {
    float gam[kC2], e[kC2], l[kC2], bt[kC2];
    float rowb[4][kC2], rowg[4][kC2];
    float colpart[2][kC2];
    float red[kGT];
    float eL;
    alignas(16) uint16_t K[kC2 * kLK2];
    alignas(16) uint16_t Q[kC2 * kLK2];
    alignas(16) union {
        struct {
            uint16_t V[kC2 * kL64];   // v rows, the step's 64 columns
            uint16_t dO[kC2 * kL64];  // do rows (unscaled)
            uint16_t Dl[kC2 * kL64];  // Delta rows
            uint16_t dR[kC2 * kL64];  // drhs rows
        } t;
        struct {
            uint16_t PD[kC2 * kL32];  // scale dP * D (diagonal included)
            uint16_t SS[kC2 * kL32];  // S + S^T, S = diag(beta) (-dA * D) strictly lower
        } d;
    } u;
    alignas(16) union {
        struct {
            uint16_t M0[64 * kLK2];   // M0^T of the step's 64 value columns: [col][key]
            uint16_t dM[64 * kLK2];   // dML^T
        } s;
        uint16_t out[2][kC2 * kLK2];  // dq, dk rows at the end
    } m;
};
static_assert(offsetof(GradSmem256, K) % 16 == 0 && offsetof(GradSmem256, u) % 16 == 0 &&
                  offsetof(GradSmem256, m) % 16 == 0 && (kC2 * kLK2 * 2) % 16 == 0 &&
                  (kC2 * kL64 * 2) % 16 == 0 && (kC2 * kL32 * 2) % 16 == 0,
              "16-byte LDS accesses need 16-byte aligned tiles");

// One value step's tiles in flight: thread t holds pieces t + 512 u of M0^T
// and dML^T (row i / 32, 16 bytes i % 32) and 8 bytes of each of the v, do,
// Delta and drhs rows (row t / 16, columns 4 (t % 16) ..); the head's gates.
struct GradPre256 {
    u32x4 m[4], d[4];
    u32x2 v, o, dl, dr;
    float g, b;
};

__device__ __forceinline__ void grads_issue256(GradPre256 &pre, const BwdArgs &a,
                                               const ChunkLoc &cl, int64_t gc, int j,
                                               int step_col, int tid) {
    const int64_t wi = gc * a.Hv + j;
    const uint16_t *m0 = a.ws_hs + (wi * a.dv + step_col) * (int64_t)256;
    const uint16_t *dm = a.ws_dhs + (wi * a.dv + step_col) * (int64_t)256;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = tid + kGT * u;
        pre.m[u] = *reinterpret_cast<const u32x4 *>(m0 + (i >> 5) * 256 + 8 * (i & 31));
        pre.d[u] = *reinterpret_cast<const u32x4 *>(dm + (i >> 5) * 256 + 8 * (i & 31));
    }
    const int row = tid >> 4, pc = tid & 15;
    const uint32_t xrow = (uint32_t)a.Hv * a.dv * 2;
    const int64_t xofs = (cl.p * a.Hv + j) * (int64_t)a.dv + step_col;
    const uint32_t span = (uint32_t)(cl.L - 1) * xrow + 128;
    const __amdgpu_buffer_rsrc_t rv =
        rsrc_uniform(static_cast<const uint16_t *>(a.v) + xofs, span);
    const __amdgpu_buffer_rsrc_t ro =
        rsrc_uniform(static_cast<const uint16_t *>(a.dout) + xofs, span);
    pre.v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, row * xrow + 8 * pc, 0, 0));
    pre.o = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(ro, row * xrow + 8 * pc, 0, 0));
    const int64_t wofs = (wi * kC2 + row) * (int64_t)a.dv + step_col + 4 * pc;
    pre.dl = *reinterpret_cast<const u32x2 *>(a.ws_delta + wofs);
    pre.dr = *reinterpret_cast<const u32x2 *>(a.ws_drhs + wofs);
    // The gates without a branch (out-of-range rows and threads read zeros).
    const uint32_t gspan = (uint32_t)(cl.L - 1) * a.Hv * 4 + 4;
    const __amdgpu_buffer_rsrc_t rg = rsrc_uniform(a.g + cl.p * a.Hv + j, gspan);
    const __amdgpu_buffer_rsrc_t rb = rsrc_uniform(a.beta + cl.p * a.Hv + j, gspan);
    const uint32_t goff = tid < kC2 ? (uint32_t)(tid * a.Hv * 4) : 0x40000000u;
    pre.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, goff, 0, 0));
    pre.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, goff, 0, 0));
}

__device__ __forceinline__ void grads_commit256(GradSmem256 &S, const GradPre256 &pre, int tid) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = tid + kGT * u;
        *reinterpret_cast<u32x4 *>(S.m.s.M0 + (i >> 5) * kLK2 + 8 * (i & 31)) = pre.m[u];
        *reinterpret_cast<u32x4 *>(S.m.s.dM + (i >> 5) * kLK2 + 8 * (i & 31)) = pre.d[u];
    }
    const int o = (tid >> 4) * kL64 + 4 * (tid & 15);
    *reinterpret_cast<u32x2 *>(S.u.t.V + o) = pre.v;
    *reinterpret_cast<u32x2 *>(S.u.t.dO + o) = pre.o;
    *reinterpret_cast<u32x2 *>(S.u.t.Dl + o) = pre.dl;
    *reinterpret_cast<u32x2 *>(S.u.t.dR + o) = pre.dr;
}

__global__ __launch_bounds__(kGT) void bwd_grads_k256(BwdArgs a) {
    __shared__ GradSmem256 S;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rb = w & 1, qd = w >> 1;
    const int G = a.Hv / a.Hqk;
    const int nsteps = a.dv / 64;
    const int steps = G * nsteps;
    const float scale = a.scale;
    const int64_t total = a.n_chunks * a.Hqk;
    auto find = [&](int64_t from, ChunkLoc &c, int64_t &g, int &h) {
        for (int64_t i = from; i < total; i += gridDim.x) {
            g = i / a.Hqk;
            h = (int)(i % a.Hqk);
            if (locate<kC2>(a, g, c))
                return i;
        }
        return total;
    };
    ChunkLoc cl;
    int64_t gc = 0;
    int hk = 0;
    int64_t item = find(blockIdx.x, cl, gc, hk);
    if (item >= total)
        return;
    GradPre256 pre;
    // An item's K and Q rows: 32 rows of 512 bytes each, two 16-byte pieces
    // per thread; rows past L, and every piece when there is no item (a
    // buffer of no bytes), read as zeros.  The first item's are loaded here,
    // each next item's at the start of the epilogue of the item before (its
    // last readers of K and Q are done; the registers stay free through the
    // value steps and the D phase), and stored at the item's start.
    u32x4 kv[2], qv[2];
    auto kq_load = [&](const ChunkLoc &c, int h, bool any) {
        const uint32_t row_bytes = (uint32_t)a.Hqk * 256 * 2;
        const uint32_t span = any ? (uint32_t)(c.L - 1) * row_bytes + 512 : 0u;
        const int64_t base = (c.p * a.Hqk + h) * (int64_t)256;
        const __amdgpu_buffer_rsrc_t rk = rsrc_uniform(static_cast<const uint16_t *>(a.k) + base, span);
        const __amdgpu_buffer_rsrc_t rq = rsrc_uniform(static_cast<const uint16_t *>(a.q) + base, span);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = tid + kGT * u;
            const uint32_t off = (i >> 5) * row_bytes + 16 * (i & 31);
            kv[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
            qv[u] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
        }
    };
    kq_load(cl, hk, true);
    grads_issue256(pre, a, cl, gc, hk * G, 0, tid);

    while (true) {
    {
        lds_barrier();  // the previous item's readers are done
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = tid + kGT * u;
            *reinterpret_cast<u32x4 *>(S.K + (i >> 5) * kLK2 + 8 * (i & 31)) = kv[u];
            *reinterpret_cast<u32x4 *>(S.Q + (i >> 5) * kLK2 + 8 * (i & 31)) = qv[u];
        }
    }
    ChunkLoc ncl;
    int64_t ngc = 0;
    int nhk = 0;
    const int64_t nitem = find(item + gridDim.x, ncl, ngc, nhk);

    f32x4 dQ[4], dK[4];  // key tiles 4 qd + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dQ[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        dK[i] = dQ[i];
    }

    for (int gi = 0; gi < G; ++gi) {
        const int j = hk * G + gi;
        f32x4 dP = {0.f, 0.f, 0.f, 0.f}, dA = dP;  // column tile qd (qd < 2)
        float pb[4] = {0.f, 0.f, 0.f, 0.f};
        float pg[4] = {0.f, 0.f, 0.f, 0.f};
        float msum = 0.0f, lsum = 0.0f;
        for (int vs = 0; vs < nsteps; ++vs) {
            const int step = gi * nsteps + vs;
            lds_barrier();  // the previous step's (or head's) readers are done
            grads_commit256(S, pre, tid);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                msum += dot8(pre.m[u], pre.d[u]);
            if (vs == 0 && w == 0) {
                // Rows past the chunk carry g = 0, so lane 31 holds gamma_{L-1}.
                const float x = wave_prefix_sum(pre.g);
                const float gL = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), kC2 - 1));
                if (lane < kC2) {
                    S.gam[lane] = x * kLog2e;
                    S.e[lane] = __expf(x);
                    S.l[lane] = __expf(gL - x);
                    S.bt[lane] = pre.b;
                }
                if (lane == 0)
                    S.eL = __expf(gL);
            }
            lds_barrier();
            {
                const bool more = step + 1 < steps, next_item = !more && nitem < total;
                const int sn = more ? step + 1 : next_item ? 0 : step;
                const int gn = sn / nsteps, vn = sn % nsteps;
                grads_issue256(pre, a, next_item ? ncl : cl, next_item ? ngc : gc,
                               (next_item ? nhk : hk) * G + gn, 64 * vn, tid);
            }
            int lrv = lane & 15, lgv = lane >> 4;
            asm volatile("" : "+v"(lrv), "+v"(lgv));
            const int lr = lrv, lg = lgv;

            // X = K M0, Y = Q M0, U = K dML on rows 16 rb, columns 16 qd.
            const int c0 = 16 * qd;
            const f32x4 b4 = ld4f(S.bt + 16 * rb + 4 * lg), e4 = ld4f(S.e + 16 * rb + 4 * lg);
            const f32x4 l4 = ld4f(S.l + 16 * rb + 4 * lg);
            f32x4 X = {0.f, 0.f, 0.f, 0.f}, Y = X, U = X;
#pragma unroll
            for (int kx = 0; kx < 8; ++kx) {
                const bf16x8 fk = frag_rows(S.K, kLK2, 16 * rb, 32 * kx, lr, lg);
                const bf16x8 fq = frag_rows(S.Q, kLK2, 16 * rb, 32 * kx, lr, lg);
                const bf16x8 bm = frag_rows(S.m.s.M0, kLK2, c0, 32 * kx, lr, lg);
                const bf16x8 bd = frag_rows(S.m.s.dM, kLK2, c0, 32 * kx, lr, lg);
                X = mma(fk, bm, X);
                Y = mma(fq, bm, Y);
                U = mma(fk, bd, U);
            }
            {
                const f32x4 vv = tile_c(S.u.t.V, kL64, 16 * rb, c0, lr, lg);
                const f32x4 oo = tile_c(S.u.t.dO, kL64, 16 * rb, c0, lr, lg);
                const f32x4 dl = tile_c(S.u.t.Dl, kL64, 16 * rb, c0, lr, lg);
                const f32x4 dr = tile_c(S.u.t.dR, kL64, 16 * rb, c0, lr, lg);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pb[r] += dr[r] * (vv[r] - e4[r] * X[r]);
                    const float lu = l4[r] * dl[r] * U[r];
                    pg[r] += e4[r] * scale * oo[r] * Y[r] - b4[r] * e4[r] * dr[r] * X[r] - lu;
                    lsum += lu;
                }
            }
            // dQ += diag(e) dO M0^T, dK += -diag(beta e) drhs M0^T + diag(l) Delta dML^T
            // (rows 16 rb, key tiles 4 qd + i); dP += do Delta^T, dA += drhs Delta^T.
            const int rrow = 16 * rb + lr;
            const float fe = scale * S.e[rrow], fx = -S.bt[rrow] * S.e[rrow], fl = S.l[rrow];
#pragma unroll 1
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 ye = frag_rows_scaled(S.u.t.dO, kL64, 16 * rb, 32 * kk, lr, lg, fe);
                const bf16x8 xe = frag_rows_scaled(S.u.t.dR, kL64, 16 * rb, 32 * kk, lr, lg, fx);
                const bf16x8 wl = frag_rows_scaled(S.u.t.Dl, kL64, 16 * rb, 32 * kk, lr, lg, fl);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int nj = 4 * qd + i;
                    const bf16x8 bm = frag_cols(S.m.s.M0, kLK2, 32 * kk, 16 * nj, lr, lg);
                    const bf16x8 bd = frag_cols(S.m.s.dM, kLK2, 32 * kk, 16 * nj, lr, lg);
                    dQ[i] = mma(ye, bm, dQ[i]);
                    dK[i] = mma(xe, bm, dK[i]);
                    dK[i] = mma(wl, bd, dK[i]);
                }
                if (qd < 2) {
                    const bf16x8 fo = frag_rows(S.u.t.dO, kL64, 16 * rb, 32 * kk, lr, lg);
                    const bf16x8 fr = frag_rows(S.u.t.dR, kL64, 16 * rb, 32 * kk, lr, lg);
                    const bf16x8 bdl = frag_rows(S.u.t.Dl, kL64, 16 * qd, 32 * kk, lr, lg);
                    dP = mma(fo, bdl, dP);
                    dA = mma(fr, bdl, dA);
                }
            }
        }
        lds_barrier();  // every read of the step tiles is done: the D-phase tiles take their space

        int lrv = lane & 15, lgv = lane >> 4;
        asm volatile("" : "+v"(lrv), "+v"(lgv));
        const int lr = lrv, lg = lgv;
        if (qd < 2) {
            // K K^T and Q K^T on tile (rb, qd), D, S = diag(beta) (-dA * D),
            // dP * D and their dbeta and dgamma terms.
            f32x4 kk4 = {0.f, 0.f, 0.f, 0.f}, qk4 = kk4;
#pragma unroll
            for (int kx = 0; kx < 8; ++kx) {
                const bf16x8 b = frag_rows(S.K, kLK2, 16 * qd, 32 * kx, lr, lg);
                kk4 = mma(frag_rows(S.K, kLK2, 16 * rb, 32 * kx, lr, lg), b, kk4);
                qk4 = mma(frag_rows(S.Q, kLK2, 16 * rb, 32 * kx, lr, lg), b, qk4);
            }
            const f32x4 grow = ld4f(S.gam + 16 * rb + 4 * lg);
            const f32x4 brow = ld4f(S.bt + 16 * rb + 4 * lg);
            const float gcol = S.gam[16 * qd + lr];
            float cp = 0.0f;
            float pdv[4], sfv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * lg + r, sc = 16 * qd + lr;
                const bool incl = sc <= row, strict = sc < row;
                // above the diagonal the exponent may overflow: selected away
                const float d = incl ? __builtin_amdgcn_exp2f(grow[r] - gcol) : 0.0f;
                const float dpv = scale * dP[r];
                const float dav = -dA[r];
                pdv[r] = incl ? dpv * d : 0.0f;
                sfv[r] = strict ? brow[r] * dav * d : 0.0f;
                if (strict)
                    pb[r] += dav * d * kk4[r];
                const float dDv = (incl ? dpv * qk4[r] : 0.0f) +
                                  (strict ? brow[r] * dav * kk4[r] : 0.0f);
                const float dDD = incl ? dDv * d : 0.0f;
                pg[r] += dDD;
                cp -= dDD;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * lg + r, sc = 16 * qd + lr;
                S.u.d.PD[row * kL32 + sc] = f2bf(pdv[r]);
                // S + S^T from S's strictly lower elements, as at dk <= 128.
                if (sc < row) {
                    const uint16_t sv = f2bf(sfv[r] + 0.0f);  // a -0 is stored as +0, the sum with S^T's zero
                    S.u.d.SS[row * kL32 + sc] = sv;
                    S.u.d.SS[sc * kL32 + row] = sv;
                } else if (sc == row) {
                    S.u.d.SS[row * kL32 + sc] = 0;
                }
            }
            cp += __shfl_xor(cp, 16);
            cp += __shfl_xor(cp, 32);
            if (lg == 0)
                S.colpart[rb][16 * qd + lr] = cp;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float xb = row16_sum(pb[r]);
            const float xg = row16_sum(pg[r]);
            if (lr == 0) {
                const int row = 16 * rb + 4 * lg + r;
                S.rowb[qd][row] = xb;
                S.rowg[qd][row] = xg;
            }
        }
        S.red[tid] = S.eL * msum + lsum;
        lds_barrier();
        if (w == 0) {
            float tot = 0.0f;
#pragma unroll
            for (int i = 0; i < kGT / 64; ++i)
                tot += S.red[64 * i + lane];
            const float gl = wave_sum(tot);
            const int rl = lane & (kC2 - 1);
            float dgm = S.rowg[0][rl] + S.rowg[1][rl] + S.rowg[2][rl] + S.rowg[3][rl] +
                        S.colpart[0][rl] + S.colpart[1][rl];
            if (lane == kC2 - 1)
                dgm += gl;
            if (lane >= kC2)
                dgm = 0.0f;
            // dg: the reverse cumulative sum over the 32 rows, as a prefix
            // scan of the row-reversed values.
            const float rev = __shfl(dgm, (kC2 - 1 - lane) & 63);
            const float ps = wave_prefix_sum(lane < kC2 ? rev : 0.0f);
            const float dgs = __shfl(ps, (kC2 - 1 - lane) & 63);
            int row = lane;
            asm volatile("" : "+v"(row));
            if (row < cl.L) {
                const int64_t o = (cl.p + row) * a.Hv + j;
                a.dbeta[o] = S.rowb[0][row] + S.rowb[1][row] + S.rowb[2][row] + S.rowb[3][row];
                a.dg[o] = dgs;
            }
        }
        // dQ += (dP * D) K; dK += (dP * D)^T Q + (S + S^T) K, over the 32 tokens
        // (wave 0's tables above are not written again before the next
        // head's barriers).
        {
            const bf16x8 pr = frag_rows(S.u.d.PD, kL32, 16 * rb, 0, lr, lg);
            const bf16x8 pc = frag_cols(S.u.d.PD, kL32, 0, 16 * rb, lr, lg);
            const bf16x8 sr = frag_rows(S.u.d.SS, kL32, 16 * rb, 0, lr, lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int nj = 4 * qd + i;
                const bf16x8 bk = frag_cols(S.K, kLK2, 0, 16 * nj, lr, lg);
                const bf16x8 bq = frag_cols(S.Q, kLK2, 0, 16 * nj, lr, lg);
                dQ[i] = mma(pr, bk, dQ[i]);
                dK[i] = mma(pc, bq, dK[i]);
                dK[i] = mma(sr, bk, dK[i]);
            }
        }
    }
    lds_barrier();  // the last head's readers of the state tiles are done
    kq_load(nitem < total ? ncl : cl, nitem < total ? nhk : hk, nitem < total);

    // dq and dk through LDS, then 16-byte stores of whole rows.
    {
        const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * lg + r, colk = 16 * (4 * qd + i) + lr;
                S.m.out[0][row * kLK2 + colk] = f2bf(dQ[i][r]);
                S.m.out[1][row * kLK2 + colk] = f2bf(dK[i][r]);
            }
    }
    lds_barrier();
    for (int e = tid; e < kC2 * 32; e += kGT) {
        const int row = e >> 5, pc = e & 31;
        if (row < cl.L) {
            const int64_t o = ((cl.p + row) * a.Hqk + hk) * (int64_t)256 + 8 * pc;
            *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.dq) + o) =
                *reinterpret_cast<const u32x4 *>(S.m.out[0] + row * kLK2 + 8 * pc);
            *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.dk_) + o) =
                *reinterpret_cast<const u32x4 *>(S.m.out[1] + row * kLK2 + 8 * pc);
        }
    }
    if (nitem >= total)
        break;
    item = nitem;
    cl = ncl;
    gc = ngc;
    hk = nhk;
    }
}

// State rows and chunk rows of the workspace: 128-key states and 64-token
// chunks at dk = 64 and 128 (zeros past dk), 256-key states and 32-token
// chunks at dk = 256.
int ws_state_width(int32_t dk) { return dk == 256 ? 256 : kDK; }
int ws_chunk_rows(int32_t dk) { return dk == 256 ? kC2 : kC; }

}  // namespace

size_t bwd_workspace_bytes(int64_t n_chunks, int32_t Hv, int32_t dk, int32_t dv) {
    const size_t ch = (size_t)n_chunks * (size_t)Hv;
    // M0^T and dML^T ([dv][width] bf16), Delta and drhs rows ([rows][dv] bf16).
    return ch * (size_t)dv * (2 * ws_state_width(dk) + 2 * ws_chunk_rows(dk)) * sizeof(uint16_t);
}

void bwd_carve(BwdArgs &a, void *workspace) {
    const size_t ch = (size_t)a.n_chunks * (size_t)a.Hv;
    const size_t sw = (size_t)ws_state_width(a.dk), cr = (size_t)ws_chunk_rows(a.dk);
    uint16_t *p = static_cast<uint16_t *>(workspace);
    a.ws_hs = p;
    p += ch * sw * a.dv;
    a.ws_dhs = p;
    p += ch * sw * a.dv;
    a.ws_delta = p;
    p += ch * cr * a.dv;
    a.ws_drhs = p;
}

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t stream) {
    if (a.n_chunks <= 0)
        return hipSuccess;
    if (a.n_chunks > 0x7fffffff)
        return hipErrorInvalidValue;
    // The two state passes on the forward kernel's pipeline.
    FwdArgs f{};
    f.q = a.q;
    f.k = a.k;
    f.v = a.v;
    f.g = a.g;
    f.beta = a.beta;
    f.h0 = a.h0;
    f.cu = a.cu;
    f.T = a.T;
    f.Hqk = a.Hqk;
    f.Hv = a.Hv;
    f.dk = a.dk;
    f.dv = a.dv;
    f.n_seqs = a.n_seqs;
    f.scale = a.scale;
    f.pieces = 1;
    f.piece_len = a.T;
    f.chunk_states = a.ws_hs;
    f.chunk_deltas = a.ws_delta;
    FwdArgs r = f;
    r.v = a.dout;
    r.h0 = nullptr;
    r.chunk_states = nullptr;
    r.chunk_deltas = nullptr;
    r.chunk_dstates = a.ws_dhs;
    r.chunk_drhs = a.ws_drhs;
    r.dv_out = a.dv_;
    r.dht = a.dht;
    r.dh0 = a.dh0;
    hipError_t e = launch_bwd_state_passes(f, r, stream);
    if (e != hipSuccess)
        return e;
    // One persistent workgroup per CU (one fits: its LDS is 146 KB, 124 KB
    // at dk = 256).
    const int64_t items = a.n_chunks * a.Hqk;
    const unsigned grid = (unsigned)(items < kGradGrid ? items : kGradGrid);
    if (a.dk == 256)
        hipLaunchKernelGGL(bwd_grads_k256, dim3(grid), dim3(kGT), 0, stream, a);
    else if (a.dk > 64)
        hipLaunchKernelGGL(bwd_grads<4>, dim3(grid), dim3(kGT), 0, stream, a);
    else
        hipLaunchKernelGGL(bwd_grads<2>, dim3(grid), dim3(kGT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gdn

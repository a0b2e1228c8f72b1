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
//             dbeta, and dgamma from e, l, exp(gamma_L) and D, then
//             dg = the reverse cumulative sum of dgamma over the chunk.
//
// Four kernels:
//   bwd_prep     per (chunk, value head), all in parallel: gamma, K K^T and
//                Q K^T (MFMA), A, T = (I + A)^-1 (the four 16 x 16 diagonal
//                inverses by fp32 forward substitution with row broadcasts,
//                the blocks below them by block recursion in fp32), and P.
//                Writes T (fp32), P (bf16) and gamma to the workspace.
//   the forward kernel (gdn_fwd_bf16.hip, launch_fwd_chunk_states) without
//                its output: the state recurrence by block substitution,
//                writing each chunk's entering state M0 to the workspace
//                (bf16, transposed to [dv][dk]).
//   bwd_dstate   per (sequence, value head, 64 value columns), chunks in
//                reverse: the state-gradient recurrence with the dense T,
//                writing each chunk's dML to the workspace (bf16, [dv][dk]);
//                dh0 is the gradient after chunk 0.  Loader waves fill the
//                next chunk's buffer while four waves run the recurrence.
//   bwd_chunk    per (chunk, q/k head), all in parallel: the token gradients
//                of the chunk from M0 and dML, summed over the value heads
//                that share the q/k head (dq, dk) and over value columns.
//
// Precision: products accumulate in fp32 on bf16 MFMA.  The state-gradient
// recurrence carries an fp32 state and uses hi + lo bf16 pairs for computed
// operands (T, dDelta, dX, e dO), as the forward does for its own; the state
// itself enters products as its hi part, as in the forward.  In bwd_chunk the
// states, Delta and the other computed operands enter as single bf16
// roundings except T, rhs and dDelta (hi + lo).
//
// MFMA v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][8(l/16)+j] and
// B[8(l/16)+j][l%16] (j = 0..7), receives C[4(l/16)+r][l%16] (r = 0..3).
// ds_read_b64_tr_b16: within 16 lanes, lane 16g+i receives element i%4 of the
// 8-byte words addressed by lanes 16g + 4j + i/4, j = 0..3.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

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
constexpr int kVT = 64;    // value columns per state workgroup
constexpr int kLK = 136;   // row stride (bf16) of K and Q tiles
constexpr int kL64 = 72;   // row stride (bf16) of 64-wide tiles
constexpr int kL32 = 40;   // row stride (bf16) of 32-wide tiles
constexpr int kLF = 65;    // row stride (fp32) of 64-wide fp32 tiles
constexpr unsigned kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit elements

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

// Sum over the 16 lanes of this lane's row.
__device__ __forceinline__ float row16_sum(float x) {
    x += __shfl_xor(x, 1, 16);
    x += __shfl_xor(x, 2, 16);
    x += __shfl_xor(x, 4, 16);
    x += __shfl_xor(x, 8, 16);
    return x;
}

// One step of the forward substitution of a diagonal block (see bwd_prep):
// x_r2 -= A[r2][R] x_R for r2 > R, the factors read from the block's fp32
// copy at addresses every lane of the 16-lane row shares (broadcast reads).
template <int R>
__device__ __forceinline__ void dinv_step(float (&x)[16], const float *blk, int ld) {
#pragma unroll
    for (int r2 = R + 1; r2 < 16; ++r2)
        x[r2] = __builtin_fmaf(-blk[r2 * ld + R], x[R], x[r2]);
}

template <int... R>
__device__ __forceinline__ void dinv_steps(float (&x)[16], const float *blk, int ld,
                                           std::integer_sequence<int, R...>) {
    (dinv_step<R>(x, blk, ld), ...);
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

// First chunk index of sequence n.
__device__ __forceinline__ int64_t chunk_base(const BwdArgs &a, int n) {
    if (!a.cu)
        return (int64_t)n * ((a.T + kC - 1) / kC);
    int64_t b = 0;
    for (int m = 0; m < n; ++m)
        b += (seq_len(a, m) + kC - 1) / kC;
    return b;
}

__device__ __forceinline__ bool locate(const BwdArgs &a, int64_t gc, ChunkLoc &cl) {
    if (!a.cu) {
        const int64_t nch = (a.T + kC - 1) / kC;
        const int64_t n = gc / nch;
        if (n >= a.n_seqs)
            return false;
        cl.n = (int)n;
        cl.c = (int)(gc % nch);
    } else {
        int64_t b = 0;
        int n = 0;
        for (; n < a.n_seqs; ++n) {
            const int64_t nc = (seq_len(a, n) + kC - 1) / kC;
            if (gc < b + nc)
                break;
            b += nc;
        }
        if (n >= a.n_seqs)
            return false;
        cl.n = n;
        cl.c = (int)(gc - b);
    }
    cl.p = seq_start(a, cl.n) + (int64_t)kC * cl.c;
    cl.L = (int)min<int64_t>(kC, seq_len(a, cl.n) - (int64_t)kC * cl.c);
    return true;
}

// Rows [p, p + L) of a [*, H, width] bf16 tensor at head h into an LDS tile
// [64][ld]; rows past L read as zeros.  256 threads, 16-byte pieces.
template <int Width>
__device__ __forceinline__ void stage_rows_bf16(uint16_t *dst, int ld, const void *src, int64_t p,
                                                int L, int H, int h, int col0, int rowlen,
                                                int tid) {
    const uint32_t row_bytes = (uint32_t)H * rowlen * 2;
    const uint16_t *base = static_cast<const uint16_t *>(src) + (p * H + h) * (int64_t)rowlen + col0;
    const __amdgpu_buffer_rsrc_t r = rsrc(base, (uint32_t)(L - 1) * row_bytes + Width * 2);
    constexpr int kPieces = Width / 8;  // 16-byte pieces per row
#pragma unroll
    for (int i = tid; i < kC * kPieces; i += 256) {
        const int row = i / kPieces, pc = i % kPieces;
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, row * row_bytes + 16 * pc, 0, 0);
        *reinterpret_cast<u32x4 *>(dst + row * ld + 8 * pc) = v;
    }
}

// Rows of q or k (dk = 64 or 128 elements) into a 128-wide LDS tile; with
// dk = 64 the upper half of every row is zero, so contractions over the key
// dimension run at 128 unchanged.  256 threads.
__device__ __forceinline__ void stage_qk_rows(uint16_t *dst, int ld, const void *src, int64_t p,
                                              int L, int H, int h, int dk, int tid) {
    if (dk == kDK) {
        stage_rows_bf16<kDK>(dst, ld, src, p, L, H, h, 0, kDK, tid);
        return;
    }
    stage_rows_bf16<kDK / 2>(dst, ld, src, p, L, H, h, 0, kDK / 2, tid);
    for (int i = tid; i < kC * 8; i += 256)
        *reinterpret_cast<u32x4 *>(dst + (i >> 3) * ld + kDK / 2 + 8 * (i & 7)) = u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// bwd_prep: per (chunk, value head).

__global__ __launch_bounds__(256) void bwd_prep(BwdArgs a) {
    // K and Q are dead once K K^T and Q K^T are in registers: A (fp32) then
    // takes K's space and T Q's, which keeps LDS under a third of a CU's.
    static_assert(kC * kLF * sizeof(float) <= kC * kLK * sizeof(uint16_t), "A, T fit K, Q");
    __shared__ __attribute__((aligned(16))) uint16_t KsAf[kC * kLK];
    __shared__ __attribute__((aligned(16))) uint16_t QsTf[kC * kLK];
    uint16_t *Ks = KsAf, *Qs = QsTf;
    float *Af = reinterpret_cast<float *>(KsAf), *Tf = reinterpret_cast<float *>(QsTf);
    __shared__ float Wf[32 * 33];
    __shared__ __attribute__((aligned(16))) uint16_t Ps[kC * kC];   // unpadded: keeps LDS under half a CU's
    __shared__ float gam[kC], bt[kC];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const int64_t gc = blockIdx.x;
    const int j = blockIdx.y;
    ChunkLoc cl;
    if (!locate(a, gc, cl))
        return;
    const int hk = j / (a.Hv / a.Hqk);
    stage_qk_rows(Ks, kLK, a.k, cl.p, cl.L, a.Hqk, hk, a.dk, tid);
    stage_qk_rows(Qs, kLK, a.q, cl.p, cl.L, a.Hqk, hk, a.dk, tid);
    if (w == 0) {
        const float gv = lane < cl.L ? a.g[(cl.p + lane) * a.Hv + j] : 0.0f;
        const float bv = lane < cl.L ? a.beta[(cl.p + lane) * a.Hv + j] : 0.0f;
        gam[lane] = wave_prefix_sum(gv);  // padded rows keep gamma_{L-1}
        bt[lane] = bv;
    }
    __syncthreads();

    // K K^T and Q K^T, rows 16w .. 16w + 15.
    f32x4 kk[4], qk[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        kk[ni] = f32x4{0.f, 0.f, 0.f, 0.f};
        qk[ni] = kk[ni];
#pragma unroll
        for (int kx = 0; kx < 4; ++kx) {
            const bf16x8 b = frag_rows(Ks, kLK, 16 * ni, 32 * kx, lr, lg);
            kk[ni] = mma(frag_rows(Ks, kLK, 16 * w, 32 * kx, lr, lg), b, kk[ni]);
            qk[ni] = mma(frag_rows(Qs, kLK, 16 * w, 32 * kx, lr, lg), b, qk[ni]);
        }
    }
    __syncthreads();  // every read of K and Q is done: A and T take their space
    for (int i = tid; i < kC * kLF; i += 256)
        Tf[i] = 0.0f;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = 16 * w + 4 * lg + rr, s = 16 * ni + lr;
            const float d = s <= r ? __expf(gam[r] - gam[s]) : 0.0f;
            Af[r * kLF + s] = s < r ? bt[r] * d * kk[ni][rr] : 0.0f;
            Ps[r * kC + s] = f2bf(s <= r ? d * qk[ni][rr] : 0.0f);
        }
    __syncthreads();

    // Diagonal blocks of T: D_i = (I + A_ii)^-1, lane row g = block g, lane c
    // = column c; once x_r is final, A[r2][r] x_r leaves every later row.
    if (w == 0) {
        const int c = lr, gb = lg;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            x[r] = r == c ? 1.0f : 0.0f;
        dinv_steps(x, Af + 16 * gb * kLF + 16 * gb, kLF, std::make_integer_sequence<int, 15>{});
#pragma unroll
        for (int r = 0; r < 16; ++r)
            Tf[(16 * gb + r) * kLF + 16 * gb + c] = x[r];
    }
    __syncthreads();
    // T_10 = -D_1 A_10 D_0 and T_32 = -D_3 A_32 D_2.
    for (int i = tid; i < 512; i += 256) {
        const int b = i >> 8, r = (i >> 4) & 15, s = i & 15;
        const float *Ar = Af + (16 + 32 * b + r) * kLF + 32 * b;
        const float *Dc = Tf + (32 * b) * kLF + 32 * b + s;
        float acc = 0.0f;
        for (int k = 0; k < 16; ++k)
            acc += Ar[k] * Dc[k * kLF];
        Wf[(16 * b + r) * 33 + s] = acc;
    }
    __syncthreads();
    for (int i = tid; i < 512; i += 256) {
        const int b = i >> 8, r = (i >> 4) & 15, s = i & 15;
        const float *Dr = Tf + (16 + 32 * b + r) * kLF + 16 + 32 * b;
        float acc = 0.0f;
        for (int k = 0; k < 16; ++k)
            acc += Dr[k] * Wf[(16 * b + k) * 33 + s];
        Tf[(16 + 32 * b + r) * kLF + 32 * b + s] = -acc;
    }
    __syncthreads();
    // T[32:64][0:32] = -T2 A[32:64][0:32] T1.
    for (int i = tid; i < 1024; i += 256) {
        const int r = i >> 5, s = i & 31;
        const float *Ar = Af + (32 + r) * kLF;
        float acc = 0.0f;
        for (int k = 0; k < 32; ++k)
            acc += Ar[k] * Tf[k * kLF + s];
        Wf[r * 33 + s] = acc;
    }
    __syncthreads();
    for (int i = tid; i < 1024; i += 256) {
        const int r = i >> 5, s = i & 31;
        const float *Tr = Tf + (32 + r) * kLF + 32;
        float acc = 0.0f;
        for (int k = 0; k < 32; ++k)
            acc += Tr[k] * Wf[k * 33 + s];
        Tf[(32 + r) * kLF + s] = -acc;
    }
    __syncthreads();

    const int64_t wi = gc * a.Hv + j;
    float *To = a.ws_T + wi * (kC * kC);
    uint16_t *Po = a.ws_P + wi * (kC * kC);
    // 16-byte stores: four fp32 of T (gathered from the padded rows), eight
    // bf16 of P.
    for (int i = tid; i < kC * kC / 4; i += 256) {
        const float *tr = Tf + (i >> 4) * kLF + 4 * (i & 15);
        *reinterpret_cast<f32x4 *>(To + 4 * i) = f32x4{tr[0], tr[1], tr[2], tr[3]};
    }
    for (int i = tid; i < kC * kC / 8; i += 256)
        *reinterpret_cast<u32x4 *>(Po + 8 * i) = *reinterpret_cast<const u32x4 *>(Ps + 8 * i);
    if (tid < kC)
        a.ws_gam[wi * kC + tid] = gam[tid];
}

// ---------------------------------------------------------------------------
// The two state recurrences: one workgroup per (sequence, value head, 64
// value columns), wave w owning columns [16w, 16w + 16).  A state slice
// [128 x 16] lives in eight C-layout tiles: tile mt holds rows 16mt ...
// 16mt + 15, lane (lr, lg) rows 16mt + 4lg + r of column lr.

struct alignas(16) StateSmem {
    uint16_t K[kC * kLK];
    uint16_t Q[kC * kLK];
    uint16_t X[kC * kL64];      // dO tile
    uint16_t Th[kC * kL64];
    uint16_t Tl[kC * kL64];
    uint16_t P[kC * kL64];
    float e[kC], l[kC], bt[kC];
    float eL;
};

// One chunk's operands in flight in registers: each of the 256 threads holds
// its share of K and Q, the value-column tile of dO, T, P and the
// gate tables, loaded while the previous chunk is computed.
struct StatePre {
    u32x4 k[4], q[4], x[2], p[2];
    f32x4 t[4];
    float gm, gL, bt;
};

__device__ __forceinline__ void state_issue(StatePre &pre, const BwdArgs &a, const ChunkLoc &cl,
                                            int hk, int j, int tile, int64_t wi, int tid) {
    // K and Q rows hold a.dk elements (64 or 128); the 16-byte slots past
    // a.dk stage zeros.
    const uint32_t krow = (uint32_t)a.Hqk * a.dk * 2;
    const int64_t kofs = (cl.p * a.Hqk + hk) * (int64_t)a.dk;
    const __amdgpu_buffer_rsrc_t rk =
        rsrc(static_cast<const uint16_t *>(a.k) + kofs, (uint32_t)(cl.L - 1) * krow + a.dk * 2);
    const __amdgpu_buffer_rsrc_t rq =
        rsrc(static_cast<const uint16_t *>(a.q) + kofs, (uint32_t)(cl.L - 1) * krow + a.dk * 2);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = tid + 256 * u;
        const uint32_t off = (uint32_t)(i >> 4) * krow + 16 * (i & 15);
        const bool in_row = 8 * (i & 15) < a.dk;
        pre.k[u] = in_row ? __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0) : u32x4{0u, 0u, 0u, 0u};
        pre.q[u] = in_row ? __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0) : u32x4{0u, 0u, 0u, 0u};
    }
    const uint32_t xrow = (uint32_t)a.Hv * a.dv * 2;
    const void *xs = a.dout;
    const __amdgpu_buffer_rsrc_t rx =
        rsrc(static_cast<const uint16_t *>(xs) + (cl.p * a.Hv + j) * (int64_t)a.dv + tile * kVT,
             (uint32_t)(cl.L - 1) * xrow + kVT * 2);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + 256 * u;
        pre.x[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(i >> 3) * xrow + 16 * (i & 7),
                                                         0, 0);
    }
    const float *Tg = a.ws_T + wi * (kC * kC);
#pragma unroll
    for (int u = 0; u < 4; ++u)
        pre.t[u] = *reinterpret_cast<const f32x4 *>(Tg + 4 * (tid + 256 * u));
    const uint16_t *Pg = a.ws_P + wi * (kC * kC);
#pragma unroll
    for (int u = 0; u < 2; ++u)
        pre.p[u] = *reinterpret_cast<const u32x4 *>(Pg + 8 * (tid + 256 * u));
    if (tid < kC) {
        pre.gm = a.ws_gam[wi * kC + tid];
        pre.gL = a.ws_gam[wi * kC + kC - 1];
        pre.bt = tid < cl.L ? a.beta[(cl.p + tid) * a.Hv + j] : 0.0f;
    }
}

__device__ __forceinline__ void state_commit(StateSmem &S, const StatePre &pre, int tid) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = tid + 256 * u;
        *reinterpret_cast<u32x4 *>(S.K + (i >> 4) * kLK + 8 * (i & 15)) = pre.k[u];
        *reinterpret_cast<u32x4 *>(S.Q + (i >> 4) * kLK + 8 * (i & 15)) = pre.q[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + 256 * u;
        *reinterpret_cast<u32x4 *>(S.X + (i >> 3) * kL64 + 8 * (i & 7)) = pre.x[u];
        *reinterpret_cast<u32x4 *>(S.P + (i >> 3) * kL64 + 8 * (i & 7)) = pre.p[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = tid + 256 * u;
        u32x2 h, l;
        split4(pre.t[u], h, l);
        *reinterpret_cast<u32x2 *>(S.Th + (i >> 4) * kL64 + 4 * (i & 15)) = h;
        *reinterpret_cast<u32x2 *>(S.Tl + (i >> 4) * kL64 + 4 * (i & 15)) = l;
    }
    if (tid < kC) {
        S.e[tid] = __expf(pre.gm);
        S.l[tid] = __expf(pre.gL - pre.gm);
        S.bt[tid] = pre.bt;
        if (tid == 0)
            S.eL = __expf(pre.gL);
    }
}

// A state slice (lane column col, rows 16mt + 4lg + r) as bf16 into the
// transposed workspace copy [dv][dk]: one 8-byte store per tile.
__device__ __forceinline__ void store_state_t(uint16_t *dst, const f32x4 (&h)[8], int col, int lg) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
        *reinterpret_cast<u32x2 *>(dst + (int64_t)col * kDK + 16 * mt + 4 * lg) = pack4(h[mt]);
}

// The state's hi part as the B operands of a contraction over dk (permuted k).
__device__ __forceinline__ void state_hi(const f32x4 (&h)[8], bf16x8 (&hb)[4]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        hb[kk] = cat(pack4(h[2 * kk]), pack4(h[2 * kk + 1]));
}

// Y = K S (S given by its hi part), rows 16mi .. of the chunk.
__device__ __forceinline__ void k_times_state(const uint16_t *Ks, const bf16x8 (&hb)[4],
                                              f32x4 (&Y)[4], int lr, int lg) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        Y[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            Y[mi] = mma(frag_rows_perm(Ks, kLK, 16 * mi, 32 * kk, lr, lg), hb[kk], Y[mi]);
    }
}

// h += X^T Z over the chunk's tokens, X = K or Q (row-major tile), Z given
// as hi and lo B operands (permuted token order).
__device__ __forceinline__ void add_xt_times(const uint16_t *Xs, const bf16x8 (&zh)[2],
                                             const bf16x8 (&zl)[2], f32x4 (&h)[8], int lr,
                                             int lg) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 f = frag_cols_perm(Xs, kLK, 32 * kk, 16 * mt, lr, lg);
            h[mt] = mma(f, zh[kk], h[mt]);
            h[mt] = mma(f, zl[kk], h[mt]);
        }
}

// Z (four C-layout tiles over the chunk's rows) as hi and lo B operands.
__device__ __forceinline__ void tiles_split(const f32x4 (&Z)[4], bf16x8 (&zh)[2], bf16x8 (&zl)[2]) {
    u32x2 h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        split4(Z[i], h[i], l[i]);
    zh[0] = cat(h[0], h[1]);
    zh[1] = cat(h[2], h[3]);
    zl[0] = cat(l[0], l[1]);
    zl[1] = cat(l[2], l[3]);
}

// Y = T Z (Trans = false) or T^T Z (Trans = true), T lower triangular given
// as hi and lo tiles, Z as hi and lo B operands; products hi*hi + hi*lo + lo*hi.
template <bool Trans>
__device__ __forceinline__ void t_times(const uint16_t *Th, const uint16_t *Tl,
                                        const bf16x8 (&zh)[2], const bf16x8 (&zl)[2],
                                        f32x4 (&Y)[4], int lr, int lg) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        Y[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // T: rows 16mi.. need columns <= their rows; T^T the reverse.
            if (!Trans && 32 * kk > 16 * mi + 15)
                continue;
            if (Trans && 32 * kk + 31 < 16 * mi)
                continue;
            const bf16x8 fh = Trans ? frag_cols_perm(Th, kL64, 32 * kk, 16 * mi, lr, lg)
                                    : frag_rows_perm(Th, kL64, 16 * mi, 32 * kk, lr, lg);
            const bf16x8 fl = Trans ? frag_cols_perm(Tl, kL64, 32 * kk, 16 * mi, lr, lg)
                                    : frag_rows_perm(Tl, kL64, 16 * mi, 32 * kk, lr, lg);
            Y[mi] = mma(fh, zh[kk], Y[mi]);
            Y[mi] = mma(fh, zl[kk], Y[mi]);
            Y[mi] = mma(fl, zh[kk], Y[mi]);
        }
    }
}

// The state-gradient recurrence, chunks in reverse, writing the gradient of
// each chunk's leaving state (dh0 at the end); the states entering the chunks
// come from the forward kernel (launch_fwd_chunk_states).  512 threads:
// waves 0..3 run the recurrence on the chunk in one
// LDS buffer while waves 4..7 fill the other with the next chunk's operands,
// whose global loads were issued a chunk earlier; one barrier per chunk.  The
// two roles run separate loops with the same number of barriers, so the
// loaders' registers and the state's never share the budget.
__device__ __forceinline__ void dstate_pass(const BwdArgs &a) {
    __shared__ StateSmem Sb[2];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const int n_tiles = a.dv / kVT;
    const int tile = blockIdx.x % n_tiles;
    const int j = (blockIdx.x / n_tiles) % a.Hv;
    const int n = blockIdx.x / (n_tiles * a.Hv);
    const int hk = j / (a.Hv / a.Hqk);
    const int64_t len = seq_len(a, n);
    const int nch = (int)((len + kC - 1) / kC);
    const int64_t base = chunk_base(a, n);
    const int64_t S_elems = (int64_t)kDK * a.dv;      // workspace states: 128 keys
    const int64_t H_elems = (int64_t)a.dk * a.dv;     // dht, dh0: a.dk keys
    const float scale = a.scale;
    auto loc = [&](int it) {
        const int c = nch - 1 - it;
        ChunkLoc cl;
        cl.n = n;
        cl.c = c;
        cl.p = seq_start(a, n) + (int64_t)kC * c;
        cl.L = (int)min<int64_t>(kC, len - (int64_t)kC * c);
        return cl;
    };
    auto wslot = [&](int it) { return (base + nch - 1 - it) * a.Hv + j; };

    if (w >= 4) {
        const int t = tid - 256;
        StatePre pre;
        if (nch > 0) {
            state_issue(pre, a, loc(0), hk, j, tile, wslot(0), t);
            state_commit(Sb[0], pre, t);
            if (nch > 1)
                state_issue(pre, a, loc(1), hk, j, tile, wslot(1), t);
        }
        __syncthreads();
        for (int it = 0; it < nch; ++it) {
            if (it + 1 < nch) {
                state_commit(Sb[(it + 1) & 1], pre, t);
                if (it + 2 < nch)
                    state_issue(pre, a, loc(it + 2), hk, j, tile, wslot(it + 2), t);
            }
            __syncthreads();
        }
        return;
    }

    const int col = tile * kVT + 16 * w + lr;   // this lane's value column
    const float *init = a.dht;
    f32x4 h[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            h[mt][r] = init && 16 * mt + 4 * lg + r < a.dk
                           ? init[((int64_t)n * a.Hv + j) * H_elems +
                                  (int64_t)(16 * mt + 4 * lg + r) * a.dv + col]
                           : 0.0f;
    __syncthreads();
    for (int it = 0; it < nch; ++it) {
        const StateSmem &S = Sb[it & 1];
        // The gradient of the state leaving the chunk.
        store_state_t(a.ws_dhs + wslot(it) * S_elems, h, col, lg);

        bf16x8 hb[4];
        state_hi(h, hb);
        f32x4 Y[4];
        k_times_state(S.K, hb, Y, lr, lg);
        const float eL = S.eL;
        {
            // dDelta = diag(l) K dML + P^T dO; drhs = T^T dDelta;
            // dM <- exp(gamma_L) dM - K^T diag(beta e) drhs + Q^T diag(e) dO.
            f32x4 dD[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                f32x4 v1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (32 * kk + 31 < 16 * mi)
                        continue;
                    v1 = mma(frag_cols(S.P, kL64, 32 * kk, 16 * mi, lr, lg),
                             frag_cols(S.X, kL64, 32 * kk, 16 * w, lr, lg), v1);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dD[mi][r] = S.l[16 * mi + 4 * lg + r] * Y[mi][r] + scale * v1[r];
            }
            bf16x8 zh[2], zl[2];
            tiles_split(dD, zh, zl);
            f32x4 dR[4];
            t_times<true>(S.Th, S.Tl, zh, zl, dR, lr, lg);
            f32x4 dX[4], eO[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * mi + 4 * lg + r;
                    dX[mi][r] = -S.bt[row] * S.e[row] * dR[mi][r];
                    eO[mi][r] = scale * S.e[row] * bf2f(S.X[row * kL64 + 16 * w + lr]);
                }
            bf16x8 xh[2], xl[2], oh[2], ol[2];
            tiles_split(dX, xh, xl);
            tiles_split(eO, oh, ol);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                h[mt] *= eL;
            add_xt_times(S.K, xh, xl, h, lr, lg);
            add_xt_times(S.Q, oh, ol, h, lr, lg);
        }
        __syncthreads();
    }
    if (a.dh0) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * mt + 4 * lg + r < a.dk)
                    a.dh0[((int64_t)n * a.Hv + j) * H_elems +
                          (int64_t)(16 * mt + 4 * lg + r) * a.dv + col] = h[mt][r];
    }
}

__global__ __launch_bounds__(512) void bwd_dstate(BwdArgs a) {
    dstate_pass(a);
}

// ---------------------------------------------------------------------------
// bwd_chunk: per (chunk, q/k head), 512 threads.  Wave w owns the chunk's
// rows [16 rb, 16 rb + 16), rb = w % 4, and the column half h = w / 4 of every
// [64 x *] result: in a 32-column tile the 16 columns 16h.., of dq and dk the
// dk tiles 4h .. 4h + 3, of the 64 x 64 products the column tiles 2h, 2h + 1.
// Two waves per SIMD hide each other's latency.

constexpr int kCT = 512;   // bwd_chunk threads

struct alignas(16) ChunkSmem {
    uint16_t K[kC * kLK];
    uint16_t Q[kC * kLK];
    uint16_t Th[kC * kL64];     // after the column tiles: dQK
    uint16_t Tl[kC * kL64];     // after the column tiles: S + S^T
    uint16_t P[kC * kL64];
    union {
        struct {
            uint16_t M0[32 * kLK];     // M0^T: [col][dk]
            uint16_t dM[32 * kLK];     // dML^T
            uint16_t V[kC * kL32];
            uint16_t dO[kC * kL32];    // do (unscaled)
            uint16_t rh[kC * kL32];
            uint16_t rl[kC * kL32];
            uint16_t Dh[kC * kL32];    // Delta
            uint16_t zh[kC * kL32];    // dDelta hi
            uint16_t zl[kC * kL32];    // dDelta lo
            uint16_t dR[kC * kL32];    // drhs
            uint16_t dY[kC * kL32];    // diag(e) dO
            uint16_t dX[kC * kL32];    // -diag(beta e) drhs
            uint16_t W[kC * kL32];     // diag(l) Delta
        } t;
        float S[kC * kLF];             // S = diag(beta) (dA * D), fp32
    } u;
    float gam[kC], e[kC], l[kC], bt[kC];
    float colpart[4][kC];
    float rowb[2][kC], rowg[2][kC];
    float red[kCT];
};

// One 32-column tile of M0^T, dML^T, V and do in flight in registers: thread
// t holds piece t of M0^T and of dML^T (row t / 16, 16 bytes t % 16), and
// threads below 256 a piece of V, the others one of do.
struct TilePre {
    u32x4 m, d, x;
};

__device__ __forceinline__ void tile_issue(TilePre &pre, const BwdArgs &a, const ChunkLoc &cl,
                                           int j, int64_t wi, int t0, int tid) {
    const int64_t sofs = wi * (int64_t)kDK * a.dv + (int64_t)t0 * kDK;
    pre.m = *reinterpret_cast<const u32x4 *>(a.ws_hs + sofs + 8 * tid);
    pre.d = *reinterpret_cast<const u32x4 *>(a.ws_dhs + sofs + 8 * tid);
    const uint32_t xrow = (uint32_t)a.Hv * a.dv * 2;
    const int64_t xofs = (cl.p * a.Hv + j) * (int64_t)a.dv + t0;
    const uint32_t span = (uint32_t)(cl.L - 1) * xrow + 64;
    const void *src = tid < 256 ? a.v : a.dout;
    const __amdgpu_buffer_rsrc_t rx = rsrc(static_cast<const uint16_t *>(src) + xofs, span);
    const int i = tid & 255;
    pre.x = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(i >> 2) * xrow + 16 * (i & 3), 0, 0);
}

__device__ __forceinline__ float dot8(u32x4 a, u32x4 b) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s += bf2f(a[i] & 0xffff) * bf2f(b[i] & 0xffff) + bf2f(a[i] >> 16) * bf2f(b[i] >> 16);
    return s;
}

// Rows [p, p + L) of a [*, H, dk] bf16 tensor (dk = 64 or 128) at head h,
// for a [64][kLK] tile: issue loads this thread's two 16-byte pieces (zeros
// past dk), commit stores them.  512 threads.
__device__ __forceinline__ void rows512_issue(u32x4 (&v)[2], const void *src, int64_t p, int L,
                                              int H, int h, int dk, int tid) {
    const uint32_t row_bytes = (uint32_t)H * dk * 2;
    const __amdgpu_buffer_rsrc_t r =
        rsrc(static_cast<const uint16_t *>(src) + (p * H + h) * (int64_t)dk,
             (uint32_t)(L - 1) * row_bytes + dk * 2);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + kCT * u;
        v[u] = 8 * (i & 15) < dk
                   ? __builtin_amdgcn_raw_buffer_load_b128(r, (i >> 4) * row_bytes + 16 * (i & 15), 0, 0)
                   : u32x4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void rows512_commit(uint16_t *dst, const u32x4 (&v)[2], int tid) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + kCT * u;
        *reinterpret_cast<u32x4 *>(dst + (i >> 4) * kLK + 8 * (i & 15)) = v[u];
    }
}

__global__ __launch_bounds__(kCT) void bwd_chunk(BwdArgs a) {
    __shared__ ChunkSmem S;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const int rb = w & 3, h = w >> 2;
    const int64_t gc = blockIdx.x;
    const int hk = blockIdx.y;
    ChunkLoc cl;
    if (!locate(a, gc, cl))
        return;
    const int G = a.Hv / a.Hqk;
    const float scale = a.scale;
    // A head's T, P and gates are loaded with its first tile before the
    // barrier that opens it, so their latency is not exposed after it.
    {
        u32x4 kv[2], qv[2];
        rows512_issue(kv, a.k, cl.p, cl.L, a.Hqk, hk, a.dk, tid);
        rows512_issue(qv, a.q, cl.p, cl.L, a.Hqk, hk, a.dk, tid);
        rows512_commit(S.K, kv, tid);
        rows512_commit(S.Q, qv, tid);
    }
    TilePre pre;
    f32x4 tv[2];
    u32x4 pv;
    float gL, gm, btv;
    auto head_issue = [&](int j, int64_t wi) {
        tile_issue(pre, a, cl, j, wi, 0, tid);
        const float *Tg = a.ws_T + wi * (kC * kC);
#pragma unroll
        for (int u = 0; u < 2; ++u)
            tv[u] = *reinterpret_cast<const f32x4 *>(Tg + 4 * (tid + kCT * u));
        pv = *reinterpret_cast<const u32x4 *>(a.ws_P + wi * (kC * kC) + 8 * tid);
        gL = a.ws_gam[wi * kC + kC - 1];
        gm = 0.0f;
        btv = 0.0f;
        if (tid < kC) {
            gm = a.ws_gam[wi * kC + tid];
            btv = tid < cl.L ? a.beta[(cl.p + tid) * a.Hv + j] : 0.0f;
        }
    };
    head_issue(hk * G, gc * a.Hv + hk * G);

    f32x4 dQ[4], dK[4];   // dk tiles 4h + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dQ[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        dK[i] = dQ[i];
    }

    for (int gi = 0; gi < G; ++gi) {
        const int j = hk * G + gi;
        const int64_t wi = gc * a.Hv + j;
        if (gi > 0)
            head_issue(j, wi);
        __syncthreads();  // the previous head's readers are done
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = tid + kCT * u;
            u32x2 hi, lo;
            split4(tv[u], hi, lo);
            *reinterpret_cast<u32x2 *>(S.Th + (i >> 4) * kL64 + 4 * (i & 15)) = hi;
            *reinterpret_cast<u32x2 *>(S.Tl + (i >> 4) * kL64 + 4 * (i & 15)) = lo;
        }
        *reinterpret_cast<u32x4 *>(S.P + (tid >> 3) * kL64 + 8 * (tid & 7)) = pv;
        if (tid < kC) {
            S.gam[tid] = gm;
            S.e[tid] = __expf(gm);
            S.l[tid] = __expf(gL - gm);
            S.bt[tid] = btv;
        }
        const float eL = __expf(gL);

        f32x4 dP[2], dA[2];   // column tiles 2h + i
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            dP[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            dA[i] = dP[i];
        }
        float pb[4] = {0.f, 0.f, 0.f, 0.f};   // dbeta parts of rows 16rb + 4lg + r
        float pg[4] = {0.f, 0.f, 0.f, 0.f};   // dgamma parts
        float dgL = 0.0f;                     // this thread's part of d gamma_L

        for (int t0 = 0; t0 < a.dv; t0 += 32) {
            // The lane indices pass through an empty asm so that the many
            // addresses formed from them are computed here, not hoisted out
            // of the loop and held (or spilled) across it.
            int lrv = lane & 15, lgv = lane >> 4;
            asm volatile("" : "+v"(lrv), "+v"(lgv));
            const int lr = lrv, lg = lgv;
            const int cc = 16 * h + lr;           // this lane's column in a tile
            __syncthreads();
            *reinterpret_cast<u32x4 *>(S.u.t.M0 + (tid >> 4) * kLK + 8 * (tid & 15)) = pre.m;
            *reinterpret_cast<u32x4 *>(S.u.t.dM + (tid >> 4) * kLK + 8 * (tid & 15)) = pre.d;
            dgL += eL * dot8(pre.m, pre.d);
            {
                const int i = tid & 255;
                uint16_t *xd = tid < 256 ? S.u.t.V : S.u.t.dO;
                *reinterpret_cast<u32x4 *>(xd + (i >> 2) * kL32 + 8 * (i & 3)) = pre.x;
            }
            __syncthreads();
            if (t0 + 32 < a.dv)
                tile_issue(pre, a, cl, j, wi, t0 + 32, tid);

            // X = K M0, Y = Q M0, U = K dML (rows 16rb.., columns 16h..).
            f32x4 X = {0.f, 0.f, 0.f, 0.f}, Y = X, U = X;
#pragma unroll
            for (int kx = 0; kx < 4; ++kx) {
                const bf16x8 fk = frag_rows(S.K, kLK, 16 * rb, 32 * kx, lr, lg);
                const bf16x8 fq = frag_rows(S.Q, kLK, 16 * rb, 32 * kx, lr, lg);
                const bf16x8 bm = frag_rows(S.u.t.M0, kLK, 16 * h, 32 * kx, lr, lg);
                const bf16x8 bd = frag_rows(S.u.t.dM, kLK, 16 * h, 32 * kx, lr, lg);
                X = mma(fk, bm, X);
                Y = mma(fq, bm, Y);
                U = mma(fk, bd, U);
            }
            // rhs = diag(beta) (V - diag(e) X), hi and lo.
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * lg + r;
                const float rhs = S.bt[row] * (bf2f(S.u.t.V[row * kL32 + cc]) - S.e[row] * X[r]);
                const uint16_t hb = f2bf(rhs);
                S.u.t.rh[row * kL32 + cc] = hb;
                S.u.t.rl[row * kL32 + cc] = f2bf(rhs - bf2f(hb));
            }
            __syncthreads();

            // Delta = T rhs; dDelta = diag(l) U + P^T dO.
            f32x4 Dl = {0.f, 0.f, 0.f, 0.f}, v1 = Dl, dD;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (32 * kk <= 16 * rb + 15) {
                    const bf16x8 th = frag_rows(S.Th, kL64, 16 * rb, 32 * kk, lr, lg);
                    const bf16x8 tl = frag_rows(S.Tl, kL64, 16 * rb, 32 * kk, lr, lg);
                    const bf16x8 bh = frag_cols(S.u.t.rh, kL32, 32 * kk, 16 * h, lr, lg);
                    const bf16x8 bl = frag_cols(S.u.t.rl, kL32, 32 * kk, 16 * h, lr, lg);
                    Dl = mma(th, bh, Dl);
                    Dl = mma(th, bl, Dl);
                    Dl = mma(tl, bh, Dl);
                }
                if (32 * kk + 31 >= 16 * rb)
                    v1 = mma(frag_cols(S.P, kL64, 32 * kk, 16 * rb, lr, lg),
                             frag_cols(S.u.t.dO, kL32, 32 * kk, 16 * h, lr, lg), v1);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * lg + r;
                dD[r] = S.l[row] * U[r] + scale * v1[r];
                S.u.t.Dh[row * kL32 + cc] = f2bf(Dl[r]);
                const uint16_t hb = f2bf(dD[r]);
                S.u.t.zh[row * kL32 + cc] = hb;
                S.u.t.zl[row * kL32 + cc] = f2bf(dD[r] - bf2f(hb));
                // d l_r = sum_c Delta dW: l_r enters dgamma_r with -l_r, gamma_L with +l_r.
                const float dlr = S.l[row] * Dl[r] * U[r];
                pg[r] -= dlr;
                dgL += dlr;
            }
            __syncthreads();

            // drhs = T^T dDelta.
            f32x4 dR = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (32 * kk + 31 < 16 * rb)
                    continue;
                const bf16x8 th = frag_cols(S.Th, kL64, 32 * kk, 16 * rb, lr, lg);
                const bf16x8 tl = frag_cols(S.Tl, kL64, 32 * kk, 16 * rb, lr, lg);
                const bf16x8 bh = frag_cols(S.u.t.zh, kL32, 32 * kk, 16 * h, lr, lg);
                const bf16x8 bl = frag_cols(S.u.t.zl, kL32, 32 * kk, 16 * h, lr, lg);
                dR = mma(th, bh, dR);
                dR = mma(th, bl, dR);
                dR = mma(tl, bh, dR);
            }
            // dV, the dbeta and dgamma parts, and the operands of the
            // products over columns.
            uint16_t *dvo = static_cast<uint16_t *>(a.dv_);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * lg + r;
                const float b = S.bt[row], e = S.e[row];
                const float vv = bf2f(S.u.t.V[row * kL32 + cc]);
                const float dov = scale * bf2f(S.u.t.dO[row * kL32 + cc]);
                const float dr = dR[r];
                if (row < cl.L)
                    dvo[((cl.p + row) * a.Hv + j) * (int64_t)a.dv + t0 + cc] = f2bf(b * dr);
                pb[r] += dr * (vv - e * X[r]);
                pg[r] += e * dov * Y[r] - b * e * dr * X[r];
                S.u.t.dR[row * kL32 + cc] = f2bf(dr);
                S.u.t.dY[row * kL32 + cc] = f2bf(e * dov);
                S.u.t.dX[row * kL32 + cc] = f2bf(-b * e * dr);
                S.u.t.W[row * kL32 + cc] = f2bf(S.l[row] * Dl[r]);
            }
            __syncthreads();

            // dQ += dY M0^T, dK += dX M0^T + W dML^T (rows 16rb.., dk tiles 4h + i).
            const bf16x8 fy = frag_rows(S.u.t.dY, kL32, 16 * rb, 0, lr, lg);
            const bf16x8 fx = frag_rows(S.u.t.dX, kL32, 16 * rb, 0, lr, lg);
            const bf16x8 fw = frag_rows(S.u.t.W, kL32, 16 * rb, 0, lr, lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int nj = 4 * h + i;
                const bf16x8 bm = frag_cols(S.u.t.M0, kLK, 0, 16 * nj, lr, lg);
                const bf16x8 bd = frag_cols(S.u.t.dM, kLK, 0, 16 * nj, lr, lg);
                dQ[i] = mma(fy, bm, dQ[i]);
                dK[i] = mma(fx, bm, dK[i]);
                dK[i] = mma(fw, bd, dK[i]);
            }
            // dP += do Delta^T (scaled later), dA += drhs Delta^T (negated later).
            const bf16x8 fo = frag_rows(S.u.t.dO, kL32, 16 * rb, 0, lr, lg);
            const bf16x8 fr = frag_rows(S.u.t.dR, kL32, 16 * rb, 0, lr, lg);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bf16x8 bdl = frag_rows(S.u.t.Dh, kL32, 16 * (2 * h + i), 0, lr, lg);
                dP[i] = mma(fo, bdl, dP[i]);
                dA[i] = mma(fr, bdl, dA[i]);
            }
        }
        __syncthreads();

        // K K^T and Q K^T again, for the gradients through A and P.
        int lrv = lane & 15, lgv = lane >> 4;
        asm volatile("" : "+v"(lrv), "+v"(lgv));
        const int lr = lrv, lg = lgv;
        f32x4 kk4[2], qk4[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            kk4[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            qk4[i] = kk4[i];
#pragma unroll
            for (int kx = 0; kx < 4; ++kx) {
                const bf16x8 b = frag_rows(S.K, kLK, 16 * (2 * h + i), 32 * kx, lr, lg);
                kk4[i] = mma(frag_rows(S.K, kLK, 16 * rb, 32 * kx, lr, lg), b, kk4[i]);
                qk4[i] = mma(frag_rows(S.Q, kLK, 16 * rb, 32 * kx, lr, lg), b, qk4[i]);
            }
        }
        float cp[2] = {0.f, 0.f};  // column parts of dgamma, columns 16(2h + i) + lr
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * lg + r, s = 16 * (2 * h + i) + lr;
                const float d = s <= row ? __expf(S.gam[row] - S.gam[s]) : 0.0f;
                const float dpv = scale * dP[i][r];
                const float dav = -dA[i][r];
                const bool incl = s <= row, strict = s < row;
                S.Th[row * kL64 + s] = f2bf(incl ? dpv * d : 0.0f);
                S.u.S[row * kLF + s] = strict ? S.bt[row] * dav * d : 0.0f;
                if (strict)
                    pb[r] += dav * d * kk4[i][r];
                const float dDv = (incl ? dpv * qk4[i][r] : 0.0f) +
                                  (strict ? S.bt[row] * dav * kk4[i][r] : 0.0f);
                const float dDD = incl ? dDv * d : 0.0f;
                pg[r] += dDD;
                cp[i] -= dDD;
            }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float x = cp[i];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            if (lg == 0)
                S.colpart[rb][16 * (2 * h + i) + lr] = x;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float xb = row16_sum(pb[r]);
            const float xg = row16_sum(pg[r]);
            if (lr == 0) {
                const int row = 16 * rb + 4 * lg + r;
                S.rowb[h][row] = xb;
                S.rowg[h][row] = xg;
            }
        }
        S.red[tid] = dgL;
        __syncthreads();
        // S + S^T; dbeta; dgamma with d gamma_L on the last row.
        for (int i = tid; i < kC * kC; i += kCT) {
            const int r = i >> 6, c = i & 63;
            S.Tl[r * kL64 + c] = f2bf(S.u.S[r * kLF + c] + S.u.S[c * kLF + r]);
        }
        if (w == 0) {
            float tot = 0.0f;
#pragma unroll
            for (int i = 0; i < kCT / 64; ++i)
                tot += S.red[64 * i + lane];
            float gl = tot;
            for (int o = 32; o >= 1; o >>= 1)
                gl += __shfl_xor(gl, o);
            float dgm = S.rowg[0][lane] + S.rowg[1][lane] + S.colpart[0][lane] +
                        S.colpart[1][lane] + S.colpart[2][lane] + S.colpart[3][lane];
            if (lane == kC - 1)
                dgm += gl;
            // dg: the reverse cumulative sum of dgamma over the 64 rows
            // (padded rows carry gamma_{L-1}), as a prefix scan of the
            // lane-reversed values.
            const float rev = __shfl(dgm, kC - 1 - lane);
            const float dgs = __shfl(wave_prefix_sum(rev), kC - 1 - lane);
            if (lane < cl.L) {
                a.dbeta[(cl.p + lane) * a.Hv + j] = S.rowb[0][lane] + S.rowb[1][lane];
                a.dg[(cl.p + lane) * a.Hv + j] = dgs;
            }
        }
        __syncthreads();
        // dQ += (dP * D) K; dK += (dP * D)^T Q + (S + S^T) K.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int nj = 4 * h + i;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 bk = frag_cols(S.K, kLK, 32 * kk, 16 * nj, lr, lg);
                const bf16x8 bq = frag_cols(S.Q, kLK, 32 * kk, 16 * nj, lr, lg);
                dQ[i] = mma(frag_rows(S.Th, kL64, 16 * rb, 32 * kk, lr, lg), bk, dQ[i]);
                dK[i] = mma(frag_cols(S.Th, kL64, 32 * kk, 16 * rb, lr, lg), bq, dK[i]);
                dK[i] = mma(frag_rows(S.Tl, kL64, 16 * rb, 32 * kk, lr, lg), bk, dK[i]);
            }
        }
    }

    // dq and dk through LDS (the union is free once the last head's S + S^T
    // pass is done), then 16-byte stores of whole rows.
    uint16_t *dqs = reinterpret_cast<uint16_t *>(&S.u);
    uint16_t *dks = dqs + kC * kLK;
    static_assert(2 * kC * kLK * sizeof(uint16_t) <= sizeof(S.u), "dq, dk tiles fit the union");
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rb + 4 * lg + r, colk = 16 * (4 * h + i) + lr;
            dqs[row * kLK + colk] = f2bf(dQ[i][r]);
            dks[row * kLK + colk] = f2bf(dK[i][r]);
        }
    __syncthreads();
    const int pieces = a.dk / 8;  // 16-byte pieces per row
    for (int e = tid; e < kC * pieces; e += kCT) {
        const int row = e / pieces, pc = e % pieces;
        if (row < cl.L) {
            const int64_t o = ((cl.p + row) * a.Hqk + hk) * (int64_t)a.dk + 8 * pc;
            *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.dq) + o) =
                *reinterpret_cast<const u32x4 *>(dqs + row * kLK + 8 * pc);
            *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.dk_) + o) =
                *reinterpret_cast<const u32x4 *>(dks + row * kLK + 8 * pc);
        }
    }
}

}  // namespace

size_t bwd_workspace_bytes(int64_t n_chunks, int32_t Hv, int32_t dk, int32_t dv) {
    const size_t ch = (size_t)n_chunks * (size_t)Hv;
    size_t b = 0;
    b += ch * kC * kC * sizeof(float);           // T
    b += ch * kC * kC * sizeof(uint16_t);        // P
    b += ch * kC * sizeof(float);                // gamma
    (void)dk;  // the states are kept 128 keys wide (zeros past dk)
    b += 2 * ch * (size_t)kDK * dv * sizeof(uint16_t);  // chunk states and their gradients
    return b;
}

void bwd_carve(BwdArgs &a, void *workspace) {
    const size_t ch = (size_t)a.n_chunks * (size_t)a.Hv;
    char *p = static_cast<char *>(workspace);
    a.ws_T = reinterpret_cast<float *>(p);
    p += ch * kC * kC * sizeof(float);
    a.ws_P = reinterpret_cast<uint16_t *>(p);
    p += ch * kC * kC * sizeof(uint16_t);
    a.ws_gam = reinterpret_cast<float *>(p);
    p += ch * kC * sizeof(float);
    a.ws_hs = reinterpret_cast<uint16_t *>(p);
    p += ch * (size_t)kDK * a.dv * sizeof(uint16_t);
    a.ws_dhs = reinterpret_cast<uint16_t *>(p);
}

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t stream) {
    if (a.n_chunks <= 0)
        return hipSuccess;
    if (a.n_chunks > 0x7fffffff)
        return hipErrorInvalidValue;
    const dim3 chunk_grid((unsigned)a.n_chunks, (unsigned)a.Hv);
    hipLaunchKernelGGL(bwd_prep, chunk_grid, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // The states entering the chunks come from the forward kernel run
    // without its output (its helper/state pipeline, block substitution).
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
    if ((e = launch_fwd_chunk_states(f, stream)) != hipSuccess)
        return e;
    const int64_t seq_blocks = (int64_t)a.n_seqs * a.Hv * (a.dv / kVT);
    hipLaunchKernelGGL(bwd_dstate, dim3((unsigned)seq_blocks), dim3(512), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(bwd_chunk, dim3((unsigned)a.n_chunks, (unsigned)a.Hqk), dim3(kCT), 0, stream,
                       a);
    return hipGetLastError();
}

}  // namespace gdn

// Chunkwise gated delta rule forward, bf16 inputs, dk = 128, for gfx950.
//
// One workgroup (4 waves) owns one (sequence, value head, 64-column value
// tile) and walks the sequence's chunks of 64 tokens in order.  Value columns
// of the state evolve independently (every step of the recurrence acts on
// them column by column), so splitting dv across workgroups is exact.  Wave w
// owns value columns [16w, 16w + 16) of the tile and keeps its [128 x 16]
// slice of the fp32 state M = S^T in MFMA accumulators for the whole
// sequence: the serial chain between chunks never leaves the wave.
//
// The chunk equations (derived from the token recurrence
// S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T of Gated DeltaNet; the
// jax-linear-attention page, "How it works", names this chunk-parallel form
// next to the token-by-token one).  With gamma the in-chunk cumulative
// log-decay and M0 the state entering the chunk:
//   A[r][s] = beta_r exp(gamma_r - gamma_s) (k_r . k_s), s < r     (a3)
//   (I + A) Delta = diag(beta) Y,  Y = V - diag(exp gamma) K M0     (a4, a5)
//   M_L = exp(gamma_L) M0 + K^T diag(exp(gamma_L - gamma)) Delta    (a6)
//   O = scale (diag(exp gamma) Q M0 + P Delta),
//       P[r][s] = exp(gamma_r - gamma_s) (q_r . k_s), s <= r        (a7)
// The UT transform is applied by block forward substitution over four
// 16-row blocks: Delta_i = D_i (diag(beta_i) Y_i - sum_{j<i} A_ij Delta_j)
// with D_i = (I + A_ii)^-1, so only the four 16 x 16 diagonal inverses are
// formed explicitly (by fp32 forward substitution, one wave each).
//
// Per chunk, four workgroup barriers (LDS only: global loads of the next
// chunk stay in flight across them):
//   stage    registers -> LDS (K, Q, V rows; wave 0: gamma tables)
//   phase 1  K M0, Q M0; K K^T and Q K^T tiles -> -A (hi/lo), A_ii, P; Y
//   phase 2  D_i
//   phase 3  Delta; state update; O += P Delta; output staging
//
// Precision: K, Q, V are exact bf16 and every product accumulates in fp32.
// Computed operands on the state chain (D_i, A_ij, the right-hand sides,
// Delta and Delta') enter the MFMA as hi + lo bf16 pairs (x = hi + lo,
// hi = bf16(x), lo = bf16(x - hi); split-bfloat16, Henry, Tang & Heinecke,
// ARITH 2019), three products per pair of split operands and two where one
// side is exact.  K M0, Q M0 and P Delta use hi parts only: their error stays
// well inside the output tolerance, and K M0's is damped by the solve.
//
// MFMA v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][8(l/16)+j] and
// B[8(l/16)+j][l%16] (j = 0..7), receives C[4(l/16)+r][l%16] (r = 0..3).  A
// C-layout tile feeds a later product as its B operand straight from
// registers when the contraction runs over the tile's rows: lane group g
// supplies rows {4g..4g+3} of two stacked 16-row tiles, and the A operand is
// read with the same permuted k order (two 8-byte reads at k = 4g and
// 16 + 4g of each 32-wide step).  K^T and V fragments come from the row-major
// tiles through the LDS transpose read ds_read_b64_tr_b16: within 16 lanes,
// lane 16g+i receives element i%4 of the 8-byte words addressed by lanes
// 16g + 4j + i/4, j = 0..3.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kC = 64;          // chunk length
constexpr int kDK = 128;        // key dimension
constexpr int kDVT = 64;        // value columns per workgroup
constexpr int kThreads = 256;   // 4 waves
constexpr int kSK = kDK + 8;    // row stride (elements) of the K and Q tiles
constexpr int kST = kC + 8;     // row stride of the 64-wide bf16 tiles
constexpr int kSD = 16 + 8;     // row stride of the D blocks

struct alignas(16) Smem {
    uint16_t K[kC * kSK];       // K chunk, [row][dk]
    uint16_t Q[kC * kSK];       // Q chunk, [row][dk]
    uint16_t V[kC * kST];       // value tile, [row][col]
    uint16_t Anh[kC * kST];     // -A hi, off-diagonal 16-blocks below the diagonal
    uint16_t Anl[kC * kST];     // -A lo
    uint16_t P[kC * kST];       // P, lower 16-blocks (upper blocks stay zero)
    uint16_t O[kC * kST];       // output staging, [row][col]
    uint16_t Dh[kC * kSD];      // D_i hi at rows 16 i .. 16 i + 15
    uint16_t Dl[kC * kSD];      // D_i lo
    float Ad[4 * 16 * 16];      // Ad[i][r][p][m] = A_ii[4 m + p][r]
    float gam[kC];              // gamma_r
    float eg[kC];               // exp(gamma_r)
    float el[kC];               // exp(gamma_L - gamma_r)
    float bt[kC];               // beta_r
    float eL;                   // exp(gamma_L)
};

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroup barrier that waits only for this wave's LDS (and scalar) accesses.
__device__ __forceinline__ void lds_barrier() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
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

// A operand in the permuted k order of a 32-wide step starting at p (p is
// already offset to the lane's row): k = 4g..4g+3 and 16+4g..16+4g+3.
__device__ __forceinline__ bf16x8 frag_perm(const uint16_t *p, int g) {
    return cat(ld8(p + 4 * g), ld8(p + 16 + 4 * g));
}

// Transpose read of 4 bf16 (see the file comment).
__device__ __forceinline__ u32x2 ld_tr(const uint16_t *p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

// Four fp32 values as 4 bf16 (hi) and the rounding residuals as 4 bf16 (lo).
__device__ __forceinline__ void split4(f32x4 x, u32x2 &hi, u32x2 &lo) {
    uint16_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = f2bf(x[i]);
        l[i] = f2bf(x[i] - bf2f(h[i]));
    }
    hi = u32x2{h[0] | (unsigned)h[1] << 16, h[2] | (unsigned)h[3] << 16};
    lo = u32x2{l[0] | (unsigned)l[1] << 16, l[2] | (unsigned)l[3] << 16};
}

__device__ __forceinline__ u32x2 pack4(f32x4 x) {
    return u32x2{f2bf(x[0]) | (unsigned)f2bf(x[1]) << 16, f2bf(x[2]) | (unsigned)f2bf(x[3]) << 16};
}

constexpr u32x2 kZero2 = {0u, 0u};

struct Prefetch {
    u32x4 k[4];   // K rows tid/16 + 16 i, columns 8 (tid % 16) .. + 7
    u32x4 q[4];
    u32x4 v[2];   // value-tile rows tid/8 + 32 i, columns 8 (tid % 8) .. + 7
    float g, b;   // wave 0: row = lane
};

__device__ __forceinline__ void load_chunk(Prefetch &pf, const FwdArgs &a, int64_t p, int L,
                                           int hk, int j, int c0, int tid) {
    const uint16_t *kq = static_cast<const uint16_t *>(a.k);
    const uint16_t *qq = static_cast<const uint16_t *>(a.q);
    const uint16_t *vq = static_cast<const uint16_t *>(a.v);
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = tid / 16 + 16 * i;
        const int col = 8 * (tid % 16);
        if (row < L) {
            const int64_t off = ((p + row) * a.Hqk + hk) * (int64_t)kDK + col;
            pf.k[i] = *reinterpret_cast<const u32x4 *>(kq + off);
            pf.q[i] = *reinterpret_cast<const u32x4 *>(qq + off);
        } else {
            pf.k[i] = zero;
            pf.q[i] = zero;
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = tid / 8 + 32 * i;
        const int col = 8 * (tid % 8);
        pf.v[i] = row < L ? *reinterpret_cast<const u32x4 *>(
                                vq + ((p + row) * a.Hv + j) * (int64_t)a.dv + c0 + col)
                          : zero;
    }
    if (tid < kC) {
        const bool ok = tid < L;
        pf.g = ok ? a.g[(p + tid) * a.Hv + j] : 0.0f;
        pf.b = ok ? a.beta[(p + tid) * a.Hv + j] : 0.0f;
    }
}

__device__ __forceinline__ void store_chunk(const Prefetch &pf, Smem &S, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = tid / 16 + 16 * i;
        const int col = 8 * (tid % 16);
        *reinterpret_cast<u32x4 *>(S.K + row * kSK + col) = pf.k[i];
        *reinterpret_cast<u32x4 *>(S.Q + row * kSK + col) = pf.q[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = tid / 8 + 32 * i;
        const int col = 8 * (tid % 8);
        *reinterpret_cast<u32x4 *>(S.V + row * kST + col) = pf.v[i];
    }
}

// (a2) In-chunk cumulative log-decay, by wave 0 (lane r holds g_r; rows past
// the valid length carry g = 0, so gamma_63 = gamma_{L-1}).
__device__ __forceinline__ void chunk_gamma(const Prefetch &pf, Smem &S, int lane) {
    float x = pf.g;
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
        const float y = __shfl_up(x, d, 64);
        if (lane >= d)
            x += y;
    }
    const float gL = __shfl(x, 63, 64);
    S.gam[lane] = x;
    S.eg[lane] = __expf(x);
    S.el[lane] = __expf(gL - x);
    S.bt[lane] = pf.b;
    if (lane == 0)
        S.eL = __expf(gL);
}

// (a3) The lower 16-blocks of K K^T and Q K^T that wave W forms: A row block
// 3 - W (blocks j = 0 .. 3 - W) and P row block W (j = 0 .. W), five in all.
// Block (i, j) is computed as K_j K_i^T (resp. K_j Q_i^T), whose C layout puts
// row 16 i + l%16, columns 16 j + 4 (l/16) .. + 3 of the wanted block in lane
// l: the row-major 8-byte pieces the A operands are read in later.
template <int W>
__device__ __forceinline__ void chunk_tiles(const bf16x8 (&kf)[4][4], const bf16x8 (&qf)[4][4],
                                            Smem &S, int lr, int lg) {
    constexpr int IA = 3 - W;
#pragma unroll
    for (int j = 0; j <= IA; ++j) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            c = mma(kf[j][kk], kf[IA][kk], c);
        const int row = 16 * IA + lr;
        const float gr = S.gam[row], br = S.bt[row];
        if (j < IA) {
            f32x4 val;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                val[r] = -br * __expf(gr - S.gam[16 * j + 4 * lg + r]) * c[r];
            u32x2 hi, lo;
            split4(val, hi, lo);
            *reinterpret_cast<u32x2 *>(S.Anh + row * kST + 16 * j + 4 * lg) = hi;
            *reinterpret_cast<u32x2 *>(S.Anl + row * kST + 16 * j + 4 * lg) = lo;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = 4 * lg + r;  // column within the block; the row is lr
                const float v = col < lr ? br * __expf(gr - S.gam[16 * IA + col]) * c[r] : 0.0f;
                S.Ad[IA * 256 + col * 16 + (lr & 3) * 4 + (lr >> 2)] = v;
            }
        }
    }
#pragma unroll
    for (int j = 0; j <= W; ++j) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            c = mma(kf[j][kk], qf[W][kk], c);
        const int row = 16 * W + lr;
        const float gr = S.gam[row];
        f32x4 val;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int col = 16 * j + 4 * lg + r;
            val[r] = col <= row ? __expf(gr - S.gam[col]) * c[r] : 0.0f;
        }
        *reinterpret_cast<u32x2 *>(S.P + row * kST + 16 * j + 4 * lg) = pack4(val);
    }
}

// x from the lane of the quad whose index is S (DPP quad_perm(S, S, S, S)).
template <int Sel>
__device__ __forceinline__ float quad_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), Sel | (Sel << 2) | (Sel << 4) | (Sel << 6), 0xF, 0xF, false));
}

__device__ __forceinline__ float quad_bcast(float x, int sel) {
    switch (sel) {
    case 0: return quad_bcast<0>(x);
    case 1: return quad_bcast<1>(x);
    case 2: return quad_bcast<2>(x);
    default: return quad_bcast<3>(x);
    }
}

// (a4) D_w = (I + A_ww)^-1 by forward substitution in fp32, by wave w: lane
// 4c + p holds rows p, p+4, p+8, p+12 of column c.  Once x_r is final it is
// broadcast within the lane quad and subtracted from the rows below.
__device__ __forceinline__ void diag_inverse(Smem &S, int w, int lane) {
    const int c = lane >> 2, p = lane & 3;
    float x[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        x[m] = (4 * m + p == c) ? 1.0f : 0.0f;
    const float *ad = S.Ad + w * 256 + p * 4;
#pragma unroll
    for (int r = 0; r < 15; ++r) {
        const f32x4 acol = *reinterpret_cast<const f32x4 *>(ad + r * 16);  // A[4m + p][r]
        const float xr = quad_bcast(x[r / 4], r % 4);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            if (4 * m + p > r)
                x[m] -= acol[m] * xr;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint16_t hi = f2bf(x[m]);
        S.Dh[(16 * w + 4 * m + p) * kSD + c] = hi;
        S.Dl[(16 * w + 4 * m + p) * kSD + c] = f2bf(x[m] - bf2f(hi));
    }
}

__global__ __launch_bounds__(kThreads, 1) void gdn_fwd_bf16_dk128(FwdArgs a) {
    __shared__ Smem S;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // Work item.  Items that read the same q/k head (the dv tiles and the
    // grouped value heads of one q/k head) are kept on one XCD: blocks are
    // dispatched round-robin over the 8 XCDs, so block b runs on XCD b % 8.
    const int n_tiles = a.dv / kDVT;
    const int G = a.Hv / a.Hqk;
    const int gs = n_tiles * G;
    const int nb = gridDim.x;
    int w = blockIdx.x;
    if (nb % (8 * gs) == 0) {
        const int xcd = w % 8, local = w / 8;
        w = ((local / gs) * 8 + xcd) * gs + local % gs;
    }
    const int tile = w % n_tiles;
    const int j = (w / n_tiles) % a.Hv;
    const int n = w / (n_tiles * a.Hv);
    const int hk = j / G;
    const int c0 = tile * kDVT;
    int64_t p0, p1;
    if (a.cu) {
        p0 = a.cu[n];
        p1 = a.cu[n + 1];
    } else {
        p0 = (int64_t)n * a.T;
        p1 = p0 + a.T;
    }

    // Upper blocks of P are read as zeros.
    for (int i = tid; i < kC * kST; i += kThreads)
        S.P[i] = 0;

    // This wave's state slice: h[mt][r] = M[16 mt + 4 lg + r][c0 + 16 wv + lr].
    const int col = c0 + 16 * wv + lr;
    const int64_t hbase = ((int64_t)n * a.Hv + j) * kDK * (int64_t)a.dv;
    f32x4 h[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            h[mt][r] = a.h0 ? a.h0[hbase + (int64_t)(16 * mt + 4 * lg + r) * a.dv + col] : 0.0f;

    Prefetch pf;
    if (p0 < p1)
        load_chunk(pf, a, p0, (int)min<int64_t>(kC, p1 - p0), hk, j, c0, tid);

    for (int64_t p = p0; p < p1; p += kC) {
        const int L = (int)min<int64_t>(kC, p1 - p);
        store_chunk(pf, S, tid);
        if (wv == 0)
            chunk_gamma(pf, S, lane);
        if (p + kC < p1)
            load_chunk(pf, a, p + kC, (int)min<int64_t>(kC, p1 - p - kC), hk, j, c0, tid);
        lds_barrier();

        // ---- phase 1 ----------------------------------------------------
        bf16x8 kf[4][4], qf[4][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int off = (16 * mi + lr) * kSK + 32 * kk;
                kf[mi][kk] = frag_perm(S.K + off, lg);
                qf[mi][kk] = frag_perm(S.Q + off, lg);
            }
        // (a5, a7) X = K M0 and Q M0 on this wave's columns (hi part of M0).
        bf16x8 hb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            hb[kk] = cat(pack4(h[2 * kk]), pack4(h[2 * kk + 1]));
        f32x4 X[4], Oa[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            X[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
            Oa[mi] = X[mi];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                X[mi] = mma(kf[mi][kk], hb[kk], X[mi]);
                Oa[mi] = mma(qf[mi][kk], hb[kk], Oa[mi]);
            }
        }
        // (a3) this wave's blocks of -A, A_ii and P.
        switch (wv) {
        case 0: chunk_tiles<0>(kf, qf, S, lr, lg); break;
        case 1: chunk_tiles<1>(kf, qf, S, lr, lg); break;
        case 2: chunk_tiles<2>(kf, qf, S, lr, lg); break;
        default: chunk_tiles<3>(kf, qf, S, lr, lg); break;
        }
        // Right-hand sides R_i = diag(beta) (V - diag(exp gamma) X); O scaled.
        f32x4 R[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const u32x2 vv = ld_tr(S.V + (16 * mi + 4 * lg + (lr >> 2)) * kST + 16 * wv + 4 * (lr & 3));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * mi + 4 * lg + r;
                const float vr = bf2f(static_cast<uint16_t>(vv[r / 2] >> (16 * (r % 2))));
                const float e = S.eg[row];
                R[mi][r] = S.bt[row] * (vr - e * X[mi][r]);
                Oa[mi][r] *= e;
            }
        }
        lds_barrier();

        // ---- phase 2 ----------------------------------------------------
        diag_inverse(S, wv, lane);
        lds_barrier();

        // ---- phase 3 ----------------------------------------------------
        // (a4, a5) Delta_i = D_i (R_i - sum_{j<i} A_ij Delta_j), split products.
        u32x2 dh[4], dl[4];
        f32x4 D[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 c = R[i];
            const int ao = (16 * i + lr) * kST;
            if (i == 1) {
                const bf16x8 ah = cat(ld8(S.Anh + ao + 4 * lg), kZero2);
                const bf16x8 al = cat(ld8(S.Anl + ao + 4 * lg), kZero2);
                c = mma(ah, cat(dh[0], kZero2), c);
                c = mma(ah, cat(dl[0], kZero2), c);
                c = mma(al, cat(dh[0], kZero2), c);
            } else if (i >= 2) {
                const bf16x8 ah = frag_perm(S.Anh + ao, lg);
                const bf16x8 al = frag_perm(S.Anl + ao, lg);
                c = mma(ah, cat(dh[0], dh[1]), c);
                c = mma(ah, cat(dl[0], dl[1]), c);
                c = mma(al, cat(dh[0], dh[1]), c);
                if (i == 3) {
                    const bf16x8 bh = cat(ld8(S.Anh + ao + 32 + 4 * lg), kZero2);
                    const bf16x8 bl = cat(ld8(S.Anl + ao + 32 + 4 * lg), kZero2);
                    c = mma(bh, cat(dh[2], kZero2), c);
                    c = mma(bh, cat(dl[2], kZero2), c);
                    c = mma(bl, cat(dh[2], kZero2), c);
                }
            }
            u32x2 rh, rl;
            split4(c, rh, rl);
            const int dofs = (16 * i + lr) * kSD + 4 * lg;
            const bf16x8 Dhi = cat(ld8(S.Dh + dofs), kZero2);
            const bf16x8 Dlo = cat(ld8(S.Dl + dofs), kZero2);
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
            d = mma(Dhi, cat(rh, kZero2), d);
            d = mma(Dhi, cat(rl, kZero2), d);
            d = mma(Dlo, cat(rh, kZero2), d);
            D[i] = d;
            split4(d, dh[i], dl[i]);
        }

        // (a6) M_L = exp(gamma_L) M0 + K^T Delta', Delta' = diag(exp(gamma_L - gamma)) Delta.
        bf16x8 dph[2], dpl[2];
        {
            u32x2 ph[4], pl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 x;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x[r] = S.el[16 * i + 4 * lg + r] * D[i][r];
                split4(x, ph[i], pl[i]);
            }
            dph[0] = cat(ph[0], ph[1]);
            dph[1] = cat(ph[2], ph[3]);
            dpl[0] = cat(pl[0], pl[1]);
            dpl[1] = cat(pl[2], pl[3]);
        }
        const float eL = S.eL;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            h[mt] *= eL;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint16_t *kp = S.K + (32 * kk + 4 * lg + (lr >> 2)) * kSK + 16 * mt + 4 * (lr & 3);
                const bf16x8 akt = cat(ld_tr(kp), ld_tr(kp + 16 * kSK));
                h[mt] = mma(akt, dph[kk], h[mt]);
                h[mt] = mma(akt, dpl[kk], h[mt]);
            }
        }

        // (a7) O += P Delta (hi parts), staged through LDS for coalesced stores.
        const bf16x8 db[2] = {cat(dh[0], dh[1]), cat(dh[2], dh[3])};
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int kk = 0; kk <= mi / 2; ++kk)
                Oa[mi] = mma(frag_perm(S.P + (16 * mi + lr) * kST + 32 * kk, lg), db[kk], Oa[mi]);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S.O[(16 * mi + 4 * lg + r) * kST + 16 * wv + lr] = f2bf(a.scale * Oa[mi][r]);
        }
        lds_barrier();

        uint16_t *o = static_cast<uint16_t *>(a.o);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = tid / 8 + 32 * i;
            const int cc = 8 * (tid % 8);
            if (row < L)
                *reinterpret_cast<u32x4 *>(o + ((p + row) * a.Hv + j) * (int64_t)a.dv + c0 + cc) =
                    *reinterpret_cast<const u32x4 *>(S.O + row * kST + cc);
        }
    }

    if (a.ht) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a.ht[hbase + (int64_t)(16 * mt + 4 * lg + r) * a.dv + col] = h[mt][r];
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream) {
    const int n_tiles = a.dv / kDVT;
    const int64_t blocks = (int64_t)a.n_seqs * a.Hv * n_tiles;
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(gdn_fwd_bf16_dk128, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gdn

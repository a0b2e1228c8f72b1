// Chunkwise gated delta rule forward, bf16 inputs, dk = 128, for gfx950.
//
// One workgroup (4 waves) owns one (sequence, value head, 64-column value
// tile) and walks the sequence's chunks of 64 tokens in order.  Value columns
// of the state evolve independently (every step of the recurrence acts on
// them column by column), so splitting dv across workgroups is exact.  Each
// wave owns 16 of the 64 columns and keeps its slice of the fp32 state,
// M = S^T restricted to [128 x 16], in MFMA accumulator registers for the
// whole sequence: the serial chain between chunks never leaves the wave.
//
// Per chunk (gamma = in-chunk cumulative log-decay, L = valid rows):
//   (a2) gamma, exp(gamma), exp(gamma_L - gamma)                   wave 0
//   (a3) A = strictly-lower (beta exp(gamma_r - gamma_s) K K^T)    MFMA, 10 tiles
//        P = lower-incl.   (exp(gamma_r - gamma_s) Q K^T)          MFMA, 10 tiles
//   (a4) T' = (I + A)^-1 diag(beta): 16x16 diagonal blocks by forward
//        substitution, off-diagonal blocks by fp32 MFMA products
//   (a5) Y = V - diag(exp gamma) K M0;  Delta = T' Y                MFMA
//   (a6) M_L = exp(gamma_L) M0 + K^T diag(exp(gamma_L - gamma)) Delta
//   (a7) O = scale (diag(exp gamma) Q M0 + P Delta)
// These are the chunk equations of the gated delta rule (derived from the
// token recurrence S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T of
// Gated DeltaNet; the jax-linear-attention page, "How it works", names the
// chunk-parallel form next to the token-by-token one).
//
// Precision: K, Q and V are exact bf16 and their products accumulate in fp32.
// Operands that are computed (the state, T', Y, Delta') are fp32; on the
// state chain they enter the MFMA as hi + lo bf16 pairs (x = hi + lo with
// hi = bf16(x), lo = bf16(x - hi); split-bfloat16, Henry, Tang & Heinecke,
// ARITH 2019): T' Y takes three products (hi hi, hi lo, lo hi), K^T Delta' two
// (K is exact).  K M0, Q M0 and P Delta use the hi part only: their error
// stays far below the output tolerance and, for K M0, is damped by T'.
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l supplies A[l%16][8*(l/16)+j] and
// B[8*(l/16)+j][l%16] (j = 0..7) and receives C[4*(l/16)+r][l%16] (r = 0..3).
// A result tile in that C layout feeds the next product as its B operand
// without leaving the registers when the contraction runs over the tile's
// rows: lane group g then supplies rows {4g..4g+3} of two stacked 16-row
// tiles, and the A operand reads the same permuted k indices (two 8-byte LDS
// reads at k = 4g and k = 16 + 4g of each 32-wide step).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kC = 64;          // chunk length
constexpr int kDK = 128;        // key dimension
constexpr int kDVT = 64;        // value columns per workgroup
constexpr int kThreads = 256;   // 4 waves; wave w owns value columns [16w, 16w + 16)
constexpr int kSK = kDK + 8;    // row stride (elements) of the [64][128] bf16 tiles
constexpr int kST = kC + 8;     // row stride of the [*][64] bf16 tiles
constexpr int kSA = kC + 4;     // row stride of the [64][64] fp32 tiles

struct Smem {
    uint16_t K[kC * kSK];       // K chunk, [row][dk]
    uint16_t Q[kC * kSK];       // Q chunk, [row][dk]; reused as Tf (fp32) by the solve
    uint16_t KT[kDK * kST];     // K chunk transposed, [dk][row]
    uint16_t VT[kDVT * kST];    // V tile transposed, [dv][row]
    uint16_t P[kC * kST];       // (Q K^T) * decay mask, [row][col]
    uint16_t Th[kC * kST];      // T' hi, [row][col]
    uint16_t Tl[kC * kST];      // T' lo
    uint16_t O[kC * kST];       // output staging, [row][dv]
    float AT[kC * kSA];         // A transposed, [col][row]
    float gam[kC];              // gamma_r
    float eg[kC];               // exp(gamma_r)
    float el[kC];               // exp(gamma_L - gamma_r)
    float bt[kC];               // beta_r
    float eL;                   // exp(gamma_L)
};
static_assert(sizeof(uint16_t) * kC * kSK == sizeof(float) * kC * kSA, "Tf must fit in Q");

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(uint16_t x) {
    return __uint_as_float(static_cast<unsigned>(x) << 16);
}

__device__ __forceinline__ uint16_t f2bf(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// A operand with the permuted k order: k = 4g .. 4g+3 and 16+4g .. 16+4g+3
// of the 32-wide step starting at `p` (p already offset to the lane's row).
__device__ __forceinline__ bf16x8 frag_perm(const uint16_t *p, int g) {
    const u32x2 lo = *reinterpret_cast<const u32x2 *>(p + 4 * g);
    const u32x2 hi = *reinterpret_cast<const u32x2 *>(p + 16 + 4 * g);
    const u32x4 v = {lo.x, lo.y, hi.x, hi.y};
    return __builtin_bit_cast(bf16x8, v);
}

// A or B operand in the plain order: k = 8g .. 8g+7 of the step at `p`.
__device__ __forceinline__ bf16x8 frag_plain(const uint16_t *p, int g) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p + 8 * g));
}

// B operand from two stacked C-layout tiles (rows 0..15 and 16..31 of a step).
__device__ __forceinline__ bf16x8 pack_hi(f32x4 a, f32x4 b) {
    bf16x8 r;
    r[0] = static_cast<__bf16>(a[0]); r[1] = static_cast<__bf16>(a[1]);
    r[2] = static_cast<__bf16>(a[2]); r[3] = static_cast<__bf16>(a[3]);
    r[4] = static_cast<__bf16>(b[0]); r[5] = static_cast<__bf16>(b[1]);
    r[6] = static_cast<__bf16>(b[2]); r[7] = static_cast<__bf16>(b[3]);
    return r;
}

__device__ __forceinline__ void split(f32x4 a, f32x4 b, bf16x8 &hi, bf16x8 &lo) {
    hi = pack_hi(a, b);
    f32x4 ra, rb;
    for (int i = 0; i < 4; ++i) {
        ra[i] = a[i] - static_cast<float>(hi[i]);
        rb[i] = b[i] - static_cast<float>(hi[4 + i]);
    }
    lo = pack_hi(ra, rb);
}

// The 10 lower-triangular 16x16 tiles of a 64x64 matrix, as (row, col) blocks.
__constant__ int8_t kLowerTiles[10][2] = {{0, 0}, {1, 0}, {1, 1}, {2, 0}, {2, 1},
                                          {2, 2}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};

struct Prefetch {
    u32x4 k[4];   // rows tid/16 + 16 i, columns 8 (tid % 16) .. + 7
    u32x4 q[4];
    u32x4 v[2];   // rows tid/8 + 32 i, columns 8 (tid % 8) .. + 7 of the value tile
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
        if (row < L)
            pf.v[i] = *reinterpret_cast<const u32x4 *>(vq + ((p + row) * a.Hv + j) * (int64_t)a.dv
                                                      + c0 + col);
        else
            pf.v[i] = zero;
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
#pragma unroll
        for (int e = 0; e < 8; ++e)
            S.KT[(col + e) * kST + row] =
                static_cast<uint16_t>(pf.k[i][e / 2] >> (16 * (e % 2)));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = tid / 8 + 32 * i;
        const int col = 8 * (tid % 8);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            S.VT[(col + e) * kST + row] =
                static_cast<uint16_t>(pf.v[i][e / 2] >> (16 * (e % 2)));
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

// (a4) T = (I + A)^-1 in fp32, A strictly lower, stored transposed in S.AT;
// result in Tf = S.Q viewed as fp32 [64][kSA].  Then T' = T diag(beta) as
// hi/lo bf16 into S.Th / S.Tl (lower blocks only; upper blocks stay zero).
__device__ __forceinline__ void solve_ut(Smem &S, int tid) {
    float *Tf = reinterpret_cast<float *>(S.Q);
    const int wv = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;

    // Diagonal blocks: wave 0, lane = 16 b + c solves column c of block b by
    // forward substitution (right-looking: once x_r is final, subtract its
    // multiple from the rows below).
    if (wv == 0) {
        const int b = lane >> 4, c = lane & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            x[i] = (i == c) ? 1.0f : 0.0f;
#pragma unroll
        for (int r = 0; r < 15; ++r) {
            const float *col = S.AT + (16 * b + r) * kSA + 16 * b;  // A[16b + *][16b + r]
            float a16[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 t = *reinterpret_cast<const f32x4 *>(col + 4 * q4);
                a16[4 * q4 + 0] = t[0]; a16[4 * q4 + 1] = t[1];
                a16[4 * q4 + 2] = t[2]; a16[4 * q4 + 3] = t[3];
            }
#pragma unroll
            for (int r2 = r + 1; r2 < 16; ++r2)
                x[r2] -= a16[r2] * x[r];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
            Tf[(16 * b + i) * kSA + 16 * b + c] = x[i];
    }
    __syncthreads();

    // Off-diagonal blocks X_ij (i > j): X_ij = -D_i sum_{k=j}^{i-1} A_ik X_kj,
    // D_i = X_ii.  fp32 MFMA 16x16x4: lane l supplies A[l%16][l/16] and
    // B[l/16][l%16], receives C[4(l/16)+r][l%16].
    auto Aik = [&](int i, int k, int kk) {  // A_ik[lr][kk]
        return S.AT[(16 * k + kk) * kSA + 16 * i + lr];
    };
    auto Tblk = [&](int i, int j, int rr, int cc) -> float & {
        return Tf[(16 * i + rr) * kSA + 16 * j + cc];
    };
    // c += A_ik X_kj (both from LDS)
    auto prod_lds = [&](int i, int k, int j, f32x4 c) {
#pragma unroll
        for (int kp = 0; kp < 4; ++kp)
            c = mma_f32(Aik(i, k, 4 * kp + lg), Tblk(k, j, 4 * kp + lg, lr), c);
        return c;
    };
    // -D_i Z with Z in C layout
    auto neg_dinv = [&](int i, f32x4 z) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < 4; ++kp)
            c = mma_f32(Tblk(i, i, lr, 4 * lg + kp), z[kp], c);
        return -c;
    };
    auto store_blk = [&](int i, int j, f32x4 c) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Tblk(i, j, 4 * lg + r, lr) = c[r];
    };
    auto load_blk = [&](int i, int j) {
        f32x4 c;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            c[r] = Tblk(i, j, 4 * lg + r, lr);
        return c;
    };
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // Level 1: X_10, X_21, X_32; wave 3 forms A_20 D_0, A_31 D_1, A_30 D_0 into
    // unused upper blocks (0,2), (1,3), (0,3).
    if (wv < 3) {
        const int i = wv + 1, j = wv;
        store_blk(i, j, neg_dinv(i, prod_lds(i, j, j, zero)));
    } else {
        store_blk(0, 2, prod_lds(2, 0, 0, zero));
        store_blk(1, 3, prod_lds(3, 1, 1, zero));
        store_blk(0, 3, prod_lds(3, 0, 0, zero));
    }
    __syncthreads();
    // Level 2: X_20, X_31; wave 2 accumulates A_31 X_10 into (0,3).
    if (wv == 0) {
        store_blk(2, 0, neg_dinv(2, prod_lds(2, 1, 0, load_blk(0, 2))));
    } else if (wv == 1) {
        store_blk(3, 1, neg_dinv(3, prod_lds(3, 2, 1, load_blk(1, 3))));
    } else if (wv == 2) {
        store_blk(0, 3, prod_lds(3, 1, 0, load_blk(0, 3)));
    }
    __syncthreads();
    // Level 3: X_30.
    if (wv == 0)
        store_blk(3, 0, neg_dinv(3, prod_lds(3, 2, 0, load_blk(0, 3))));
    __syncthreads();

    // T' = T diag(beta) as hi + lo bf16, lower blocks.
    for (int e = tid; e < 10 * 256; e += kThreads) {
        const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        const int r = 16 * kLowerTiles[blk][0] + rr, s = 16 * kLowerTiles[blk][1] + cc;
        const float t = (s <= r) ? Tf[r * kSA + s] * S.bt[s] : 0.0f;
        const uint16_t hi = f2bf(t);
        S.Th[r * kST + s] = hi;
        S.Tl[r * kST + s] = f2bf(t - bf2f(hi));
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

    // Upper blocks of P and T' are read as zeros by the products below.
    for (int i = tid; i < kC * kST; i += kThreads) {
        S.P[i] = 0;
        S.Th[i] = 0;
        S.Tl[i] = 0;
    }

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
        __syncthreads();

        // (a5, a7 first half) X = K M0 and Q M0 on this wave's 16 columns.
        bf16x8 hb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            hb[kk] = pack_hi(h[2 * kk], h[2 * kk + 1]);
        f32x4 X[4], Oa[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            X[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
            Oa[mi] = X[mi];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int off = (16 * mi + lr) * kSK + 32 * kk;
                X[mi] = mma(frag_perm(S.K + off, lg), hb[kk], X[mi]);
                Oa[mi] = mma(frag_perm(S.Q + off, lg), hb[kk], Oa[mi]);
            }
        }

        // (a3) K K^T -> A (transposed, fp32) and Q K^T -> P (bf16), lower tiles.
#pragma unroll
        for (int tt = wv; tt < 20; tt += 4) {
            const int isq = tt >= 10;
            const int mi = kLowerTiles[tt % 10][0], ni = kLowerTiles[tt % 10][1];
            const uint16_t *src = isq ? S.Q : S.K;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = mma(frag_plain(src + (16 * mi + lr) * kSK + 32 * kk, lg),
                          frag_plain(S.K + (16 * ni + lr) * kSK + 32 * kk, lg), acc);
            const int s = 16 * ni + lr;
            const float gs_ = S.gam[s];
            if (!isq) {
                f32x4 outv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * mi + 4 * lg + r;
                    outv[r] = (s < row) ? S.bt[row] * __expf(S.gam[row] - gs_) * acc[r] : 0.0f;
                }
                *reinterpret_cast<f32x4 *>(S.AT + s * kSA + 16 * mi + 4 * lg) = outv;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * mi + 4 * lg + r;
                    const float pv = (s <= row) ? __expf(S.gam[row] - gs_) * acc[r] : 0.0f;
                    S.P[row * kST + s] = f2bf(pv);
                }
            }
        }

        // Y = V - diag(exp gamma) X as hi/lo B operands; O scaled by exp(gamma).
        bf16x8 yh[2], yl[2];
        {
            f32x4 Y[4];
            const int vc = 16 * wv + lr;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const int row0 = 16 * mi + 4 * lg;
                const u32x2 vv = *reinterpret_cast<const u32x2 *>(S.VT + vc * kST + row0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float vr = bf2f(static_cast<uint16_t>(vv[r / 2] >> (16 * (r % 2))));
                    const float e = S.eg[row0 + r];
                    Y[mi][r] = vr - e * X[mi][r];
                    Oa[mi][r] *= e;
                }
            }
            split(Y[0], Y[1], yh[0], yl[0]);
            split(Y[2], Y[3], yh[1], yl[1]);
        }
        __syncthreads();

        // (a4) UT transform.
        solve_ut(S, tid);
        __syncthreads();

        // (a5) Delta = T' Y, three products per step (T' lower triangular:
        // row tiles 0, 1 need only the first 32-wide step).
        f32x4 D[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            D[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk <= mi / 2; ++kk) {
                const int off = (16 * mi + lr) * kST + 32 * kk;
                const bf16x8 th = frag_perm(S.Th + off, lg);
                const bf16x8 tl = frag_perm(S.Tl + off, lg);
                D[mi] = mma(th, yh[kk], D[mi]);
                D[mi] = mma(th, yl[kk], D[mi]);
                D[mi] = mma(tl, yh[kk], D[mi]);
            }
        }
        bf16x8 dh[2], dl[2], db[2];
        {
            f32x4 Dp[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Dp[mi][r] = S.el[16 * mi + 4 * lg + r] * D[mi][r];
            split(Dp[0], Dp[1], dh[0], dl[0]);
            split(Dp[2], Dp[3], dh[1], dl[1]);
            db[0] = pack_hi(D[0], D[1]);
            db[1] = pack_hi(D[2], D[3]);
        }

        // (a6) M_L = exp(gamma_L) M0 + K^T Delta'.
        const float eL = S.eL;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            h[mt] *= eL;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 akt = frag_perm(S.KT + (16 * mt + lr) * kST + 32 * kk, lg);
                h[mt] = mma(akt, dh[kk], h[mt]);
                h[mt] = mma(akt, dl[kk], h[mt]);
            }
        }

        // (a7) O += P Delta, scaled, staged through LDS for coalesced stores.
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int kk = 0; kk <= mi / 2; ++kk)
                Oa[mi] = mma(frag_perm(S.P + (16 * mi + lr) * kST + 32 * kk, lg), db[kk], Oa[mi]);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S.O[(16 * mi + 4 * lg + r) * kST + 16 * wv + lr] = f2bf(a.scale * Oa[mi][r]);
        }
        __syncthreads();
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

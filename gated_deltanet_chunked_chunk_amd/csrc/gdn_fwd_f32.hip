// Chunkwise gated delta rule forward, fp32 inputs, for gfx950.
//
// The same chunk equations as the bf16 kernel, evaluated entirely in fp32
// vector arithmetic (products, the triangular solve and the state), with the
// accurate expf.  fp32 inputs come with tolerances tighter than a bf16 MFMA
// path can meet, and the workloads that use them are small: one workgroup
// per (sequence, value head, 32 value columns), every step a loop over
// register tiles of LDS-staged operands, separated by barriers.  Chunks are
// 64 tokens, or 32 with dk = 256 (so that the K and Q tiles fit in LDS).
//
// Per chunk of L <= C tokens starting from state M0 ([dk][dv], M = S^T):
//   gamma_r = g_1 + ... + g_r
//   A[r][s] = beta_r exp(gamma_r - gamma_s) (k_r . k_s),  s < r
//   T' = (I + A)^-1 diag(beta)              (forward substitution per column)
//   Delta = T' (V - diag(exp gamma) K M0)
//   O = scale (diag(exp gamma) Q M0 + ((Q K^T) * D) Delta),  D[r][s] = exp(gamma_r - gamma_s), s <= r
//   M_L = exp(gamma_L) M0 + K^T diag(exp(gamma_L - gamma)) Delta
// derived from the token recurrence of the gated delta rule (Gated DeltaNet;
// chunk-parallel form per the jax-linear-attention page, "How it works").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kDVT = 32;
constexpr int kThreads = 512;

template <int DK>
constexpr int chunk_f32() {
    return DK == 256 ? 32 : 64;
}

// K, Q, P and T' are held transposed (a column of the row-major matrix is a
// row here), so that a thread's register tile of consecutive rows reads one
// 16-byte word per step of the contraction; rows are 16-byte aligned.
template <int DK, int kC = chunk_f32<DK>()>
struct SmemF32 {
    alignas(16) float KT[DK][kC + 4];    // KT[d][r] = K[r][d]
    alignas(16) float QT[DK][kC + 4];    // QT[d][r] = Q[r][d]
    alignas(16) float V[kC][kDVT + 4];   // V rows, then Delta
    alignas(16) float M[DK][kDVT + 4];   // state slice
    alignas(16) float A[kC][kC + 4];     // A (strictly lower), row r's column s at (s % 4) C/4 + s / 4
    alignas(16) float TT[kC][kC + 4];    // TT[s][r] = T'[r][s], T' = (I + A)^-1 diag(beta)
    alignas(16) float PT[kC][kC + 4];    // PT[s][r] = P[r][s], P = (Q K^T) * D
    alignas(16) float Y[kC][kDVT + 4];   // V - diag(exp gamma) K M0
    alignas(16) float gam[kC], bt[kC], el[kC], eg[kC];
};

typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ float4 ld4(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}

__device__ __forceinline__ float2 ld2(const float *p) {
    return *reinterpret_cast<const float2 *>(p);
}

// Thread (h, i, j) = (tid / 256, tid / 16 % 16, tid % 16) owns register
// tiles of consecutive rows TR i .. of the chunk (TR = C / 16) and, for
// [C x 32] results, the value column 2 j + h; for the C x C products the
// columns TR j + TR/2 h .. + TR/2 - 1 of the other operand; for the state
// update the keys TD i .. (TD = dk / 16).  Two waves share each SIMD, so one
// waits for LDS while the other computes.  Each element is still one running
// sum in the order of its contraction index.
template <int DK>
__global__ __launch_bounds__(kThreads) void gdn_fwd_f32_kernel(FwdArgs a) {
    constexpr int kC = chunk_f32<DK>();
    constexpr int TR = kC / 16, TD = DK / 16;
    constexpr int TH = TR / 2;  // columns of the C x C tile per thread
    typedef __attribute__((ext_vector_type(TR))) float rowv;
    typedef __attribute__((ext_vector_type(TH))) float colv;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SmemF32<DK> &S = *reinterpret_cast<SmemF32<DK> *>(smem_raw);
    const int tid = threadIdx.x;
    const int th = tid >> 8, ti = (tid >> 4) & 15, tj = tid & 15;
    const int vc = 2 * tj + th;  // value column of the [C x 32] tiles
    const int n_tiles = a.dv / kDVT;
    const int G = a.Hv / a.Hqk;
    const int w = blockIdx.x;
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
    const float *q = static_cast<const float *>(a.q);
    const float *k = static_cast<const float *>(a.k);
    const float *v = static_cast<const float *>(a.v);
    float *o = static_cast<float *>(a.o);
    const int64_t hbase = ((int64_t)n * a.Hv + j) * DK * (int64_t)a.dv;
    auto rows = [](const float *p) {  // TR consecutive entries of a 16-byte aligned row
        if constexpr (TR == 4) {
            const float4 x = ld4(p);
            return rowv{x.x, x.y, x.z, x.w};
        } else {
            const float2 x = ld2(p);
            return rowv{x.x, x.y};
        }
    };

    auto cols = [](const float *p) {  // TH consecutive entries, 8-byte aligned when TH = 2
        if constexpr (TH == 2) {
            const float2 x = ld2(p);
            return colv{x.x, x.y};
        } else {
            return colv{p[0]};
        }
    };

    for (int e = tid; e < DK * kDVT; e += kThreads) {
        const int i = e / kDVT, c = e % kDVT;
        S.M[i][c] = a.h0 ? a.h0[hbase + (int64_t)i * a.dv + c0 + c] : 0.0f;
    }

    for (int64_t p = p0; p < p1; p += kC) {
        const int L = (int)min<int64_t>(kC, p1 - p);
        __syncthreads();
        // Every load of the chunk is issued before any is stored, so their
        // latencies overlap instead of adding up.  K and Q: a wave-wide load
        // covers 16 rows x 16 keys (a 16-byte piece per lane) and stores it
        // transposed with no two lanes on one LDS bank.  Rows past the
        // chunk's end load row L - 1 and are replaced by zeros (a select of
        // values: the loads stay unconditional).
        {
            constexpr int KPT = kC * DK / (4 * kThreads);
            constexpr int VPT = (kC * kDVT / 4 + kThreads - 1) / kThreads;
            f32x4 kr[KPT], qr[KPT], vr[VPT];
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const int e = tid + kThreads * i, blk = e >> 6, l = e & 63;
                const int r = 16 * (blk % (kC / 16)) + (l & 15), d = 16 * (blk / (kC / 16)) + 4 * (l >> 4);
                const int64_t off = ((p + min(r, L - 1)) * a.Hqk + hk) * DK + d;
                const f32x4 kx = *reinterpret_cast<const f32x4 *>(k + off);
                const f32x4 qx = *reinterpret_cast<const f32x4 *>(q + off);
                const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                kr[i] = r < L ? kx : z;
                qr[i] = r < L ? qx : z;
            }
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                // pieces past the tile (at 32-token chunks, half the threads
                // have none) load row 0 and are not stored
                const int e = tid + kThreads * i, r = min(e / (kDVT / 4), kC - 1), c = 4 * (e % (kDVT / 4));
                const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                const f32x4 vx = *reinterpret_cast<const f32x4 *>(
                    v + ((p + min(r, L - 1)) * a.Hv + j) * (int64_t)a.dv + c0 + c);
                vr[i] = r < L ? vx : z;
            }
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const int e = tid + kThreads * i, blk = e >> 6, l = e & 63;
                const int r = 16 * (blk % (kC / 16)) + (l & 15), d = 16 * (blk / (kC / 16)) + 4 * (l >> 4);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    S.KT[d + u][r] = kr[i][u];
                    S.QT[d + u][r] = qr[i][u];
                }
            }
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int e = tid + kThreads * i, r = e / (kDVT / 4), c = 4 * (e % (kDVT / 4));
                if (e < kC * kDVT / 4)
                    *reinterpret_cast<f32x4 *>(&S.V[r][c]) = vr[i];
            }
        }
        if (tid < 64) {
            // Gates of row r = lane, loaded in parallel (rows past the
            // chunk's end read as zero).  gamma is summed in row order, the
            // same sequence of fp32 additions in every lane (lane r keeps the
            // partial sum after row r): gamma_L - gamma_r then carries only
            // the rounding of rows r+1..L, which a tree-shaped scan would not.
            const int r = tid;
            const bool ok = r < L;
            float gv = ok ? a.g[(p + r) * a.Hv + j] : 0.0f;
            float bv = ok ? a.beta[(p + r) * a.Hv + j] : 0.0f;
            if ((a.flags & kStepGateAct) && ok) {
                gv = logsigmoid_f32(gv);
                bv = sigmoid_f32(bv);
            }
            float acc = 0.0f, mine = 0.0f;
#pragma unroll
            for (int i = 0; i < kC; ++i) {
                acc += __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                     __builtin_bit_cast(int, gv), i));
                if (i == r)
                    mine = acc;
            }
            if (r < kC) {
                S.gam[r] = mine;
                S.bt[r] = bv;
                S.el[r] = expf(acc - mine);
                S.eg[r] = expf(mine);
            }
        }
        __syncthreads();
        if (a.flags & kStepL2Norm) {
            // In-op L2 normalisation: one wave per row of K or Q (fp32).
            const int lane = tid & 63;
            for (int row = tid >> 6; row < 2 * kC; row += kThreads / 64) {
                float(*x)[kC + 4] = row < kC ? S.KT : S.QT;
                const int rr = row < kC ? row : row - kC;
                float ss = 0.0f;
                for (int d = lane; d < DK; d += 64)
                    ss += x[d][rr] * x[d][rr];
                for (int o = 32; o >= 1; o >>= 1)
                    ss += __shfl_xor(ss, o);
                const float inv = inv_l2_norm(ss);
                for (int d = lane; d < DK; d += 64)
                    x[d][rr] *= inv;
            }
            __syncthreads();
        }

        // A (strictly lower) and P (lower incl. diagonal) on the register
        // tile rows TR ti .., columns TR tj .. (tiles above the diagonal
        // are never read and not formed).
        if (tj <= ti) {
            const int s0 = TR * tj + TH * th;  // this thread's first column
            colv kk[TR], qk[TR];  // [row t][column u]
#pragma unroll
            for (int t = 0; t < TR; ++t) {
                kk[t] = colv{};
                qk[t] = colv{};
            }
#pragma unroll 8
            for (int d = 0; d < DK; ++d) {
                const rowv kr = rows(&S.KT[d][TR * ti]), qr = rows(&S.QT[d][TR * ti]);
                const colv ks = cols(&S.KT[d][s0]);
#pragma unroll
                for (int t = 0; t < TR; ++t)
#pragma unroll
                    for (int u = 0; u < TH; ++u) {
                        kk[t][u] = __builtin_fmaf(kr[t], ks[u], kk[t][u]);
                        qk[t][u] = __builtin_fmaf(qr[t], ks[u], qk[t][u]);
                    }
            }
#pragma unroll
            for (int t = 0; t < TR; ++t)
#pragma unroll
                for (int u = 0; u < TH; ++u) {
                    const int r = TR * ti + t, s = s0 + u;
                    const float dec = s <= r ? expf(S.gam[r] - S.gam[s]) : 0.0f;
                    S.A[r][(s & 3) * (kC / 4) + (s >> 2)] = s < r ? S.bt[r] * dec * kk[t][u] : 0.0f;
                    S.PT[s][r] = dec * qk[t][u];
                }
        }
        // Y = V - diag(exp gamma) K M0 on rows TR ti .., columns 2 tj, 2 tj + 1.
        {
            rowv x0 = rowv{};
#pragma unroll 8
            for (int d = 0; d < DK; ++d) {
                const rowv kr = rows(&S.KT[d][TR * ti]);
                const float m = S.M[d][vc];
#pragma unroll
                for (int t = 0; t < TR; ++t)
                    x0[t] = __builtin_fmaf(kr[t], m, x0[t]);
            }
#pragma unroll
            for (int t = 0; t < TR; ++t) {
                const int r = TR * ti + t;
                S.Y[r][vc] = S.V[r][vc] - S.eg[r] * x0[t];
            }
        }
        __syncthreads();

        // T = (I + A)^-1 column by column, x = (I + A)^-1 e_c by forward
        // substitution: x_r = [r == c] - sum_{s < r} A[r][s] x_s.  Four lanes
        // share column c: lane q of the quad sums the terms s = q, q + 4, ..
        // in order and keeps those x_s, and the quad adds its four partial
        // sums as (p0 + p1) + (p2 + p3) (the same value in every lane).  A's
        // residue-permuted rows make each lane's terms one run of 16-byte
        // words, read the same by every column (broadcast reads).  Column c
        // of T' = T diag(beta) is written as row c of TT.
        if (tid < 4 * kC) {
            constexpr int MQ = kC / 4;  // terms per lane
            const int c = tid >> 2, qd = tid & 3;
            float xq[MQ];
#pragma unroll
            for (int m = 0; m < MQ; ++m)
                xq[m] = 0.0f;
#pragma unroll
            for (int r = 0; r < kC; ++r) {
                // terms s = 4 m + qd < r: m < (r - qd + 3) / 4
                const int mq = (r - qd + 3) >> 2;
                float part = 0.0f;
#pragma unroll
                for (int u = 0; 4 * u < (r + 3) / 4; ++u) {
                    const float4 a4 = ld4(&S.A[r][qd * MQ + 4 * u]);
                    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (4 * u + i < (r + 3) / 4)
                            part = 4 * u + i < mq ? __builtin_fmaf(av[i], xq[4 * u + i], part) : part;
                }
                float sum = part + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                              0, __builtin_bit_cast(int, part), 0xB1, 0xF, 0xF, false));
                sum = sum + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                          0, __builtin_bit_cast(int, sum), 0x4E, 0xF, 0xF, false));
                const float acc = ((r == c) ? 1.0f : 0.0f) - sum;
                const float xr = (r < c) ? 0.0f : acc;
                if ((r & 3) == qd)
                    xq[r >> 2] = xr;
            }
            const float b = S.bt[c];
#pragma unroll
            for (int m = 0; m < MQ; ++m)
                S.TT[c][4 * m + qd] = xq[m] * b;
        }
        __syncthreads();

        // Delta = T' Y (into V's storage): row r sums s = 0 .. r in order.
        {
            rowv d0 = rowv{};
            for (int sb = 0; sb <= ti; ++sb) {
                rowv tt[TR];
                float y[TR];
#pragma unroll
                for (int u = 0; u < TR; ++u) {
                    tt[u] = rows(&S.TT[TR * sb + u][TR * ti]);
                    y[u] = S.Y[TR * sb + u][vc];
                }
#pragma unroll
                for (int u = 0; u < TR; ++u)
#pragma unroll
                    for (int t = 0; t < TR; ++t) {
                        const bool on = TR * sb + u <= TR * ti + t;
                        d0[t] = on ? __builtin_fmaf(tt[u][t], y[u], d0[t]) : d0[t];
                    }
            }
#pragma unroll
            for (int t = 0; t < TR; ++t)
                S.V[TR * ti + t][vc] = d0[t];
        }
        __syncthreads();
        // O = scale (diag(exp gamma) Q M0 + P Delta), rows of this chunk only.
        {
            rowv q0 = rowv{}, p0v = rowv{};
#pragma unroll 8
            for (int d = 0; d < DK; ++d) {
                const rowv qr = rows(&S.QT[d][TR * ti]);
                const float m = S.M[d][vc];
#pragma unroll
                for (int t = 0; t < TR; ++t)
                    q0[t] = __builtin_fmaf(qr[t], m, q0[t]);
            }
            for (int sb = 0; sb <= ti; ++sb) {
                rowv pr[TR];
                float dl[TR];
#pragma unroll
                for (int u = 0; u < TR; ++u) {
                    pr[u] = rows(&S.PT[TR * sb + u][TR * ti]);
                    dl[u] = S.V[TR * sb + u][vc];
                }
#pragma unroll
                for (int u = 0; u < TR; ++u)
#pragma unroll
                    for (int t = 0; t < TR; ++t) {
                        const bool on = TR * sb + u <= TR * ti + t;
                        p0v[t] = on ? __builtin_fmaf(pr[u][t], dl[u], p0v[t]) : p0v[t];
                    }
            }
#pragma unroll
            for (int t = 0; t < TR; ++t) {
                const int r = TR * ti + t;
                if (r < L)
                    o[((p + r) * a.Hv + j) * (int64_t)a.dv + c0 + vc] = a.scale * (S.eg[r] * q0[t] + p0v[t]);
            }
        }
        __syncthreads();
        // M_L = exp(gamma_L) M0 + K^T diag(exp(gamma_L - gamma)) Delta on keys
        // TD ti .., columns 2 tj, 2 tj + 1, summed over the rows in order.
        {
            const float eL = expf(S.gam[kC - 1]);
            float m0[TD];
#pragma unroll
            for (int t = 0; t < TD; ++t)
                m0[t] = 0.0f;
#pragma unroll 4
            for (int r = 0; r < kC; r += 4) {
                const float4 el4 = ld4(&S.el[r]);
                const float elv[4] = {el4.x, el4.y, el4.z, el4.w};
                float dl[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    dl[u] = S.V[r + u][vc];
#pragma unroll
                for (int t = 0; t < TD; ++t) {
                    const float4 k4 = ld4(&S.KT[TD * ti + t][r]);
                    const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        m0[t] = __builtin_fmaf(kv[u] * elv[u], dl[u], m0[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < TD; ++t) {
                float *mp = &S.M[TD * ti + t][vc];
                *mp = eL * *mp + m0[t];
            }
        }
    }
    __syncthreads();
    if (a.ht) {
        for (int e = tid; e < DK * kDVT; e += kThreads) {
            const int i = e / kDVT, c = e % kDVT;
            a.ht[hbase + (int64_t)i * a.dv + c0 + c] = S.M[i][c];
        }
    }
}

template <int DK>
hipError_t launch_dk(const FwdArgs &a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.n_seqs * a.Hv * (a.dv / kDVT);
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    const size_t smem = sizeof(SmemF32<DK>);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gdn_fwd_f32_kernel<DK>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(gdn_fwd_f32_kernel<DK>, dim3((unsigned)blocks), dim3(kThreads), smem,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream) {
    if (a.dk == 64)
        return launch_dk<64>(a, stream);
    if (a.dk == 256)
        return launch_dk<256>(a, stream);
    return launch_dk<128>(a, stream);
}

}  // namespace gdn

// Chunkwise gated delta rule forward, fp32 inputs, for gfx950.
//
// The same chunk equations as the bf16 kernel, evaluated entirely in fp32
// vector arithmetic (products, the triangular solve and the state), with the
// accurate expf.  fp32 inputs come with tolerances tighter than a bf16 MFMA
// path can meet, and the workloads that use them are small, so this kernel
// favours plainness: one workgroup per (sequence, value head, 32 value
// columns), every step an LDS-staged loop separated by barriers.  Chunks are
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
constexpr int kThreads = 256;

template <int DK>
constexpr int chunk_f32() {
    return DK == 256 ? 32 : 64;
}

template <int DK, int kC = chunk_f32<DK>()>
struct SmemF32 {
    float K[kC][DK + 1];
    float Q[kC][DK + 1];
    float V[kC][kDVT + 1];
    float M[DK][kDVT + 1];      // state slice
    alignas(16) float T[kC][kC + 4];  // A, then T' = (I + A)^-1 diag(beta); 16-byte rows
    float P[kC][kC + 1];        // (Q K^T) * D
    float Y[kC][kDVT + 1];      // V - diag(exp gamma) K M0, then Delta
    float gam[kC], bt[kC], el[kC];
};

template <int DK>
__global__ __launch_bounds__(kThreads) void gdn_fwd_f32_kernel(FwdArgs a) {
    constexpr int kC = chunk_f32<DK>();
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SmemF32<DK> &S = *reinterpret_cast<SmemF32<DK> *>(smem_raw);
    const int tid = threadIdx.x;
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

    for (int e = tid; e < DK * kDVT; e += kThreads) {
        const int i = e / kDVT, c = e % kDVT;
        S.M[i][c] = a.h0 ? a.h0[hbase + (int64_t)i * a.dv + c0 + c] : 0.0f;
    }

    for (int64_t p = p0; p < p1; p += kC) {
        const int L = (int)min<int64_t>(kC, p1 - p);
        __syncthreads();
        // Every load of the chunk is issued before any is stored, so their
        // latencies overlap instead of adding up.
        {
            constexpr int KPT = kC * DK / kThreads, VPT = kC * kDVT / kThreads;
            float kr[KPT], qr[KPT], vr[VPT];
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const int e = tid + kThreads * i, r = e / DK, d = e % DK;
                const int64_t off = ((p + r) * a.Hqk + hk) * DK + d;
                kr[i] = r < L ? k[off] : 0.0f;
                qr[i] = r < L ? q[off] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int e = tid + kThreads * i, r = e / kDVT, c = e % kDVT;
                vr[i] = r < L ? v[((p + r) * a.Hv + j) * (int64_t)a.dv + c0 + c] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const int e = tid + kThreads * i, r = e / DK, d = e % DK;
                S.K[r][d] = kr[i];
                S.Q[r][d] = qr[i];
            }
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int e = tid + kThreads * i, r = e / kDVT, c = e % kDVT;
                S.V[r][c] = vr[i];
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
            }
        }
        __syncthreads();
        if (a.flags & kStepL2Norm) {
            // In-op L2 normalisation: one wave per row of K or Q (fp32).
            const int lane = tid & 63;
            for (int row = tid >> 6; row < 2 * kC; row += kThreads / 64) {
                float *x = row < kC ? S.K[row] : S.Q[row - kC];
                float ss = 0.0f;
                for (int d = lane; d < DK; d += 64)
                    ss += x[d] * x[d];
                for (int o = 32; o >= 1; o >>= 1)
                    ss += __shfl_xor(ss, o);
                const float inv = inv_l2_norm(ss);
                for (int d = lane; d < DK; d += 64)
                    x[d] *= inv;
            }
            __syncthreads();
        }

        // A (strictly lower) and P (lower incl. diagonal).
        for (int e = tid; e < kC * kC; e += kThreads) {
            const int r = e / kC, s = e % kC;
            float kk = 0.0f, qk = 0.0f;
            if (s <= r) {
                for (int d = 0; d < DK; ++d) {
                    kk += S.K[r][d] * S.K[s][d];
                    qk += S.Q[r][d] * S.K[s][d];
                }
            }
            const float dec = s <= r ? expf(S.gam[r] - S.gam[s]) : 0.0f;
            S.T[r][s] = s < r ? S.bt[r] * dec * kk : 0.0f;
            S.P[r][s] = dec * qk;
        }
        // Y = V - diag(exp gamma) K M0
        for (int e = tid; e < kC * kDVT; e += kThreads) {
            const int r = e / kDVT, c = e % kDVT;
            float x = 0.0f;
            for (int d = 0; d < DK; ++d)
                x += S.K[r][d] * S.M[d][c];
            S.Y[r][c] = S.V[r][c] - expf(S.gam[r]) * x;
        }
        __syncthreads();

        // T = (I + A)^-1 column by column: thread c of wave 0 solves column c
        // by forward substitution, reading only A (every thread reads the
        // same A[r][s]: broadcast reads); T' = T diag(beta) replaces A after
        // the barrier.  The loops are unrolled so x stays in registers; its
        // entries above the diagonal are zero, so the sums can start at 0.
        // Each row's sum runs in four interleaved partial sums over 16-byte
        // reads of the row, so the loads and the multiply-adds pipeline.
        float x[kC];
        if (tid < kC) {
            const int c = tid;
#pragma unroll
            for (int r = 0; r < kC; ++r) {
                float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s4 = 0; 4 * s4 < r; ++s4) {
                    const float4 a4 = *reinterpret_cast<const float4 *>(&S.T[r][4 * s4]);
                    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (4 * s4 + i < r)
                            part[i] = __builtin_fmaf(av[i], x[4 * s4 + i], part[i]);
                }
                const float acc = ((r == c) ? 1.0f : 0.0f) - ((part[0] + part[1]) + (part[2] + part[3]));
                x[r] = (r < c) ? 0.0f : acc;
            }
        }
        __syncthreads();
        if (tid < kC)
#pragma unroll
            for (int r = 0; r < kC; ++r)
                S.T[r][tid] = x[r] * S.bt[tid];
        __syncthreads();

        // Delta = T' Y (into V's storage), then the output and the state.
        for (int e = tid; e < kC * kDVT; e += kThreads) {
            const int r = e / kDVT, c = e % kDVT;
            float acc = 0.0f;
            for (int s = 0; s <= r; ++s)
                acc += S.T[r][s] * S.Y[s][c];
            S.V[r][c] = acc;
        }
        __syncthreads();
        for (int e = tid; e < kC * kDVT; e += kThreads) {
            const int r = e / kDVT, c = e % kDVT;
            if (r >= L)
                continue;
            float qm = 0.0f;
            for (int d = 0; d < DK; ++d)
                qm += S.Q[r][d] * S.M[d][c];
            float pd = 0.0f;
            for (int s = 0; s <= r; ++s)
                pd += S.P[r][s] * S.V[s][c];
            o[((p + r) * a.Hv + j) * (int64_t)a.dv + c0 + c] = a.scale * (expf(S.gam[r]) * qm + pd);
        }
        __syncthreads();
        const float gL = S.gam[kC - 1];
        for (int e = tid; e < DK * kDVT; e += kThreads) {
            const int d = e / kDVT, c = e % kDVT;
            float acc = 0.0f;
            for (int r = 0; r < kC; ++r)
                acc += S.K[r][d] * S.el[r] * S.V[r][c];
            S.M[d][c] = expf(gL) * S.M[d][c] + acc;
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

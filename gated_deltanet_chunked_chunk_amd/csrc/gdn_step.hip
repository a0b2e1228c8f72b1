// Single-token recurrent step (decode) and the in-op input preparation of
// the gated delta rule, for gfx950.
//
// The recurrent step advances each sequence's state by one token, the
// token-by-token form the jax-linear-attention page lists next to the chunked
// one ("How it works"), used for decoding one token at a time:
//
//     y = M^T k,  delta = beta (v - a y),  M <- a M + k delta^T,  o = scale M^T q
//
// with M = S^T the fp32 [dk][dv] state and a = exp(g).  The step is bound by
// HBM: it reads and writes the whole state once.  One workgroup of 256
// threads owns (sequence, value head, 64 value columns).  Each lane moves 16
// bytes (4 columns) of a state row per access, so a wave touches four 256-byte
// row segments per instruction; the partial products of y and o are summed
// over the lanes and waves that share a column.
//
// The preparation is the in-op option of the "Quick start" call on the same
// page (q and k divided by their L2 norms inside the op) and the gate
// activations its example applies to raw gate values (g = logsigmoid(raw),
// beta = sigmoid(raw)); the norms are taken in fp32 and the normalised rows
// stored back in the input dtype.  Rows whose size is a power-of-two number
// of 16-byte pieces are spread over that many lanes, several rows in flight
// per wave; other sizes take one wave per row.
//
// The reverse of the preparation, with the same row layout: for y = x / n,
// n = ||x||, dx = (dy - (dy . y) y) / n (a zero row gets zero); for the gates
// d logsigmoid(x) = sigmoid(-x) and d sigmoid(x) = sigmoid(x) sigmoid(-x).
// Both row sums (x . x and dy . x) come from one read of the two rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ __forceinline__ float load_el(const void *p, int64_t i, bool bf16) {
    if (bf16)
        return __uint_as_float(static_cast<unsigned>(static_cast<const uint16_t *>(p)[i]) << 16);
    return static_cast<const float *>(p)[i];
}

__device__ __forceinline__ void store_el(void *p, int64_t i, float x, bool bf16) {
    if (bf16)
        static_cast<uint16_t *>(p)[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
    else
        static_cast<float *>(p)[i] = x;
}

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(a)) |
           (unsigned)__builtin_bit_cast(uint16_t, static_cast<__bf16>(b)) << 16;
}

// Four consecutive elements (8 bytes of bf16 or 16 of fp32) as fp32.
__device__ __forceinline__ f32x4 load4(const void *p, int64_t i, bool bf16) {
    if (bf16) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(p) + i);
        return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
    }
    return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(p) + i);
}

__device__ __forceinline__ void store4(void *p, int64_t i, f32x4 x, bool bf16) {
    if (bf16)
        *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p) + i) =
            u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    else
        *reinterpret_cast<f32x4 *>(static_cast<float *>(p) + i) = x;
}

// Sum over the four lanes l, l + 16, l + 32, l + 48 of a wave.
__device__ __forceinline__ f32x4 sum_row_quads(f32x4 x) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        x[c] += __shfl_xor(x[c], 16);
        x[c] += __shfl_xor(x[c], 32);
    }
    return x;
}

template <int DK>
__global__ __launch_bounds__(256) void recurrent_step(StepArgs a) {
    __shared__ float ks[DK], qs[DK], nrm[2];
    __shared__ f32x4 ypart[4][16], opart[4][16];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int cg = lane & 15, rq = lane >> 4;  // 4-column group; row within the wave's four
    const int n_tiles = a.dv / 64;
    const int tile = blockIdx.x % n_tiles;
    const int j = (blockIdx.x / n_tiles) % a.Hv;
    const int64_t n = blockIdx.x / (n_tiles * a.Hv);
    const int hk = j / (a.Hv / a.Hqk);
    const bool bf = a.bf16;
    const int64_t qk_row = (n * a.Hqk + hk) * (int64_t)DK;
    if (tid < DK) {
        ks[tid] = load_el(a.k, qk_row + tid, bf);
        qs[tid] = load_el(a.q, qk_row + tid, bf);
    }
    __syncthreads();
    if (a.flags & kStepL2Norm) {
        // Wave 0 reduces k, wave 1 reduces q.
        if (w < 2) {
            const float *x = w == 0 ? ks : qs;
            float s = 0.0f;
            for (int i = lane; i < DK; i += 64)
                s += x[i] * x[i];
            for (int o = 32; o >= 1; o >>= 1)
                s += __shfl_xor(s, o);
            if (lane == 0)
                nrm[w] = inv_l2_norm(s);
        }
        __syncthreads();
        if (tid < DK) {
            ks[tid] *= nrm[0];
            qs[tid] *= nrm[1];
        }
        __syncthreads();
    }
    float gv = a.g[n * a.Hv + j], bv = a.beta[n * a.Hv + j];
    if (a.flags & kStepGateAct) {
        gv = logsigmoid_f32(gv);
        bv = sigmoid_f32(bv);
    }
    const float av = expf(gv);
    // The sequence's cache slot (uniform over the workgroup); one out of range
    // starts from a zero state and keeps nothing.
    const int64_t slot = a.slots ? (int64_t)__builtin_amdgcn_readfirstlane(a.slots[n]) : n;
    const bool cached = slot >= 0 && slot < a.n_slots;
    const int col = tile * 64 + 4 * cg;
    // This lane's rows: 16 it + 4 w + rq, it < DK / 16.
    constexpr int R = DK / 16;
    const int row0 = 4 * w + rq;
    const int rs4 = a.dv / 4;  // f32x4 per state row
    f32x4 *st = reinterpret_cast<f32x4 *>(
        a.state + ((cached ? slot : 0) * a.Hv + j) * (int64_t)DK * a.dv + col) + row0 * rs4;
    f32x4 m[R];
    if (cached) {
#pragma unroll
        for (int it = 0; it < R; ++it)
            m[it] = st[16 * it * rs4];
    } else {
#pragma unroll
        for (int it = 0; it < R; ++it)
            m[it] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < R; ++it)
        y += m[it] * ks[row0 + 16 * it];
    y = sum_row_quads(y);
    if (rq == 0)
        ypart[w][cg] = y;
    __syncthreads();
    y = ypart[0][cg] + ypart[1][cg] + ypart[2][cg] + ypart[3][cg];
    const int64_t vo = (n * a.Hv + j) * (int64_t)a.dv + col;
    const f32x4 delta = bv * (load4(a.v, vo, bf) - av * y);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < R; ++it) {
        m[it] = av * m[it] + ks[row0 + 16 * it] * delta;
        o += m[it] * qs[row0 + 16 * it];
    }
    if (cached) {
#pragma unroll
        for (int it = 0; it < R; ++it)
            st[16 * it * rs4] = m[it];
    }
    o = sum_row_quads(o);
    if (rq == 0)
        opart[w][cg] = o;
    __syncthreads();
    if (w == 0 && rq == 0)
        store4(a.o, vo, a.scale * (opart[0][cg] + opart[1][cg] + opart[2][cg] + opart[3][cg]),
               bf);
}

// Rows of q and k divided by their L2 norms, one wave per row (any dk up to
// 256), and the gate activations.
__global__ __launch_bounds__(256) void preprocess(PrepArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const bool bf = a.bf16;
    if (wave < 2 * a.qk_rows && (a.flags & kStepL2Norm)) {
        const bool isq = wave >= a.qk_rows;
        const int64_t row = isq ? wave - a.qk_rows : wave;
        const void *src = isq ? a.q : a.k;
        void *dst = isq ? a.q_out : a.k_out;
        float x[4], s = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = lane + 64 * u;
            x[u] = i < a.dk ? load_el(src, row * a.dk + i, bf) : 0.0f;
            s += x[u] * x[u];
        }
        for (int o = 32; o >= 1; o >>= 1)
            s += __shfl_xor(s, o);
        const float inv = inv_l2_norm(s);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = lane + 64 * u;
            if (i < a.dk)
                store_el(dst, row * a.dk + i, x[u] * inv, bf);
        }
    }
    if (a.flags & kStepGateAct) {
        const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
        if (i < a.gate_n) {
            a.g_out[i] = logsigmoid_f32(a.g[i]);
            a.beta_out[i] = sigmoid_f32(a.beta[i]);
        }
    }
}

// The same with 16-byte pieces: a row of Lpr pieces (8 bf16 or 4 fp32 each)
// on Lpr consecutive lanes, 64 / Lpr rows per wave and kPrepGroups such
// groups per wave, all loaded before any is reduced.
constexpr int kPrepGroups = 4;

template <int Lpr, bool Bf16>
__global__ __launch_bounds__(256) void preprocess_vec(PrepArgs a) {
    constexpr int kRowsPerWave = 64 / Lpr;
    constexpr int kPer = Bf16 ? 8 : 4;  // elements per lane
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (a.flags & kStepL2Norm) {
        const int64_t total = 2 * a.qk_rows;
        u32x4 x[kPrepGroups];
        int64_t rows[kPrepGroups];
#pragma unroll
        for (int u = 0; u < kPrepGroups; ++u) {
            rows[u] = (wave * kPrepGroups + u) * kRowsPerWave + lane / Lpr;
            if (rows[u] < total) {
                const bool isq = rows[u] >= a.qk_rows;
                const int64_t r = isq ? rows[u] - a.qk_rows : rows[u];
                const u32x4 *src = reinterpret_cast<const u32x4 *>(isq ? a.q : a.k);
                x[u] = src[r * Lpr + lane % Lpr];
            } else {
                x[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < kPrepGroups; ++u) {
            float f[kPer];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (Bf16) {
                    f[2 * e] = __uint_as_float(x[u][e] << 16);
                    f[2 * e + 1] = __uint_as_float(x[u][e] & 0xffff0000u);
                } else {
                    f[e] = __uint_as_float(x[u][e]);
                }
            }
            float s = 0.0f;
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                s = fmaf(f[e], f[e], s);
#pragma unroll
            for (int o = Lpr / 2; o >= 1; o >>= 1)
                s += __shfl_xor(s, o);
            const float inv = inv_l2_norm(s);
            u32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                y[e] = Bf16 ? pack_bf16x2(f[2 * e] * inv, f[2 * e + 1] * inv)
                            : __float_as_uint(f[e] * inv);
            if (rows[u] < total) {
                const bool isq = rows[u] >= a.qk_rows;
                const int64_t r = isq ? rows[u] - a.qk_rows : rows[u];
                u32x4 *dst = reinterpret_cast<u32x4 *>(isq ? a.q_out : a.k_out);
                dst[r * Lpr + lane % Lpr] = y;
            }
        }
    }
    if (a.flags & kStepGateAct) {
        const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
        if (i < a.gate_n) {
            a.g_out[i] = logsigmoid_f32(a.g[i]);
            a.beta_out[i] = sigmoid_f32(a.beta[i]);
        }
    }
}

// Reverse of the gate activations, one gate per thread.
__device__ __forceinline__ void gates_bwd(const PrepBwdArgs &a, int64_t i) {
    if (i < a.gate_n) {
        const float b = a.beta[i];
        a.dg_out[i] = a.dg[i] * sigmoid_f32(-a.g[i]);
        a.dbeta_out[i] = a.dbeta[i] * (sigmoid_f32(b) * sigmoid_f32(-b));
    }
}

// Gradient of one normalised row: with inv = 1 / n and p = (dy . x) inv, the
// projection dy . y, dx = inv (dy - p inv x).
__device__ __forceinline__ float l2_bwd_el(float x, float dy, float inv, float p) {
    return inv * fmaf(-p * inv, x, dy);
}

// One wave per row (any dk up to 256).
__global__ __launch_bounds__(256) void preprocess_bwd(PrepBwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const bool bf = a.bf16;
    if (wave < 2 * a.qk_rows && (a.flags & kStepL2Norm)) {
        const bool isq = wave >= a.qk_rows;
        const int64_t row = isq ? wave - a.qk_rows : wave;
        const void *xs = isq ? a.q : a.k;
        const void *ds = isq ? a.dq : a.dk;
        void *dst = isq ? a.dq_out : a.dk_out;
        float x[4], d[4], s = 0.0f, t = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = lane + 64 * u;
            x[u] = i < a.dk_dim ? load_el(xs, row * a.dk_dim + i, bf) : 0.0f;
            d[u] = i < a.dk_dim ? load_el(ds, row * a.dk_dim + i, bf) : 0.0f;
            s = fmaf(x[u], x[u], s);
            t = fmaf(d[u], x[u], t);
        }
        for (int o = 32; o >= 1; o >>= 1) {
            s += __shfl_xor(s, o);
            t += __shfl_xor(t, o);
        }
        const float inv = inv_l2_norm(s);
        const float p = t * inv;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = lane + 64 * u;
            if (i < a.dk_dim)
                store_el(dst, row * a.dk_dim + i, l2_bwd_el(x[u], d[u], inv, p), bf);
        }
    }
    if (a.flags & kStepGateAct)
        gates_bwd(a, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// 16-byte pieces, as preprocess_vec: a row on Lpr lanes, kPrepGroups groups
// of rows per wave with all of their loads issued before any reduction.
template <int Lpr, bool Bf16>
__global__ __launch_bounds__(256) void preprocess_bwd_vec(PrepBwdArgs a) {
    constexpr int kRowsPerWave = 64 / Lpr;
    constexpr int kPer = Bf16 ? 8 : 4;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (a.flags & kStepL2Norm) {
        const int64_t total = 2 * a.qk_rows;
        u32x4 x[kPrepGroups], d[kPrepGroups];
        int64_t rows[kPrepGroups];
#pragma unroll
        for (int u = 0; u < kPrepGroups; ++u) {
            rows[u] = (wave * kPrepGroups + u) * kRowsPerWave + lane / Lpr;
            if (rows[u] < total) {
                const bool isq = rows[u] >= a.qk_rows;
                const int64_t r = isq ? rows[u] - a.qk_rows : rows[u];
                const int64_t at = r * Lpr + lane % Lpr;
                x[u] = reinterpret_cast<const u32x4 *>(isq ? a.q : a.k)[at];
                d[u] = reinterpret_cast<const u32x4 *>(isq ? a.dq : a.dk)[at];
            } else {
                x[u] = u32x4{0u, 0u, 0u, 0u};
                d[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < kPrepGroups; ++u) {
            float fx[kPer], fd[kPer];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (Bf16) {
                    fx[2 * e] = __uint_as_float(x[u][e] << 16);
                    fx[2 * e + 1] = __uint_as_float(x[u][e] & 0xffff0000u);
                    fd[2 * e] = __uint_as_float(d[u][e] << 16);
                    fd[2 * e + 1] = __uint_as_float(d[u][e] & 0xffff0000u);
                } else {
                    fx[e] = __uint_as_float(x[u][e]);
                    fd[e] = __uint_as_float(d[u][e]);
                }
            }
            float s = 0.0f, t = 0.0f;
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                s = fmaf(fx[e], fx[e], s);
                t = fmaf(fd[e], fx[e], t);
            }
#pragma unroll
            for (int o = Lpr / 2; o >= 1; o >>= 1) {
                s += __shfl_xor(s, o);
                t += __shfl_xor(t, o);
            }
            const float inv = inv_l2_norm(s);
            const float p = t * inv;
            u32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                y[e] = Bf16 ? pack_bf16x2(l2_bwd_el(fx[2 * e], fd[2 * e], inv, p),
                                          l2_bwd_el(fx[2 * e + 1], fd[2 * e + 1], inv, p))
                            : __float_as_uint(l2_bwd_el(fx[e], fd[e], inv, p));
            if (rows[u] < total) {
                const bool isq = rows[u] >= a.qk_rows;
                const int64_t r = isq ? rows[u] - a.qk_rows : rows[u];
                reinterpret_cast<u32x4 *>(isq ? a.dq_out : a.dk_out)[r * Lpr + lane % Lpr] = y;
            }
        }
    }
    if (a.flags & kStepGateAct)
        gates_bwd(a, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// Blocks of 256 threads covering `rows` rows at `rows_per_block` and the
// gates at one per thread; 0 when there is nothing to do, -1 past the grid.
int64_t prep_blocks(int64_t rows, int64_t rows_per_block, int64_t gates) {
    const int64_t by_rows = (rows + rows_per_block - 1) / rows_per_block;
    const int64_t by_gates = (gates + 255) / 256;
    const int64_t blocks = by_rows > by_gates ? by_rows : by_gates;
    return blocks > 0x7fffffff ? -1 : blocks;
}

template <int Lpr, bool Bf16>
hipError_t launch_bwd_vec(const PrepBwdArgs &a, hipStream_t stream) {
    const int64_t rows = (a.flags & kStepL2Norm) ? 2 * a.qk_rows : 0;
    const int64_t gates = (a.flags & kStepGateAct) ? a.gate_n : 0;
    const int64_t blocks = prep_blocks(rows, 4 * kPrepGroups * (64 / Lpr), gates);
    if (blocks == 0)
        return hipSuccess;
    if (blocks < 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((preprocess_bwd_vec<Lpr, Bf16>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

template <int Lpr, bool Bf16>
hipError_t launch_vec(const PrepArgs &a, hipStream_t stream) {
    constexpr int64_t kRowsPerBlock = 4 * kPrepGroups * (64 / Lpr);
    const int64_t by_rows = (2 * a.qk_rows + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t by_gates = (a.gate_n + 255) / 256;
    const int64_t blocks = by_rows > by_gates ? by_rows : by_gates;
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((preprocess_vec<Lpr, Bf16>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_recurrent_step(const StepArgs &a, hipStream_t stream) {
    const int64_t blocks = a.N * a.Hv * (a.dv / 64);
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    if (a.dk == 128)
        hipLaunchKernelGGL(recurrent_step<128>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else if (a.dk == 64)
        hipLaunchKernelGGL(recurrent_step<64>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else if (a.dk == 256)
        hipLaunchKernelGGL(recurrent_step<256>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_preprocess(const PrepArgs &a, hipStream_t stream) {
    // 16-byte pieces per row, when the row is a power-of-two number of them.
    const int row_bytes = a.dk * (a.bf16 ? 2 : 4);
    const int lpr = row_bytes % 16 == 0 ? row_bytes / 16 : 0;
    if (a.bf16) {
        switch (lpr) {
        case 4: return launch_vec<4, true>(a, stream);
        case 8: return launch_vec<8, true>(a, stream);
        case 16: return launch_vec<16, true>(a, stream);
        case 32: return launch_vec<32, true>(a, stream);
        }
    } else {
        switch (lpr) {
        case 4: return launch_vec<4, false>(a, stream);
        case 8: return launch_vec<8, false>(a, stream);
        case 16: return launch_vec<16, false>(a, stream);
        case 32: return launch_vec<32, false>(a, stream);
        case 64: return launch_vec<64, false>(a, stream);
        }
    }
    const int64_t by_rows = (2 * a.qk_rows + 3) / 4;
    const int64_t by_gates = (a.gate_n + 255) / 256;
    const int64_t blocks = by_rows > by_gates ? by_rows : by_gates;
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(preprocess, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_preprocess_bwd(const PrepBwdArgs &a, hipStream_t stream) {
    const int row_bytes = a.dk_dim * (a.bf16 ? 2 : 4);
    const int lpr = row_bytes % 16 == 0 ? row_bytes / 16 : 0;
    if (a.bf16) {
        switch (lpr) {
        case 4: return launch_bwd_vec<4, true>(a, stream);
        case 8: return launch_bwd_vec<8, true>(a, stream);
        case 16: return launch_bwd_vec<16, true>(a, stream);
        case 32: return launch_bwd_vec<32, true>(a, stream);
        }
    } else {
        switch (lpr) {
        case 4: return launch_bwd_vec<4, false>(a, stream);
        case 8: return launch_bwd_vec<8, false>(a, stream);
        case 16: return launch_bwd_vec<16, false>(a, stream);
        case 32: return launch_bwd_vec<32, false>(a, stream);
        case 64: return launch_bwd_vec<64, false>(a, stream);
        }
    }
    const int64_t rows = (a.flags & kStepL2Norm) ? 2 * a.qk_rows : 0;
    const int64_t gates = (a.flags & kStepGateAct) ? a.gate_n : 0;
    const int64_t blocks = prep_blocks(rows, 4, gates);
    if (blocks == 0)
        return hipSuccess;
    if (blocks < 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(preprocess_bwd, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gdn

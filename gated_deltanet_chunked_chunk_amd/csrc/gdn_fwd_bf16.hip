// Chunkwise gated delta rule forward, bf16 inputs, for gfx950.  The
// description below is for dk = 128; dk = 64 stages its rows into the same
// 128-wide layout, and dk = 256 walks chunks of 32 tokens laid into it (see
// chunk_len).
//
// One workgroup owns one (sequence, value head, 64-column value tile) and
// walks the sequence's chunks of 64 tokens in order.  Value columns of the
// state evolve independently (every step of the recurrence acts on them
// column by column), so splitting dv across workgroups is exact.
//
// The workgroup has eight waves in two roles, one of each on every SIMD:
//   state waves 0..3   wave s owns value columns [16s, 16s + 16) and keeps
//                      its [128 x 16] slice of the fp32 state M = S^T in MFMA
//                      accumulators for the whole sequence; per chunk it runs
//                      the state-dependent steps (a5)-(a7).
//   helper waves 4..7  prepare the next chunk while the state waves work on
//                      the current one: all four stage K, Q, V and the gates
//                      from HBM into LDS; helper 3 forms the cumulative decay
//                      (a2); helpers 1..3 the off-diagonal blocks of K K^T
//                      and Q K^T (a3); helper 0 the diagonal blocks and their
//                      inverses (a4).
// Chunk c is read from LDS buffer c % 2 while chunk c + 1 is written into the
// other, and one LDS-only workgroup barrier per chunk hands the buffers over.
// The helper waves meet once more among themselves per chunk (an LDS
// counter) between staging and the products that read the staged rows.
//
// The Prep instance also applies the in-op preparation options as the
// helpers stage a chunk: the gate activations, and the q/k rows' inverse L2
// norms, applied as fp32 factors in the blocks and the decay tables (the
// rows themselves are never rescaled).
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
// formed explicitly (fp32 forward substitution; one helper wave does all
// four, one 16-lane row per block).
//
// Precision: K, Q, V are exact bf16 and every product accumulates in fp32.
// Computed operands on the state chain (D_i, A_ij, the right-hand sides,
// Delta and Delta') enter the MFMA as hi + lo bf16 pairs (x = hi + lo,
// hi = bf16(x), lo = bf16(x - hi); split-bfloat16, Henry, Tang & Heinecke,
// ARITH 2019).  In the block substitution a split product A x takes two
// 32-deep MFMAs whose A operand holds A's (hi | lo) halves, one against
// (x_hi | x_hi) and one against (x_lo | x_lo), so all four hi/lo terms are
// summed with no zero padding.  Q M0 and P Delta feed only the output and
// use hi parts, well inside its tolerance.  K M0 uses the hi part of M0 at
// dk = 128 and 256 and hi + lo at dk = 64.  A hi-only M0 there puts a
// relative error of about 2^-9 into every chunk's right-hand side, which the
// state keeps for about 1 / (1 - a) tokens; a chunk of 64 keys spans the whole
// key space at dk = 64 (half of it at dk = 128), so that is where, under slow
// decay, the error nears the state tolerance.  The low part costs the 128-key
// kernel about 7% of its time, which is why it is not taken there.
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
//
// Global loads are raw buffer loads whose range ends at the chunk's last
// valid row, so rows past the end of a sequence read as zeros (zero k, q,
// v, g and beta: they contribute nothing) without branches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kC = 64;          // chunk length
constexpr int kDK = 128;        // key dimension
constexpr int kDVT = 64;        // value columns per workgroup
constexpr int kThreads = 512;   // 4 state waves + 4 helper waves
// LDS is 64 banks of 4 bytes, 256 bytes per cycle.  Measured on gfx950 with
// the bank-conflict counter: a 16-byte-per-lane access serves 16 lanes per
// cycle, those of one half-wave with equal parity of lane bits 2..4; an
// 8-byte access serves 32 lanes per cycle.  Row strides of the padded tiles are 4 (mod 8)
// 4-byte words, so that the 8-byte fragment reads (16 rows x 2 column groups
// per cycle) fall in distinct banks.
constexpr int kSP = kC + 8;     // P
constexpr int kSN = 48 + 8;     // -A (rows 16..63, columns 0..47)
constexpr int kSDT = 16;        // D blocks, transposed (one 32-byte row per column)
constexpr int kAD = 20;         // column stride of the helpers' A_ii copies (conflict-free column reads)
constexpr unsigned kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit elements
constexpr float kLog2e = 1.44269504088896341f;

// Tokens per chunk.  With dk = 256 a chunk is 32 tokens, and the two key
// halves of its rows take the places of rows 0..31 and 32..63 of the
// 64 x 128 K and Q tiles: key 128 h + x of row r is column x of tile row
// 32 h + r.  Every tile layout, fragment read and LDS size stays as it is.
template <int DK>
constexpr int chunk_len() {
    return DK == 256 ? 32 : kC;
}
// Accumulator tiles of the state slice (16 keys each).
template <int DK>
constexpr int state_tiles() {
    return DK == 256 ? 16 : 8;
}

// K, Q (64 x 128) and V (64 x 64) tiles are unpadded, with the pieces of each
// row permuted.  A K or Q row is 256 bytes, one bank cycle: its 16-byte slot c
// is stored at slot c ^ sigma(r), where sigma permutes the bits of r % 16
// (bits 0, 1, 2, 3 of r become bits 0, 2, 3, 1).  Then MFMA fragment reads
// (16 rows, slot 4 kk + lane group) are conflict-free for the lanes served
// together, and the transpose reads of K (8 rows x 4 half-slots at the same
// offset) meet at most two to a bank.  A V row is 128 bytes: its 8-byte chunk
// c is stored at c ^ 4 ((r / 2) % 4), which makes the transpose reads (8 rows
// x 4 chunks) conflict-free.
__device__ __forceinline__ int sig_kq(int row) {
    return (row & 1) | ((row >> 2) & 2) | ((row & 2) << 1) | ((row & 4) << 1);
}
__device__ __forceinline__ int kq_slot(int row, int slot) {  // element offset of a 16-byte slot
    return row * kDK + ((slot ^ sig_kq(row & 15)) << 3);
}
__device__ __forceinline__ int v_at(int row, int chunk) {  // element offset of an 8-byte chunk
    return row * kDVT + ((chunk ^ (((row >> 1) & 3) << 2)) << 2);
}

// The fp32 state is kept with its key rows permuted: accumulator tile mt, row
// 4g + r holds key dimension pi(16 mt + 4g + r) = 32 (mt / 2) + 8 g + 4 (mt % 2)
// + r.  Then the two stacked accumulator tiles 2k, 2k+1 of lane group g hold
// key dims 32 k + 8 g .. + 7 in order: the B operand of K M0 in natural k order.
__device__ __forceinline__ int key_of(int mt, int g, int r) {
    return 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + r;
}

// One chunk's worth of shared operands.
struct alignas(16) ChunkBuf {
    uint16_t K[kC * kDK];       // K rows, [row][dk], chunks permuted
    uint16_t Q[kC * kDK];       // Q rows, [row][dk], chunks permuted
    uint16_t V[kC * kDVT];      // value tile, [row][col], chunks permuted
    uint16_t P[kC * kSP];       // P, lower 16-blocks (upper blocks stay zero)
    uint16_t Anh[48 * kSN];     // -A hi, row r - 16, blocks below the diagonal
    uint16_t Anl[48 * kSN];     // -A lo
    uint16_t DhT[kC * kSDT];    // D_i^T hi: row 16 i + c is column c of D_i
    uint16_t DlT[kC * kSDT];    // D_i^T lo
    float gam[kC];              // gamma_r log2(e): the decay factors are exp2 of differences
    float eg[kC];               // exp(gamma_r)
    float el[kC];               // exp(gamma_L - gamma_r)
    float bt[kC];               // beta_r
    float nu[kC];               // in-op L2 norm: 1 / ||k_r|| (Prep instance only)
    float mu[kC];               // in-op L2 norm: 1 / ||q_r|| (Prep instance only)
    float egq[kC];              // exp(gamma_r) mu_r (Prep instance only)
    float eL;                   // exp(gamma_L)
    float pad_[3];
};

// The fixed-address parts first: below 64 KiB their addresses fit the
// immediate offset of LDS instructions.
struct alignas(16) Smem {
    float Ad[4][16 * kAD];      // -A_ii of the diagonal blocks, column-major (helpers 1..3 write, 0 reads)
    uint16_t Ost[4][16 * kC];   // state wave s: output staging, [col][row], words permuted
    int hsync;                  // helper-wave meeting counter
    int dsync;                  // diagonal blocks written (helpers 1..3, three per chunk)
    ChunkBuf buf[2];
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

// Fragment addressing in a slot-permuted K or Q tile.  A fragment of row
// 16 m + lr, k-step kk is the 16-byte slot 4 kk + lg (key dims 32 kk + 8 lg ..
// + 7).  The permutation of rows 16 m + lr depends on lr only, and the slot
// index 4 kk + lg = 4 kk ^ lg, so the element offset is base ^ (32 kk) with
// base the offset of slot lg: the fragment is at t + 2048 m + (base ^ 32 kk).
struct KqBase {
    int b;
};

// The base is passed through an empty asm so that the four XORed offsets are
// formed where they are used instead of being hoisted out of the chunk loop
// and kept live through it.
__device__ __forceinline__ KqBase kq_base(int lr, int lg) {
    int b = kq_slot(lr, lg);
    asm volatile("" : "+v"(b));
    return KqBase{b};
}

__device__ __forceinline__ bf16x8 frag_kq(const uint16_t *t, const KqBase &kb, int m, int kk) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(t + 2048 * m + (kb.b ^ (32 * kk))));
}

// Transpose read of 4 bf16 (see the file comment).
__device__ __forceinline__ u32x2 ld_tr(const uint16_t *p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

// A packed bf16 pair held in an SGPR.  Used for the constant operands of
// v_dot2c_f32_bf16: given as a compile-time constant, (-1, 0) is encoded as
// the inline constant -1.0, which the hardware reads as the fp32 bit pattern
// 0xbf800000, i.e. the pair (0, -1).
template <unsigned V>
__device__ __forceinline__ bf16x2 packed_bf16_sgpr() {
    unsigned r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(V));
    return __builtin_bit_cast(bf16x2, r);
}

// Four fp32 values as 4 bf16 (hi, round to nearest even) and the rounding
// residuals as 4 bf16 (lo).  x - hi is exact in fp32; it is formed by a bf16
// dot product of the packed pair with (-1, 0) or (0, -1) accumulated onto x.
__device__ __forceinline__ void split4(f32x4 x, u32x2 &hi, u32x2 &lo) {
    const bf16x2 h01 = {static_cast<__bf16>(x[0]), static_cast<__bf16>(x[1])};
    const bf16x2 h23 = {static_cast<__bf16>(x[2]), static_cast<__bf16>(x[3])};
    const bf16x2 m0 = packed_bf16_sgpr<0x0000bf80u>();  // (-1, 0)
    const bf16x2 m1 = packed_bf16_sgpr<0xbf800000u>();  // (0, -1)
    const bf16x2 l01 = {static_cast<__bf16>(__builtin_amdgcn_fdot2_f32_bf16(h01, m0, x[0], false)),
                        static_cast<__bf16>(__builtin_amdgcn_fdot2_f32_bf16(h01, m1, x[1], false))};
    const bf16x2 l23 = {static_cast<__bf16>(__builtin_amdgcn_fdot2_f32_bf16(h23, m0, x[2], false)),
                        static_cast<__bf16>(__builtin_amdgcn_fdot2_f32_bf16(h23, m1, x[3], false))};
    hi = u32x2{__builtin_bit_cast(unsigned, h01), __builtin_bit_cast(unsigned, h23)};
    lo = u32x2{__builtin_bit_cast(unsigned, l01), __builtin_bit_cast(unsigned, l23)};
}

__device__ __forceinline__ u32x2 pack4(f32x4 x) {
    const bf16x2 h01 = {static_cast<__bf16>(x[0]), static_cast<__bf16>(x[1])};
    const bf16x2 h23 = {static_cast<__bf16>(x[2]), static_cast<__bf16>(x[3])};
    return u32x2{__builtin_bit_cast(unsigned, h01), __builtin_bit_cast(unsigned, h23)};
}

constexpr u32x2 kZero2 = {0u, 0u};

// K = 16 product: lane l supplies A[l%16][4(l/16)+j] and B[4(l/16)+j][l%16]
// (j = 0..3), the rows 4g..4g+3 a C-layout tile gives lane group g.
__device__ __forceinline__ f32x4 mma16(u32x2 a, u32x2 b, f32x4 c) {
    return mma(cat(a, kZero2), cat(b, kZero2), c);
}

__device__ __forceinline__ f32x4 ld4f(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}

template <int Ctrl, int RowMask>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl, RowMask, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes (row_shr within rows of 16, then
// row_bcast:15 and row_bcast:31 across rows).
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp<0x111, 0xF>(x);
    x += dpp<0x112, 0xF>(x);
    x += dpp<0x114, 0xF>(x);
    x += dpp<0x118, 0xF>(x);
    x += dpp<0x142, 0xA>(x);
    x += dpp<0x143, 0xC>(x);
    return x;
}

// Sum over the 16 lanes of a DPP row: quad xor 1, quad xor 2, the half-row
// mirror (quad against quad), the row mirror (half against half).
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1, 0xF>(x);
    x += dpp<0x4E, 0xF>(x);
    x += dpp<0x141, 0xF>(x);
    x += dpp<0x140, 0xF>(x);
    return x;
}

// In-op L2 norm of a staged q or k row: the 16 lanes of a DPP row hold its
// 128 bf16 values, 8 each; returns 1 / ||row|| (fp32) in every lane of the
// row.  The rows stay as they are: the factors are applied where the rows
// enter the chunk equations.
__device__ __forceinline__ float sum_sq8(const u32x4 &x, float s) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // The element goes through a scalar: a bit cast of the vector
        // element itself read element 0 every time.
        const unsigned w = x[e];
        const bf16x2 p = __builtin_bit_cast(bf16x2, w);
        s = __builtin_amdgcn_fdot2_f32_bf16(p, p, s, false);
    }
    return s;
}

__device__ __forceinline__ float row_inv_norm(const u32x4 &x) {
    return inv_l2_norm(row16_sum(sum_sq8(x, 0.0f)));
}

// The same for a 256-wide row held as two 128-wide halves by the same lanes.
__device__ __forceinline__ float row_inv_norm(const u32x4 &x0, const u32x4 &x1) {
    return inv_l2_norm(row16_sum(sum_sq8(x1, sum_sq8(x0, 0.0f))));
}

// x from the lane of the quad whose index is Sel.
template <int Sel>
__device__ __forceinline__ float quad_bcast(float x) {
    return dpp<Sel | (Sel << 2) | (Sel << 4) | (Sel << 6), 0xF>(x);
}

__device__ __forceinline__ float quad_bcast(float x, int sel) {
    switch (sel) {
    case 0: return quad_bcast<0>(x);
    case 1: return quad_bcast<1>(x);
    case 2: return quad_bcast<2>(x);
    default: return quad_bcast<3>(x);
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// Everything a workgroup needs to address its sequence.
struct Item {
    int64_t p0;      // first token (flattened over the rows)
    int nchunks;
    int len;         // tokens in the sequence (or in the piece)
    int j, hk, c0, n;
    int piece;       // piece of the row (0 without the piece scan)
    bool ident;      // a transition tile: V = 0, starting from identity columns
    int64_t chunk0;  // the backward's passes: the sequence's first chunk in the chunk numbering
};

// Helper-wave registers holding the next chunk's global data.
struct Stage {
    u32x4 k[4];   // K rows t/16 + 16 i, columns 8 (t % 16) .. + 7 (t = helper thread)
    u32x4 q[4];
    u32x4 v[2];   // value-tile rows t/8 + 32 i, columns 8 (t % 8) .. + 7
    float g, b;   // row = lane
};

// The schedule of packed documents: slot r of the work order is document
// order[r] (longest first) when the order is given, else document r.
__device__ __forceinline__ int doc_at(const FwdArgs &a, int64_t r) {
    return a.order ? a.order[r] : (int)r;
}

// Packed documents split into pieces of a.piece_len tokens: the pieces of
// document n (a document no longer than one piece, empty ones included, is
// one piece).
__device__ __forceinline__ int64_t doc_pieces(const FwdArgs &a, int n) {
    const int64_t len = (int64_t)a.cu[n + 1] - a.cu[n];
    return len > a.piece_len ? (len + a.piece_len - 1) / a.piece_len : 1;
}

// The first slot of document n in the piece arrays: every piece but a
// document's last has one, in document index order.
__device__ __forceinline__ int64_t doc_slot_base(const FwdArgs &a, int n) {
    int64_t b = 0;
    for (int m = 0; m < n; ++m)
        b += doc_pieces(a, m) - 1;
    return b;
}

// Document and piece of the r-th piece of a pass (ends: every piece but a
// document's last; otherwise all), documents taken in schedule order.
// False when r is past the last piece.
__device__ __forceinline__ bool locate_piece(const FwdArgs &a, int64_t r, bool ends, int &n,
                                             int64_t &p) {
    for (int i = 0; i < a.n_seqs; ++i) {
        n = doc_at(a, i);
        const int64_t cnt = doc_pieces(a, n) - (ends ? 1 : 0);
        if (r < cnt) {
            p = r;
            return true;
        }
        r -= cnt;
    }
    return false;
}

// Without Full (the piece ends, which form no output) Q is not loaded.  DK
// is the key dimension in HBM; with DK = 64 the LDS rows keep their 128
// columns and the lanes of the upper 64 stage zeros.  With DK = 256, tile
// row t/16 + 16 i is key half i / 2 of chunk row t/16 + 16 (i % 2), and only
// the 32 value rows of the chunk are staged.
template <bool Full, int DK>
__device__ __forceinline__ void stage_load(Stage &st, const FwdArgs &a, const Item &it, int c,
                                           int t, int lane) {
    constexpr int CL = chunk_len<DK>();
    const int64_t p = it.p0 + (int64_t)CL * c;
    const int L = min(CL, it.len - CL * c);
    const uint32_t krow = (uint32_t)a.Hqk * DK * 2;  // bytes between tokens
    const uint32_t vrow = (uint32_t)a.Hv * a.dv * 2;
    const uint32_t grow = (uint32_t)a.Hv * 4;
    const uint16_t *kb = static_cast<const uint16_t *>(a.k) + (p * a.Hqk + it.hk) * DK;
    const uint16_t *qb = static_cast<const uint16_t *>(a.q) + (p * a.Hqk + it.hk) * DK;
    const uint16_t *vb = static_cast<const uint16_t *>(a.v) + (p * a.Hv + it.j) * a.dv +
                         (it.ident ? 0 : it.c0);
    const __amdgpu_buffer_rsrc_t rk = rsrc(kb, (L - 1) * krow + DK * 2);
    const __amdgpu_buffer_rsrc_t rq = rsrc(qb, (L - 1) * krow + DK * 2);
    const bool kq_pad = DK < kDK && (t % 16) * 8 >= DK;  // a column slot past DK
    const __amdgpu_buffer_rsrc_t rv = rsrc(vb, it.ident ? 0u : (L - 1) * vrow + kDVT * 2);
    const __amdgpu_buffer_rsrc_t rg = rsrc(a.g + p * a.Hv + it.j, (L - 1) * grow + 4);
    const __amdgpu_buffer_rsrc_t rb = rsrc(a.beta + p * a.Hv + it.j, (L - 1) * grow + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t off = DK == 256 ? (t / 16 + 16 * (i % 2)) * krow + 16 * (t % 16 + 16 * (i / 2))
                                       : (t / 16 + 16 * i) * krow + 16 * (t % 16);
        if (kq_pad) {
            st.k[i] = u32x4{0u, 0u, 0u, 0u};
            st.q[i] = st.k[i];
            continue;
        }
        st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        if (Full)
            st.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
        st.v[i] = 32 * i < CL ? __builtin_amdgcn_raw_buffer_load_b128(rv, (t / 8 + 32 * i) * vrow + 16 * (t % 8), 0, 0)
                              : u32x4{0u, 0u, 0u, 0u};
    st.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, lane * grow, 0, 0));
    st.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, lane * grow, 0, 0));
}

// (a3) The lower 16-blocks of K K^T and Q K^T.  Block (i, j) is computed as
// K_j X_i^T (X = K or Q), whose C layout puts row 16 i + l%16, columns
// 16 j + 4 (l/16) .. + 3 of the wanted block in lane l: the row-major 8-byte
// pieces the A operands of the solve are read in.
// KK: the 32-wide k-steps that carry data (DK / 32; with DK = 64 the upper
// half of each staged row is zero and skipped).
template <int KK = 4>
__device__ __forceinline__ void load_block(bf16x8 (&f)[4], const uint16_t *t, const KqBase &kb, int m) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        f[kk] = frag_kq(t, kb, m, kk);
}

template <int KK = 4>
__device__ __forceinline__ f32x4 block_product(const bf16x8 (&xi)[4], const bf16x8 (&kj)[4]) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        c = mma(kj[kk], xi[kk], c);
    return c;
}

// -A block (I, J), I > J, from c = the block of K K^T: -beta_r exp(gamma_r - gamma_s)
// (k_r . k_s), hi + lo.  Nrm: k_r . k_s scaled by nu_r nu_s (the in-op L2 norm).
template <int I, int J, bool Nrm>
__device__ __forceinline__ void a_finish(ChunkBuf &B, f32x4 c, int lr, int lg) {
    if (Nrm)
        c = c * (B.nu[16 * I + lr] * ld4f(B.nu + 16 * J + 4 * lg));
    const float g = B.gam[16 * I + lr], b = B.bt[16 * I + lr];
    const f32x4 gc = ld4f(B.gam + 16 * J + 4 * lg);
    f32x4 val;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        val[r] = -b * __builtin_amdgcn_exp2f(g - gc[r]) * c[r];
    u32x2 hi, lo;
    split4(val, hi, lo);
    const int o = (16 * I + lr - 16) * kSN + 16 * J + 4 * lg;
    *reinterpret_cast<u32x2 *>(B.Anh + o) = hi;
    *reinterpret_cast<u32x2 *>(B.Anl + o) = lo;
}

template <int I, int J, bool Nrm, int DK>
__device__ __forceinline__ void a_block(ChunkBuf &B, const bf16x8 (&ki)[4], const bf16x8 (&kj)[4],
                                        int lr, int lg) {
    a_finish<I, J, Nrm>(B, block_product<DK / 32>(ki, kj), lr, lg);
}

// P block (I, J), I >= J, from c = the block of Q K^T: exp(gamma_r - gamma_s)
// (q_r . k_s), s <= r.  Nrm: q_r . k_s scaled by mu_r nu_s (the in-op L2 norm).
template <int I, int J, bool Nrm>
__device__ __forceinline__ void p_finish(ChunkBuf &B, f32x4 c, int lr, int lg) {
    if (Nrm)
        c = c * (B.mu[16 * I + lr] * ld4f(B.nu + 16 * J + 4 * lg));
    const float g = B.gam[16 * I + lr];
    const f32x4 gc = ld4f(B.gam + 16 * J + 4 * lg);
    f32x4 val;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (J < I) {
            val[r] = __builtin_amdgcn_exp2f(g - gc[r]) * c[r];
        } else {
            const float e = __builtin_amdgcn_exp2f(fminf(g - gc[r], 0.0f));
            val[r] = 4 * lg + r <= lr ? e * c[r] : 0.0f;
        }
    }
    *reinterpret_cast<u32x2 *>(B.P + (16 * I + lr) * kSP + 16 * J + 4 * lg) = pack4(val);
}

template <int I, int J, bool Nrm, int DK>
__device__ __forceinline__ void p_block(ChunkBuf &B, const bf16x8 (&qi)[4], const bf16x8 (&kj)[4],
                                        int lr, int lg) {
    p_finish<I, J, Nrm>(B, block_product<DK / 32>(qi, kj), lr, lg);
}

// Diagonal block A_II (strictly lower part, negated) into ad, column-major,
// from c = the block of K K^T.
template <int I, bool Nrm>
__device__ __forceinline__ void diag_finish(float *ad, const ChunkBuf &B, f32x4 c, int lr, int lg) {
    if (Nrm)
        c = c * (B.nu[16 * I + lr] * ld4f(B.nu + 16 * I + 4 * lg));
    const float g = B.gam[16 * I + lr], b = B.bt[16 * I + lr];
    const f32x4 gc = ld4f(B.gam + 16 * I + 4 * lg);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int col = 4 * lg + r;  // column within the block; the row is lr
        const float e = __builtin_amdgcn_exp2f(fminf(g - gc[r], 0.0f));
        ad[col * kAD + lr] = col < lr ? -(b * e * c[r]) : 0.0f;
    }
}

// (a4) D_i = (I + A_ii)^-1 by forward substitution in fp32, the four blocks
// in one wave: lane row g works on block g (from its copy of -A_gg in Ad[g],
// column-major) and lane c of the row computes column c.  Once x_r is final,
// -A[r2][r] x_r is added to every row r2 > r; the factors -A[r2][r] are
// column r of the copy, which every lane of the row reads at the same
// addresses (a broadcast read, one 16-byte read per four factors).  The
// reads run a few steps ahead of the multiply-adds, so the dependent steps
// do not each wait for LDS.  Column c is stored, as hi and lo bf16, as
// row 16 g + c of D^T.
template <int R>
__device__ __forceinline__ void dinv_load(f32x4 (&col)[15][4], const float *ad) {
    if constexpr (R < 15) {
#pragma unroll
        for (int q = (R + 1) / 4; q < 4; ++q)
            col[R][q] = ld4f(ad + R * kAD + 4 * q);
    }
}

template <int Ahead, int R>
__device__ __forceinline__ void dinv_step(float (&x)[16], f32x4 (&col)[15][4], const float *ad) {
    dinv_load<R + Ahead>(col, ad);
#pragma unroll
    for (int r2 = R + 1; r2 < 16; ++r2)
        x[r2] = __builtin_fmaf(col[R][r2 / 4][r2 % 4], x[R], x[r2]);
}

template <int... R>
__device__ __forceinline__ void dinv_loads(f32x4 (&col)[15][4], const float *ad,
                                           std::integer_sequence<int, R...>) {
    (dinv_load<R>(col, ad), ...);
}

template <int Ahead, int... R>
__device__ __forceinline__ void dinv_steps(float (&x)[16], f32x4 (&col)[15][4], const float *ad,
                                           std::integer_sequence<int, R...>) {
    (dinv_step<Ahead, R>(x, col, ad), ...);
}

// Ahead: how many steps the reads run ahead of the multiply-adds.
template <int Ahead>
__device__ __forceinline__ void diag_inverse_all(ChunkBuf &B, const Smem &S, int lane) {
    const int c = lane & 15, g = lane >> 4;
    const float *ad = S.Ad[g];
    f32x4 col[15][4];  // col[r][q]: rows 4 q .. 4 q + 3 of column r (quads holding a row > r)
    dinv_loads(col, ad, std::make_integer_sequence<int, Ahead>{});
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        x[r] = (r == c) ? 1.0f : 0.0f;
    dinv_steps<Ahead>(x, col, ad, std::make_integer_sequence<int, 15>{});
    u32x4 hi[2], lo[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        u32x2 h2, l2;
        split4(f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]}, h2, l2);
        hi[q >> 1][2 * (q & 1)] = h2.x;
        hi[q >> 1][2 * (q & 1) + 1] = h2.y;
        lo[q >> 1][2 * (q & 1)] = l2.x;
        lo[q >> 1][2 * (q & 1) + 1] = l2.y;
    }
    u32x4 *dh = reinterpret_cast<u32x4 *>(B.DhT + (16 * g + c) * kSDT);
    u32x4 *dl = reinterpret_cast<u32x4 *>(B.DlT + (16 * g + c) * kSDT);
    dh[0] = hi[0];
    dh[1] = hi[1];
    dl[0] = lo[0];
    dl[1] = lo[1];
}

// The per-chunk products, split over the helper waves.  The diagonal blocks
// of A come first on helpers 1..3 (A11; A00, A22; A33), each from row blocks
// of K the helper loads for its other products anyway; once a helper's are in
// LDS it counts itself on dsync.  Helper 0 forms P00, waits for the three
// counts and inverts the four blocks, the longest dependent piece of work;
// the rest of A and P is spread so that helpers 1..3 end at about the same
// time.  Without WithP (no output is formed) the P blocks are skipped; Nrm
// folds the in-op L2 norms of the rows into the blocks.  dmeet counts the
// diagonal-block signals helper 0 has waited for.
template <bool WithP, bool Nrm, int DK>
__device__ __forceinline__ void helper_products(Smem &S, ChunkBuf &B, int hw, int lr, int lg,
                                                int lane, int &dmeet) {
    constexpr int KK = DK / 32;
    const KqBase kb = kq_base(lr, lg);
    auto diag_done = [&]() {
        if (lane == 0)
            __hip_atomic_fetch_add(&S.dsync, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    dmeet += 3;
    if (hw == 0) {  // P00, then the inverses
        if constexpr (WithP) {
            bf16x8 q0[4], k0[4];
            load_block<KK>(q0, B.Q, kb, 0);
            load_block<KK>(k0, B.K, kb, 0);
            p_block<0, 0, Nrm, DK>(B, q0, k0, lr, lg);
        }
        while (__hip_atomic_load(&S.dsync, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < dmeet)
            __builtin_amdgcn_s_sleep(1);
        diag_inverse_all<4>(B, S, lane);
    } else if (hw == 1) {  // A11; A31 A30 A32, P10 P11
        bf16x8 k1[4], k3[4], kj[4], q1[4];
        load_block<KK>(k1, B.K, kb, 1);
        load_block<KK>(k3, B.K, kb, 3);
        diag_finish<1, Nrm>(S.Ad[1], B, block_product<KK>(k1, k1), lr, lg);
        diag_done();
        load_block<KK>(kj, B.K, kb, 0);
        load_block<KK>(q1, B.Q, kb, 1);
        a_block<3, 1, Nrm, DK>(B, k3, k1, lr, lg);
        a_block<3, 0, Nrm, DK>(B, k3, kj, lr, lg);
        if constexpr (WithP)
            p_block<1, 0, Nrm, DK>(B, q1, kj, lr, lg);
        load_block<KK>(kj, B.K, kb, 2);
        if constexpr (WithP)
            p_block<1, 1, Nrm, DK>(B, q1, k1, lr, lg);
        a_block<3, 2, Nrm, DK>(B, k3, kj, lr, lg);
    } else if (hw == 2) {  // A00 A22; A20 A21, P20 P21 P22
        bf16x8 k0[4], k2[4], q2[4], k1[4];
        load_block<KK>(k0, B.K, kb, 0);
        load_block<KK>(k2, B.K, kb, 2);
        diag_finish<0, Nrm>(S.Ad[0], B, block_product<KK>(k0, k0), lr, lg);
        diag_finish<2, Nrm>(S.Ad[2], B, block_product<KK>(k2, k2), lr, lg);
        diag_done();
        load_block<KK>(q2, B.Q, kb, 2);
        load_block<KK>(k1, B.K, kb, 1);
        a_block<2, 0, Nrm, DK>(B, k2, k0, lr, lg);
        if constexpr (WithP)
            p_block<2, 0, Nrm, DK>(B, q2, k0, lr, lg);
        a_block<2, 1, Nrm, DK>(B, k2, k1, lr, lg);
        if constexpr (WithP) {
            p_block<2, 1, Nrm, DK>(B, q2, k1, lr, lg);
            p_block<2, 2, Nrm, DK>(B, q2, k2, lr, lg);
        }
    } else {  // A33; A10, P33 P30 P31 P32
        bf16x8 k3[4], q3[4], k1[4], kj[4];
        load_block<KK>(k3, B.K, kb, 3);
        if constexpr (WithP)
            load_block<KK>(q3, B.Q, kb, 3);
        diag_finish<3, Nrm>(S.Ad[3], B, block_product<KK>(k3, k3), lr, lg);
        diag_done();
        load_block<KK>(k1, B.K, kb, 1);
        load_block<KK>(kj, B.K, kb, 0);
        if constexpr (WithP)
            p_block<3, 3, Nrm, DK>(B, q3, k3, lr, lg);
        a_block<1, 0, Nrm, DK>(B, k1, kj, lr, lg);
        if constexpr (WithP) {
            p_block<3, 0, Nrm, DK>(B, q3, kj, lr, lg);
            p_block<3, 1, Nrm, DK>(B, q3, k1, lr, lg);
            load_block<KK>(kj, B.K, kb, 2);
            p_block<3, 2, Nrm, DK>(B, q3, kj, lr, lg);
        }
    }
}

// dk = 256: block (I, J) of X K^T over the 256 keys, both key halves
// (tile row blocks I, J and I + 2, J + 2).
template <int I, int J>
__device__ __forceinline__ f32x4 gram256(const uint16_t *X, const uint16_t *K, const KqBase &kb) {
    bf16x8 x[4], k[4];
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        load_block<4>(x, X, kb, I + 2 * hf);
        load_block<4>(k, K, kb, J + 2 * hf);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            c = mma(k[kk], x[kk], c);
    }
    return c;
}

// The per-chunk products of a 32-token chunk (dk = 256): helper 0 the two
// diagonal blocks of A and their inverses, helper 1 A10 and P00, helper 2
// P10, helper 3 P11.  Without WithP (no output is formed) the P blocks are
// skipped.
template <bool WithP, bool Nrm>
__device__ __forceinline__ void helper_products_k256(Smem &S, ChunkBuf &B, int hw, int lr, int lg,
                                                     int lane) {
    const KqBase kb = kq_base(lr, lg);
    if (hw == 0) {
        diag_finish<0, Nrm>(S.Ad[0], B, gram256<0, 0>(B.K, B.K, kb), lr, lg);
        diag_finish<1, Nrm>(S.Ad[1], B, gram256<1, 1>(B.K, B.K, kb), lr, lg);
        // blocks 2, 3 invert the identity left in Ad[2], Ad[3]
        diag_inverse_all<3>(B, S, lane);
    } else if (hw == 1) {
        a_finish<1, 0, Nrm>(B, gram256<1, 0>(B.K, B.K, kb), lr, lg);
        if constexpr (WithP)
            p_finish<0, 0, Nrm>(B, gram256<0, 0>(B.Q, B.K, kb), lr, lg);
    } else if (WithP && hw == 2) {
        p_finish<1, 0, Nrm>(B, gram256<1, 0>(B.Q, B.K, kb), lr, lg);
    } else if (WithP) {
        p_finish<1, 1, Nrm>(B, gram256<1, 1>(B.Q, B.K, kb), lr, lg);
    }
}

// Helper waves: put chunk c (already in `st`) into LDS buffer B with its
// decay tables, A blocks, P and diagonal inverses.  Once `st` is in LDS it is
// refilled with chunk `next` (if next >= 0), so those loads are in flight
// during the products below and the state waves' whole next chunk.
template <bool Prep, bool Full, int DK>
__device__ __forceinline__ void helper_prepare(Smem &S, ChunkBuf &B, Stage &st, int hw, int t,
                                               int lane, int &meet, int &dmeet, const FwdArgs &a,
                                               const Item &it, int L, int next) {
    hw = __builtin_amdgcn_readfirstlane(hw);  // uniform: scalar branches below
    const int lr = lane & 15, lg = lane >> 4;
    if (Prep && DK == 256) {
        // The rows' inverse L2 norms (1 without the option): the lanes that
        // stage row t/16 + 16 i (i < 2) hold both of its key halves.
        const bool l2 = a.flags & kStepL2Norm;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float nk = l2 ? row_inv_norm(st.k[i], st.k[i + 2]) : 1.0f;
            const float nq = l2 && Full ? row_inv_norm(st.q[i], st.q[i + 2]) : 1.0f;
            if (t % 16 == 0) {
                B.nu[t / 16 + 16 * i] = nk;
                B.mu[t / 16 + 16 * i] = nq;
            }
        }
    } else if (Prep) {
        // The rows' inverse L2 norms (1 without the option), one lane per row.
        const bool l2 = a.flags & kStepL2Norm;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float nk = l2 ? row_inv_norm(st.k[i]) : 1.0f;
            const float nq = l2 && Full ? row_inv_norm(st.q[i]) : 1.0f;
            if (t % 16 == 0) {
                B.nu[t / 16 + 16 * i] = nk;
                B.mu[t / 16 + 16 * i] = nq;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int at = kq_slot(t / 16 + 16 * i, t % 16);
        *reinterpret_cast<u32x4 *>(B.K + at) = st.k[i];
        if (Full)
            *reinterpret_cast<u32x4 *>(B.Q + at) = st.q[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
        *reinterpret_cast<u32x4 *>(B.V + v_at(t / 8 + 32 * i, 2 * (t % 8))) = st.v[i];
    const bool gate_act = Prep && (a.flags & kStepGateAct);
    if (hw == 3) {
        // (a2) gamma; padded rows carry g = 0, so gamma_63 = gamma_{L-1}.
        // With the gate activation, g = logsigmoid(raw) with the hardware
        // exp and log: gamma is a sum of these, so their absolute error
        // (about 1e-7) is what counts, and beta's sigmoid runs on helper 2.
        float gv = st.g;
        if (gate_act)
            gv = lane < L ? fminf(gv, 0.0f) - __logf(1.0f + __expf(-fabsf(gv))) : 0.0f;
        const float x = wave_prefix_sum(gv);
        const float gL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
        B.gam[lane] = x * kLog2e;
        B.eg[lane] = __expf(x);
        B.el[lane] = __expf(gL - x);
        if (!gate_act)
            B.bt[lane] = st.b;
        if (lane == 0)
            B.eL = __expf(gL);
    } else if (gate_act && hw == 2) {
        const float e = __expf(-fabsf(st.b));
        B.bt[lane] = lane < L ? (st.b >= 0.0f ? 1.0f : e) / (1.0f + e) : 0.0f;
    }
    // Meet the other helper waves: the staged rows and gamma are in LDS.
    meet += 4;
    if (lane == 0)
        __hip_atomic_fetch_add(&S.hsync, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (next >= 0)
        stage_load<Full, DK>(st, a, it, next, t, lane);
    while (__hip_atomic_load(&S.hsync, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < meet)
        __builtin_amdgcn_s_sleep(1);
    if (Prep && hw == 3) {
        // Every row's norms are in LDS now: fold them into the tables the
        // state waves read (K M0 and the update through nu, Q M0 through mu).
        const float nu = B.nu[lane];
        B.egq[lane] = B.eg[lane] * B.mu[lane];
        B.eg[lane] *= nu;
        B.el[lane] *= nu;
    }

    if constexpr (DK == 256)
        helper_products_k256<Full, Prep>(S, B, hw, lr, lg, lane);
    else
        helper_products<Full, Prep, DK>(S, B, hw, lr, lg, lane, dmeet);
}

// Writes a wave's 64 x 16 block, given as four C-layout tiles of bf16 pairs
// (v[mi]: rows 16 mi + 4 g .. + 3 of column lr in lane (lr, g)), as rows of
// 16 columns: dst points at row 0, column 0 of the block, rows are
// row_stride elements apart, and rows >= rows_valid are not written.  The
// block goes through the wave's own LDS staging area column-major (word w of
// column c at w ^ x(c)); four transpose reads then give lane L the 16
// columns of row L, stored as two 16-byte pieces.
__device__ __forceinline__ void stage_store_rows(uint16_t *ost, const u32x2 (&v)[4], int lane,
                                                 uint16_t *dst, int64_t row_stride,
                                                 int rows_valid) {
    const int lr = lane & 15, lg = lane >> 4;
    auto ost_x = [](int col) {
        return (((col >> 1) & 1) << 3) ^ (((col >> 2) & 1) << 1) ^ (((col >> 3) & 1) << 2);
    };
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
        *reinterpret_cast<u32x2 *>(ost + lr * kC + 4 * ((4 * mi + lg) ^ ost_x(lr))) = v[mi];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int c0 = 8 * hf + (lr >> 2), c1 = c0 + 4;
        const int w = 4 * lg + (lr & 3);
        const u32x2 r0 = ld_tr(ost + c0 * kC + 4 * (w ^ ost_x(c0)));
        const u32x2 r1 = ld_tr(ost + c1 * kC + 4 * (w ^ ost_x(c1)));
        if (lane < rows_valid)
            *reinterpret_cast<u32x4 *>(dst + lane * row_stride + 8 * hf) =
                u32x4{r0.x, r0.y, r1.x, r1.y};
    }
}

// State waves: one chunk of (a5)-(a7) for value columns [16 s, 16 s + 16);
// without Out only the state advances (the output is not formed).
// Nrm: Q M0 is scaled by the egq table (exp(gamma) mu); the in-op L2 norms
// of K (nu) are already in the eg and el tables.
template <bool Out, bool Nrm, int DK, bool SaveDelta = false>
__device__ __forceinline__ void state_chunk(Smem &S, const ChunkBuf &B, const FwdArgs &a,
                                            const Item &it, int c, int s, int lane, f32x4 (&h)[8]) {
    const int lr = lane & 15, lg = lane >> 4;
    // (a5, a7) X = K M0 and Q M0 on this wave's columns (hi part of M0; at
    // dk = 64 K M0 adds the lo part), fragments loaded one row block ahead
    // of the products.
    // Key tiles 0 .. DK/16 - 1 hold the state; with DK = 64 the rest stay
    // zero and are skipped, as are the zero upper halves of the K, Q rows.
    constexpr int KK = DK / 32, MT = DK / 16;
    // At dk = 64, K M0 also takes the low part of M0 (LoKM).
    constexpr bool LoKM = DK == 64;
    bf16x8 hb[4], hl[4];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        if constexpr (LoKM) {
            u32x2 h0, l0, h1, l1;
            split4(h[2 * kk], h0, l0);
            split4(h[2 * kk + 1], h1, l1);
            hb[kk] = cat(h0, h1);
            hl[kk] = cat(l0, l1);
        } else {
            hb[kk] = cat(pack4(h[2 * kk]), pack4(h[2 * kk + 1]));
        }
    }
    f32x4 X[4], Oa[4];
    bf16x8 fk[2][4], fq[2][4];
    const KqBase kb = kq_base(lr, lg);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        fk[0][kk] = frag_kq(B.K, kb, 0, kk);
        fq[0][kk] = frag_kq(B.Q, kb, 0, kk);
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if (mi < 3) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                fk[(mi + 1) & 1][kk] = frag_kq(B.K, kb, mi + 1, kk);
                fq[(mi + 1) & 1][kk] = frag_kq(B.Q, kb, mi + 1, kk);
            }
        }
        X[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
        Oa[mi] = X[mi];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            X[mi] = mma(fk[mi & 1][kk], hb[kk], X[mi]);
            if constexpr (LoKM)
                X[mi] = mma(fk[mi & 1][kk], hl[kk], X[mi]);
            Oa[mi] = mma(fq[mi & 1][kk], hb[kk], Oa[mi]);
        }
    }
    // Right-hand sides R_i = diag(beta) (V - diag(exp gamma) X); O scaled.
    const int vbase = v_at(4 * lg + (lr >> 2), 4 * s + (lr & 3));  // row block 0; + 16 rows per mi
    f32x4 R[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const f32x4 eg4 = ld4f(B.eg + 16 * mi + 4 * lg);  // with Nrm: exp(gamma) nu
        const f32x4 egq = Nrm ? ld4f(B.egq + 16 * mi + 4 * lg) : eg4;
        const f32x4 bt4 = ld4f(B.bt + 16 * mi + 4 * lg);
        const u32x2 vv = ld_tr(B.V + vbase + 16 * kDVT * mi);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float vr = bf2f(static_cast<uint16_t>(vv[r / 2] >> (16 * (r % 2))));
            R[mi][r] = bt4[r] * (vr - eg4[r] * X[mi][r]);
            Oa[mi][r] *= egq[r];
        }
    }
    // Operands of the solve.  Each block of -A and each D_i is one A operand
    // holding its hi part in k positions 8g..8g+3 and its lo part in
    // 8g+4..8g+7 (lane group g, columns 4g..4g+3 of row lr); multiplied by a
    // B operand that holds one bf16 part of the right-hand side twice, one
    // 32-deep product gives (hi + lo) x part.
    bf16x8 An[6], Dd[4];  // blocks (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
#pragma unroll
    for (int i = 1, n = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < i; ++j, ++n) {
            const int o = (16 * (i - 1) + lr) * kSN + 16 * j + 4 * lg;
            An[n] = cat(ld8(B.Anh + o), ld8(B.Anl + o));
        }
    // D_i fragments (row lr, columns 4 lg .. + 3) from the transposed
    // copy: lane 4 j + m of each 16-lane group points at column 4 lg + j,
    // rows 4 m .. 4 m + 3.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int dofs = (16 * i + 4 * lg + (lr >> 2)) * kSDT + 4 * (lr & 3);
        Dd[i] = cat(ld_tr(B.DhT + dofs), ld_tr(B.DlT + dofs));
    }

    // (a4, a5) Delta_i = D_i (R_i - sum_{j<i} A_ij Delta_j).  Once Delta_j is
    // known its products go into every later right-hand side, the next one
    // first: the dependent chain is two products per block step.
    u32x2 dh[4], dl[4];
    f32x4 D[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u32x2 rh, rl;
        split4(R[i], rh, rl);
        f32x4 d = mma(Dd[i], cat(rh, rh), f32x4{0.f, 0.f, 0.f, 0.f});
        d = mma(Dd[i], cat(rl, rl), d);
        D[i] = d;
        split4(d, dh[i], dl[i]);
        const bf16x8 bh = cat(dh[i], dh[i]), bl = cat(dl[i], dl[i]);
#pragma unroll
        for (int r = i + 1; r < 4; ++r) {
            const int n = (r - 1) * r / 2 + i;  // block (r, i)
            R[r] = mma(An[n], bh, R[r]);
            R[r] = mma(An[n], bl, R[r]);
        }
    }

    // (a6) M_L = exp(gamma_L) M0 + K^T Delta', Delta' = diag(exp(gamma_L - gamma)) Delta,
    // K^T fragments loaded one tile ahead of the products.
    bf16x8 dph[2], dpl[2];
    {
        u32x2 ph[4], pl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 el4 = ld4f(B.el + 16 * i + 4 * lg);  // with Nrm: times nu
            split4(el4 * D[i], ph[i], pl[i]);
        }
        dph[0] = cat(ph[0], ph[1]);
        dph[1] = cat(ph[2], ph[3]);
        dpl[0] = cat(pl[0], pl[1]);
        dpl[1] = cat(pl[2], pl[3]);
    }
    const float eL = B.eL;
    // K^T fragment of accumulator tile mt, k-step kk: rows 32 kk + 4 lg + j
    // (+16), key dim pi(16 mt + lr).  Lane 4 j + q of each 16-lane group points
    // at row 32 kk + 4 lg + j, key dims 32 (mt / 2) + 8 q + 4 (mt % 2) .. + 3:
    // half (mt % 2) of slot 4 (mt / 2) + q.
    const int ktrow = 4 * lg + (lr >> 2);
    int ktb = kq_slot(ktrow, lr & 3);  // slot 4 a + (lr & 3) is at ktb ^ (32 a)
    asm volatile("" : "+v"(ktb));
    auto ktf = [&](int mt, int kk) {
        const uint16_t *p = B.K + (ktb ^ (32 * (mt >> 1))) + 4 * (mt & 1) + 32 * kk * kDK;
        return cat(ld_tr(p), ld_tr(p + 16 * kDK));
    };
    bf16x8 kt[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        kt[0][kk] = ktf(0, kk);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        if (mt < MT - 1) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                kt[(mt + 1) & 1][kk] = ktf(mt + 1, kk);
        }
        h[mt] *= eL;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            h[mt] = mma(kt[mt & 1][kk], dph[kk], h[mt]);
            h[mt] = mma(kt[mt & 1][kk], dpl[kk], h[mt]);
        }
    }

    if constexpr (SaveDelta) {
        // The backward's forward pass: the chunk's Delta rows (hi part),
        // after the update, which does not wait for them.
        uint16_t *dst = a.chunk_deltas + ((it.chunk0 + c) * a.Hv + it.j) * (int64_t)kC * a.dv +
                        it.c0 + 16 * s;
        stage_store_rows(S.Ost[s], dh, lane, dst, a.dv, kC);
    }
    if constexpr (!Out)
        return;
    // (a7) O += P Delta (hi parts); this wave's 64 x 16 block to HBM through
    // its own LDS staging area (no other wave touches it).  The staging copy
    // is column-major: lane (g, c) writes its four rows 16 mi + 4 g .. + 3 of
    // column c as one 8-byte word; four transpose reads then give lane L the
    // 16 columns of row L.  Word w of column c is stored at w ^ ost_x(c).
    const bf16x8 db[2] = {cat(dh[0], dh[1]), cat(dh[2], dh[3])};
    bf16x8 pf[6];
#pragma unroll
    for (int mi = 0, n = 0; mi < 4; ++mi)
#pragma unroll
        for (int kk = 0; kk <= mi / 2; ++kk, ++n)
            pf[n] = frag_perm(B.P + (16 * mi + lr) * kSP + 32 * kk, lg);
    uint16_t *ost = S.Ost[s];
    auto ost_x = [](int col) {
        return (((col >> 1) & 1) << 3) ^ (((col >> 2) & 1) << 1) ^ (((col >> 3) & 1) << 2);
    };
#pragma unroll
    for (int mi = 0, n = 0; mi < 4; ++mi) {
#pragma unroll
        for (int kk = 0; kk <= mi / 2; ++kk, ++n)
            Oa[mi] = mma(pf[n], db[kk], Oa[mi]);
        *reinterpret_cast<u32x2 *>(ost + lr * kC + 4 * ((4 * mi + lg) ^ ost_x(lr))) =
            pack4(a.scale * Oa[mi]);
    }
    const int L = min(kC, it.len - kC * c);
    const int64_t p = it.p0 + (int64_t)kC * c;
    uint16_t *o = static_cast<uint16_t *>(a.o) + ((p + lane) * a.Hv + it.j) * (int64_t)a.dv + it.c0 + 16 * s;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int c0 = 8 * hf + (lr >> 2), c1 = c0 + 4;
        const int w = 4 * lg + (lr & 3);
        const u32x2 r0 = ld_tr(ost + c0 * kC + 4 * (w ^ ost_x(c0)));
        const u32x2 r1 = ld_tr(ost + c1 * kC + 4 * (w ^ ost_x(c1)));
        if (lane < L)
            *reinterpret_cast<u32x4 *>(o + 8 * hf) = u32x4{r0.x, r0.y, r1.x, r1.y};
    }
}

// State waves, the backward's reverse pass: one chunk of the state-gradient
// recurrence for value columns [16 s, 16 s + 16).  h holds the wave's slice
// of dM, the gradient of the state leaving the chunk, in the forward's
// layout; the value tile holds dO (the upstream gradient of o) instead of V.
// From the forward's chunk equations (M0 -> Delta -> O, M_L), by the chain
// rule:
//   dDelta = diag(l) K dM + scale P^T dO,        l = exp(gamma_L - gamma)
//   (I + A)^T drhs = dDelta                      (T^T dDelta, T = (I + A)^-1)
//   dM0 = exp(gamma_L) dM - K^T diag(beta e) drhs + scale Q^T diag(e) dO
// The transposed solve is the forward's block substitution run backwards,
// drhs_i = D_i^T (dDelta_i - sum_{j>i} A_ji^T drhs_j), with D_i^T and the
// A_ji^T read from the forward's tiles by plain and transposing LDS reads,
// split products as in state_chunk.  K dM and P^T dO use single bf16
// roundings of dM and P (as the forward's K M0 and P Delta do).  drhs is
// stored as bf16 rows (the parallel gradient pass reads it) and dV =
// diag(beta) drhs as the gradient of v.
template <int DK>
__device__ __forceinline__ void state_chunk_rev(Smem &S, const ChunkBuf &B, const FwdArgs &a,
                                                const Item &it, int c, int s, int lane,
                                                f32x4 (&h)[8]) {
    const int lr = lane & 15, lg = lane >> 4;
    constexpr int KK = DK / 32, MT = DK / 16;
    // Z = K dM (hi part of dM), fragments loaded one row block ahead.
    bf16x8 hb[4];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        hb[kk] = cat(pack4(h[2 * kk]), pack4(h[2 * kk + 1]));
    f32x4 Z[4];
    bf16x8 fk[2][4];
    const KqBase kb = kq_base(lr, lg);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        fk[0][kk] = frag_kq(B.K, kb, 0, kk);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if (mi < 3) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                fk[(mi + 1) & 1][kk] = frag_kq(B.K, kb, mi + 1, kk);
        }
        Z[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            Z[mi] = mma(fk[mi & 1][kk], hb[kk], Z[mi]);
    }
    // W = P^T dO.  A operand of row block mi of P^T: column 16 mi + lr of P,
    // tokens 32 kk + 8 lg .. + 7 (two transpose reads); B operand: dO at the
    // same tokens, column 16 s + lr of the value tile.
    bf16x8 dob[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int r0 = 32 * kk + 8 * lg + (lr >> 2);
        dob[kk] = cat(ld_tr(B.V + v_at(r0, 4 * s + (lr & 3))), ld_tr(B.V + v_at(r0 + 4, 4 * s + (lr & 3))));
    }
    f32x4 dD[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        f32x4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (32 * kk + 31 < 16 * mi)
                continue;  // P is zero above the diagonal
            const uint16_t *pp = B.P + (32 * kk + 8 * lg + (lr >> 2)) * kSP + 16 * mi + 4 * (lr & 3);
            w = mma(cat(ld_tr(pp), ld_tr(pp + 4 * kSP)), dob[kk], w);
        }
        const f32x4 el4 = ld4f(B.el + 16 * mi + 4 * lg);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dD[mi][r] = el4[r] * Z[mi][r] + a.scale * w[r];
    }
    // Operands of the transposed solve: D_i^T (row lr of D_i^T is row
    // 16 i + lr of the stored D_i^T copy, hi | lo) and (-A_ji)^T for j > i
    // (transpose reads of the stored -A_ji, hi | lo).
    bf16x8 Dt[4], At[6];  // At: blocks (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int o = (16 * i + lr) * kSDT + 4 * lg;
        Dt[i] = cat(ld8(B.DhT + o), ld8(B.DlT + o));
    }
#pragma unroll
    for (int j = 1, n = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < j; ++i, ++n) {
            const int o = (16 * (j - 1) + 4 * lg + (lr >> 2)) * kSN + 16 * i + 4 * (lr & 3);
            At[n] = cat(ld_tr(B.Anh + o), ld_tr(B.Anl + o));
        }
    // drhs_i = D_i^T (dDelta_i - sum_{j>i} A_ji^T drhs_j), i = 3 .. 0; once
    // drhs_j is known its products go into every earlier right-hand side.
    f32x4 DR[4];
#pragma unroll
    for (int i = 3; i >= 0; --i) {
        u32x2 xh, xl;
        split4(dD[i], xh, xl);
        f32x4 d = mma(Dt[i], cat(xh, xh), f32x4{0.f, 0.f, 0.f, 0.f});
        d = mma(Dt[i], cat(xl, xl), d);
        DR[i] = d;
        u32x2 dh, dl;
        split4(d, dh, dl);
        const bf16x8 bh = cat(dh, dh), bl = cat(dl, dl);
#pragma unroll
        for (int r = i - 1; r >= 0; --r) {
            const int n = (i - 1) * i / 2 + r;  // block (i, r)
            dD[r] = mma(At[n], bh, dD[r]);
            dD[r] = mma(At[n], bl, dD[r]);
        }
    }
    // dM0 = exp(gamma_L) dM + K^T x + Q^T y, x = -diag(beta e) drhs,
    // y = scale diag(e) dO (hi | lo B operands over the chunk's rows).
    const int vbase = v_at(4 * lg + (lr >> 2), 4 * s + (lr & 3));
    u32x2 xh[4], xl[4], yh[4], yl[4], dvv[4], drb[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const f32x4 bt4 = ld4f(B.bt + 16 * mi + 4 * lg);
        const f32x4 eg4 = ld4f(B.eg + 16 * mi + 4 * lg);
        const u32x2 vv = ld_tr(B.V + vbase + 16 * kDVT * mi);
        f32x4 x, y, dv4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float dov = bf2f(static_cast<uint16_t>(vv[r / 2] >> (16 * (r % 2))));
            x[r] = -(bt4[r] * eg4[r]) * DR[mi][r];
            y[r] = a.scale * eg4[r] * dov;
            dv4[r] = bt4[r] * DR[mi][r];
        }
        split4(x, xh[mi], xl[mi]);
        split4(y, yh[mi], yl[mi]);
        dvv[mi] = pack4(dv4);
        drb[mi] = pack4(DR[mi]);
    }
    const bf16x8 xbh[2] = {cat(xh[0], xh[1]), cat(xh[2], xh[3])};
    const bf16x8 xbl[2] = {cat(xl[0], xl[1]), cat(xl[2], xl[3])};
    const bf16x8 ybh[2] = {cat(yh[0], yh[1]), cat(yh[2], yh[3])};
    const bf16x8 ybl[2] = {cat(yl[0], yl[1]), cat(yl[2], yl[3])};
    const float eL = B.eL;
    const int ktrow = 4 * lg + (lr >> 2);
    int ktb = kq_slot(ktrow, lr & 3);
    asm volatile("" : "+v"(ktb));
    auto tf = [&](const uint16_t *X, int mt, int kk) {
        const uint16_t *p = X + (ktb ^ (32 * (mt >> 1))) + 4 * (mt & 1) + 32 * kk * kDK;
        return cat(ld_tr(p), ld_tr(p + 16 * kDK));
    };
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        h[mt] *= eL;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 kt = tf(B.K, mt, kk), qt = tf(B.Q, mt, kk);
            h[mt] = mma(kt, xbh[kk], h[mt]);
            h[mt] = mma(kt, xbl[kk], h[mt]);
            h[mt] = mma(qt, ybh[kk], h[mt]);
            h[mt] = mma(qt, ybl[kk], h[mt]);
        }
    }
    // drhs rows to the workspace (all 64), dV rows to the output (valid rows).
    uint16_t *dr = a.chunk_drhs + ((it.chunk0 + c) * a.Hv + it.j) * (int64_t)kC * a.dv +
                   it.c0 + 16 * s;
    stage_store_rows(S.Ost[s], drb, lane, dr, a.dv, kC);
    const int L = min(kC, it.len - kC * c);
    uint16_t *dvo = static_cast<uint16_t *>(a.dv_out) +
                    ((it.p0 + (int64_t)kC * c) * a.Hv + it.j) * (int64_t)a.dv + it.c0 + 16 * s;
    stage_store_rows(S.Ost[s], dvv, lane, dvo, (int64_t)a.Hv * a.dv, L);
}

// State waves, dk = 256: one 32-token chunk of (a5)-(a7) for value columns
// [16 s, 16 s + 16), with the wave's [256 x 16] state slice in 16
// accumulator tiles.  The steps are those of state_chunk over two row
// blocks: K M0 and Q M0 take eight k-steps (key half h of row block i is
// tile row block i + 2 h), the solve one substitution step, and the update
// one 32-deep k-step per key tile (keys 128 h + x from tile rows 32 h ..).
template <bool Out, bool Nrm, bool SaveDelta = false>
__device__ __forceinline__ void state_chunk_k256(Smem &S, const ChunkBuf &B, const FwdArgs &a,
                                                 const Item &it, int c, int s, int lane,
                                                 f32x4 (&h)[16]) {
    constexpr int CL = 32;
    const int lr = lane & 15, lg = lane >> 4;
    bf16x8 hb[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
        hb[kk] = cat(pack4(h[2 * kk]), pack4(h[2 * kk + 1]));
    // (a5, a7) X = K M0 and Q M0, in four segments (row block sg / 2, key
    // half sg % 2), fragments loaded one segment ahead.
    f32x4 X[2], Oa[2];
    bf16x8 fk[2][4], fq[2][4];
    const KqBase kb = kq_base(lr, lg);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        fk[0][kk] = frag_kq(B.K, kb, 0, kk);
        fq[0][kk] = frag_kq(B.Q, kb, 0, kk);
    }
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
        if (sg < 3) {
            const int m = ((sg + 1) >> 1) + 2 * ((sg + 1) & 1);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                fk[(sg + 1) & 1][kk] = frag_kq(B.K, kb, m, kk);
                fq[(sg + 1) & 1][kk] = frag_kq(B.Q, kb, m, kk);
            }
        }
        const int mi = sg >> 1, hf = sg & 1;
        if (hf == 0) {
            X[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
            Oa[mi] = X[mi];
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            X[mi] = mma(fk[sg & 1][kk], hb[4 * hf + kk], X[mi]);
            Oa[mi] = mma(fq[sg & 1][kk], hb[4 * hf + kk], Oa[mi]);
        }
    }
    // Right-hand sides R_i = diag(beta) (V - diag(exp gamma) X); O scaled.
    const int vbase = v_at(4 * lg + (lr >> 2), 4 * s + (lr & 3));
    f32x4 R[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const f32x4 eg4 = ld4f(B.eg + 16 * mi + 4 * lg);
        const f32x4 egq = Nrm ? ld4f(B.egq + 16 * mi + 4 * lg) : eg4;
        const f32x4 bt4 = ld4f(B.bt + 16 * mi + 4 * lg);
        const u32x2 vv = ld_tr(B.V + vbase + 16 * kDVT * mi);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float vr = bf2f(static_cast<uint16_t>(vv[r / 2] >> (16 * (r % 2))));
            R[mi][r] = bt4[r] * (vr - eg4[r] * X[mi][r]);
            Oa[mi][r] *= egq[r];
        }
    }
    // (a4, a5) Delta_0 = D_0 R_0, Delta_1 = D_1 (R_1 - A_10 Delta_0), split
    // products as in state_chunk.
    const bf16x8 An = cat(ld8(B.Anh + lr * kSN + 4 * lg), ld8(B.Anl + lr * kSN + 4 * lg));
    bf16x8 Dd[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int dofs = (16 * i + 4 * lg + (lr >> 2)) * kSDT + 4 * (lr & 3);
        Dd[i] = cat(ld_tr(B.DhT + dofs), ld_tr(B.DlT + dofs));
    }
    u32x2 dh[2], dl[2];
    f32x4 D[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        u32x2 rh, rl;
        split4(R[i], rh, rl);
        f32x4 d = mma(Dd[i], cat(rh, rh), f32x4{0.f, 0.f, 0.f, 0.f});
        d = mma(Dd[i], cat(rl, rl), d);
        D[i] = d;
        split4(d, dh[i], dl[i]);
        if (i == 0) {
            R[1] = mma(An, cat(dh[0], dh[0]), R[1]);
            R[1] = mma(An, cat(dl[0], dl[0]), R[1]);
        }
    }
    // (a6) M_L = exp(gamma_L) M0 + K^T Delta'; the K^T fragment of key tile
    // mt is tile mt % 8 of tile rows 32 (mt / 8) .., loaded one tile ahead.
    bf16x8 dph, dpl;
    {
        u32x2 ph[2], pl[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const f32x4 el4 = ld4f(B.el + 16 * i + 4 * lg);
            split4(el4 * D[i], ph[i], pl[i]);
        }
        dph = cat(ph[0], ph[1]);
        dpl = cat(pl[0], pl[1]);
    }
    const float eL = B.eL;
    const int ktrow = 4 * lg + (lr >> 2);
    int ktb = kq_slot(ktrow, lr & 3);
    asm volatile("" : "+v"(ktb));
    auto ktf = [&](int mt) {
        const uint16_t *p = B.K + (ktb ^ (32 * ((mt & 7) >> 1))) + 4 * (mt & 1) + 32 * (mt >> 3) * kDK;
        return cat(ld_tr(p), ld_tr(p + 16 * kDK));
    };
    bf16x8 kt[2];
    kt[0] = ktf(0);
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
        if (mt < 15)
            kt[(mt + 1) & 1] = ktf(mt + 1);
        h[mt] *= eL;
        h[mt] = mma(kt[mt & 1], dph, h[mt]);
        h[mt] = mma(kt[mt & 1], dpl, h[mt]);
    }

    if constexpr (SaveDelta) {
        // The backward's forward pass: the chunk's 32 Delta rows (hi part),
        // after the update, which does not wait for them.
        uint16_t *dst = a.chunk_deltas + ((it.chunk0 + c) * a.Hv + it.j) * (int64_t)CL * a.dv +
                        it.c0 + 16 * s;
        const u32x2 rows[4] = {dh[0], dh[1], kZero2, kZero2};
        stage_store_rows(S.Ost[s], rows, lane, dst, a.dv, CL);
    }
    if constexpr (!Out)
        return;
    // (a7) O += P Delta (hi parts), staged through LDS as in state_chunk.
    const bf16x8 db = cat(dh[0], dh[1]);
    bf16x8 pf[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
        pf[mi] = frag_perm(B.P + (16 * mi + lr) * kSP, lg);
    uint16_t *ost = S.Ost[s];
    auto ost_x = [](int col) {
        return (((col >> 1) & 1) << 3) ^ (((col >> 2) & 1) << 1) ^ (((col >> 3) & 1) << 2);
    };
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        Oa[mi] = mma(pf[mi], db, Oa[mi]);
        *reinterpret_cast<u32x2 *>(ost + lr * kC + 4 * ((4 * mi + lg) ^ ost_x(lr))) =
            pack4(a.scale * Oa[mi]);
    }
    const int L = min(CL, it.len - CL * c);
    const int64_t p = it.p0 + (int64_t)CL * c;
    uint16_t *o = static_cast<uint16_t *>(a.o) + ((p + lane) * a.Hv + it.j) * (int64_t)a.dv + it.c0 + 16 * s;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int c0 = 8 * hf + (lr >> 2), c1 = c0 + 4;
        const int w = 4 * lg + (lr & 3);
        const u32x2 r0 = ld_tr(ost + c0 * kC + 4 * (w ^ ost_x(c0)));
        const u32x2 r1 = ld_tr(ost + c1 * kC + 4 * (w ^ ost_x(c1)));
        if (lane < L)
            *reinterpret_cast<u32x4 *>(o + 8 * hf) = u32x4{r0.x, r0.y, r1.x, r1.y};
    }
}

// The reverse pass at dk = 256: state_chunk_rev over a chunk of 32 tokens
// laid into the tiles as in state_chunk_k256 (key half h of chunk row r is
// tile row 32 h + r): Z = K dM over eight k-steps in four segments, W = P^T
// dO over the chunk's 32 tokens, one transposed substitution step, and the
// update of the sixteen key tiles with one 32-deep k-step each.
__device__ __forceinline__ void state_chunk_rev_k256(Smem &S, const ChunkBuf &B, const FwdArgs &a,
                                                     const Item &it, int c, int s, int lane,
                                                     f32x4 (&h)[16]) {
    constexpr int CL = 32;
    const int lr = lane & 15, lg = lane >> 4;
    bf16x8 hb[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
        hb[kk] = cat(pack4(h[2 * kk]), pack4(h[2 * kk + 1]));
    // Z = K dM (hi part of dM): segment sg is row block sg / 2 and key half
    // sg % 2 (tile row block m = row block + 2 key half), fragments loaded one
    // segment ahead.
    f32x4 Z[2];
    bf16x8 fk[2][4];
    const KqBase kb = kq_base(lr, lg);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        fk[0][kk] = frag_kq(B.K, kb, 0, kk);
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
        if (sg < 3) {
            const int m = ((sg + 1) >> 1) + 2 * ((sg + 1) & 1);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                fk[(sg + 1) & 1][kk] = frag_kq(B.K, kb, m, kk);
        }
        const int mi = sg >> 1, hf = sg & 1;
        if (hf == 0)
            Z[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            Z[mi] = mma(fk[sg & 1][kk], hb[4 * hf + kk], Z[mi]);
    }
    // W = P^T dO over the 32 tokens (A operand: column 16 mi + lr of P,
    // tokens 8 lg .. + 7; B operand: dO at those tokens, column 16 s + lr).
    const int r0 = 8 * lg + (lr >> 2);
    const bf16x8 dob = cat(ld_tr(B.V + v_at(r0, 4 * s + (lr & 3))),
                           ld_tr(B.V + v_at(r0 + 4, 4 * s + (lr & 3))));
    f32x4 dD[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const uint16_t *pp = B.P + r0 * kSP + 16 * mi + 4 * (lr & 3);
        const f32x4 w = mma(cat(ld_tr(pp), ld_tr(pp + 4 * kSP)), dob, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 el4 = ld4f(B.el + 16 * mi + 4 * lg);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dD[mi][r] = el4[r] * Z[mi][r] + a.scale * w[r];
    }
    // drhs_1 = D_1^T dDelta_1, drhs_0 = D_0^T (dDelta_0 - A_10^T drhs_1).
    bf16x8 Dt[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int o = (16 * i + lr) * kSDT + 4 * lg;
        Dt[i] = cat(ld8(B.DhT + o), ld8(B.DlT + o));
    }
    const int ao = (4 * lg + (lr >> 2)) * kSN + 4 * (lr & 3);
    const bf16x8 At = cat(ld_tr(B.Anh + ao), ld_tr(B.Anl + ao));
    f32x4 DR[2];
#pragma unroll
    for (int i = 1; i >= 0; --i) {
        u32x2 xh, xl;
        split4(dD[i], xh, xl);
        f32x4 d = mma(Dt[i], cat(xh, xh), f32x4{0.f, 0.f, 0.f, 0.f});
        d = mma(Dt[i], cat(xl, xl), d);
        DR[i] = d;
        if (i == 1) {
            u32x2 dh, dl;
            split4(d, dh, dl);
            dD[0] = mma(At, cat(dh, dh), dD[0]);
            dD[0] = mma(At, cat(dl, dl), dD[0]);
        }
    }
    // dM0 = exp(gamma_L) dM + K^T x + Q^T y, x = -diag(beta e) drhs,
    // y = scale diag(e) dO, as in state_chunk_rev.
    const int vbase = v_at(4 * lg + (lr >> 2), 4 * s + (lr & 3));
    u32x2 xh[2], xl[2], yh[2], yl[2], dvv[4], drb[4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const f32x4 bt4 = ld4f(B.bt + 16 * mi + 4 * lg);
        const f32x4 eg4 = ld4f(B.eg + 16 * mi + 4 * lg);
        const u32x2 vv = ld_tr(B.V + vbase + 16 * kDVT * mi);
        f32x4 x, y, dv4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float dov = bf2f(static_cast<uint16_t>(vv[r / 2] >> (16 * (r % 2))));
            x[r] = -(bt4[r] * eg4[r]) * DR[mi][r];
            y[r] = a.scale * eg4[r] * dov;
            dv4[r] = bt4[r] * DR[mi][r];
        }
        split4(x, xh[mi], xl[mi]);
        split4(y, yh[mi], yl[mi]);
        dvv[mi] = pack4(dv4);
        drb[mi] = pack4(DR[mi]);
    }
    dvv[2] = dvv[3] = drb[2] = drb[3] = kZero2;
    const bf16x8 xbh = cat(xh[0], xh[1]), xbl = cat(xl[0], xl[1]);
    const bf16x8 ybh = cat(yh[0], yh[1]), ybl = cat(yl[0], yl[1]);
    const float eL = B.eL;
    const int ktrow = 4 * lg + (lr >> 2);
    int ktb = kq_slot(ktrow, lr & 3);
    asm volatile("" : "+v"(ktb));
    // The transposed fragment of key tile mt: tile mt % 8 of tile rows
    // 32 (mt / 8) .., as in state_chunk_k256.
    auto tf = [&](const uint16_t *X, int mt) {
        const uint16_t *p = X + (ktb ^ (32 * ((mt & 7) >> 1))) + 4 * (mt & 1) + 32 * (mt >> 3) * kDK;
        return cat(ld_tr(p), ld_tr(p + 16 * kDK));
    };
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
        h[mt] *= eL;
        const bf16x8 kt = tf(B.K, mt), qt = tf(B.Q, mt);
        h[mt] = mma(kt, xbh, h[mt]);
        h[mt] = mma(kt, xbl, h[mt]);
        h[mt] = mma(qt, ybh, h[mt]);
        h[mt] = mma(qt, ybl, h[mt]);
    }
    // drhs rows to the workspace (all 32), dV rows to the output (valid rows).
    uint16_t *dr = a.chunk_drhs + ((it.chunk0 + c) * a.Hv + it.j) * (int64_t)CL * a.dv +
                   it.c0 + 16 * s;
    stage_store_rows(S.Ost[s], drb, lane, dr, a.dv, CL);
    const int L = min(CL, it.len - CL * c);
    uint16_t *dvo = static_cast<uint16_t *>(a.dv_out) +
                    ((it.p0 + (int64_t)CL * c) * a.Hv + it.j) * (int64_t)a.dv + it.c0 + 16 * s;
    stage_store_rows(S.Ost[s], dvv, lane, dvo, (int64_t)a.Hv * a.dv, L);
}

// Prep: the in-op preparation options of a.flags are honoured (a separate
// instance, so the plain kernel carries none of their code).  Mode 4: the
// backward's reverse pass (state_chunk_rev), chunks from the last, with dO in
// place of V; it stores the gradient of every chunk's leaving state, drhs,
// dV and dh0.
// Mode 0: the output pass over whole rows.  Mode 2: the same over pieces
// that start from the states of piece_starts (an instance of its own, so
// traces tell the two apart).  Mode 3: no output; the state entering every
// chunk is stored (bf16, [dv][dk]) to a.chunk_states for the backward.  Mode 1: the piece
// ends, for every piece but the last: F from a zero start and real V, and
// (extra "identity" tiles) the transition Phi, the end state of dk unit
// columns with V = 0; no output is formed.
template <bool Prep, int Mode, int DK>
__global__ __launch_bounds__(kThreads, 1) void gdn_fwd_bf16(FwdArgs a) {
    __shared__ Smem S;
    constexpr int CL = chunk_len<DK>(), NH = state_tiles<DK>();
    // Modes that form P (and stage Q): the output passes and the reverse pass.
    constexpr bool kFull = Mode == 0 || Mode == 2 || Mode == 4;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

    // Work item.  Items that read the same q/k head (the dv tiles and the
    // grouped value heads of one q/k head) are kept on one XCD: blocks are
    // dispatched round-robin over the 8 XCDs, so block b runs on XCD b % 8.
    const int n_val = a.dv / kDVT;
    const int n_tiles = Mode == 1 ? n_val + DK / kDVT : n_val;
    const bool packed_pieces = a.cu && a.pieces > 1;
    // Batch rows: pieces of a row in this pass.
    const int np = a.pieces > 1 && !a.cu ? (Mode == 1 ? a.pieces - 1 : a.pieces) : 1;
    const int G = a.Hv / a.Hqk;
    const int gs = n_tiles * G;
    const int nb = gridDim.x;
    int w = blockIdx.x;
    if (nb % (8 * gs) == 0) {
        const int xcd = w % 8, local = w / 8;
        w = ((local / gs) * 8 + xcd) * gs + local % gs;
    }
    Item it;
    const int tile = w % n_tiles;
    it.j = (w / n_tiles) % a.Hv;
    const int64_t rest = w / (n_tiles * a.Hv);
    it.hk = it.j / G;
    it.ident = Mode == 1 && tile >= n_val;
    it.c0 = (it.ident ? tile - n_val : tile) * kDVT;
    int64_t p1;
    int64_t slot_base = 0;  // the sequence's first slot in the piece arrays
    int64_t seq_pieces = 1; // pieces of the sequence
    if (packed_pieces) {
        int n = 0;
        int64_t pc = 0;
        if (!locate_piece(a, rest, Mode == 1, n, pc))
            return;  // past the last piece (a host copy of cu that disagrees with the device's)
        it.n = n;
        it.piece = (int)pc;
        seq_pieces = doc_pieces(a, n);
        slot_base = doc_slot_base(a, n);
        if (slot_base + seq_pieces - 1 > a.n_slots)
            return;  // more pieces than the workspace holds (the same disagreement)
        it.p0 = a.cu[n] + pc * a.piece_len;
        p1 = pc + 1 < seq_pieces ? it.p0 + a.piece_len : a.cu[n + 1];
    } else if (a.cu) {
        it.piece = 0;
        it.n = doc_at(a, rest);
        it.p0 = a.cu[it.n];
        p1 = a.cu[it.n + 1];
    } else {
        it.piece = (int)(rest % np);
        it.n = (int)(rest / np);
        seq_pieces = a.pieces > 1 ? a.pieces : 1;
        slot_base = (int64_t)it.n * (seq_pieces - 1);
        const int64_t row0 = (int64_t)it.n * a.T;
        const int64_t s0 = a.pieces > 1 ? it.piece * a.piece_len : 0;
        const int64_t s1 = a.pieces > 1 && it.piece < a.pieces - 1 ? s0 + a.piece_len : a.T;
        it.p0 = row0 + s0;
        p1 = row0 + s1;
    }
    it.len = (int)(p1 - it.p0);
    it.nchunks = (it.len + CL - 1) / CL;

    for (int i = tid; i < kC * kSP; i += kThreads) {
        S.buf[0].P[i] = 0;
        S.buf[1].P[i] = 0;
    }
    if (DK == 256) {  // blocks 2, 3 of the inverses: the identity, never read
        for (int i = tid; i < 16 * kAD; i += kThreads) {
            S.Ad[2][i] = 0.0f;
            S.Ad[3][i] = 0.0f;
        }
    }
    if (tid == 0) {
        S.hsync = 0;
        S.dsync = 0;
    }
    __syncthreads();

    const bool state = wv < 4;
    const int s = wv & 3;      // state wave: value-column group; helper wave: helper index
    const int t = tid - 256;   // helper thread index
    const int lg = lane >> 4, lr = lane & 15;
    const int col = it.c0 + 16 * s + lr;
    const int64_t hbase = ((int64_t)it.n * a.Hv + it.j) * DK * (int64_t)a.dv;
    // The slot of (sequence, piece, head) in the piece arrays.
    const int64_t pslot = (slot_base + it.piece) * a.Hv + it.j;

    f32x4 h[NH];
    Stage st;
    int meet = 0, dmeet = 0;
    // Issue priority on the shared SIMDs follows the critical paths.  Where
    // the state waves form an output (Modes 0, 2) or run the reverse chain
    // (Mode 4), their chain is the longest: state waves first, then helper 0
    // (diagonal blocks and their inverses), helpers 1..3 filling the gaps.
    // Where they form no output (piece ends, Mode 1; the backward's forward
    // state pass, Mode 3) they finish their chunk step before helper 0 does,
    // so helper 0 goes first there.  With the in-op preparation helpers 1..3
    // carry the row norms as well and go before the default.
    constexpr bool kHelper0First = Mode == 1 || Mode == 3;
    if (state)
        __builtin_amdgcn_s_setprio(kHelper0First ? 2 : 3);
    else if (s == 0)
        __builtin_amdgcn_s_setprio(kHelper0First ? 3 : 2);
    else if (Prep)
        __builtin_amdgcn_s_setprio(1);
    if (state) {
        const float *src = nullptr;
        if (Mode == 4)  // the reverse pass starts from the final state's gradient
            src = a.dht ? a.dht + hbase : nullptr;
        else if (Mode != 1 && it.piece > 0)  // the state entering this piece: slot (n, piece - 1, j)
            src = a.piece_starts + (pslot - a.Hv) * DK * (int64_t)a.dv;
        else if (Mode != 1 && a.h0)
            src = a.h0 + hbase;
        if (src) {
#pragma unroll
            for (int mt = 0; mt < NH; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = key_of(mt, lg, r);
                    h[mt][r] = key < DK ? src[(int64_t)key * a.dv + col] : 0.f;
                }
        } else {
#pragma unroll
            for (int mt = 0; mt < NH; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h[mt][r] = it.ident && key_of(mt, lg, r) == col ? 1.f : 0.f;
        }
    } else if (it.nchunks > 0) {
        // The reverse pass (Mode 4) walks the chunks from the last.
        const int c0 = Mode == 4 ? it.nchunks - 1 : 0;
        const int c1 = Mode == 4 ? it.nchunks - 2 : 1;
        stage_load<kFull, DK>(st, a, it, c0, t, lane);
        helper_prepare<Prep, kFull, DK>(S, S.buf[0], st, s, t, lane, meet, dmeet, a, it,
                                        min(CL, it.len - CL * c0), it.nchunks > 1 ? c1 : -1);
    }
    lds_barrier();

    // Modes 3 and 4: this sequence's first chunk in the chunk numbering.
    int64_t chunk0 = 0;
    if (Mode == 3 || Mode == 4) {
        if (a.cu) {
            for (int m = 0; m < it.n; ++m)
                chunk0 += (a.cu[m + 1] - a.cu[m] + CL - 1) / CL;
        } else {
            chunk0 = (int64_t)it.n * ((a.T + CL - 1) / CL);
        }
    }
    it.chunk0 = chunk0;
    // One chunk loop per role (the barrier counts match): the state slice and
    // the helpers' prefetch registers are then never live together.
    // Iteration i works on chunk c(i): in order, or from the last (Mode 4).
    auto cidx = [&](int i) { return Mode == 4 ? it.nchunks - 1 - i : i; };
    if (state) {
        for (int i = 0; i < it.nchunks; ++i) {
            const int c = cidx(i);
            if (Mode == 3 || Mode == 4) {
                // The state entering the chunk (Mode 3) or the gradient of
                // the state leaving it (Mode 4): the tiles 2 k and 2 k + 1
                // hold keys 32 k + 8 lg .. + 7 of column col in order, one
                // 16-byte store.  The rows are 128 keys wide at dk = 64 and
                // 128 (zeros past DK), 256 at dk = 256.  Non-temporal: the
                // gradient kernel reads them once, after the other pass has
                // streamed its own data through the caches (dk = 256
                // backward 3.26 -> 3.19 ms; the same for the Delta, drhs and
                // dV rows made the dk = 128 backward twice as slow).
                constexpr int SW = DK == 256 ? 256 : kDK;
                uint16_t *dst = (Mode == 3 ? a.chunk_states : a.chunk_dstates) +
                                ((chunk0 + c) * a.Hv + it.j) * (int64_t)a.dv * SW +
                                (int64_t)col * SW;
#pragma unroll
                for (int mt = 0; mt < NH; mt += 2) {
                    const u32x2 lo = pack4(h[mt]), hi = pack4(h[mt + 1]);
                    __builtin_nontemporal_store(u32x4{lo.x, lo.y, hi.x, hi.y},
                                                reinterpret_cast<u32x4 *>(dst + key_of(mt, lg, 0)));
                }
            }
            if constexpr (Mode == 4 && DK == 256)
                state_chunk_rev_k256(S, S.buf[i & 1], a, it, c, s, lane, h);
            else if constexpr (Mode == 4)
                state_chunk_rev<DK>(S, S.buf[i & 1], a, it, c, s, lane, h);
            else if constexpr (DK == 256)
                state_chunk_k256<Mode == 0 || Mode == 2, Prep, Mode == 3>(S, S.buf[i & 1], a, it, c,
                                                                         s, lane, h);
            else
                state_chunk<Mode == 0 || Mode == 2, Prep, DK, Mode == 3>(S, S.buf[i & 1], a, it, c, s,
                                                                         lane, h);
            lds_barrier();
        }
    } else {
        for (int i = 0; i < it.nchunks; ++i) {
            if (i + 1 < it.nchunks)
                helper_prepare<Prep, kFull, DK>(S, S.buf[(i + 1) & 1], st, s, t, lane, meet, dmeet, a,
                                                it, min(CL, it.len - CL * cidx(i + 1)),
                                                i + 2 < it.nchunks ? cidx(i + 2) : -1);
            lds_barrier();
        }
    }

    if (state) {
        float *dst = nullptr;
        int64_t stride = a.dv, dcol = col;
        if (Mode == 1) {
            stride = a.dv + DK;
            dst = a.piece_ends + pslot * DK * stride;
            dcol = (it.ident ? a.dv : 0) + col;
        } else if (Mode == 4) {
            dst = a.dh0 ? a.dh0 + hbase : nullptr;
        } else if (Mode != 3 && a.ht && it.piece == seq_pieces - 1) {
            dst = a.ht + hbase;
        }
        if (dst) {
#pragma unroll
            for (int mt = 0; mt < NH; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = key_of(mt, lg, r);
                    if (key < DK)
                        dst[(int64_t)key * stride + dcol] = h[mt][r];
                }
        }
    }
}

// The piece scan between the two passes: for row n, head j and value columns
// [16 y, 16 y + 16), M_0 = h0 (or zero) and M_{p+1} = Phi_p M_p + F_p for
// p < pieces - 1, written to piece_starts.  The state map of a piece is
// affine in its start state (the recurrence is linear in S), so this is
// exact; fp32 with one fused multiply-add per term, summed in key order.
// Thread (rg, cg) owns rows dk/64 * rg .. + dk/64 - 1 and columns 4 cg .. + 3
// of the product; Phi_p is staged transposed in LDS, 64 of its columns at a
// time, so both operands are read as 16-byte vectors.
constexpr int kScanCols = 16;

template <int DK>
__global__ __launch_bounds__(256) void piece_scan(FwdArgs a) {
    constexpr int R = DK / 64;   // rows per thread
    constexpr int KB = 64;       // columns of Phi staged at a time
    typedef __attribute__((ext_vector_type(R))) float rowv;
    __shared__ __attribute__((aligned(16))) float Ms[DK][kScanCols + 4];
    __shared__ __attribute__((aligned(16))) float PhT[KB][DK + 4];
    const int tid = threadIdx.x, cg = tid % 4, rg = tid / 4;
    const int n = blockIdx.x / a.Hv, j = blockIdx.x % a.Hv;
    const int c0 = blockIdx.y * kScanCols;
    const int64_t hbase = ((int64_t)n * a.Hv + j) * DK * (int64_t)a.dv;
    // The sequence's slots: batch rows have pieces - 1 each; a packed
    // document one per piece but its last.
    const int64_t count = a.cu ? doc_pieces(a, n) - 1 : a.pieces - 1;
    const int64_t base = a.cu ? doc_slot_base(a, n) : (int64_t)n * (a.pieces - 1);
    if (count <= 0 || base + count > a.n_slots)
        return;
    for (int e = tid; e < DK * kScanCols; e += 256) {
        const int i = e / kScanCols, c = e % kScanCols;
        Ms[i][c] = a.h0 ? a.h0[hbase + (int64_t)i * a.dv + c0 + c] : 0.0f;
    }
    const int64_t estride = a.dv + DK;
    for (int64_t p = 0; p < count; ++p) {
        const int64_t pslot = (base + p) * a.Hv + j;
        const float *ends = a.piece_ends + pslot * DK * estride;
        f32x4 acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = *reinterpret_cast<const f32x4 *>(ends + (R * rg + r) * estride + c0 + 4 * cg);
        for (int k0 = 0; k0 < DK; k0 += KB) {
            __syncthreads();  // the previous reads of PhT, and the last step's writes of Ms
            for (int e = tid; e < DK * KB / 4; e += 256) {
                const int r = e / (KB / 4), q4 = e % (KB / 4);
                const f32x4 x = *reinterpret_cast<const f32x4 *>(ends + r * estride + a.dv + k0 + 4 * q4);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    PhT[4 * q4 + i][r] = x[i];
            }
            __syncthreads();
            for (int kk = 0; kk < KB; ++kk) {
                const f32x4 m = *reinterpret_cast<const f32x4 *>(&Ms[k0 + kk][4 * cg]);
                const rowv ph = *reinterpret_cast<const rowv *>(&PhT[kk][R * rg]);
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[r][c] = fmaf(ph[r], m[c], acc[r][c]);
            }
        }
        __syncthreads();  // every read of Ms is done
        float *out = a.piece_starts + pslot * DK * (int64_t)a.dv;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            *reinterpret_cast<f32x4 *>(&Ms[R * rg + r][4 * cg]) = acc[r];
            *reinterpret_cast<f32x4 *>(out + (R * rg + r) * (int64_t)a.dv + c0 + 4 * cg) = acc[r];
        }
    }
}

template <bool Prep, int DK>
hipError_t launch_passes(const FwdArgs &a, hipStream_t stream) {
    const int n_val = a.dv / kDVT;
    if (a.pieces <= 1) {
        const int64_t blocks = (int64_t)a.n_seqs * a.Hv * n_val;
        if (blocks > 0x7fffffff)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL((gdn_fwd_bf16<Prep, 0, DK>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, a);
        return hipGetLastError();
    }
    const int64_t items_a = a.cu ? a.items_ends : (int64_t)a.n_seqs * (a.pieces - 1);
    const int64_t items_b = a.cu ? a.items_all : (int64_t)a.n_seqs * a.pieces;
    const int64_t blocks_a = items_a * a.Hv * (n_val + DK / kDVT);
    const int64_t blocks_b = items_b * a.Hv * n_val;
    const int64_t scan_rows = (int64_t)a.n_seqs * a.Hv;
    if (blocks_a > 0x7fffffff || blocks_b > 0x7fffffff || scan_rows > 0x7fffffff)
        return hipErrorInvalidValue;
    if (blocks_a > 0)
        hipLaunchKernelGGL((gdn_fwd_bf16<Prep, 1, DK>), dim3((unsigned)blocks_a), dim3(kThreads), 0,
                           stream, a);
    hipLaunchKernelGGL(piece_scan<DK>, dim3((unsigned)scan_rows, (unsigned)(a.dv / kScanCols)),
                       dim3(256), 0, stream, a);
    hipLaunchKernelGGL((gdn_fwd_bf16<Prep, 2, DK>), dim3((unsigned)blocks_b), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <bool Prep>
hipError_t launch_dk(const FwdArgs &a, hipStream_t stream) {
    if (a.dk == 128)
        return launch_passes<Prep, 128>(a, stream);
    if (a.dk == 64)
        return launch_passes<Prep, 64>(a, stream);
    if (a.dk == 256)
        return launch_passes<Prep, 256>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_state_passes(const FwdArgs &fwd, const FwdArgs &rev, hipStream_t stream) {
    const int64_t blocks = (int64_t)fwd.n_seqs * fwd.Hv * (fwd.dv / kDVT);
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0x7fffffff || (fwd.dk != 128 && fwd.dk != 64 && fwd.dk != 256) ||
        fwd.pieces > 1 || fwd.flags || !fwd.chunk_states || !fwd.chunk_deltas ||
        !rev.chunk_dstates || !rev.chunk_drhs || !rev.dv_out)
        return hipErrorInvalidValue;
    if (fwd.dk == 256) {
        hipLaunchKernelGGL((gdn_fwd_bf16<false, 3, 256>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, fwd);
        hipLaunchKernelGGL((gdn_fwd_bf16<false, 4, 256>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, rev);
    } else if (fwd.dk == 128) {
        hipLaunchKernelGGL((gdn_fwd_bf16<false, 3, 128>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, fwd);
        hipLaunchKernelGGL((gdn_fwd_bf16<false, 4, 128>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, rev);
    } else {
        hipLaunchKernelGGL((gdn_fwd_bf16<false, 3, 64>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, fwd);
        hipLaunchKernelGGL((gdn_fwd_bf16<false, 4, 64>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, rev);
    }
    return hipGetLastError();
}

size_t fwd_piece_starts_offset(int64_t slots, int32_t Hv, int32_t dk, int32_t dv) {
    const size_t per = (size_t)slots * Hv * dk;
    return (per * (dv + dk) * 4 + 255) / 256 * 256;
}

size_t fwd_piece_bytes(int64_t slots, int32_t Hv, int32_t dk, int32_t dv) {
    if (slots <= 0)
        return 0;
    return fwd_piece_starts_offset(slots, Hv, dk, dv) + (size_t)slots * Hv * dk * dv * 4;
}

namespace {

// Documents ranked by length, longest first, ties by index: each thread
// ranks its documents by counting the longer ones among all (lengths staged
// in LDS, read by every thread at the same address).
__global__ __launch_bounds__(1024) void doc_order(const int32_t *cu, int32_t n_seqs,
                                                  int32_t *order) {
    __shared__ int32_t len[kMaxOrderedDocs];
    for (int i = threadIdx.x; i < n_seqs; i += blockDim.x)
        len[i] = cu[i + 1] - cu[i];
    __syncthreads();
    for (int n = threadIdx.x; n < n_seqs; n += blockDim.x) {
        const int32_t ln = len[n];
        int rank = 0;
        for (int m = 0; m < n_seqs; ++m) {
            const int32_t lm = len[m];
            rank += (lm > ln) | ((lm == ln) & (m < n));
        }
        order[rank] = n;
    }
}

}  // namespace

hipError_t launch_doc_order(const int32_t *cu, int32_t n_seqs, int32_t *order,
                            hipStream_t stream) {
    if (n_seqs < 1 || n_seqs > kMaxOrderedDocs)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(doc_order, dim3(1), dim3(1024), 0, stream, cu, n_seqs, order);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream) {
    if ((int64_t)a.n_seqs * a.Hv <= 0)
        return hipSuccess;
    return a.flags ? launch_dk<true>(a, stream) : launch_dk<false>(a, stream);
}

}  // namespace gdn

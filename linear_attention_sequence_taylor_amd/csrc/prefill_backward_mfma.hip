// prefill_backward_mfma.hip -- gradients of causal Taylor linear attention on
// the gfx950 matrix cores (bf16 inputs, feature dim 16, fp32 accumulation).
//
// Same quantities as prefill_backward.hip ("Simple linear attention language
// models balance the recall-throughput tradeoff", s5 and s4 "Taylor Linear
// Attention"): with s_ij = q_i.k_j/4, a_ij = 1 + s_ij + s_ij^2/2,
// y_i = N_i / D_i, g_i = dy_i / D_i, h_i = -(dy_i . y_i) / D_i and
// e_ij = (g_i . v_j + h_i)(1 + s_ij)/4:
//   dq_i = sum_{j<=i} e_ij k_j,  dk_j = sum_{i>=j} e_ij q_i,
//   dv_j = sum_{i>=j} a_ij g_i.
//
// Every product is a 16-row MFMA tile per wave (16 rows of its own side, 16
// or 32 of the other side per instruction).  The operand layouts line up
// without register shuffles: a score tile computed as K Q^T (keys x queries)
// leaves lane (g, r) with query r and keys 4g..4g+3, which is the A operand
// of a product over those keys for query row r.  Operands that need a column
// of a row-major tile (V, K, Q and g as B operands) come from gfx950's
// transposed LDS read, so every tile is staged once, row-major.  q, k, v are
// exact in bf16; the weights a, e and g enter as bf16 hi/lo pairs (about 16
// significant bits); accumulation is fp32.  The 1/4 of s is folded into this
// wave's own q (or k) row, an exact power-of-two scale of a bf16 value, and
// the 1/4 of e into the final dq (dk).
//
// Query side (one workgroup per 64 queries, wave w: queries 16w..16w+15):
//   pass 1 over the key tiles at or before the queries: N and D, then g, h
//   (g as bf16 hi/lo planes to the workspace, h in fp32);
//   pass 2: ga^T = V g^T, e, dq += e K.
// Key side (one workgroup per 64 keys): over the query tiles at or after the
// keys: s = Q K^T, ga = g V^T, e, dv += a^T g, dk += e^T Q.
// Only the diagonal tile needs the causal mask; rows past L are staged as
// zeros (their g and h are zero, so they add nothing on the key side) and
// never stored.
#include "common.hpp"
#include "kernels.hpp"

namespace based {
namespace {

constexpr int kT = 64;  // rows per tile (queries or keys)
constexpr int kD = 16;  // feature dim of this path

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define BWD_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 ld4(const uint16_t* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// LDS tiles are row-major bf16 with W columns and no padding; element
// (row, col) sits at tile_at<W>(row, col).  Rows are permuted in pieces so
// that the two read shapes below both hit distinct banks (64 banks of 4
// bytes; a 16-byte read serves 16 lanes at a time, an 8-byte read 32):
// 16 consecutive rows at one column piece (the row-operand reads), and 8
// consecutive rows (from a multiple of 16, or 8 past it) at two adjacent
// 16-byte pieces (the transposed reads).
//  - W = 16 (Q, K): four 8-byte slots per row; rows 8..15 of every 16 swap
//    slots 0,1 with 2,3.
//  - W = 64, 128 (V, g): 16-byte units; unit index XOR h(row), with h
//    distinct over 16 rows and h/2 distinct over each aligned 8 rows (and,
//    for W = 64, over the rows of one parity, which share banks).
template <int W>
__device__ __forceinline__ int tile_at(int row, int col) {
    if constexpr (W == kD) {
        return row * kD + ((((col >> 2) ^ ((row >> 2) & 2))) << 2) + (col & 3);
    } else {
        static_assert(W == 64 || W == 128, "tile width");
        const int h = W == 64 ? ((((row >> 1) & 3) << 1) | ((row >> 3) & 1)) : (((row & 7) << 1) | ((row >> 3) & 1));
        return row * W + ((((col >> 3) ^ h)) << 3) + (col & 7);
    }
}

// Transposed read of a bf16 tile in LDS: lane c of each 16-lane group
// passes the address of row rb + c/4, columns col0 + 4(c%4) .. +3, and
// receives rows rb .. rb+3 of column col0 + c (rb may differ between the
// groups).
template <int W>
__device__ __forceinline__ uint2 tr4(const uint16_t* tile, int rb, int col0, int c) {
    const uint16_t* p = tile + tile_at<W>(rb + (c >> 2), col0 + 4 * (c & 3));
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(BWD_LDS(s16x4, p)));
}
// B operand of a 16x16x32 product whose k index 8g + i stands for row
// rb + 4g + i (i < 4) and rb + 16 + 4g + i - 4 (i >= 4): the pairing of the
// A operands built from two 16-row score tiles (join_tiles).
template <int W>
__device__ __forceinline__ bf16x8 tr_b8(const uint16_t* tile, int rb, int col0, int g, int c) {
    const uint2 a = tr4<W>(tile, rb + 4 * g, col0, c);
    const uint2 b = tr4<W>(tile, rb + 16 + 4 * g, col0, c);
    return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// hi = bf16(x), lo = bf16(x - hi).  Each x - hi is one v_dot2_f32_bf16 of
// the packed hi pair against (-1, -0) or (-0, -1), plus x: the products are
// exact and x - hi is representable, so the one rounding changes nothing.
// (The selectors keep a -0 in the other half: the pair (-1, +0) has the bit
// pattern of a small integer that is emitted as an inline float constant.)
__device__ __forceinline__ void hilo8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
    const bf16x2 sel_lo = __builtin_bit_cast(bf16x2, 0x8000bf80u);
    const bf16x2 sel_hi = __builtin_bit_cast(bf16x2, 0xbf808000u);
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t hp = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        const bf16x2 hb = __builtin_bit_cast(bf16x2, hp);
        h[i] = hp;
        l[i] = pack_bf16x2(__builtin_amdgcn_fdot2_f32_bf16(hb, sel_lo, x[2 * i], false),
                           __builtin_amdgcn_fdot2_f32_bf16(hb, sel_hi, x[2 * i + 1], false));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}
// The four values of score tile 2p and the four of tile 2p + 1 as one
// 8-vector (k index 8g + i of tr_b8).
__device__ __forceinline__ void join_tiles(const float (&a)[4], const float (&b)[4], float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = a[i];
        x[4 + i] = b[i];
    }
}

// Four bf16 values times 1/4 (exact unless they underflow).
__device__ __forceinline__ bf16x4 quarter(uint2 u) {
    const float f[4] = {bf16lo_f32(u.x), bf16hi_f32(u.x), bf16lo_f32(u.y), bf16hi_f32(u.y)};
    return __builtin_bit_cast(bf16x4, make_uint2(pack_bf16x2(0.25f * f[0], 0.25f * f[1]),
                                                 pack_bf16x2(0.25f * f[2], 0.25f * f[3])));
}

// A [64][W] bf16 tile (rows row0.. of a [L][W] matrix, rows past L zero)
// held in registers across the workgroup, 16 bytes per piece: loaded from
// global memory while the previous tile is in use, then stored to LDS in
// the tile_at<W> layout.
template <int W>
struct TileRegs {
    static constexpr int kU = W / 8;                    // pieces per row
    static constexpr int kPer = (kT * kU + 255) / 256;  // pieces per thread
    u32x4 x[kPer];

    __device__ __forceinline__ void load(const uint16_t* mat, int L, int row0) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = threadIdx.x + 256 * i, row = e / kU, u = e % kU;
            x[i] = u32x4{0u, 0u, 0u, 0u};
            if (e < kT * kU && row0 + row < L)
                x[i] = *reinterpret_cast<const u32x4*>(mat + (size_t)(row0 + row) * W + 8 * u);
        }
    }
    __device__ __forceinline__ void store(uint16_t* dst) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = threadIdx.x + 256 * i, row = e / kU, u = e % kU;
            if (e < kT * kU) *reinterpret_cast<u32x4*>(dst + tile_at<W>(row, 8 * u)) = x[i];
        }
    }
};

// ---------------------------------------------------------------- query side
template <int DV>
struct BwdQSmem {
    alignas(16) uint16_t k[kT * kD];
    alignas(16) uint16_t v[kT * DV];
    alignas(16) uint16_t ghi[4][16 * DV];  // per wave: g of its 16 queries
    alignas(16) uint16_t glo[4][16 * DV];
    float h[4][16];
};

// Pass 1 on one key tile: N (yacc: rows = queries 4g+m, columns 16ct + r)
// and D - eps (dsum: the same rows, every column) as the product with a
// column of ones.
template <int DV, bool DIAG>
__device__ __forceinline__ void q_pass1(const BwdQSmem<DV>& sm, const bf16x4& qb, int w, int g, int r,
                                        f32x4 (&yacc)[DV / 16], f32x4& dsum) {
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    float a[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        const f32x4 st = mfma16(ld4(&sm.k[tile_at<kD>(16 * kt + r, 4 * g)]), qb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float s = st[m];
            float x = fmaf(s, fmaf(s, 0.5f, 1.f), 1.f);
            if (DIAG) x = 16 * kt + 4 * g + m <= 16 * w + r ? x : 0.f;
            a[kt][m] = x;
        }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        float x[8];
        join_tiles(a[2 * p], a[2 * p + 1], x);
        bf16x8 ahi, alo;
        hilo8(x, ahi, alo);
        dsum = mfma32(ahi, ones, dsum);
        dsum = mfma32(alo, ones, dsum);
#pragma unroll
        for (int ct = 0; ct < DV / 16; ++ct) {
            const bf16x8 vb = tr_b8<DV>(sm.v, 32 * p, 16 * ct, g, r);
            yacc[ct] = mfma32(ahi, vb, yacc[ct]);
            yacc[ct] = mfma32(alo, vb, yacc[ct]);
        }
    }
}

// Pass 2 on one key tile: dq (rows = queries 4g+m, columns = feature r) +=
// e4 K with e4 = 4 e.
template <int DV, bool DIAG>
__device__ __forceinline__ void q_pass2(const BwdQSmem<DV>& sm, const bf16x4& qb, int w, int g, int r,
                                        f32x4& dqacc) {
    const float hr = sm.h[w][r];
    float e[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        const f32x4 st = mfma16(ld4(&sm.k[tile_at<kD>(16 * kt + r, 4 * g)]), qb, f32x4{0.f, 0.f, 0.f, 0.f});
        // ga^T: rows = keys 16kt + 4g + m, columns = queries r
        f32x4 ga = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cs = 0; cs < DV / 32; ++cs) {
            const bf16x8 va = ld8(&sm.v[tile_at<DV>(16 * kt + r, 32 * cs + 8 * g)]);
            ga = mfma32(va, ld8(&sm.ghi[w][tile_at<DV>(r, 32 * cs + 8 * g)]), ga);
            ga = mfma32(va, ld8(&sm.glo[w][tile_at<DV>(r, 32 * cs + 8 * g)]), ga);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float gh = ga[m] + hr;
            float x = fmaf(gh, st[m], gh);
            if (DIAG) x = 16 * kt + 4 * g + m <= 16 * w + r ? x : 0.f;
            e[kt][m] = x;
        }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        float x[8];
        join_tiles(e[2 * p], e[2 * p + 1], x);
        bf16x8 ehi, elo;
        hilo8(x, ehi, elo);
        const bf16x8 kb = tr_b8<kD>(sm.k, 32 * p, 0, g, r);
        dqacc = mfma32(ehi, kb, dqacc);
        dqacc = mfma32(elo, kb, dqacc);
    }
}

template <int DV>
__global__ __launch_bounds__(256) void bwd_query_mfma_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             const float* __restrict__ dy, int L, int ntiles,
                                                             float eps, float* __restrict__ dq,
                                                             uint16_t* __restrict__ ghi_ws,
                                                             uint16_t* __restrict__ glo_ws,
                                                             float* __restrict__ h_ws) {
    constexpr int kNV = DV / 16;  // column tiles
    __shared__ BwdQSmem<DV> sm;
    const int BH = gridDim.x / ntiles;
    const int head = blockIdx.x % BH;
    const int ti = ntiles - 1 - (int)(blockIdx.x / BH);  // the longest rows first, every head
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const uint16_t* kh = k + (size_t)head * L * kD;
    const uint16_t* vh = v + (size_t)head * L * DV;
    const int qw0 = ti * kT + 16 * w;  // first query of this wave
    const int qr = qw0 + r;            // this lane's query in score tiles

    // B operand of the scores: this lane's query row, dims 4g..4g+3, times 1/4
    bf16x4 qb = __builtin_bit_cast(bf16x4, make_uint2(0u, 0u));
    if (qr < L) qb = quarter(*reinterpret_cast<const uint2*>(q + ((size_t)head * L + qr) * kD + 4 * g));

    // ---- pass 1: the key tiles before the diagonal, the next one loading
    // while the current one is in use, then the diagonal tile
    f32x4 yacc[kNV];
#pragma unroll
    for (int ct = 0; ct < kNV; ++ct) yacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 dsum = {0.f, 0.f, 0.f, 0.f};
    TileRegs<kD> kreg;
    TileRegs<DV> vreg;
    kreg.load(kh, L, 0);
    vreg.load(vh, L, 0);
    for (int tj = 0; tj < ti; ++tj) {
        __syncthreads();
        kreg.store(sm.k);
        vreg.store(sm.v);
        __syncthreads();
        kreg.load(kh, L, (tj + 1) * kT);
        vreg.load(vh, L, (tj + 1) * kT);
        q_pass1<DV, false>(sm, qb, w, g, r, yacc, dsum);
    }
    __syncthreads();
    kreg.store(sm.k);
    vreg.store(sm.v);
    __syncthreads();
    kreg.load(kh, L, 0);  // pass 2's first off-diagonal tile
    vreg.load(vh, L, 0);
    q_pass1<DV, true>(sm, qb, w, g, r, yacc, dsum);

    // ---- g = dy/D and h = -(dy.N)/D^2 for queries qw0 + 4g + m, columns
    // 16ct + r: g to this wave's LDS rows as bf16 hi/lo, h to LDS and the
    // workspace.  The dy loads all go out at once (rows past L read row L-1
    // and are zeroed), not one per use.
    float dyv[4][kNV];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int qi = qw0 + 4 * g + m;
        const float* dyr = dy + ((size_t)head * L + min(qi, L - 1)) * DV + r;
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) dyv[m][ct] = dyr[16 * ct];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int qi = qw0 + 4 * g + m;
        const float inv = 1.f / (dsum[m] + eps);
        float dyy = 0.f;
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) {
            const float dyc = qi < L ? dyv[m][ct] : 0.f;
            dyy = fmaf(dyc, yacc[ct][m], dyy);
            const float gv = dyc * inv;
            const uint32_t hb = pack_bf16x2(gv, 0.f);
            const uint32_t lb = pack_bf16x2(gv - bf16lo_f32(hb), 0.f);
            sm.ghi[w][tile_at<DV>(4 * g + m, 16 * ct + r)] = (uint16_t)(hb & 0xffffu);
            sm.glo[w][tile_at<DV>(4 * g + m, 16 * ct + r)] = (uint16_t)(lb & 0xffffu);
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) dyy += __shfl_xor(dyy, off, 64);
        const float hq = -dyy * inv * inv;
        if (r == 0) {
            sm.h[w][4 * g + m] = hq;
            if (qi < L) h_ws[(size_t)head * L + qi] = hq;
        }
    }
    __syncthreads();
    // this wave's g rows to the workspace in 16-byte pieces
    {
        constexpr int kU = DV / 8;
        for (int e = lane; e < 16 * kU; e += 64) {
            const int row = e / kU, u = e % kU;
            const int qi = qw0 + row;
            if (qi < L) {
                const size_t off = ((size_t)head * L + qi) * DV + 8 * u;
                *reinterpret_cast<u32x4*>(ghi_ws + off) =
                    *reinterpret_cast<const u32x4*>(&sm.ghi[w][tile_at<DV>(row, 8 * u)]);
                *reinterpret_cast<u32x4*>(glo_ws + off) =
                    *reinterpret_cast<const u32x4*>(&sm.glo[w][tile_at<DV>(row, 8 * u)]);
            }
        }
    }

    // ---- pass 2: the diagonal tile (still in LDS), then the tiles before it
    f32x4 dqacc = {0.f, 0.f, 0.f, 0.f};
    q_pass2<DV, true>(sm, qb, w, g, r, dqacc);
    for (int tj = 0; tj < ti; ++tj) {
        __syncthreads();
        kreg.store(sm.k);
        vreg.store(sm.v);
        __syncthreads();
        kreg.load(kh, L, (tj + 1) * kT);
        vreg.load(vh, L, (tj + 1) * kT);
        q_pass2<DV, false>(sm, qb, w, g, r, dqacc);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int qi = qw0 + 4 * g + m;
        if (qi < L) dq[((size_t)head * L + qi) * kD + r] = 0.25f * dqacc[m];
    }
}

// ---------------------------------------------------------------- key side
template <int DV>
struct BwdKSmem {
    alignas(16) uint16_t q[kT * kD];
    alignas(16) uint16_t ghi[kT * DV];  // g of the query tile, hi / lo
    alignas(16) uint16_t glo[kT * DV];
    alignas(16) float h[kT];
};

// One query tile: dv (rows = keys 4g+m, columns 16ct + r) += a^T g and
// dk (columns = feature r) += e4^T Q with e4 = 4 e.
template <int DV, bool DIAG>
__device__ __forceinline__ void k_tile(const BwdKSmem<DV>& sm, const bf16x4& kb, const bf16x8 (&vb)[DV / 32], int w,
                                       int g, int r, f32x4 (&dvacc)[DV / 16], f32x4& dkacc) {
    float a[4][4], e[4][4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
        // scores and ga: rows = queries 16qt + 4g + m, columns = keys r
        const f32x4 st = mfma16(ld4(&sm.q[tile_at<kD>(16 * qt + r, 4 * g)]), kb, f32x4{0.f, 0.f, 0.f, 0.f});
        f32x4 ga = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cs = 0; cs < DV / 32; ++cs) {
            ga = mfma32(ld8(&sm.ghi[tile_at<DV>(16 * qt + r, 32 * cs + 8 * g)]), vb[cs], ga);
            ga = mfma32(ld8(&sm.glo[tile_at<DV>(16 * qt + r, 32 * cs + 8 * g)]), vb[cs], ga);
        }
        const f32x4 hq = *reinterpret_cast<const f32x4*>(&sm.h[16 * qt + 4 * g]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float s = st[m], gh = ga[m] + hq[m];
            float xa = fmaf(s, fmaf(s, 0.5f, 1.f), 1.f), xe = fmaf(gh, s, gh);
            if (DIAG) {
                const bool ok = 16 * qt + 4 * g + m >= 16 * w + r;
                xa = ok ? xa : 0.f;
                xe = ok ? xe : 0.f;
            }
            a[qt][m] = xa;
            e[qt][m] = xe;
        }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        float xa[8], xe[8];
        join_tiles(a[2 * p], a[2 * p + 1], xa);
        join_tiles(e[2 * p], e[2 * p + 1], xe);
        bf16x8 ahi, alo, ehi, elo;
        hilo8(xa, ahi, alo);
        hilo8(xe, ehi, elo);
#pragma unroll
        for (int ct = 0; ct < DV / 16; ++ct) {
            const bf16x8 gbh = tr_b8<DV>(sm.ghi, 32 * p, 16 * ct, g, r);
            const bf16x8 gbl = tr_b8<DV>(sm.glo, 32 * p, 16 * ct, g, r);
            dvacc[ct] = mfma32(ahi, gbh, dvacc[ct]);
            dvacc[ct] = mfma32(alo, gbh, dvacc[ct]);
            dvacc[ct] = mfma32(ahi, gbl, dvacc[ct]);
        }
        const bf16x8 qb = tr_b8<kD>(sm.q, 32 * p, 0, g, r);
        dkacc = mfma32(ehi, qb, dkacc);
        dkacc = mfma32(elo, qb, dkacc);
    }
}

template <int DV>
__global__ __launch_bounds__(256) void bwd_key_mfma_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, int L, int ntiles,
                                                           const uint16_t* __restrict__ ghi_ws,
                                                           const uint16_t* __restrict__ glo_ws,
                                                           const float* __restrict__ h_ws, float* __restrict__ dk,
                                                           float* __restrict__ dvo) {
    constexpr int kNV = DV / 16;
    __shared__ BwdKSmem<DV> sm;
    const int BH = gridDim.x / ntiles;
    const int head = blockIdx.x % BH;
    const int tj = blockIdx.x / BH;  // the first keys (the longest loops) first, every head
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const uint16_t* qh = q + (size_t)head * L * kD;
    const uint16_t* gh = ghi_ws + (size_t)head * L * DV;
    const uint16_t* gl = glo_ws + (size_t)head * L * DV;
    const float* hh = h_ws + (size_t)head * L;
    const int kw0 = tj * kT + 16 * w;  // first key of this wave
    const int kr = kw0 + r;            // this lane's key in score tiles

    // this lane's key row (times 1/4) and value row pieces: the B operands
    // of Q K^T and g V^T
    bf16x4 kb = __builtin_bit_cast(bf16x4, make_uint2(0u, 0u));
    bf16x8 vb[DV / 32];
#pragma unroll
    for (int cs = 0; cs < DV / 32; ++cs) vb[cs] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    if (kr < L) {
        kb = quarter(*reinterpret_cast<const uint2*>(k + ((size_t)head * L + kr) * kD + 4 * g));
#pragma unroll
        for (int cs = 0; cs < DV / 32; ++cs) vb[cs] = ld8(v + ((size_t)head * L + kr) * DV + 32 * cs + 8 * g);
    }
    f32x4 dvacc[kNV];
#pragma unroll
    for (int ct = 0; ct < kNV; ++ct) dvacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 dkacc = {0.f, 0.f, 0.f, 0.f};

    // the diagonal tile, then the query tiles after it, the next one loading
    // while the current one is in use
    TileRegs<kD> qreg;
    TileRegs<DV> ghreg, glreg;
    float hreg = 0.f;
    auto load = [&](int ti) {
        qreg.load(qh, L, ti * kT);
        ghreg.load(gh, L, ti * kT);
        glreg.load(gl, L, ti * kT);
        if (threadIdx.x < kT) hreg = ti * kT + (int)threadIdx.x < L ? hh[ti * kT + threadIdx.x] : 0.f;
    };
    auto store = [&]() {
        qreg.store(sm.q);
        ghreg.store(sm.ghi);
        glreg.store(sm.glo);
        if (threadIdx.x < kT) sm.h[threadIdx.x] = hreg;
    };
    load(tj);
    store();
    __syncthreads();
    load(tj + 1);
    k_tile<DV, true>(sm, kb, vb, w, g, r, dvacc, dkacc);
    for (int ti = tj + 1; ti < ntiles; ++ti) {
        __syncthreads();
        store();
        __syncthreads();
        load(ti + 1);
        k_tile<DV, false>(sm, kb, vb, w, g, r, dvacc, dkacc);
    }
    // rows = keys kw0 + 4g + m; dv columns 16ct + r, dk feature r
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int kj = kw0 + 4 * g + m;
        if (kj < L) {
#pragma unroll
            for (int ct = 0; ct < kNV; ++ct) dvo[((size_t)head * L + kj) * DV + 16 * ct + r] = dvacc[ct][m];
            dk[((size_t)head * L + kj) * kD + r] = 0.25f * dkacc[m];
        }
    }
}

}  // namespace

// The workspace of prefill_backward.hip (BH*L*DV fp32 for g, then BH*L fp32
// for h) holds g here as two bf16 planes of BH*L*DV each (hi, then lo).
template <int DV>
static void launch_both(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* dy, int BH, int L,
                        float eps, float* dq, float* dk, float* dvo, float* g_ws, float* h_ws, hipStream_t st) {
    const int ntiles = (L + kT - 1) / kT;
    const dim3 grid((unsigned)(ntiles * BH));
    uint16_t* ghi = reinterpret_cast<uint16_t*>(g_ws);
    uint16_t* glo = ghi + (size_t)BH * L * DV;
    hipLaunchKernelGGL((bwd_query_mfma_kernel<DV>), grid, dim3(256), 0, st, q, k, v, dy, L, ntiles, eps, dq, ghi,
                       glo, h_ws);
    hipLaunchKernelGGL((bwd_key_mfma_kernel<DV>), grid, dim3(256), 0, st, q, k, v, L, ntiles, ghi, glo, h_ws, dk,
                       dvo);
}

hipError_t launch_prefill_backward_mfma(const void* q, const void* k, const void* v, const float* dy, int BH, int L,
                                        int dv, float eps, float* dq, float* dk, float* dvo, float* g_ws,
                                        float* h_ws, hipStream_t st) {
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* vv = static_cast<const uint16_t*>(v);
    if (dv == 64) launch_both<64>(qq, kk, vv, dy, BH, L, eps, dq, dk, dvo, g_ws, h_ws, st);
    else launch_both<128>(qq, kk, vv, dy, BH, L, eps, dq, dk, dvo, g_ws, h_ws, st);
    return hipGetLastError();
}

}  // namespace based

// prefill_backward_mfma.hip -- gradients of causal Taylor linear attention on
// the gfx950 matrix cores (bf16 inputs, feature dim 16, fp32 accumulation),
// in two forms: the direct form below (pair by pair, O(L^2) per head) and the
// chunked form further down (linear in L through the carried state; d_v 64,
// and 128 as one pass per column half).
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

// A [64][W] bf16 tile (rows row0.. of a [L][ld] matrix, ld = W unless
// given, rows past L zero) held in registers across the workgroup, 16 bytes
// per piece: loaded from global memory while the previous tile is in use,
// then stored to LDS in the tile_at<W> layout.
template <int W>
struct TileRegs {
    static constexpr int kU = W / 8;                    // pieces per row
    static constexpr int kPer = (kT * kU + 255) / 256;  // pieces per thread
    u32x4 x[kPer];

    __device__ __forceinline__ void load(const uint16_t* mat, int L, int row0, int ld = W) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = threadIdx.x + 256 * i, row = e / kU, u = e % kU;
            x[i] = u32x4{0u, 0u, 0u, 0u};
            if (e < kT * kU && row0 + row < L)
                x[i] = *reinterpret_cast<const u32x4*>(mat + (size_t)(row0 + row) * ld + 8 * u);
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
    // On the diagonal tile, key pair p (tiles 2p, 2p + 1) meets this wave's
    // queries only if 2p <= w (w is wave-uniform).
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        if (DIAG && 2 * (kt >> 1) > w) continue;
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
        if (DIAG && 2 * p > w) continue;
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
        if (DIAG && 2 * (kt >> 1) > w) continue;  // as in q_pass1
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
        if (DIAG && 2 * p > w) continue;
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
    // On the diagonal tile, query pair p (tiles 2p, 2p + 1) meets this
    // wave's keys only if 2p + 1 >= w (w is wave-uniform).
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
        if (DIAG && 2 * (qt >> 1) + 1 < w) continue;
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
        if (DIAG && 2 * p + 1 < w) continue;
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

// ================================================================ chunked form
// The same gradients in time linear in L, through the recurrent form of the
// output ("Simple linear attention language models balance the
// recall-throughput tradeoff", s2 "Preliminaries": the prefix state
// S_i = sum_{j<=i} phi(k_j) v_j^T, z_i = sum_{j<=i} phi(k_j)):
//   dq_i = J(q_i)^T (S_i g_i + h_i z_i),
//   dk_j = J(k_j)^T (R_j v_j + r_j),   dv_j = R_j^T phi(k_j),
// with R_j = sum_{i>=j} phi(q_i) g_i^T and r_j = sum_{i>=j} phi(q_i) h_i.
// Pairs inside one 64-token chunk are the direct form's diagonal tile
// (q_pass1, q_pass2 and k_tile above); the carried state stands for the
// earlier chunks (S, z) or the later ones (R, r).
//
// Features are the symmetric monomials m(x) of the raw 16-vector x, in ten
// rotation tiles of 16 rows (slot (t, r)):
//   t = 0: x_r^2;  t = 1..7: x_r x_((r+t) mod 16);  t = 8: x_r x_(r+8) on
//   rows r < 8, the constant 1 on row 8, nothing on rows 9..15;  t = 9: x_r.
// Each unordered pair a != b appears once (one of (b - a) mod 16 and its
// complement lies in 1..8).  With the coefficients c = 1/32 (squares), 1/16
// (pairs), 1/4 (linear terms) and 1 (constant), sum_f c_f m_f(q) m_f(k) is
// 1 + s + s^2/2 for s = q.k/4.  The states hold raw monomial sums; the
// coefficients, powers of two and so exact, are applied when a state is
// published to LDS (S^c = c S, z^c = c z and likewise for R, r).  Then
// y_i D_i = m(q_i) S^c + intra, D_i = m(q_i) z^c + intra + eps, and
// J(q)^T (S g + h z) above becomes J_m(q)^T (S^c g + h z^c) with J_m the
// Jacobian of the raw monomials (likewise for k with R^c, r^c).
//
// Three products on the matrix cores (16x16x32 bf16, fp32 accumulation):
//   update       state += m(X)^T M over a chunk's tokens (M = V or g): lane
//                (g, r) builds feature row r for 8 tokens of a k-step from a
//                transposed read of X and its DPP row rotations;
//   readout      Y = m(X) S^c for a wave's 16 tokens (A = the lane's token's
//                features, B = the published state);
//   contraction  U = M S^c^T (A = rows of M, B = the published state by
//                transposed reads), then J_m^T U on the vector ALUs with DPP
//                row rotations (lane r = feature row r = component r).
// Every operand that is not an exact bf16 input is a bf16 hi/lo pair
// (features, g, published states): with single bf16 operands the gradients
// of early tokens, where D is small, miss the tolerance.
//
// Launches (segments of cps chunks; one workgroup per (segment, head)):
//   1. segment sums of m(k) v^T and m(k) (every segment but the last);
//   2. exclusive prefix over the segments: S, z at each segment start;
//   3. query sweep, chunk by chunk: y and D, g and h (to the workspace), dq;
//   4. segment sums of m(q) g^T and m(q) h (every segment but the first);
//   5. exclusive suffix over the segments: R, r after each segment;
//   6. key sweep, last chunk first: dk, dv.
// With one segment per head, 1, 2, 4 and 5 are skipped; with at most
// kFoldSegments segments, 2 and 5 are: each sweep adds up the earlier (or
// later) segments' sums itself when it loads its carried-in state.
constexpr int kNTile = 10;
constexpr int kSlot = 16 * kNTile;                   // 160 state rows
constexpr int kStateFloats = kSlot * 64 + kSlot;     // one (segment, head) state, d_v = 64

// Value of lane (r - N) mod 16 of this lane's 16-lane row (1 <= N <= 15).
// A rotation reads a valid lane everywhere, so no old value is kept (a
// kept old value would cost a register move before every rotation).
template <int N>
__device__ __forceinline__ float ror16(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xf, 0xf, true));
}

// Coefficient of slot (t, row).
__device__ __forceinline__ float slot_coef(int t, int row) {
    if (t == 0) return 1.f / 32.f;
    if (t < 8) return 1.f / 16.f;
    if (t == 9) return 0.25f;
    return row < 8 ? 1.f / 16.f : (row == 8 ? 1.f : 0.f);
}
// Published position of slot (t, row): the readout's k-step J covers tiles
// 2J and 2J + 1, its k = 8g + i being row 4g + (i & 3) of tile 2J + (i >> 2).
__device__ __forceinline__ int slot_pos(int t, int row) {
    return 32 * (t >> 1) + 8 * (row >> 2) + 4 * (t & 1) + (row & 3);
}
// A published plane holds value column c at row c (160 bf16 per row),
// position p at 16-byte unit (p >> 3) XOR ((c >> 2) & 3), so that the
// readout's 16-byte reads (16 columns, one unit), the contraction's
// transposed reads (4 columns x 4 units) and the publish writes (16
// columns) each hit 16 distinct 4-bank groups (PubLane below).

// Per-lane LDS offsets into a published plane, fixed for the kernel: with
// them every access of the readout, the publish and the contraction is the
// lane's offset plus a constant.
//  - rw: column r at unit g, swizzled: readout k-step J and column tile ct
//    read rw + 2560 ct + 32 J; publish of tile t at column tile ct writes
//    rw + 2560 ct + 32 (t >> 1) + 4 (t & 1).
//  - tr[h]: the contraction's transposed read of rows 8g + 4h + j (j =
//    c16 / 4) at slot group 4 (c16 % 4); tile T, k-step cs read
//    tr[h] + 5120 cs + 32 (T >> 1) + 4 (T & 1).
struct PubLane {
    int rw, tr[2], zp;
    __device__ __forceinline__ PubLane(int g, int r) {
        rw = r * kSlot + ((g ^ (r >> 2)) << 3);
        const int j = r >> 2, qq = r & 3;
#pragma unroll
        for (int h = 0; h < 2; ++h) tr[h] = (8 * g + 4 * h + j) * kSlot + ((qq ^ ((2 * g + h) & 3)) << 3);
        zp = 8 * (r >> 2) + (r & 3);  // slot_pos(T, r) - 32 (T >> 1) - 4 (T & 1)
    }
};

// A state published for the readout and the contraction.
struct PubState {
    alignas(16) uint16_t hi[64 * kSlot];
    alignas(16) uint16_t lo[64 * kSlot];
    alignas(16) uint16_t zhi[kSlot];  // normaliser, position order
    alignas(16) uint16_t zlo[kSlot];
    alignas(16) float z[kSlot];
};

// ---- update: feature rows of one tile for 8 tokens (x[i] = x_r of token i)
template <int T>
__device__ __forceinline__ void mono_rows(const float (&x)[8], int r, float (&a)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if constexpr (T == 0) {
            a[i] = x[i] * x[i];
        } else if constexpr (T < 8) {
            a[i] = x[i] * ror16<16 - T>(x[i]);
        } else if constexpr (T == 8) {
            const float p = x[i] * ror16<8>(x[i]);
            a[i] = r < 8 ? p : (r == 8 ? 1.f : 0.f);
        } else {
            a[i] = x[i];
        }
    }
}

__device__ __forceinline__ void unpack_b8(const bf16x8& b, float (&x)[8]) {
    const u32x4 u = __builtin_bit_cast(u32x4, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16lo_f32(u[i]);
        x[2 * i + 1] = bf16hi_f32(u[i]);
    }
}

// One tile T of the update at k-step ks: acc[ct] += m(X)_T^T M for the
// column tiles [CT0, CT0 + NCT), and zacc += sum_i m_i w_i (if ZSUM).
template <int T, int CT0, int NCT, bool MHILO, bool ZSUM>
__device__ __forceinline__ void update_tile(const float (&x)[8], const float (&w8)[8], const bf16x8 (&bh)[4],
                                            const bf16x8 (&bl)[4], int r, f32x4* acc, float& zacc) {
    float a[8];
    mono_rows<T>(x, r, a);
    if constexpr (ZSUM) {
        // key side (M exact): the plain feature sums; query side: weighted by h
#pragma unroll
        for (int i = 0; i < 8; ++i) zacc = MHILO ? fmaf(a[i], w8[i], zacc) : zacc + a[i];
    }
    bf16x8 ah, al;
    hilo8(a, ah, al);
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
        acc[j] = mfma32(ah, bh[CT0 + j], acc[j]);
        acc[j] = mfma32(al, bh[CT0 + j], acc[j]);
        if constexpr (MHILO) acc[j] = mfma32(ah, bl[CT0 + j], acc[j]);
    }
}

// The update of wave W over one staged chunk (d_v = 64).  Wave W owns
// tiles 2W and 2W + 1 at every column tile (acc[0..3], acc[4..7]) and tile
// 8 + W/2 at column tiles 2(W%2), 2(W%2) + 1 (acc[8], acc[9]); zacc[0..2]
// are the matching normaliser rows (the third only on even W, so that each
// row is summed once).  X is [64][16] in tile_at<16> layout, M [64][64] in
// tile_at<64> layout (hi, and lo if MHILO).  The key side (M = V, exact)
// sums plain features: padded tokens have x = 0 and v = 0, so only the
// constant row counts them, and that row is replaced by the token count
// when published or stored.  The query side (M = g hi/lo) weights the
// normaliser by h (wtok, LDS), zero on padded tokens.
template <int W, bool MHILO>
__device__ __forceinline__ void update_wave(const uint16_t* xt, const uint16_t* mhi, const uint16_t* mlo,
                                            const float* wtok, int g, int r, f32x4 (&acc)[10], float (&zacc)[3]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        float x[8], w8[8];
        unpack_b8(tr_b8<kD>(xt, 32 * ks, 0, g, r), x);
        if constexpr (MHILO) {
            const f32x4 w0 = *reinterpret_cast<const f32x4*>(&wtok[32 * ks + 4 * g]);
            const f32x4 w1 = *reinterpret_cast<const f32x4*>(&wtok[32 * ks + 16 + 4 * g]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w8[i] = w0[i];
                w8[4 + i] = w1[i];
            }
        }
        bf16x8 bh[4], bl[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            bh[ct] = tr_b8<64>(mhi, 32 * ks, 16 * ct, g, r);
            if constexpr (MHILO) bl[ct] = tr_b8<64>(mlo, 32 * ks, 16 * ct, g, r);
        }
        update_tile<2 * W, 0, 4, MHILO, true>(x, w8, bh, bl, r, &acc[0], zacc[0]);
        update_tile<2 * W + 1, 0, 4, MHILO, true>(x, w8, bh, bl, r, &acc[4], zacc[1]);
        update_tile<8 + W / 2, 2 * (W % 2), 2, MHILO, W % 2 == 0>(x, w8, bh, bl, r, &acc[8], zacc[2]);
    }
}
template <bool MHILO>
__device__ __forceinline__ void update_any(int w, const uint16_t* xt, const uint16_t* mhi, const uint16_t* mlo,
                                           const float* wtok, int g, int r, f32x4 (&acc)[10], float (&zacc)[3]) {
    switch (w) {
        case 0: update_wave<0, MHILO>(xt, mhi, mlo, wtok, g, r, acc, zacc); break;
        case 1: update_wave<1, MHILO>(xt, mhi, mlo, wtok, g, r, acc, zacc); break;
        case 2: update_wave<2, MHILO>(xt, mhi, mlo, wtok, g, r, acc, zacc); break;
        default: update_wave<3, MHILO>(xt, mhi, mlo, wtok, g, r, acc, zacc); break;
    }
}

// Tile t and column tile ct of the acc index j of wave w (see update_wave).
__device__ __forceinline__ int acc_tile(int w, int j) { return j < 8 ? 2 * w + (j >> 2) : 8 + (w >> 1); }
__device__ __forceinline__ int acc_ct(int w, int j) { return j < 8 ? (j & 3) : 2 * (w & 1) + (j - 8); }
__device__ __forceinline__ int z_tile(int w, int i) { return i < 2 ? 2 * w + i : 8 + (w >> 1); }
__device__ __forceinline__ bool z_owned(int w, int i) { return i < 2 || (w & 1) == 0; }

// Publish the wave's part of the state (times the slot coefficients) as
// bf16 hi/lo planes, and its normaliser rows (the lane-group partial sums
// added up) in fp32 and hi/lo.
// zconst >= 0 replaces the constant feature's normaliser row (the number of
// tokens summed, which the key-side update counts with the padding).
template <int W>
__device__ __forceinline__ void publish_wave(const f32x4 (&acc)[10], const float (&zacc)[3], PubState& ps,
                                             const PubLane& pl, int g, int r, float zconst) {
#pragma unroll
    for (int j = 0; j < 10; ++j) {
        const int t = j < 8 ? 2 * W + (j >> 2) : 8 + (W >> 1), ct = j < 8 ? (j & 3) : 2 * (W & 1) + (j - 8);
        float v[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) v[m] = slot_coef(t, 4 * g + m) * acc[j][m];
        const uint32_t h0 = pack_bf16x2(v[0], v[1]), h1 = pack_bf16x2(v[2], v[3]);
        const int off = pl.rw + 2560 * ct + 32 * (t >> 1) + 4 * (t & 1);
        *reinterpret_cast<uint2*>(&ps.hi[off]) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(&ps.lo[off]) = make_uint2(lo_pair_of(h0, v[0], v[1]), lo_pair_of(h1, v[2], v[3]));
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        if (i == 2 && (W & 1)) continue;
        float zt = zacc[i] + __shfl_xor(zacc[i], 16, 64);
        zt += __shfl_xor(zt, 32, 64);
        const int t = i < 2 ? 2 * W + i : 8 + (W >> 1);
        if (t == 8 && r == 8 && zconst >= 0.f) zt = zconst;
        if (g == 0) {
            const int p = slot_pos(t, r);
            const float zc = slot_coef(t, r) * zt;
            const uint32_t hp = pack_bf16x2(zc, 0.f);
            ps.z[p] = zc;
            ps.zhi[p] = (uint16_t)(hp & 0xffffu);
            ps.zlo[p] = (uint16_t)(pack_bf16x2(zc - bf16lo_f32(hp), 0.f) & 0xffffu);  // zc - hi is exact
        }
    }
}
__device__ __forceinline__ void publish_state(int w, const f32x4 (&acc)[10], const float (&zacc)[3], PubState& ps,
                                              const PubLane& pl, int g, int r, float zconst) {
    switch (w) {
        case 0: publish_wave<0>(acc, zacc, ps, pl, g, r, zconst); break;
        case 1: publish_wave<1>(acc, zacc, ps, pl, g, r, zconst); break;
        case 2: publish_wave<2>(acc, zacc, ps, pl, g, r, zconst); break;
        default: publish_wave<3>(acc, zacc, ps, pl, g, r, zconst); break;
    }
}

// A (segment, head) state in the workspace: raw sums S[f][c] (f = 16t + row)
// then z[f], fp32.
__device__ __forceinline__ void state_load(int w, const float* slot, int g, int r, f32x4 (&acc)[10],
                                           float (&zacc)[3]) {
#pragma unroll
    for (int j = 0; j < 10; ++j) {
        const int t = acc_tile(w, j), ct = acc_ct(w, j);
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[j][m] = slot ? slot[(16 * t + 4 * g + m) * 64 + 16 * ct + r] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 3; ++i)
        zacc[i] = slot && g == 0 && z_owned(w, i) ? slot[kSlot * 64 + 16 * z_tile(w, i) + r] : 0.f;
}
// The sum of n states at first, first + step, ... (n = 0: zero): a
// sweep's carried-in state straight from the segment sums, without a scan
// launch, when there are few segments.
__device__ __forceinline__ void state_load_sum(int w, const float* first, size_t step, int n, int g, int r,
                                               f32x4 (&acc)[10], float (&zacc)[3]) {
    state_load(w, n > 0 ? first : nullptr, g, r, acc, zacc);
    for (int i = 1; i < n; ++i) {
        f32x4 a2[10];
        float z2[3];
        state_load(w, first + i * step, g, r, a2, z2);
#pragma unroll
        for (int j = 0; j < 10; ++j) acc[j] += a2[j];
#pragma unroll
        for (int j = 0; j < 3; ++j) zacc[j] += z2[j];
    }
}
__device__ __forceinline__ void state_store(int w, const f32x4 (&acc)[10], const float (&zacc)[3], float* slot,
                                            int g, int r, float zconst) {
#pragma unroll
    for (int j = 0; j < 10; ++j) {
        const int t = acc_tile(w, j), ct = acc_ct(w, j);
#pragma unroll
        for (int m = 0; m < 4; ++m) slot[(16 * t + 4 * g + m) * 64 + 16 * ct + r] = acc[j][m];
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        float zt = zacc[i] + __shfl_xor(zacc[i], 16, 64);
        zt += __shfl_xor(zt, 32, 64);
        if (z_tile(w, i) == 8 && r == 8 && zconst >= 0.f) zt = zconst;
        if (g == 0 && z_owned(w, i)) slot[kSlot * 64 + 16 * z_tile(w, i) + r] = zt;
    }
}

// ---- readout: Y (rows = the wave's tokens 4g + m, columns 16ct + r) +=
// m(x) S^c, and D - eps += m(x) z^c (every column) if WITH_D.
// xr[j] = x_((j + 4g) mod 16) of the lane's token (row r of the wave).
template <int J>
__device__ __forceinline__ void mono_readout(const float (&xr)[16], int g, float (&a)[8]) {
    constexpr int T0 = 2 * J, T1 = 2 * J + 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (T0 == 0) a[i] = xr[i] * xr[i];
        else if constexpr (T0 < 8) a[i] = xr[i] * xr[i + T0];
        else a[i] = g < 2 ? xr[i] * xr[i + 8] : ((g == 2 && i == 0) ? 1.f : 0.f);
        if constexpr (T1 < 8) a[4 + i] = xr[i] * xr[i + T1];
        else a[4 + i] = xr[i];
    }
}
template <int J, bool WITH_D>
__device__ __forceinline__ void readout_step(const PubState& ps, const PubLane& pl, const float (&xr)[16], int g,
                                             f32x4 (&y)[4], f32x4& dsum) {
    float a[8];
    mono_readout<J>(xr, g, a);
    bf16x8 ah, al;
    hilo8(a, ah, al);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int off = pl.rw + 2560 * ct + 32 * J;
        const bf16x8 bh = ld8(&ps.hi[off]), bl = ld8(&ps.lo[off]);
        y[ct] = mfma32(ah, bh, y[ct]);
        y[ct] = mfma32(al, bh, y[ct]);
        y[ct] = mfma32(ah, bl, y[ct]);
    }
    if constexpr (WITH_D) {
        const bf16x8 zh = ld8(&ps.zhi[32 * J + 8 * g]), zl = ld8(&ps.zlo[32 * J + 8 * g]);
        dsum = mfma32(ah, zh, dsum);
        dsum = mfma32(al, zh, dsum);
        dsum = mfma32(ah, zl, dsum);
    }
}
template <bool WITH_D>
__device__ __forceinline__ void readout(const PubState& ps, const PubLane& pl, const float (&xr)[16], int g,
                                        f32x4 (&y)[4], f32x4& dsum) {
    readout_step<0, WITH_D>(ps, pl, xr, g, y, dsum);
    readout_step<1, WITH_D>(ps, pl, xr, g, y, dsum);
    readout_step<2, WITH_D>(ps, pl, xr, g, y, dsum);
    readout_step<3, WITH_D>(ps, pl, xr, g, y, dsum);
    readout_step<4, WITH_D>(ps, pl, xr, g, y, dsum);
}

// ---- contraction and Jacobian
// B operand of U = M S^c^T for tile T and k-step cs: lane (g, c16) gets
// columns 32cs + 8g + i of slot (T, c16).  Each transposed read hands lane
// c16 rows j = 0..3 of the element that lane 4j + c16/4 addressed at its
// position c16 % 4, so lane 4j + q addresses column c0 + j at the four
// consecutive positions of slots (T, 4q .. 4q + 3).
template <int T>
__device__ __forceinline__ bf16x8 pub_tr(const uint16_t* plane, const PubLane& pl, int cs) {
    constexpr int kc = 32 * (T >> 1) + 4 * (T & 1);
    const uint2 a = __builtin_bit_cast(
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(BWD_LDS(s16x4, plane + pl.tr[0] + 5120 * cs + kc)));
    const uint2 b = __builtin_bit_cast(
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(BWD_LDS(s16x4, plane + pl.tr[1] + 5120 * cs + kc)));
    return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// dx[m] += J_m(x)^T u for tile T: lane (g, r) holds u[m] at slot (T, r) of
// token 4g + m and xj[m] = x_r of that token; dx[m] is component r.
template <int T>
__device__ __forceinline__ void jac_tile(const f32x4& u, const float (&xj)[4], int r, float (&dx)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float uu = u[m];
        if constexpr (T == 0) {
            dx[m] = fmaf(2.f * xj[m], uu, dx[m]);
        } else if constexpr (T < 8) {
            // x_r x_(r+T): d/dx_r = x_(r+T) here, d/dx_(r+T) = x_r moved T lanes on
            dx[m] = fmaf(ror16<16 - T>(xj[m]), uu, dx[m]);
            dx[m] += ror16<T>(xj[m] * uu);
        } else if constexpr (T == 8) {
            const float u8 = r < 8 ? uu : 0.f;
            dx[m] = fmaf(ror16<8>(xj[m]), u8, dx[m]);
            dx[m] += ror16<8>(xj[m] * u8);
        } else {
            dx[m] += uu;
        }
    }
}

template <int T, bool AHILO>
__device__ __forceinline__ void contract_tile(const PubState& ps, const PubLane& pl, const bf16x8 (&ah)[2],
                                              const bf16x8 (&al)[2], const float (&zw)[4], const float (&xj)[4],
                                              int r, float (&dx)[4]) {
    f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
        const bf16x8 bh = pub_tr<T>(ps.hi, pl, cs), bl = pub_tr<T>(ps.lo, pl, cs);
        u = mfma32(ah[cs], bh, u);
        u = mfma32(ah[cs], bl, u);
        if constexpr (AHILO) u = mfma32(al[cs], bh, u);
    }
    const float zc = ps.z[pl.zp + 32 * (T >> 1) + 4 * (T & 1)];
#pragma unroll
    for (int m = 0; m < 4; ++m) u[m] = fmaf(zw[m], zc, u[m]);
    jac_tile<T>(u, xj, r, dx);
}
// dx += J_m^T (M S^c^T + zw z^c) over all ten tiles.  M's rows are the
// wave's tokens: ah/al[cs] = M[row r][32cs + 8g .. +7] (hi/lo if AHILO).
// (A loop over the tiles rather than an unrolled sequence: unrolled, the
// compiler issues every tile's LDS reads up front and runs out of
// registers.)
template <bool AHILO>
__device__ __forceinline__ void contract_all(const PubState& ps, const PubLane& pl, const bf16x8 (&ah)[2],
                                             const bf16x8 (&al)[2], const float (&zw)[4], const float (&xj)[4],
                                             int r, float (&dx)[4]) {
#pragma unroll 1
    for (int t = 0; t < kNTile; ++t) {
        switch (t) {
            case 0: contract_tile<0, AHILO>(ps, pl, ah, al, zw, xj, r, dx); break;
            case 1: contract_tile<1, AHILO>(ps, pl, ah, al, zw, xj, r, dx); break;
            case 2: contract_tile<2, AHILO>(ps, pl, ah, al, zw, xj, r, dx); break;
            case 3: contract_tile<3, AHILO>(ps, pl, ah, al, zw, xj, r, dx); break;
            case 4: contract_tile<4, AHILO>(ps, pl, ah, al, zw, xj, r, dx); break;
            case 5: contract_tile<5, AHILO>(ps, pl, ah, al, zw, xj, r, dx); break;
            case 6: contract_tile<6, AHILO>(ps, pl, ah, al, zw, xj, r, dx); break;
            case 7: contract_tile<7, AHILO>(ps, pl, ah, al, zw, xj, r, dx); break;
            case 8: contract_tile<8, AHILO>(ps, pl, ah, al, zw, xj, r, dx); break;
            default: contract_tile<9, AHILO>(ps, pl, ah, al, zw, xj, r, dx); break;
        }
    }
}

// The global-memory inputs of one wave's 16 tokens for a chunk, loaded one
// chunk ahead of their use: this lane's token row rotated by 4g (pieces of
// 4 dims), x_r of tokens base + 4g + m, and the 4 dims 4g..4g+3 of the
// lane's token (the score operand).  Zero past L.
struct TokenRegs {
    uint2 rot[4];
    uint16_t xj[4];
    uint2 sc;
    __device__ __forceinline__ void load(const uint16_t* xh, int tok, int base, int L, int g, int r) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            rot[pp] = make_uint2(0u, 0u);
            if (tok < L) rot[pp] = *reinterpret_cast<const uint2*>(xh + (size_t)tok * kD + 4 * ((pp + g) & 3));
        }
        // the score operand is piece g of the row, which is rot[0]
        sc = rot[0];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int t = base + 4 * g + m;
            xj[m] = t < L ? xh[(size_t)t * kD + r] : (uint16_t)0;
        }
    }
    // xr[j] = x_((j + 4g) mod 16) of the lane's token; xj[m] = x_r of token 4g + m
    __device__ __forceinline__ void unpack(float (&xr)[16], float (&xjf)[4]) const {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            xr[4 * pp] = bf16lo_f32(rot[pp].x);
            xr[4 * pp + 1] = bf16hi_f32(rot[pp].x);
            xr[4 * pp + 2] = bf16lo_f32(rot[pp].y);
            xr[4 * pp + 3] = bf16hi_f32(rot[pp].y);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) xjf[m] = bf16_bits_to_f32(xj[m]);
    }
};

// Make this wave's LDS writes visible to its own later reads (no other
// wave takes part): LDS serves one wave's accesses in order, so only the
// compiler's ordering is at stake.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------- segment sums
// Launch 1 (KEYS: m(k) v^T, m(k) over the valid tokens) or 4 (m(q) g^T,
// m(q) h) for segments seg0 .. seg0 + gridDim.x/BH - 1.
template <bool KEYS>
__global__ __launch_bounds__(256) void bwd_segsum_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ mhi,
                                                         const uint16_t* __restrict__ mlo,
                                                         const float* __restrict__ hw, int BH, int L, int ldv,
                                                         int nch, int cps, int seg0, float* __restrict__ states) {
    __shared__ BwdKSmem<64> sm[2];  // per chunk parity; q: X, ghi/glo: M, h: token weights
    const int head = blockIdx.x % BH, seg = seg0 + (int)(blockIdx.x / BH);
    const int c_begin = seg * cps, c_end = min(nch, c_begin + cps);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const uint16_t* xh = x + (size_t)head * L * kD;
    const uint16_t* mh = KEYS ? mhi + (size_t)head * L * ldv : mhi + (size_t)head * L * 64;
    const uint16_t* ml = KEYS ? nullptr : mlo + (size_t)head * L * 64;
    const float* hh = KEYS ? nullptr : hw + (size_t)head * L;
    f32x4 acc[10];
    float zacc[3];
    state_load(w, nullptr, g, r, acc, zacc);
    TileRegs<kD> xreg;
    TileRegs<64> mreg, lreg;
    float hreg = 0.f;
    auto load = [&](int c) {
        xreg.load(xh, L, c * kT);
        mreg.load(mh, L, c * kT, KEYS ? ldv : 64);
        if (!KEYS) {
            lreg.load(ml, L, c * kT);
            if (threadIdx.x < kT) hreg = c * kT + (int)threadIdx.x < L ? hh[c * kT + threadIdx.x] : 0.f;
        }
    };
    auto store = [&](BwdKSmem<64>& b) {
        xreg.store(b.q);
        mreg.store(b.ghi);
        if (!KEYS) {
            lreg.store(b.glo);
            if (threadIdx.x < kT) b.h[threadIdx.x] = hreg;
        }
    };
    // chunk c is staged in sm[c & 1] one iteration ahead, its global loads
    // two iterations ahead; one barrier per chunk
    load(c_begin);
    store(sm[c_begin & 1]);
    if (c_begin + 1 < c_end) load(c_begin + 1);
    for (int c = c_begin; c < c_end; ++c) {
        __syncthreads();
        if (c + 1 < c_end) {
            store(sm[(c + 1) & 1]);
            if (c + 2 < c_end) load(c + 2);
        }
        const BwdKSmem<64>& b = sm[c & 1];
        update_any<!KEYS>(w, b.q, b.ghi, b.glo, b.h, g, r, acc, zacc);
    }
    state_store(w, acc, zacc, states + ((size_t)seg * BH + head) * kStateFloats, g, r,
                KEYS ? (float)(min(L, c_end * kT) - c_begin * kT) : -1.f);
}

// Launches 2 and 5: each (segment, head) state becomes the sum of the
// states of the segments before it (REVERSE: after it).  Segments without
// a sum of their own (the last one forward, the first one in reverse)
// count as zero.
__global__ __launch_bounds__(256) void bwd_scan_kernel(float* __restrict__ states, int BH, int nseg, int reverse) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)BH * kStateFloats) return;
    const size_t head = i / kStateFloats, e = i % kStateFloats;
    float run = 0.f;
    for (int n = 0; n < nseg; ++n) {
        const int s = reverse ? nseg - 1 - n : n;
        float* p = states + ((size_t)s * BH + head) * kStateFloats + e;
        const bool has = reverse ? s > 0 : s < nseg - 1;
        const float xv = has ? *p : 0.f;
        *p = run;
        run += xv;
    }
}

// ---------------------------------------------------------------- query sweep
// kSweepBuf = 2: the staged chunk and the published state double-buffered
// by chunk parity, one barrier per chunk, but 1 workgroup per CU by LDS;
// kSweepBuf = 1: single buffers and a second barrier before they are
// rewritten, 2 workgroups per CU.  A sweep is a chain of dependent steps,
// so the second workgroup's latency hiding wins (about 1.4x measured on
// the 360M-shaped layer).
constexpr int kSweepBuf = 1;
__device__ __forceinline__ int sbuf(int c) { return c & (kSweepBuf - 1); }
struct QSweepSmem {
    BwdQSmem<64> t[kSweepBuf];
    PubState s[kSweepBuf];
};

__global__ __launch_bounds__(256, 3 - kSweepBuf) void bwd_qsweep_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const float* __restrict__ dy, int BH, int L, int ldv,
                                                         int nch, int cps, float eps, const float* __restrict__ s_init,
                                                         int fold, int accumulate, float* __restrict__ dq,
                                                         uint16_t* __restrict__ ghi_ws,
                                                         uint16_t* __restrict__ glo_ws, float* __restrict__ h_ws) {
    constexpr int DV = 64, kNV = 4;
    __shared__ QSweepSmem sm;
    const int head = blockIdx.x % BH, seg = blockIdx.x / BH;
    const int c_begin = seg * cps, c_end = min(nch, c_begin + cps);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const uint16_t* qh = q + (size_t)head * L * kD;
    const uint16_t* kh = k + (size_t)head * L * kD;
    const uint16_t* vh = v + (size_t)head * L * ldv;

    f32x4 acc[10];
    float zacc[3];
    // the state before this segment: its scanned slot, or (fold) the sum of
    // the earlier segments' slots
    if (fold)
        state_load_sum(w, s_init ? s_init + (size_t)head * kStateFloats : nullptr, (size_t)BH * kStateFloats,
                       s_init ? seg : 0, g, r, acc, zacc);
    else
        state_load(w, s_init && seg > 0 ? s_init + ((size_t)seg * BH + head) * kStateFloats : nullptr, g, r, acc,
                   zacc);
    TileRegs<kD> kreg;
    TileRegs<DV> vreg;
    kreg.load(kh, L, c_begin * kT);
    vreg.load(vh, L, c_begin * kT, ldv);
    // this wave's queries, one chunk ahead
    TokenRegs qreg;
    auto load_q = [&](int c) {
        const int qw0 = c * kT + 16 * w;
        qreg.load(qh, qw0 + r, qw0, L, g, r);
    };
    load_q(c_begin);
    kreg.store(sm.t[sbuf(c_begin)].k);
    vreg.store(sm.t[sbuf(c_begin)].v);
    const PubLane pl(g, r);
    publish_state(w, acc, zacc, sm.s[sbuf(c_begin)], pl, g, r, (float)(c_begin * kT));
    __syncthreads();
    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * kT;
        BwdQSmem<DV>& tt = sm.t[sbuf(c)];
        const PubState& ss = sm.s[sbuf(c)];
        if (c + 1 < c_end) {
            kreg.load(kh, L, t0 + kT);
            vreg.load(vh, L, t0 + kT, ldv);
        }
        const int qw0 = t0 + 16 * w;  // first query of this wave
        float xr[16], xj[4];
        qreg.unpack(xr, xj);
        const bf16x4 qb = quarter(qreg.sc);  // this lane's query, dims 4g..4g+3, times 1/4
        // dy rows qw0 + 4g + m, columns 16ct + r (zero past L), in flight
        // during the products below
        float dyc[4][kNV];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int qi = qw0 + 4 * g + m;
            const float* dyr = dy + ((size_t)head * L + min(qi, L - 1)) * ldv + r;
#pragma unroll
            for (int ct = 0; ct < kNV; ++ct) dyc[m][ct] = qi < L ? dyr[16 * ct] : 0.f;
        }
        if (c + 1 < c_end) load_q(c + 1);

        // y D and D: the chunk's own keys (diagonal tile), then the state
        f32x4 yacc[kNV];
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) yacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 dsum = {0.f, 0.f, 0.f, 0.f};
        q_pass1<DV, true>(tt, qb, w, g, r, yacc, dsum);
        readout<true>(ss, pl, xr, g, yacc, dsum);

        // g = dy/D, h = -(dy.y D)/D^2 (rows qw0 + 4g + m, columns 16ct + r)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int qi = qw0 + 4 * g + m;
            const float inv = 1.f / (dsum[m] + eps);
            float dyy = 0.f, gv[kNV];
#pragma unroll
            for (int ct = 0; ct < kNV; ++ct) {
                dyy = fmaf(dyc[m][ct], yacc[ct][m], dyy);
                gv[ct] = dyc[m][ct] * inv;
            }
            // hi/lo pairs two columns at a time (one conversion per pair)
#pragma unroll
            for (int ct = 0; ct < kNV; ct += 2) {
                const uint32_t hb = pack_bf16x2(gv[ct], gv[ct + 1]);
                const uint32_t lb = lo_pair_of(hb, gv[ct], gv[ct + 1]);
                tt.ghi[w][tile_at<DV>(4 * g + m, 16 * ct + r)] = (uint16_t)(hb & 0xffffu);
                tt.ghi[w][tile_at<DV>(4 * g + m, 16 * ct + 16 + r)] = (uint16_t)(hb >> 16);
                tt.glo[w][tile_at<DV>(4 * g + m, 16 * ct + r)] = (uint16_t)(lb & 0xffffu);
                tt.glo[w][tile_at<DV>(4 * g + m, 16 * ct + 16 + r)] = (uint16_t)(lb >> 16);
            }
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) dyy += __shfl_xor(dyy, off, 64);
            const float hq = -dyy * inv * inv;
            if (r == 0) {
                tt.h[w][4 * g + m] = hq;
                if (qi < L) h_ws[(size_t)head * L + qi] = hq;
            }
        }
        wave_lds_fence();
        {
            constexpr int kU = DV / 8;
            for (int e = lane; e < 16 * kU; e += 64) {
                const int row = e / kU, u = e % kU;
                const int qi = qw0 + row;
                if (qi < L) {
                    const size_t off = ((size_t)head * L + qi) * DV + 8 * u;
                    *reinterpret_cast<u32x4*>(ghi_ws + off) =
                        *reinterpret_cast<const u32x4*>(&tt.ghi[w][tile_at<DV>(row, 8 * u)]);
                    *reinterpret_cast<u32x4*>(glo_ws + off) =
                        *reinterpret_cast<const u32x4*>(&tt.glo[w][tile_at<DV>(row, 8 * u)]);
                }
            }
        }

        // dq: the state part J_m^T (S^c g + h z^c), then the diagonal tile
        bf16x8 gah[2], gal[2];
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
            gah[cs] = ld8(&tt.ghi[w][tile_at<DV>(r, 32 * cs + 8 * g)]);
            gal[cs] = ld8(&tt.glo[w][tile_at<DV>(r, 32 * cs + 8 * g)]);
        }
        float hz[4], dx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) hz[m] = tt.h[w][4 * g + m];
        contract_all<true>(ss, pl, gah, gal, hz, xj, r, dx);
        f32x4 dqacc = {0.f, 0.f, 0.f, 0.f};
        q_pass2<DV, true>(tt, qb, w, g, r, dqacc);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int qi = qw0 + 4 * g + m;
            if (qi < L) {
                float* o = &dq[((size_t)head * L + qi) * kD + r];
                *o = fmaf(0.25f, dqacc[m], dx[m]) + (accumulate ? *o : 0.f);
            }
        }

        // the state after this chunk
        update_any<false>(w, tt.k, tt.v, nullptr, nullptr, g, r, acc, zacc);
        if (kSweepBuf == 1) __syncthreads();
        if (c + 1 < c_end) {
            kreg.store(sm.t[sbuf(c + 1)].k);
            vreg.store(sm.t[sbuf(c + 1)].v);
            publish_state(w, acc, zacc, sm.s[sbuf(c + 1)], pl, g, r, (float)(t0 + kT));
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- key sweep
struct KSweepSmem {
    BwdKSmem<64> t[kSweepBuf];
    PubState s[kSweepBuf];
};

__global__ __launch_bounds__(256, 3 - kSweepBuf) void bwd_ksweep_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, int BH, int L, int ldv,
                                                         int nch, int cps, const uint16_t* __restrict__ ghi_ws,
                                                         const uint16_t* __restrict__ glo_ws,
                                                         const float* __restrict__ h_ws,
                                                         const float* __restrict__ r_init, int fold, int accumulate,
                                                         float* __restrict__ dk,
                                                         float* __restrict__ dvo) {
    constexpr int DV = 64, kNV = 4;
    __shared__ KSweepSmem sm;
    const int head = blockIdx.x % BH, seg = blockIdx.x / BH;
    const int nseg = (nch + cps - 1) / cps;
    const int c_begin = seg * cps, c_end = min(nch, c_begin + cps);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const uint16_t* qh = q + (size_t)head * L * kD;
    const uint16_t* kh = k + (size_t)head * L * kD;
    const uint16_t* vh = v + (size_t)head * L * ldv;
    const uint16_t* gh = ghi_ws + (size_t)head * L * DV;
    const uint16_t* gl = glo_ws + (size_t)head * L * DV;
    const float* hh = h_ws + (size_t)head * L;

    f32x4 acc[10];
    float zacc[3];
    // the sums after this segment: its scanned slot, or (fold) the sum of
    // the later segments' slots
    if (fold)
        state_load_sum(w, r_init ? r_init + ((size_t)(seg + 1) * BH + head) * kStateFloats : nullptr,
                       (size_t)BH * kStateFloats, r_init ? nseg - 1 - seg : 0, g, r, acc, zacc);
    else
        state_load(w, r_init && seg < nseg - 1 ? r_init + ((size_t)seg * BH + head) * kStateFloats : nullptr, g, r,
                   acc, zacc);
    TileRegs<kD> qreg;
    TileRegs<DV> ghreg, glreg;
    float hreg = 0.f;
    auto load = [&](int c) {
        qreg.load(qh, L, c * kT);
        ghreg.load(gh, L, c * kT);
        glreg.load(gl, L, c * kT);
        if (threadIdx.x < kT) hreg = c * kT + (int)threadIdx.x < L ? hh[c * kT + threadIdx.x] : 0.f;
    };
    auto store = [&](BwdKSmem<DV>& b) {
        qreg.store(b.q);
        ghreg.store(b.ghi);
        glreg.store(b.glo);
        if (threadIdx.x < kT) b.h[threadIdx.x] = hreg;
    };
    // this wave's keys and their value rows, one chunk ahead
    TokenRegs kregs;
    u32x4 vrow[2];
    auto load_k = [&](int c) {
        const int kw0 = c * kT + 16 * w, kr = kw0 + r;
        kregs.load(kh, kr, kw0, L, g, r);
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
            vrow[cs] = u32x4{0u, 0u, 0u, 0u};
            if (kr < L) vrow[cs] = *reinterpret_cast<const u32x4*>(vh + (size_t)kr * ldv + 32 * cs + 8 * g);
        }
    };
    load(c_end - 1);
    load_k(c_end - 1);
    store(sm.t[sbuf(c_end - 1)]);
    const PubLane pl(g, r);
    publish_state(w, acc, zacc, sm.s[sbuf(c_end - 1)], pl, g, r, -1.f);
    __syncthreads();
    for (int c = c_end - 1; c >= c_begin; --c) {
        const int t0 = c * kT;
        const BwdKSmem<DV>& tt = sm.t[sbuf(c)];
        const PubState& ss = sm.s[sbuf(c)];
        if (c > c_begin) load(c - 1);
        const int kw0 = t0 + 16 * w;  // first key of this wave
        const bf16x4 kb = quarter(kregs.sc);  // this lane's key, dims 4g..4g+3, times 1/4
        bf16x8 vb[2];
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) vb[cs] = __builtin_bit_cast(bf16x8, vrow[cs]);
        float xr[16], xj[4];
        kregs.unpack(xr, xj);
        if (c > c_begin) load_k(c - 1);

        // dv: the chunk's own queries (diagonal tile), then m(k) R^c
        f32x4 dvacc[kNV];
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) dvacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 dkacc = {0.f, 0.f, 0.f, 0.f}, unused = {0.f, 0.f, 0.f, 0.f};
        k_tile<DV, true>(tt, kb, vb, w, g, r, dvacc, dkacc);
        readout<false>(ss, pl, xr, g, dvacc, unused);
        // dk: J_m^T (R^c v + r^c)
        const float ones[4] = {1.f, 1.f, 1.f, 1.f};
        float dx[4] = {0.f, 0.f, 0.f, 0.f};
        contract_all<false>(ss, pl, vb, vb, ones, xj, r, dx);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int kj = kw0 + 4 * g + m;
            if (kj < L) {
#pragma unroll
                for (int ct = 0; ct < kNV; ++ct) dvo[((size_t)head * L + kj) * ldv + 16 * ct + r] = dvacc[ct][m];
                float* o = &dk[((size_t)head * L + kj) * kD + r];
                *o = fmaf(0.25f, dkacc[m], dx[m]) + (accumulate ? *o : 0.f);
            }
        }

        // R, r with this chunk's queries
        update_any<true>(w, tt.q, tt.ghi, tt.glo, tt.h, g, r, acc, zacc);
        if (kSweepBuf == 1) __syncthreads();
        if (c > c_begin) {
            store(sm.t[sbuf(c - 1)]);
            publish_state(w, acc, zacc, sm.s[sbuf(c - 1)], pl, g, r, -1.f);
        }
        __syncthreads();
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

// ---------------------------------------------------------------- chunked launch plan
// Segments of cps chunks so that (segments x heads) fills the chip about
// twice with 256-thread workgroups.
static void chunk_plan(int BH, int L, int& nch, int& cps, int& nseg) {
    nch = (L + kT - 1) / kT;
    const long long want = ((long long)nch * BH + 511) / 512;
    cps = (int)(want < 1 ? 1 : want);
    nseg = (nch + cps - 1) / cps;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Up to this many segments the sweeps add up the segment sums themselves.
static constexpr int kFoldSegments = 8;

size_t prefill_backward_chunked_workspace_bytes(int BH, int L) {
    int nch, cps, nseg;
    chunk_plan(BH, L, nch, cps, nseg);
    const size_t base = align256((size_t)BH * L * (64 + 1) * sizeof(float));
    return nseg > 1 ? base + 2 * align256((size_t)nseg * BH * kStateFloats * sizeof(float)) : base;
}

// d_v = 128 runs the d_v = 64 pipeline on each half of the value columns:
// with half c's own y_c, g_c = dy_c / D and h_c = -(dy_c . y_c) / D (D does
// not depend on the columns), the gradients are linear in (g, h) = sums of
// the halves' terms, so dq and dk are the sums of the two passes' (the
// second pass adds into them) and dv is the two halves side by side.  The
// passes reuse the workspace one after the other on the stream.
hipError_t launch_prefill_backward_chunked(const void* q, const void* k, const void* v, const float* dy, int BH,
                                           int L, int dv, float eps, float* dq, float* dk, float* dvo,
                                           void* workspace, hipStream_t st) {
    int nch, cps, nseg;
    chunk_plan(BH, L, nch, cps, nseg);
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    char* base = static_cast<char*>(workspace);
    uint16_t* ghi = reinterpret_cast<uint16_t*>(base);
    uint16_t* glo = ghi + (size_t)BH * L * 64;
    float* h_ws = reinterpret_cast<float*>(glo + (size_t)BH * L * 64);
    const size_t sbytes = align256((size_t)nseg * BH * kStateFloats * sizeof(float));
    float* s_states = reinterpret_cast<float*>(base + align256((size_t)BH * L * (64 + 1) * sizeof(float)));
    float* r_states = reinterpret_cast<float*>(reinterpret_cast<char*>(s_states) + sbytes);
    const unsigned scan_blocks = (unsigned)(((size_t)BH * kStateFloats + 255) / 256);
    // With few segments each sweep sums the earlier (later) segments' slots
    // itself instead of a scan launch.
    const int fold = nseg <= kFoldSegments;
    for (int half = 0; half < dv / 64; ++half) {
        const uint16_t* vv = static_cast<const uint16_t*>(v) + 64 * half;
        const float* dyh = dy + 64 * half;
        float* dvh = dvo + 64 * half;
        if (nseg > 1) {
            hipLaunchKernelGGL((bwd_segsum_kernel<true>), dim3((unsigned)(BH * (nseg - 1))), dim3(256), 0, st, kk, vv,
                               nullptr, nullptr, BH, L, dv, nch, cps, 0, s_states);
            if (!fold) hipLaunchKernelGGL(bwd_scan_kernel, dim3(scan_blocks), dim3(256), 0, st, s_states, BH, nseg, 0);
        }
        hipLaunchKernelGGL(bwd_qsweep_kernel, dim3((unsigned)(BH * nseg)), dim3(256), 0, st, qq, kk, vv, dyh, BH, L,
                           dv, nch, cps, eps, nseg > 1 ? s_states : nullptr, fold, half, dq, ghi, glo, h_ws);
        if (nseg > 1) {
            hipLaunchKernelGGL((bwd_segsum_kernel<false>), dim3((unsigned)(BH * (nseg - 1))), dim3(256), 0, st, qq,
                               ghi, glo, h_ws, BH, L, 64, nch, cps, 1, r_states);
            if (!fold) hipLaunchKernelGGL(bwd_scan_kernel, dim3(scan_blocks), dim3(256), 0, st, r_states, BH, nseg, 1);
        }
        hipLaunchKernelGGL(bwd_ksweep_kernel, dim3((unsigned)(BH * nseg)), dim3(256), 0, st, qq, kk, vv, BH, L, dv,
                           nch, cps, ghi, glo, h_ws, nseg > 1 ? r_states : nullptr, fold, half, dk, dvh);
    }
    return hipGetLastError();
}

}  // namespace based

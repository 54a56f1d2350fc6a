// prefill_mfma_kernels.hpp -- chunked causal Taylor linear attention on the gfx950
// matrix cores (bf16 operands, fp32 accumulation), chunk length 64.
//
// Method: "Simple linear attention language models balance the
// recall-throughput tradeoff", App. B "Forward / Generation Prefill" and s5:
// the feature map and the causal dot product are fused (features never
// reach HBM); per chunk, the on-diagonal term uses the causally masked
// pairwise weights, the off-diagonal term reads the cumulative Taylor-order
// state, and the state is carried to the next chunk ("Gated Slot Attention
// ...", App. A, chunkwise form, has the same inter/intra split).
//
// MI355X design
//  * One workgroup of 12 waves per (batch, head, value-column group[,
//    sequence segment]) walks the 64-token chunks in order, one barrier
//    per chunk.  The state lives in MFMA accumulators (fp32) for the whole
//    sequence.  Waves w, w + 4 and w + 8 share a SIMD:
//      - waves 0..3, off-diagonal: psi(Q) of query tile w (16 rows) times
//        the state before the chunk, handed to the on-diagonal wave of the
//        same tile through LDS; they also stage Q and K of the next chunk;
//      - waves 4..7, update: rotation tiles w-4, w and (for w-4 < 2) w+4
//        of [S | z] += psi(K)^T [V | 1], then the state rounded to bf16
//        into LDS for the next chunk's readout; they stage V^T;
//      - waves 8..11, on-diagonal: the causal intra-chunk term of query
//        tile w-8, then (one chunk later) the sum with the hand-off, the
//        normalisation and the fp32 stores.  Only these waves store to
//        global memory, so the other waves' waits on the vector-memory
//        counter (which counts loads and stores in issue order) never
//        cover output stores.
//  * Symmetric features.  phi(q).phi(k) only needs the 136 distinct
//    products k_a k_b (a <= b) plus 16 linear terms and the constant:
//    153 feature rows, padded to 160 = 10 "rotation tiles" of 16 rows.
//    Tile t < 8 row r holds the pair (r, (r+t) mod 16); tile 8 holds the
//    pairs (r, r+8) for r < 8 and the constant in row 8; tile 9 holds the
//    linear terms.  Features are built from raw bf16 values; the pre-scale
//    d'^(-1/4) = 1/2, the 1/sqrt2 and the pair multiplicity are exact
//    powers of two (and one 1/sqrt2 pair) folded into the state scaling.
//  * psi(K)^T (row = feature, 8 tokens per lane) is formed in registers
//    with DPP row rotations: lane r of a 16-lane row holds k_r of its 8
//    tokens, and row_ror brings k_(r+t) from lane (r+t) mod 16.
//  * The normaliser z is an extra 16-column accumulator tile driven by a
//    ones operand, so phi(q).z and the on-diagonal row sums come out of the
//    same MFMAs in the same register layout as the numerator.
//  * Readout of chunk c uses the state before c, double-buffered in LDS.
//    The linear/constant rows (the last feature k-step) are stored as a
//    hi/lo bf16 pair and read against a single-bf16 psi(Q) (exact for the
//    constant and linear terms); the on-diagonal weights 1 + s + s^2/2
//    are a hi/lo bf16 pair.
//  * Q, K, V of chunk c+1 are fetched into registers two chunks ahead and
//    written to the other LDS buffer during chunk c (V and K transposed).
//
// This header holds the device code.  It is compiled in two units:
// prefill_mfma.hip (the launch plans and most kernel instances) and
// prefill_mfma_ilp.hip (the instances that the instruction-level-
// parallelism scheduler serves better; see there).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace based {
namespace {

constexpr int kC = 64;        // chunk length
constexpr int kSlots = 160;   // 10 rotation tiles x 16 feature rows
constexpr int kSRow = 176;    // LDS row stride (bf16) of the state operand [col][slot]
constexpr int kLoSlots = 32;  // slots of the last feature k-step (tiles 8, 9)
constexpr int kLoRow = 48;    // LDS row stride (bf16) of their lo parts
constexpr int kTRow = 64;     // LDS row stride (bf16) of V^T [col][token]
constexpr int kQRow = 24;     // LDS row stride (bf16) of Q and K [token][dim]
constexpr int kKtRow = 72;    // LDS row stride (fp32) of K^T/4 [dim][token]
constexpr int kQfRow = 16;    // LDS row stride (fp32) of Q [token][dim]
constexpr float kSqrt2 = 1.41421356237309504880f;

// Staging layouts.  Each row is cut into 16-byte units whose order is
// XOR-swizzled by a few row bits, chosen (by the gfx950 LDS bank mapping:
// 64 banks for 16-byte reads serviced 16 lanes at a time, 32 banks for
// writes) so that every read and write pattern below is conflict-free or
// at most two-way.  All vector accesses stay inside one unit.
__device__ __forceinline__ int vt_idx(int row, int tok) {  // V^T: 8 tokens per unit
    return row * kTRow + 8 * ((tok >> 3) ^ ((row >> 1) & 7)) + (tok & 7);
}
// Position in V^T of token t of a chunk: within each 32-token half, the
// 4-token groups g and g + 4 (tokens 4g..4g+3 and 16+4g..16+4g+3) sit side
// by side, the k-slice that lane group g of a 16x16x32 product takes on
// both the intra-chunk weights (two 16-key score tiles) and the update.
__device__ __forceinline__ int vt_pos(int t) {
    return (t & 32) | (((t >> 2) & 3) << 3) | (((t >> 4) & 1) << 2) | (t & 3);
}
__device__ __forceinline__ int kt_idx(int row, int tok) {  // K^T fp32: 4 tokens per unit
    return row * kKtRow + 4 * ((tok >> 2) ^ (row & 1)) + (tok & 3);
}
__device__ __forceinline__ int qf_idx(int row, int dim) {  // Q fp32: 4 dims per unit
    return row * kQfRow + 4 * ((dim >> 2) ^ ((row >> 1) & 3)) + (dim & 3);
}
__device__ __forceinline__ int qk_idx(int row, int dim) {  // Q, K bf16: 8 dims per unit
    return row * kQRow + 8 * ((dim >> 3) ^ ((row >> 3) & 1)) + (dim & 7);
}

template <int DV>
struct PrefillSmem {
    static_assert(DV == 32 || DV == 64, "column group width");
    static constexpr int kSBufs = 2;  // state operand buffers
    alignas(16) uint16_t q[2][kC * kQRow];
    alignas(16) uint16_t k[2][kC * kQRow];
    alignas(16) float ktf[2][kDFeat * kKtRow];  // K^T scaled by 1/4 (update waves)
    alignas(16) float qf[2][kC * kQfRow];       // Q as fp32 (readout features)
    alignas(16) uint16_t vt[2][DV * kTRow];
    alignas(16) uint16_t s_hi[kSBufs][DV * kSRow];
    alignas(16) uint16_t s_lo[kSBufs][DV * kLoRow];
    alignas(16) uint16_t z_hi[kSBufs][kSlots];
    alignas(16) uint16_t z_lo[kSBufs][kLoSlots];
    // off-diagonal hand-off: [chunk parity][query tile][column tile][lane] f32x4
    alignas(16) float hand[2][4][(DV / 16 + 1) * 64 * 4];
};

// ---- fused window branch (the hybrid layer): LDS of the four window waves.
// K of the window branch as [64][64] bf16 tiles (16-byte units XOR-swizzled
// by the row's low bits) and V (the workgroup's 32 value columns) as
// row-major [64][32], each in a ring of three chunks: c-1 and c in use,
// c+1 being written.  The normalised window output of chunk c goes to the
// on-diagonal wave of its query tile through `hand` (chunk parity).
constexpr int kWinD = 64;     // window q/k dim
constexpr int kWinCols = 32;  // value columns per workgroup of the fused layer
struct WinSmem {
    alignas(16) uint16_t k[3][kC * kWinD];
    alignas(16) uint16_t v[3][kC * kWinCols];
    alignas(16) float hand[2][4][2 * 64 * 4];  // [parity][query tile][column tile][lane] f32x4
};
struct WinNone {
    int unused;
};
__device__ __forceinline__ int win_idx(int row, int col) {
    return row * kWinD + 8 * ((col >> 3) ^ (row & 7)) + (col & 7);
}

enum { kModeFull = 0, kModeSegment = 2 };

template <int T, int DV>
__device__ __forceinline__ void ws_store(const f32x4 (&acc)[DV / 16 + 1], float* slot, int lane);
template <int T, int DV>
__device__ __forceinline__ void ws_load(f32x4 (&acc)[DV / 16 + 1], const float* slot, int lane, int slot_nct,
                                        int ct0);

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Value of lane (r - N) mod 16 of this lane's 16-lane row.
template <int N>
__device__ __forceinline__ float row_ror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

__device__ __forceinline__ bf16x8 pack8(const float (&a)[8]) {
    u32x4 u = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]),
               pack_bf16x2(a[6], a[7])};
    return __builtin_bit_cast(bf16x8, u);
}
// hi = bf16(a), lo = bf16(a - hi): a ~= hi + lo to ~16 mantissa bits.
__device__ __forceinline__ void pack8_hilo(const float (&a)[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = pack_bf16x2(a[2 * i], a[2 * i + 1]);
        l[i] = lo_pair_of(h[i], a[2 * i], a[2 * i + 1]);
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}
__device__ __forceinline__ void unpack8(const u32x4& u, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16lo_f32(u[i]);
        x[2 * i + 1] = bf16hi_f32(u[i]);
    }
}
__device__ __forceinline__ bf16x8 lds_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x4 lds_bf16x4(const uint16_t* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ bf16x8 ones8() {
    u32x4 u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    return __builtin_bit_cast(bf16x8, u);
}

// State operand layout.  The contraction index of readout k-step J
// (32 slots) is k = 8g + i: tile J (i < 4) or J + 4 (i >= 4) for J < 4,
// tiles 8 and 9 for J = 4, row 4g + (i & 3).  Those are exactly the rows
// update lane (g, r) holds in its accumulators for tiles U and U + 4, so
// each lane publishes a whole 16-byte unit (unit 4J + g of row r).  Within
// a row the 16-byte units are XOR-swizzled by bit 2 of the row so that the
// readout's 16-byte reads (row r = lane & 15) and the publish writes are
// free of LDS bank conflicts.
__device__ __forceinline__ int unit_swz(int u, int row) { return u ^ ((row >> 2) & 1); }

// ---------------------------------------------------------------- 273-row state map
// Rows of the caller's state for rotation tile T, row r.  Returns the
// number of rows (0, 1 or 2: a pair a != b has two mirror rows).
template <int T>
__device__ __forceinline__ int state_rows(int r, int& r0, int& r1) {
    if (T == 9) { r0 = 1 + r; return 1; }
    if (T == 8 && r == 8) { r0 = 0; return 1; }
    if (T == 8 && r > 8) return 0;
    const int a = r, b = (r + T) & 15;
    r0 = 1 + kDFeat + a * kDFeat + b;
    r1 = 1 + kDFeat + b * kDFeat + a;
    return T == 0 ? 1 : 2;
}
// ---------------------------------------------------------------- feature operands
// psi(Q) for readout k-step J: lane (query row, group g) holds the
// features k = 8g + i of the state operand layout above.
// qr[m] = raw q_((4g + m) mod 16) of the lane's query.
template <int J>
__device__ __forceinline__ void psi_q(const float (&qr)[16], int g, float (&a)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int m = i & 3;
        if (J < 4) {
            const int T = i < 4 ? J : J + 4;  // pair (row, row + T)
            a[i] = T == 0 ? (0.5f * qr[m]) * qr[m] : qr[m] * qr[m + T];
        } else if (i < 4) {
            // tile 8: pairs (row, row + 8) for rows < 8, the constant at row 8
            a[i] = g < 2 ? qr[m] * qr[m + 8] : ((g == 2 && m == 0) ? 1.f : 0.f);
        } else {
            a[i] = qr[m];  // tile 9: linear terms
        }
    }
}

// ---------------------------------------------------------------- per-wave bodies
// Accumulators hold the state in readout units (the k pre-scale 1/4 and
// the pair multiplicity are folded in when the features of K are formed,
// the 1/2 of the diagonal terms into the query features), so publishing
// the state operand is a plain rounding to bf16.  state_scale converts to the caller's 273-row units
// (one mirror row of a pair).
template <int T>
__device__ __forceinline__ float state_scale(int r) {
    if (T == 0) return 2.f * kSqrt2;
    if (T == 9) return 2.f;
    if (T == 8 && r == 8) return 1.f;
    return 2.f * kSqrt2;
}

// Tiles J and J + 4 (J < 4): one 16-byte unit per lane and column tile.
template <int J, int DV>
__device__ __forceinline__ void publish_pair(const f32x4 (&a)[DV / 16 + 1], const f32x4 (&b)[DV / 16 + 1],
                                             PrefillSmem<DV>& sm, int sbuf, int g, int r) {
    constexpr int kNV = DV / 16;
    const int u = 4 * J + g;
#pragma unroll
    for (int ct = 0; ct <= kNV; ++ct) {
        if (ct == kNV && r != 0) continue;  // the normaliser tile has 16 equal columns
        const u32x4 x = {pack_bf16x2(a[ct][0], a[ct][1]), pack_bf16x2(a[ct][2], a[ct][3]),
                         pack_bf16x2(b[ct][0], b[ct][1]), pack_bf16x2(b[ct][2], b[ct][3])};
        u32x4* dst = ct < kNV ? reinterpret_cast<u32x4*>(&sm.s_hi[sbuf][(16 * ct + r) * kSRow + 8 * unit_swz(u, r)])
                              : reinterpret_cast<u32x4*>(&sm.z_hi[sbuf][8 * u]);
        *dst = x;
    }
}
// Tile 8 (H = 0) or 9 (H = 1): half H of unit 16 + g, as a hi/lo pair.
template <int H, int DV>
__device__ __forceinline__ void publish_last(const f32x4 (&a)[DV / 16 + 1], PrefillSmem<DV>& sm, int sbuf, int g,
                                             int r) {
    constexpr int kNV = DV / 16;
#pragma unroll
    for (int ct = 0; ct <= kNV; ++ct) {
        if (ct == kNV && r != 0) continue;
        const uint32_t h01 = pack_bf16x2(a[ct][0], a[ct][1]);
        const uint32_t h23 = pack_bf16x2(a[ct][2], a[ct][3]);
        const uint32_t l01 = lo_pair_of(h01, a[ct][0], a[ct][1]);
        const uint32_t l23 = lo_pair_of(h23, a[ct][2], a[ct][3]);
        uint2* hi = ct < kNV
                        ? reinterpret_cast<uint2*>(&sm.s_hi[sbuf][(16 * ct + r) * kSRow + 8 * unit_swz(16 + g, r) + 4 * H])
                        : reinterpret_cast<uint2*>(&sm.z_hi[sbuf][8 * (16 + g) + 4 * H]);
        uint2* lo = ct < kNV ? reinterpret_cast<uint2*>(&sm.s_lo[sbuf][(16 * ct + r) * kLoRow + 8 * unit_swz(g, r) + 4 * H])
                             : reinterpret_cast<uint2*>(&sm.z_lo[sbuf][8 * g + 4 * H]);
        *hi = make_uint2(h01, h23);
        *lo = make_uint2(l01, l23);
    }
}

template <int T, int DV>
__device__ __forceinline__ void load_initial(f32x4 (&acc)[DV / 16 + 1], const float* Sh, const float* zh,
                                             int ldv, int g, int r) {
    constexpr int kNV = DV / 16;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        int r0 = 0, r1 = 0;
        const int n = state_rows<T>(4 * g + m, r0, r1);
        const float inv = 1.f / state_scale<T>(4 * g + m);
#pragma unroll
        for (int ct = 0; ct <= kNV; ++ct) {
            float x = 0.f;
            if (n > 0) {
                if (ct < kNV) {
                    const int col = 16 * ct + r;
                    x = Sh[(size_t)r0 * ldv + col];
                    if (n == 2) x = 0.5f * (x + Sh[(size_t)r1 * ldv + col]);
                } else {
                    x = zh[r0];
                    if (n == 2) x = 0.5f * (x + zh[r1]);
                }
            }
            acc[ct][m] = x * inv;
        }
    }
}

template <int T, int DV>
__device__ __forceinline__ void store_final(const f32x4 (&acc)[DV / 16 + 1], float* Sh, float* zh,
                                            int ldv, bool own_z, int use_init, int g, int r) {
    constexpr int kNV = DV / 16;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        int r0 = 0, r1 = 0;
        const int n = state_rows<T>(4 * g + m, r0, r1);
        if (n == 0) continue;
        const float sc = state_scale<T>(4 * g + m);
#pragma unroll
        for (int ct = 0; ct <= kNV; ++ct) {
            if (ct == kNV && (r != 0 || !own_z)) continue;
            float* base = ct < kNV ? Sh + 16 * ct + r : zh;
            const size_t stride = ct < kNV ? (size_t)ldv : 1;
            if (!use_init) {
                base[r0 * stride] = acc[ct][m] * sc;
                if (n == 2) base[r1 * stride] = acc[ct][m] * sc;
            } else {
                // Initial rows were folded in as their symmetric mean; add
                // only this call's increment so an asymmetric initial state
                // keeps its antisymmetric part.
                const float x0 = base[r0 * stride];
                const float x1 = n == 2 ? base[r1 * stride] : x0;
                const float mean = n == 2 ? 0.5f * (x0 + x1) : x0;
                const float inc = acc[ct][m] * sc - mean;
                base[r0 * stride] = x0 + inc;
                if (n == 2) base[r1 * stride] = x1 + inc;
            }
        }
    }
}

// Tile 8 rows: d = k_r * k_(r+8) on lanes r < 8 of each 16-lane row (DPP
// bank mask); lanes r >= 8 keep their old value, which holds the constant
// feature (1 on row 8, 0 below it).  The s_nop covers the DPP read hazard.
__device__ __forceinline__ void tile8_rows(const float (&kv)[8], float (&d)[8]) {
    asm volatile(
        "s_nop 1\n\t"
        "v_mul_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_mul_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_mul_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_mul_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_mul_f32_dpp %4, %12, %12 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_mul_f32_dpp %5, %13, %13 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_mul_f32_dpp %6, %14, %14 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_mul_f32_dpp %7, %15, %15 row_ror:8 row_mask:0xf bank_mask:0x3"
        : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]), "+v"(d[4]), "+v"(d[5]), "+v"(d[6]), "+v"(d[7])
        : "v"(kv[0]), "v"(kv[1]), "v"(kv[2]), "v"(kv[3]), "v"(kv[4]), "v"(kv[5]), "v"(kv[6]), "v"(kv[7]));
}

// psi(K)^T for rotation tile T: lane (row r, group g) holds feature row r
// for 8 tokens; kv[] = k_r / 4 of those tokens.  Tile 8 comes from
// tile8_rows (t8); its constant row is 1 for every token of the chunk,
// padding included (padded tokens have v = 0, so only the normaliser's
// constant row counts them; that count is taken off before the state
// leaves the kernel).
template <int T>
__device__ __forceinline__ bf16x8 psi_k(const float (&kv)[8], float (&t8)[8]) {
    float a[8];
    if constexpr (T == 8) {
        tile8_rows(kv, t8);
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = t8[i];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (T == 0) {
                a[i] = kv[i] * kv[i];  // the 1/2 of the diagonal is on the query side
            } else if (T < 8) {
                a[i] = kv[i] * row_ror<16 - T>(kv[i]);
            } else {
                a[i] = kv[i];
            }
        }
    }
    return pack8(a);
}

// ---- staging split: readout waves stage Q and K (+K^T), update waves V^T.
struct QKStage {
    u32x4 a;
};
template <int DV>
struct VStage {
    static constexpr int kPass = DV >= 64 ? DV / 64 : 1;
    u32x4 v0[kPass], v1[kPass];
};

__device__ __forceinline__ u32x4 keep_if(const u32x4& x, bool ok) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = ok ? x[i] : 0u;
    return r;
}
// (a & 0xffff) | (b << 16) and (a >> 16) | (b & 0xffff0000), one byte
// permute each (v_perm_b32 numbers src1's bytes 0-3 and src0's 4-7)
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Unconditional 16-byte loads: rows past the end are clamped to the last
// row and zeroed when stored, so no branch sits between prefetch and use.
// t (0..255 of the off-diagonal waves): t < 128 stages K, else Q; token
// (t & 127) >> 1, dims 8*(t & 1) .. +8.
__device__ __forceinline__ void qk_load(QKStage& st, const uint16_t* qh, const uint16_t* kh, int t0, int L,
                                        int t) {
    const int tok = min(t0 + ((t & 127) >> 1), L - 1);
    const uint16_t* src = t < 128 ? kh : qh;
    st.a = *reinterpret_cast<const u32x4*>(src + (size_t)tok * kDFeat + 8 * (t & 1));
}
// MASK: the chunk runs past L and its rows there are zeroed (a full chunk
// takes the branch without the selects).
template <int DV, bool MASK>
__device__ __forceinline__ void qk_store(const QKStage& in, PrefillSmem<DV>& sm, int buf, int t0, int L, int t) {
    const int tok = (t & 127) >> 1, half = t & 1;
    const u32x4 a = MASK ? keep_if(in.a, t0 + tok < L) : in.a;
    uint16_t* rowm = t < 128 ? &sm.k[buf][0] : &sm.q[buf][0];
    *reinterpret_cast<u32x4*>(rowm + qk_idx(tok, 8 * half)) = a;
    if (t < 128) {
        float* kt = &sm.ktf[buf][0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kt[kt_idx(8 * half + 2 * e, tok)] = 0.25f * bf16lo_f32(a[e]);
            kt[kt_idx(8 * half + 2 * e + 1, tok)] = 0.25f * bf16hi_f32(a[e]);
        }
    } else {
        float* qf = &sm.qf[buf][0];
        *reinterpret_cast<f32x4*>(qf + qf_idx(tok, 8 * half)) =
            f32x4{bf16lo_f32(a[0]), bf16hi_f32(a[0]), bf16lo_f32(a[1]), bf16hi_f32(a[1])};
        *reinterpret_cast<f32x4*>(qf + qf_idx(tok, 8 * half + 4)) =
            f32x4{bf16lo_f32(a[2]), bf16hi_f32(a[2]), bf16lo_f32(a[3]), bf16hi_f32(a[3])};
    }
}
// u (0..255, or 0..127 for a 32-column group): token pair p = u & 31,
// column blocks (u >> 5) + 8*pass of 8 columns.
// ldv is the row stride of v in the caller's tensor.
template <int DV>
__device__ __forceinline__ void v_load(VStage<DV>& st, const uint16_t* vh, int ldv, int t0, int L, int u) {
    const int p = u & 31;
    const int ta = min(t0 + 2 * p, L - 1), tb = min(t0 + 2 * p + 1, L - 1);
#pragma unroll
    for (int ps = 0; ps < VStage<DV>::kPass; ++ps) {
        const int cb = (u >> 5) + 8 * ps;
        if (8 * cb >= DV) continue;
        st.v0[ps] = *reinterpret_cast<const u32x4*>(vh + (size_t)ta * ldv + 8 * cb);
        st.v1[ps] = *reinterpret_cast<const u32x4*>(vh + (size_t)tb * ldv + 8 * cb);
    }
}
template <int DV, bool MASK>
__device__ __forceinline__ void v_store(const VStage<DV>& st, PrefillSmem<DV>& sm, int buf, int t0, int L, int u) {
    const int p = u & 31;
    const bool oka = t0 + 2 * p < L, okb = t0 + 2 * p + 1 < L;
    uint32_t* vt = reinterpret_cast<uint32_t*>(&sm.vt[buf][0]);
#pragma unroll
    for (int ps = 0; ps < VStage<DV>::kPass; ++ps) {
        const int cb = (u >> 5) + 8 * ps;
        if (8 * cb >= DV) continue;
        const u32x4 v0 = MASK ? keep_if(st.v0[ps], oka) : st.v0[ps];
        const u32x4 v1 = MASK ? keep_if(st.v1[ps], okb) : st.v1[ps];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vt[vt_idx(8 * cb + 2 * e, vt_pos(2 * p)) >> 1] = lo_pair(v0[e], v1[e]);
            vt[vt_idx(8 * cb + 2 * e + 1, vt_pos(2 * p)) >> 1] = hi_pair(v0[e], v1[e]);
        }
    }
}

// ---- staging pipeline: chunk c+1 is written to LDS during interval c from
// registers loaded two intervals earlier; two register sets alternate (set
// A holds the odd chunks, set B the even ones), so no register copy waits on
// a load in flight.  V^T is staged by update-wave threads (vu >= 0), Q and K
// by off-diagonal-wave threads (t >= 0, K for t < 128).
template <int DV, bool DO_V, bool DO_QK>
struct StagePipe {
    struct Regs {
        VStage<DV> v;
        QKStage qk;
    };
    Regs a, b;
    int vu, t;
    const uint16_t *qh, *kh, *vh;
    int ldv, L;

    __device__ __forceinline__ void load(Regs& rg, int t0) {
        if (DO_V && vu >= 0) v_load<DV>(rg.v, vh, ldv, t0, L, vu);
        if (DO_QK && t >= 0) qk_load(rg.qk, qh, kh, t0, L, t);
    }
    __device__ __forceinline__ void store(const Regs& rg, PrefillSmem<DV>& sm, int buf, int t0) {
        if (t0 + kC <= L) {  // uniform: a full chunk needs no zeroing
            if (DO_V && vu >= 0) v_store<DV, false>(rg.v, sm, buf, t0, L, vu);
            if (DO_QK && t >= 0) qk_store<DV, false>(rg.qk, sm, buf, t0, L, t);
        } else {
            if (DO_V && vu >= 0) v_store<DV, true>(rg.v, sm, buf, t0, L, vu);
            if (DO_QK && t >= 0) qk_store<DV, true>(rg.qk, sm, buf, t0, L, t);
        }
    }
    // chunk 0 into LDS buffer 0; chunks 1 and 2 in flight
    __device__ __forceinline__ void prologue(PrefillSmem<DV>& sm, int nchunks) {
        load(b, 0);
        if (nchunks > 1) load(a, kC);
        store(b, sm, 0, 0);
        if (nchunks > 2) load(b, 2 * kC);
    }
    // interval c: stage chunk c+1 (held in rg) and refill rg with chunk c+3
    __device__ __forceinline__ void advance(Regs& rg, PrefillSmem<DV>& sm, int c, int nchunks) {
        if (c + 1 < nchunks) {
            store(rg, sm, (c + 1) & 1, (c + 1) * kC);
            if (c + 3 < nchunks) load(rg, (c + 3) * kC);
        }
    }
};

// ---- on-diagonal term of query tile DQ (rows 16DQ..16DQ+15) of one chunk:
// for key tiles 0..DQ, t = 4 + q.k (raw q, k: the MFMA accumulator starts
// at 4), so that t^2 + 16 = 16(1 + s)^2 + 16 = 32(1 + s + s^2/2) with
// s = q.k/4: one FMA per causal weight, which enters (as a hi/lo bf16 pair)
// times V and the ones column, in MFMA accumulator layout.  The sums are
// 32 times the method's on-diagonal numerator and denominator; the
// off-diagonal part is scaled to match when the two are combined.
template <int DQ, int DV>
__device__ __forceinline__ void diag_block(const PrefillSmem<DV>& sm, int buf, int lane, int g, int r,
                                          f32x4 (&y)[DV / 16 + 1]) {
    constexpr int kNV = DV / 16, kNCT = kNV + 1;
    const uint16_t* q_l = &sm.q[buf][0];
    const uint16_t* k_l = &sm.k[buf][0];
    const uint16_t* vt_l = &sm.vt[buf][0];
    const bf16x8 ones = ones8();
#pragma unroll
    for (int ct = 0; ct < kNCT; ++ct) y[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x4 qb = lds_bf16x4(q_l + qk_idx(16 * DQ + r, 4 * g));
    float wgt[DQ + 1][4];
#pragma unroll
    for (int j = 0; j <= DQ; ++j) {
        const bf16x4 ka = lds_bf16x4(k_l + qk_idx(16 * j + r, 4 * g));
        const f32x4 t = mfma16(ka, qb, f32x4{4.f, 4.f, 4.f, 4.f});
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // t[m] = 4 + q_query . k_key (raw), key = 16j + 4g + m, query = 16DQ + r
            const float w = fmaf(t[m], t[m], 16.f);
            wgt[j][m] = (j == DQ && 4 * g + m > r) ? 0.f : w;
        }
    }
#pragma unroll
    for (int p = 0; p <= DQ / 2; ++p) {
        float a[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            a[m] = wgt[2 * p][m];
            a[4 + m] = (2 * p + 1 <= DQ) ? wgt[(2 * p + 1 <= DQ) ? 2 * p + 1 : 0][m] : 0.f;
        }
        bf16x8 ahi, alo;
        pack8_hilo(a, ahi, alo);
        bf16x8 vb[kNV];
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct)
            vb[ct] = lds_bf16x8(vt_l + vt_idx(16 * ct + r, 32 * p + 8 * g));  // tokens 32p + {4g.., 16+4g..}
        // hi parts of every column tile first, then the lo parts, so
        // consecutive MFMAs never depend on each other
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) y[ct] = mfma32(ahi, vb[ct], y[ct]);
        y[kNV] = mfma32(ahi, ones, y[kNV]);
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) y[ct] = mfma32(alo, vb[ct], y[ct]);
        y[kNV] = mfma32(alo, ones, y[kNV]);
    }
}

// ---- off-diagonal wave W: psi(Q_c) x S_c (state before chunk c) for query
// tile W (rows 16W..16W+15), handed to the on-diagonal wave of that tile.
template <int W, int DV, int MODE>
__device__ __forceinline__ void offdiag_wave(const uint16_t* __restrict__ qh, const uint16_t* __restrict__ kh, int L,
                                             PrefillSmem<DV>& sm) {
    constexpr int kNV = DV / 16, kNCT = kNV + 1;
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const int nchunks = (L + kC - 1) / kC;
    // Q and K staging: waves 0, 1 (K) and 2, 3 (Q)
    StagePipe<DV, false, true> pipe;
    pipe.vu = -1;
    pipe.t = (int)threadIdx.x;
    pipe.qh = qh;
    pipe.kh = kh;
    pipe.vh = nullptr;
    pipe.ldv = 0;
    pipe.L = L;
    pipe.prologue(sm, nchunks);

    __syncthreads();  // first chunk staged, initial state published
    auto step = [&](int c, typename StagePipe<DV, false, true>::Regs& regs) {
        const int buf = c & 1;
        f32x4 y[kNCT];
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct) y[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        float qr[16];
        const float* qf = &sm.qf[buf][0];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(qf + qf_idx(16 * W + r, 4 * ((g + cc) & 3)));
            qr[4 * cc + 0] = x[0];
            qr[4 * cc + 1] = x[1];
            qr[4 * cc + 2] = x[2];
            qr[4 * cc + 3] = x[3];
        }
        const uint16_t* shi = &sm.s_hi[buf][0];
        const uint16_t* slo = &sm.s_lo[buf][0];
#define BASED_READOUT_STEP(J)                                                                             \
{                                                                                                     \
    float a[8];                                                                                       \
    psi_q<J>(qr, g, a);                                                                               \
    const bf16x8 ahi = pack8(a);                                                                      \
    _Pragma("unroll") for (int ct = 0; ct < kNV; ++ct)                                                \
        y[ct] = mfma32(ahi, lds_bf16x8(shi + (16 * ct + r) * kSRow + 8 * unit_swz(4 * (J) + g, r)), y[ct]); \
    y[kNV] = mfma32(ahi, lds_bf16x8(&sm.z_hi[buf][8 * (4 * (J) + g)]), y[kNV]);                       \
}
        BASED_READOUT_STEP(0)
        BASED_READOUT_STEP(1)
        BASED_READOUT_STEP(2)
        BASED_READOUT_STEP(3)
#undef BASED_READOUT_STEP
        // last feature k-step (pairs (r, r+8), constant, linear): the state
        // side as a hi/lo pair (its constant and linear rows carry the
        // largest sums); the features in single bf16, where the constant
        // and the linear terms (raw bf16 q) are exact and the pairs are
        // rounded like every other pair feature
        float a[8];
        psi_q<4>(qr, g, a);
        const bf16x8 ahi = pack8(a);
        bf16x8 sb[kNCT];
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) sb[ct] = lds_bf16x8(shi + (16 * ct + r) * kSRow + 8 * unit_swz(16 + g, r));
        sb[kNV] = lds_bf16x8(&sm.z_hi[buf][8 * (16 + g)]);
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct) y[ct] = mfma32(ahi, sb[ct], y[ct]);
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct)
            y[ct] = mfma32(ahi, lds_bf16x8(slo + (16 * ct + r) * kLoRow + 8 * unit_swz(g, r)), y[ct]);
        y[kNV] = mfma32(ahi, lds_bf16x8(&sm.z_lo[buf][8 * g]), y[kNV]);
        f32x4* dst = reinterpret_cast<f32x4*>(&sm.hand[buf][W][0]);
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct) dst[ct * 64 + lane] = y[ct];
        pipe.advance(regs, sm, c, nchunks);
        __syncthreads();
    };
    for (int c = 0; c < nchunks; c += 2) {
        step(c, pipe.a);
        if (c + 1 < nchunks) step(c + 1, pipe.b);
    }
}

// ---- window wave DQ of the fused layer: the w <= 64 softmax window of
// query tile DQ ("Simple linear attention language models balance the
// recall-throughput tradeoff", s4 "Local Exact Attention") over the keys of
// chunks c-1 and c.  Interval c stages chunk c+1 (K and V through
// registers; this wave's q rows of chunk c+1 into registers), computes
// chunk c and hands the normalised output to the on-diagonal wave of the
// tile, which adds it when it finishes chunk c in interval c+1.
struct WinRegs {
    u32x4 k0, k1, v;
};
// t = 0..255 (thread of the window waves): K units t and t + 256 (row =
// unit / 8, 16-byte unit = unit % 8), V unit t (row t / 4, unit t % 4).
// Rows are clamped into [0, L): rows outside it only ever meet masked
// weights (which are exactly 0).
__device__ __forceinline__ void win_load(WinRegs& rg, const uint16_t* k2h, const uint16_t* v2h, int ldv, int t0,
                                         int L, int t) {
    const int rk0 = min(max(t0 + (t >> 3), 0), L - 1);
    const int rk1 = min(max(t0 + 32 + (t >> 3), 0), L - 1);
    const int rv = min(max(t0 + (t >> 2), 0), L - 1);
    rg.k0 = *reinterpret_cast<const u32x4*>(k2h + (size_t)rk0 * kWinD + 8 * (t & 7));
    rg.k1 = *reinterpret_cast<const u32x4*>(k2h + (size_t)rk1 * kWinD + 8 * (t & 7));
    rg.v = *reinterpret_cast<const u32x4*>(v2h + (size_t)rv * ldv + 8 * (t & 3));
}
__device__ __forceinline__ void win_store(const WinRegs& rg, WinSmem& ws, int slot, int t) {
    *reinterpret_cast<u32x4*>(&ws.k[slot][win_idx(t >> 3, 8 * (t & 7))]) = rg.k0;
    *reinterpret_cast<u32x4*>(&ws.k[slot][win_idx(32 + (t >> 3), 8 * (t & 7))]) = rg.k1;
    *reinterpret_cast<u32x4*>(&ws.v[slot][(t >> 2) * kWinCols + 8 * (t & 3)]) = rg.v;
}
// This lane's query row (dims 8g..8g+7 and 32+8g..32+8g+7): the B operand
// of the two k-steps of the scores.
__device__ __forceinline__ void win_qload(bf16x8 (&qb)[2], const uint16_t* q2h, int tok, int L, int g) {
    const uint16_t* row = q2h + (size_t)min(tok, L - 1) * kWinD;
    qb[0] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 8 * g));
    qb[1] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 32 + 8 * g));
}
// Transposed LDS read (ds_read_b64_tr_b16) of a row-major [64][32] V slot:
// lane c of each 16-lane group passes the address of row rb + c/4, columns
// col0 + 4(c%4) .. +3, and receives rows rb .. rb+3 of column col0 + c.
__device__ __forceinline__ uint2 win_vtr(const uint16_t* vs, int rb, int col0, int c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const uint16_t* p = vs + (rb + (c >> 2)) * kWinCols + col0 + 4 * (c & 3);
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) s16x4*)(p)));
}
// Window output of query tile DQ for one chunk: o[ct] = sum_j p_ij v_j
// (rows = queries 4g+m, columns 16ct + r) and o[2] = sum_j p_ij, with
// p_ij = exp(scale q_i.k_j - max_j) over j in [i - window + 1, i], j >= 0.
// Key tiles DQ-4 .. DQ of 16 keys (relative to the chunk; negative = the
// previous chunk) cover every window of the tile.  kg0 is the chunk's first
// token (global).  Scores are computed as K Q^T: lane (g, r) holds query r,
// keys 4g..4g+3 of each tile, the A operand of P V.
// FULL64: window == 64 and the chunk is not the sequence's first, so every
// key tile but the first (keys 4g+m > r in the window) and the last
// (4g+m <= r, causal) is wholly inside every query's window.
template <int DQ, bool FULL64>
__device__ __forceinline__ void win_block(const WinSmem& ws, int cur, int prev, const bf16x8 (&qb)[2], int kg0,
                                          int window, float sl2, int g, int r, f32x4 (&o)[3]) {
    const bf16x8 ones = ones8();
    const int rho = 16 * DQ + r;
    float p[5][4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int jt = DQ - 4 + i;
        const uint16_t* kt = &ws.k[jt < 0 ? prev : cur][0];
        const int row = 16 * ((jt + 4) & 3) + r;
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
        sc = mfma32(lds_bf16x8(kt + win_idx(row, 8 * g)), qb[0], sc);
        sc = mfma32(lds_bf16x8(kt + win_idx(row, 32 + 8 * g)), qb[1], sc);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int kap = 16 * jt + 4 * g + m;
            bool ok;
            if constexpr (FULL64) ok = i == 0 ? 4 * g + m > r : (i == 4 ? 4 * g + m <= r : true);
            else ok = kap <= rho && kap > rho - window && kg0 + kap >= 0;
            p[i][m] = ok ? sc[m] * sl2 : -INFINITY;
            mx = fmaxf(mx, p[i][m]);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));  // finite: the query's own key is always in
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) p[i][m] = __builtin_amdgcn_exp2f(p[i][m] - mx);
#pragma unroll
    for (int ct = 0; ct < 3; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
        const bool two = 2 * ks + 1 < 5;
        float x[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            x[m] = p[2 * ks][m];
            x[4 + m] = two ? p[two ? 2 * ks + 1 : 0][m] : 0.f;
        }
        bf16x8 ahi, alo;
        pack8_hilo(x, ahi, alo);
        const int j0 = DQ - 4 + 2 * ks, j1 = j0 + 1;
        const uint16_t* v0 = &ws.v[j0 < 0 ? prev : cur][0];
        const uint16_t* v1 = &ws.v[j1 < 0 ? prev : cur][0];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const uint2 a = win_vtr(v0, 16 * ((j0 + 4) & 3) + 4 * g, 16 * ct, r);
            const uint2 b = two ? win_vtr(v1, 16 * ((j1 + 4) & 3) + 4 * g, 16 * ct, r) : make_uint2(0u, 0u);
            const bf16x8 vb = __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
            o[ct] = mfma32(ahi, vb, o[ct]);
            o[ct] = mfma32(alo, vb, o[ct]);
        }
        o[2] = mfma32(ahi, ones, o[2]);
        o[2] = mfma32(alo, ones, o[2]);
    }
}

template <int DQ, int MODE>
__device__ __forceinline__ void window_wave(const uint16_t* __restrict__ q2h, const uint16_t* __restrict__ k2h,
                                            const uint16_t* __restrict__ v2h, int ldv, int L, int tb, int len,
                                            int window, float sl2, WinSmem& ws) {
    const int t = threadIdx.x - 768;  // 0..255
    const int lane = t & 63, g = lane >> 4, r = lane & 15;
    const int nchunks = (len + kC - 1) / kC;
    WinRegs rg;
    bf16x8 qc[2], qn[2];
    // prologue: chunk -1 (the halo of the first chunk) into slot 2, chunk 0 into slot 0
    win_load(rg, k2h, v2h, ldv, tb - kC, L, t);
    win_store(rg, ws, 2, t);
    win_load(rg, k2h, v2h, ldv, tb, L, t);
    win_store(rg, ws, 0, t);
    win_qload(qc, q2h, tb + 16 * DQ + r, L, g);
    __syncthreads();  // first chunk staged
    for (int c = 0; c < nchunks; ++c) {
        const bool more = c + 1 < nchunks;
        // unconditional (past the last chunk the rows are clamped and the
        // data unused): a load inside `if (more)` made the join wait for it
        // before this chunk's products
        win_load(rg, k2h, v2h, ldv, tb + (c + 1) * kC, L, t);
        win_qload(qn, q2h, tb + (c + 1) * kC + 16 * DQ + r, L, g);
        f32x4 o[3];
        if (window == kWinD && tb + c * kC >= kC)
            win_block<DQ, true>(ws, c % 3, (c + 2) % 3, qc, tb + c * kC, window, sl2, g, r, o);
        else
            win_block<DQ, false>(ws, c % 3, (c + 2) % 3, qc, tb + c * kC, window, sl2, g, r, o);
        f32x4* dst = reinterpret_cast<f32x4*>(&ws.hand[c & 1][DQ][0]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            f32x4 x;
#pragma unroll
            for (int m = 0; m < 4; ++m) x[m] = o[ct][m] * __builtin_amdgcn_rcpf(o[2][m]);  // o[2] >= 1
            dst[ct * 64 + lane] = x;
        }
        if (more) {
            win_store(rg, ws, (c + 1) % 3, t);
            qc[0] = qn[0];
            qc[1] = qn[1];
        }
        __syncthreads();
    }
}

// ---- on-diagonal wave DQ: the intra-chunk term of query tile DQ.  Interval
// c computes it for chunk c and finishes chunk c-1: the off-diagonal part
// (handed over during interval c-1) is added, the rows are normalised and
// stored.
template <int DQ, int DV, int MODE, bool HYB, class WinT>
__device__ __forceinline__ void ondiag_wave(int L, int ldv, float eps,
                                            float* __restrict__ yh, PrefillSmem<DV>& sm, const WinT& wsm) {
    constexpr int kNV = DV / 16, kNCT = kNV + 1;
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const int nchunks = (L + kC - 1) / kC;

    __syncthreads();  // first chunk staged, initial state published
    // Chunk c's rows: add the off-diagonal part, normalise, store.  nrows
    // is the number of valid rows of the chunk (64 except at the end).  The
    // on-diagonal sums yd are 32 times the method's (see diag_block): the
    // off-diagonal part is scaled by 32 and so is eps (exact powers of two).
    const float eps32 = 32.f * eps;
    auto finish = [&](int c, const f32x4 (&yd)[kNCT], int nrows) {
        const f32x4* src = reinterpret_cast<const f32x4*>(&sm.hand[c & 1][DQ][0]);
        f32x4 y[kNCT];
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct) {
            const f32x4 x = src[ct * 64 + lane];
#pragma unroll
            for (int m = 0; m < 4; ++m) y[ct][m] = fmaf(x[m], 32.f, yd[ct][m]);
        }
        float* ybase = yh + (size_t)c * kC * ldv;
        if constexpr (HYB) {
            // fused layer: plus the window output of the same rows
            // (normalised on its own), one column tile at a time
            const f32x4* hw = reinterpret_cast<const f32x4*>(&wsm.hand[c & 1][DQ][0]);
            float inv[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) inv[m] = __builtin_amdgcn_rcpf(y[kNV][m] + eps32);
#pragma unroll
            for (int ct = 0; ct < kNV; ++ct) {
                const f32x4 yw = hw[ct * 64 + lane];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int tq = 16 * DQ + 4 * g + m;
                    if (tq < nrows)
                        __builtin_nontemporal_store(fmaf(y[ct][m], inv[m], yw[m]), &ybase[tq * ldv + 16 * ct + r]);
                }
            }
            return;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int tq = 16 * DQ + 4 * g + m;
            const float inv = __builtin_amdgcn_rcpf(y[kNV][m] + eps32);
            if (tq < nrows) {
#pragma unroll
                for (int ct = 0; ct < kNV; ++ct)
                    __builtin_nontemporal_store(y[ct][m] * inv, &ybase[tq * ldv + 16 * ct + r]);
            }
        }
    };
    // Two chunks per iteration with two accumulator sets, so that no
    // register copy carries a chunk's term to the next interval.
    f32x4 ya[kNCT], yb[kNCT];
    for (int c = 0; c < nchunks; c += 2) {
        diag_block<DQ, DV>(sm, 0, lane, g, r, ya);  // chunk c (even: buffer 0)
        if (c > 0) finish(c - 1, yb, kC);
        __syncthreads();
        if (c + 1 < nchunks) {
            diag_block<DQ, DV>(sm, 1, lane, g, r, yb);
            finish(c, ya, kC);
            __syncthreads();
        }
    }
    if (nchunks & 1) finish(nchunks - 1, ya, L - (nchunks - 1) * kC);
    else finish(nchunks - 1, yb, L - (nchunks - 1) * kC);
}

// ---- update wave U: state rotation tiles U, U+4 (, U+8).
template <int U, int DV, int MODE>
__device__ __forceinline__ void update_wave(const uint16_t* __restrict__ qh, const uint16_t* __restrict__ kh,
                                            const uint16_t* __restrict__ vh, int L, int ldv, float* __restrict__ Sh,
                                            float* __restrict__ zh, bool own_z, int use_init, PrefillSmem<DV>& sm,
                                            const float* ws_in, bool write_final, int ws_nct, int ws_ct0) {
    constexpr int kNV = DV / 16, kNCT = kNV + 1;
    constexpr int kNT = U < 2 ? 3 : 2;
    const int u = threadIdx.x - 256;  // 0..255
    const int lane = u & 63, g = lane >> 4, r = lane & 15;
    const int nchunks = (L + kC - 1) / kC;
    // rotation tile 8: rows 0..7 are the pairs (r, r+8), row 8 the constant
    float t8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t8[i] = r == 8 ? 1.f : 0.f;

    f32x4 acc[kNT][kNCT];
#pragma unroll
    for (int ti = 0; ti < kNT; ++ti)
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct) acc[ti][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (MODE == kModeSegment) {
        ws_load<U, DV>(acc[0], ws_in, lane, ws_nct, ws_ct0);
        ws_load<U + 4, DV>(acc[1], ws_in, lane, ws_nct, ws_ct0);
        if constexpr (kNT == 3) ws_load<U + 8, DV>(acc[2], ws_in, lane, ws_nct, ws_ct0);
    } else if (MODE == kModeFull && use_init) {
        load_initial<U, DV>(acc[0], Sh, zh, ldv, g, r);
        load_initial<U + 4, DV>(acc[1], Sh, zh, ldv, g, r);
        if constexpr (kNT == 3) load_initial<U + 8, DV>(acc[2], Sh, zh, ldv, g, r);
    }

    // V^T staging (a 32-column group uses update waves 2 and 3 only)
    StagePipe<DV, true, false> pipe;
    pipe.vu = DV == 32 ? u - 128 : u;
    pipe.t = -1;
    pipe.qh = qh;
    pipe.kh = kh;
    pipe.vh = vh;
    pipe.ldv = ldv;
    pipe.L = L;
    pipe.prologue(sm, nchunks);
    publish_pair<U, DV>(acc[0], acc[1], sm, 0, g, r);
    if constexpr (kNT == 3) publish_last<U, DV>(acc[2], sm, 0, g, r);
    __syncthreads();

    const bf16x8 ones = ones8();
    // One chunk: update with chunk c, stage chunk c+1 from `regs` and
    // refill it with chunk c+3, publish the state after chunk c.  (Staging
    // stays on waves without global stores: on gfx9 the vector-memory
    // counter also counts stores, so a wave that stores outputs would wait
    // for them before it could use its prefetched loads.)
    auto step = [&](int c, typename StagePipe<DV, true, false>::Regs& regs) {
        const int buf = c & 1;
        const float* kt_l = &sm.ktf[buf][0];
        const uint16_t* vt_l = &sm.vt[buf][0];

        // ---- S += psi(K)^T V, z += psi(K)^T 1 over this chunk's 64 tokens
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float kv[8];
            // tokens 32s + 4g.. and 32s + 16 + 4g.. (the V^T slice at 32s + 8g)
            const f32x4 k0 = *reinterpret_cast<const f32x4*>(kt_l + kt_idx(r, 32 * s + 4 * g));
            const f32x4 k1 = *reinterpret_cast<const f32x4*>(kt_l + kt_idx(r, 32 * s + 16 + 4 * g));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kv[i] = k0[i];
                kv[4 + i] = k1[i];
            }
            bf16x8 vb[kNV];
#pragma unroll
            for (int ct = 0; ct < kNV; ++ct)
                vb[ct] = lds_bf16x8(vt_l + vt_idx(16 * ct + r, 32 * s + 8 * g));
            {
                const bf16x8 a = psi_k<U>(kv, t8);
#pragma unroll
                for (int ct = 0; ct < kNV; ++ct) acc[0][ct] = mfma32(a, vb[ct], acc[0][ct]);
                acc[0][kNV] = mfma32(a, ones, acc[0][kNV]);
            }
            {
                const bf16x8 a = psi_k<U + 4>(kv, t8);
#pragma unroll
                for (int ct = 0; ct < kNV; ++ct) acc[1][ct] = mfma32(a, vb[ct], acc[1][ct]);
                acc[1][kNV] = mfma32(a, ones, acc[1][kNV]);
            }
            if constexpr (kNT == 3) {
                const bf16x8 a = psi_k<U + 8>(kv, t8);
#pragma unroll
                for (int ct = 0; ct < kNV; ++ct) acc[2][ct] = mfma32(a, vb[ct], acc[2][ct]);
                acc[2][kNV] = mfma32(a, ones, acc[2][kNV]);
            }
        }

        pipe.advance(regs, sm, c, nchunks);

        // ---- publish the state after this chunk for the next readout
        publish_pair<U, DV>(acc[0], acc[1], sm, buf ^ 1, g, r);
        if constexpr (kNT == 3) publish_last<U, DV>(acc[2], sm, buf ^ 1, g, r);
        __syncthreads();
    };
    for (int c = 0; c < nchunks; c += 2) {
        step(c, pipe.a);                           // chunk c+1 (odd) is in set A
        if (c + 1 < nchunks) step(c + 1, pipe.b);  // chunk c+2 (even) is in set B
    }

    // padded tokens of the last chunk entered the constant row of the
    // normaliser (tile 8, row 8 = lane group 2, element 0)
    if constexpr (U == 0) {
        if (g == 2) acc[2][kNV][0] -= (float)(nchunks * kC - L);
    }
    if (write_final) {
        store_final<U, DV>(acc[0], Sh, zh, ldv, own_z, use_init, g, r);
        store_final<U + 4, DV>(acc[1], Sh, zh, ldv, own_z, use_init, g, r);
        if constexpr (kNT == 3) store_final<U + 8, DV>(acc[2], Sh, zh, ldv, own_z, use_init, g, r);
    }
}

// Workspace: one state per (segment slot, head) in accumulator layout,
// [slot][head][tile 0..9][column tile][lane] f32x4, readout units.
template <int DV>
__host__ __device__ constexpr size_t ws_slot_floats() {
    return (size_t)10 * (DV / 16 + 1) * 64 * 4;
}
template <int T, int DV>
__device__ __forceinline__ void ws_store(const f32x4 (&acc)[DV / 16 + 1], float* slot, int lane) {
    constexpr int kNCT = DV / 16 + 1;
    f32x4* p = reinterpret_cast<f32x4*>(slot) + (size_t)T * kNCT * 64 + lane;
#pragma unroll
    for (int ct = 0; ct < kNCT; ++ct) p[ct * 64] = acc[ct];
}
// A slot may be wider than the reader: slot_nct column tiles per rotation
// tile (the last one the normaliser), of which the reader takes ct0 ..
// ct0 + DV/16 - 1 and the normaliser (a 32-column group reading a 64-column
// slot).  slot_nct = DV/16 + 1, ct0 = 0 is the reader's own layout.
template <int T, int DV>
__device__ __forceinline__ void ws_load(f32x4 (&acc)[DV / 16 + 1], const float* slot, int lane, int slot_nct,
                                        int ct0) {
    constexpr int kNV = DV / 16;
    const f32x4* p = reinterpret_cast<const f32x4*>(slot) + (size_t)T * slot_nct * 64 + lane;
#pragma unroll
    for (int ct = 0; ct < kNV; ++ct) acc[ct] = p[(ct0 + ct) * 64];
    acc[kNV] = p[(slot_nct - 1) * 64];
}

// One workgroup = 12 waves (roles above).  MODE
//   kModeFull:    one workgroup per (head, column group) walks the whole
//                 sequence.
//   kModeSegment: workgroup (head, s): outputs of segment s starting from
//                 slot s (after the prefix sum); the last segment writes the
//                 final state.
//   HYB:          the fused hybrid layer (32-column groups only): four more
//                 waves (12..15) run the w <= 64 window of the same rows with
//                 their own q2, k2 and the shared v, and the on-diagonal
//                 waves store y_LA + y_window.
template <int DV, int MODE, bool HYB = false>
__global__ __launch_bounds__(HYB ? 1024 : 768, 1) void prefill_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int L, int ldv,
    int ncg, int seg_len, int nseg, float eps, float* __restrict__ y, float* __restrict__ S, float* __restrict__ z,
    int use_init, float* __restrict__ ws, const uint16_t* __restrict__ q2, const uint16_t* __restrict__ k2,
    int window, float win_scale) {
    static_assert(!HYB || DV == kWinCols, "the fused layer uses 32-column groups");
    using WinT = std::conditional_t<HYB, WinSmem, WinNone>;
    __shared__ PrefillSmem<DV> sm;
    __shared__ WinT wsm;
    // Workgroup -> (head, segment, column group), column group fastest.  The
    // 8 XCDs take workgroups round-robin; the remap gives each XCD a
    // contiguous run, so the column groups of a head (same Q, K) share an L2.
    const int total = gridDim.x;
    int b = blockIdx.x;
    if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);
    const int cg = b % ncg;
    const int hs = b / ncg;
    const int seg = MODE == kModeFull ? 0 : hs % nseg;
    const int head = MODE == kModeFull ? hs : hs / nseg;
    const int BH = total / (ncg * (MODE == kModeFull ? 1 : nseg));
    const int tb = seg * seg_len;
    const int len = MODE == kModeFull ? L : min(seg_len, L - tb);
    const int col0 = cg * DV;
    const uint16_t* qh = q + ((size_t)head * L + tb) * kDFeat;
    const uint16_t* kh = k + ((size_t)head * L + tb) * kDFeat;
    const uint16_t* vh = v + ((size_t)head * L + tb) * ldv + col0;
    float* yh = y + ((size_t)head * L + tb) * ldv + col0;
    float* Sh = S + (size_t)head * kNumFeat * ldv + col0;
    float* zh = z + (size_t)head * kNumFeat;
    const bool own_z = cg == 0;  // every column group carries z; the first writes it
    float* ws_in = nullptr;
    // The fused layer's segment pass reads the state of a 64-column state
    // pass (one slot per head, segment and 64-column group): its column
    // group's tiles of it.
    int ws_nct = DV / 16 + 1, ws_ct0 = 0;
    if (MODE != kModeFull) {
        if (HYB) {
            ws_nct = 64 / 16 + 1;
            ws_ct0 = (DV / 16) * (cg % 2);
            ws_in = ws + (((size_t)seg * BH + head) * (ldv / 64) + cg / 2) * ws_slot_floats<64>();
        } else {
            ws_in = ws + (((size_t)seg * BH + head) * ncg + cg) * ws_slot_floats<DV>();
        }
    }
    const int w = threadIdx.x >> 6;
    const bool write_final = MODE == kModeFull || seg == nseg - 1;
    // Waves w, w + 4 and w + 8 share a SIMD: the off-diagonal wave of query
    // tile w, update wave w (three state tiles for w < 2) and the
    // on-diagonal wave of query tile w (heavier for larger w).
    switch (w) {
        case 0: offdiag_wave<0, DV, MODE>(qh, kh, len, sm); break;
        case 1: offdiag_wave<1, DV, MODE>(qh, kh, len, sm); break;
        case 2: offdiag_wave<2, DV, MODE>(qh, kh, len, sm); break;
        case 3: offdiag_wave<3, DV, MODE>(qh, kh, len, sm); break;
        case 8: ondiag_wave<0, DV, MODE, HYB>(len, ldv, eps, yh, sm, wsm); break;
        case 9: ondiag_wave<1, DV, MODE, HYB>(len, ldv, eps, yh, sm, wsm); break;
        case 10: ondiag_wave<2, DV, MODE, HYB>(len, ldv, eps, yh, sm, wsm); break;
        case 11: ondiag_wave<3, DV, MODE, HYB>(len, ldv, eps, yh, sm, wsm); break;
        case 4: update_wave<0, DV, MODE>(qh, kh, vh, len, ldv, Sh, zh, own_z, use_init, sm, ws_in, write_final, ws_nct, ws_ct0); break;
        case 5: update_wave<1, DV, MODE>(qh, kh, vh, len, ldv, Sh, zh, own_z, use_init, sm, ws_in, write_final, ws_nct, ws_ct0); break;
        case 6: update_wave<2, DV, MODE>(qh, kh, vh, len, ldv, Sh, zh, own_z, use_init, sm, ws_in, write_final, ws_nct, ws_ct0); break;
        case 7: update_wave<3, DV, MODE>(qh, kh, vh, len, ldv, Sh, zh, own_z, use_init, sm, ws_in, write_final, ws_nct, ws_ct0); break;
        default: break;
    }
    if constexpr (HYB) {
        // window waves: head-based pointers, global token indices
        const uint16_t* q2h = q2 + (size_t)head * L * kWinD;
        const uint16_t* k2h = k2 + (size_t)head * L * kWinD;
        const uint16_t* v2h = v + (size_t)head * L * ldv + col0;
        const float sl2 = win_scale * 1.4426950408889634f;
        switch (w) {
            case 12: window_wave<0, MODE>(q2h, k2h, v2h, ldv, L, tb, len, window, sl2, wsm); break;
            case 13: window_wave<1, MODE>(q2h, k2h, v2h, ldv, L, tb, len, window, sl2, wsm); break;
            case 14: window_wave<2, MODE>(q2h, k2h, v2h, ldv, L, tb, len, window, sl2, wsm); break;
            case 15: window_wave<3, MODE>(q2h, k2h, v2h, ldv, L, tb, len, window, sl2, wsm); break;
            default: break;
        }
    }
}

// ---- state pass of the segment split.  A segment's state increment is a
// plain sum over its tokens, sum_t psi(k_t) [v_t | 1]^T, with no order to
// respect between chunks, so it needs none of the prefill's roles.  Ten
// waves: wave w owns the rotation tiles 2p, 2p + 1 (p = w mod 5; all their
// column tiles) over the k-step h = w / 5 of every chunk (tokens 32h ..
// 32h + 31), and the two waves of a tile pair add their sums at the end.
// The chunks come from a ring of LDS slots filled by asynchronous global ->
// LDS copies several chunks ahead (the pass is bound by reading K and V;
// the prefill's two-chunk register prefetch left it waiting on memory).
// Operands come straight from the row-major copies through transposed LDS
// reads (ds_read_b64_tr_b16): K^T gives each lane its feature dim for 8
// tokens (the DPP products of psi_k), V^T the B operand.  The contraction
// index k = 8g + i of lane group g stands for token 4g + i (i < 4) or
// 16 + 4g + (i - 4) of the k-step, so that the 32 lanes a read serves at
// once cover 8 consecutive rows: no bank conflicts with the row swizzle of
// the V slots.  K is used raw, so quadratic rows come out 16 times and
// linear rows 4 times the readout units; the scale is applied once before
// the store.  Segments handled here are whole (a multiple of 64 tokens,
// inside the sequence): only the last segment can be ragged, and it needs
// no state pass.
constexpr int kStateWaves = 10;

template <int DV>
struct StateRingT {
    static constexpr int kRing = DV == 64 ? 8 : 12;  // 80 KB / 72 KB
    static constexpr int kGroup = 2;                 // chunks per barrier interval
    alignas(16) uint16_t k[kRing][kC * kDFeat];      // [64][16] row-major
    alignas(16) uint16_t v[kRing][kC * DV];           // [64][DV], 16-byte units XOR-swizzled by row
};

#define BASED_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Element offset of (row, col) in a [64][DV] V slot.  DV = 64: 8 units per
// row, swizzled by row & 7; DV = 32: 4 units, rows r and r + 4 (which share
// banks) get the unit pairs {0,1} and {2,3} swapped.
template <int DV>
__device__ __forceinline__ int sv_idx(int row, int col) {
    const int sw = DV == 64 ? (row & 7) : (((row >> 2) & 1) << 1);
    return row * DV + 8 * ((col >> 3) ^ sw) + (col & 7);
}

// Copy of 1 KB block b of chunk t (64 tokens from t0) into its ring slot:
// blocks 0, 1 are K (32 rows each), blocks 2.. are V (64 / (DV/8) rows
// each).  The DMA writes lane l's 16 bytes at byte 16 l of the block, so a
// lane fetches the source unit the swizzle stores there.
template <int DV>
__device__ __forceinline__ void state_dma(const uint16_t* kh, const uint16_t* vh, int ldv, int t0,
                                          StateRingT<DV>& rg, int slot, int b, int lane) {
    if (b < 2) {
        const int row = 32 * b + (lane >> 1);
        __builtin_amdgcn_global_load_lds(kh + (size_t)(t0 + row) * kDFeat + 8 * (lane & 1),
                                         BASED_LDS_PTR(void, &rg.k[slot][512 * b]), 16, 0, 0);
    } else {
        constexpr int kUnits = DV / 8, kRows = 64 / kUnits;
        const int vb = b - 2;
        const int row = kRows * vb + lane / kUnits;
        const int pu = lane % kUnits;  // the unit this lane's 16 bytes land in
        const int gu = (sv_idx<DV>(row, 8 * pu) - row * DV) >> 3;  // the swizzle is an involution
        __builtin_amdgcn_global_load_lds(vh + (size_t)(t0 + row) * ldv + 8 * gu,
                                         BASED_LDS_PTR(void, &rg.v[slot][512 * vb]), 16, 0, 0);
    }
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)BASED_LDS_PTR(const void, p);
}

// LDS byte addresses of this lane's reads in ring slot 0 for one k-step (32
// tokens from row tb): its 8 K values (feature dim r of its group's tokens,
// see above) and the B operand of each value column tile (the same tokens,
// column 16ct + r).  Slot s lies s slot sizes further on, which the reads
// add as an immediate offset, so the addresses are computed once.
template <int DV>
struct StateReadBase {
    uint32_t k0, k1, va[DV / 16][2];
};
template <int DV>
__device__ __forceinline__ StateReadBase<DV> state_read_base(const StateRingT<DV>& rg, int tb, int g, int r) {
    StateReadBase<DV> b;
    const int row0 = tb + 4 * g + (r >> 2), row1 = row0 + 16, col = 4 * (r & 3);
    b.k0 = lds_addr(&rg.k[0][row0 * kDFeat + col]);
    b.k1 = lds_addr(&rg.k[0][row1 * kDFeat + col]);
#pragma unroll
    for (int ct = 0; ct < DV / 16; ++ct) {
        b.va[ct][0] = lds_addr(&rg.v[0][sv_idx<DV>(row0, 16 * ct + col)]);
        b.va[ct][1] = lds_addr(&rg.v[0][sv_idx<DV>(row1, 16 * ct + col)]);
    }
    return b;
}

// The reads of one k-step in ring slot SLOT.  One asm block with its own
// wait: the compiler cannot tell these reads from the copies in flight into
// other slots and would otherwise wait for all of them.
template <int DV, int SLOT>
__device__ __forceinline__ void state_reads(const StateReadBase<DV>& b, uint2 (&kk)[2], bf16x8 (&vb)[DV / 16]) {
    constexpr int kOff = SLOT * kC * kDFeat * 2, vOff = SLOT * kC * DV * 2;  // bytes
    static_assert(kOff < 65536 && vOff < 65536, "slot offset fits the immediate field");
    uint2 x[DV / 8];
    if constexpr (DV == 64) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %10 offset:%20\n\t"
            "ds_read_b64_tr_b16 %1, %11 offset:%20\n\t"
            "ds_read_b64_tr_b16 %2, %12 offset:%21\n\t"
            "ds_read_b64_tr_b16 %3, %13 offset:%21\n\t"
            "ds_read_b64_tr_b16 %4, %14 offset:%21\n\t"
            "ds_read_b64_tr_b16 %5, %15 offset:%21\n\t"
            "ds_read_b64_tr_b16 %6, %16 offset:%21\n\t"
            "ds_read_b64_tr_b16 %7, %17 offset:%21\n\t"
            "ds_read_b64_tr_b16 %8, %18 offset:%21\n\t"
            "ds_read_b64_tr_b16 %9, %19 offset:%21\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(kk[0]), "=&v"(kk[1]), "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]),
              "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
            : "v"(b.k0), "v"(b.k1), "v"(b.va[0][0]), "v"(b.va[0][1]), "v"(b.va[1][0]), "v"(b.va[1][1]),
              "v"(b.va[2][0]), "v"(b.va[2][1]), "v"(b.va[3][0]), "v"(b.va[3][1]), "i"(kOff), "i"(vOff)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %6 offset:%12\n\t"
            "ds_read_b64_tr_b16 %1, %7 offset:%12\n\t"
            "ds_read_b64_tr_b16 %2, %8 offset:%13\n\t"
            "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
            "ds_read_b64_tr_b16 %4, %10 offset:%13\n\t"
            "ds_read_b64_tr_b16 %5, %11 offset:%13\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(kk[0]), "=&v"(kk[1]), "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
            : "v"(b.k0), "v"(b.k1), "v"(b.va[0][0]), "v"(b.va[0][1]), "v"(b.va[1][0]), "v"(b.va[1][1]),
              "i"(kOff), "i"(vOff)
            : "memory");
    }
#pragma unroll
    for (int ct = 0; ct < DV / 16; ++ct)
        vb[ct] = __builtin_bit_cast(bf16x8, u32x4{x[2 * ct].x, x[2 * ct].y, x[2 * ct + 1].x, x[2 * ct + 1].y});
}

// s_waitcnt with vmcnt = n (0..15) and the other counters left alone.
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
#define BASED_WVM(N) \
    case N: __builtin_amdgcn_s_waitcnt((N) | 0x70 | 0xF00); break;
        BASED_WVM(0) BASED_WVM(1) BASED_WVM(2) BASED_WVM(3) BASED_WVM(4) BASED_WVM(5) BASED_WVM(6) BASED_WVM(7)
        BASED_WVM(8) BASED_WVM(9) BASED_WVM(10)
#undef BASED_WVM
        default: __builtin_amdgcn_s_waitcnt(11 | 0x70 | 0xF00); break;
    }
}

// f(integral_constant<Q>, cb + QG) for Q = Q0 .. NQ - 1 while cb + QG < nch.
template <int Q, int NQ, int G, typename F>
__device__ __forceinline__ void for_groups(F& f, int cb, int nch) {
    if constexpr (Q < NQ) {
        if (cb + Q * G < nch) {
            f(std::integral_constant<int, Q>{}, cb + Q * G);
            for_groups<Q + 1, NQ, G>(f, cb, nch);
        }
    }
}

__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Readout units of rotation tile T from the raw-k sums: quadratic rows
// 1/16, linear rows (tile 9) 1/4, the constant (tile 8, row 8) 1.
template <int T>
__device__ __forceinline__ float raw_scale(int row) {
    if (T == 9) return 0.25f;
    if (T == 8 && row == 8) return 1.f;
    return 1.f / 16.f;
}

// Tiles T0 = 2P, 2P + 1 over k-step H of every chunk; the H = 1 wave hands
// its sums to the H = 0 wave, which writes the slot.
template <int P, int H, int DV>
__device__ __forceinline__ void state_pair(const uint16_t* kh, const uint16_t* vh, int ldv, int nch,
                                           StateRingT<DV>& rg, float* ws_out) {
    constexpr int kNV = DV / 16, kNCT = kNV + 1, kRing = StateRingT<DV>::kRing;
    constexpr int T0 = 2 * P, T1 = 2 * P + 1;
    constexpr int kBlocks = 2 + DV / 8;  // 1 KB copies per chunk
    const int w = P + 5 * H;
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const bf16x8 ones = ones8();
    f32x4 a0[kNCT], a1[kNCT];
#pragma unroll
    for (int ct = 0; ct < kNCT; ++ct) a0[ct] = a1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float t8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t8[i] = r == 8 ? 1.f : 0.f;
    constexpr int G = StateRingT<DV>::kGroup;
    const bool copies = w < kBlocks;
    // chunks are taken G per barrier interval (the last group of an odd
    // chunk count has one); the copies of the chunks up to kRing - G ahead
    // are in flight meanwhile
    const int first = min(kRing - G, nch);
    for (int c = 0; c < first; ++c)
        if (copies) state_dma<DV>(kh, vh, ldv, c * kC, rg, c, w, lane);
    const StateReadBase<DV> rb = state_read_base<DV>(rg, 32 * H, g, r);
    // the products of one chunk, staged in ring slot S
    auto chunk = [&](auto slot) {
        constexpr int S = decltype(slot)::value;
        uint2 kk[2];
        bf16x8 vb[kNV];
        state_reads<DV, S>(rb, kk, vb);
        float kv[8];
        kv[0] = bf16lo_f32(kk[0].x);
        kv[1] = bf16hi_f32(kk[0].x);
        kv[2] = bf16lo_f32(kk[0].y);
        kv[3] = bf16hi_f32(kk[0].y);
        kv[4] = bf16lo_f32(kk[1].x);
        kv[5] = bf16hi_f32(kk[1].x);
        kv[6] = bf16lo_f32(kk[1].y);
        kv[7] = bf16hi_f32(kk[1].y);
        const bf16x8 f0 = psi_k<T0>(kv, t8);
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) a0[ct] = mfma32(f0, vb[ct], a0[ct]);
        a0[kNV] = mfma32(f0, ones, a0[kNV]);
        const bf16x8 f1 = psi_k<T1>(kv, t8);
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) a1[ct] = mfma32(f1, vb[ct], a1[ct]);
        a1[kNV] = mfma32(f1, ones, a1[kNV]);
    };
    // group Q of a ring turn: chunks c0 = cb + QG .. + G - 1 (slots QG..),
    // the copies of the chunks kRing - G further on issued first.  The loop
    // runs whole ring turns, so every slot index is a constant.
    auto group = [&](auto q, int c0) {
        constexpr int Q = decltype(q)::value;
        // this wave's copies of chunks c0 .. c0 + G - 1 have landed once at
        // most the copies of the chunks after them are outstanding; the
        // barrier makes every wave's copies visible and frees the slots of
        // the previous group
        if (copies) wait_vm(min(c0 + kRing - G, nch) - min(c0 + G, nch));
        raw_barrier();
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int cn = c0 + kRing - G + j;
            if (copies && cn < nch) state_dma<DV>(kh, vh, ldv, cn * kC, rg, (Q * G + kRing - G + j) % kRing, w, lane);
        }
        chunk(std::integral_constant<int, (Q * G) % kRing>{});
        if (c0 + 1 < nch) chunk(std::integral_constant<int, (Q * G + 1) % kRing>{});
    };
    static_assert(G == 2 && kRing % G == 0, "two chunks per interval, whole groups per ring turn");
    for (int cb = 0; cb < nch; cb += kRing) for_groups<0, kRing / G, G>(group, cb, nch);
    // the H = 1 waves' sums through LDS (the ring is free after the barrier)
    raw_barrier();
    f32x4* xch = reinterpret_cast<f32x4*>(&rg.k[0][0]) + (size_t)P * 2 * kNCT * 64;
    if (H == 1) {
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct) {
            xch[ct * 64 + lane] = a0[ct];
            xch[(kNCT + ct) * 64 + lane] = a1[ct];
        }
    }
    __syncthreads();
    if (H == 0) {
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct) {
            a0[ct] += xch[ct * 64 + lane];
            a1[ct] += xch[(kNCT + ct) * 64 + lane];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                a0[ct][m] *= raw_scale<T0>(4 * g + m);
                a1[ct][m] *= raw_scale<T1>(4 * g + m);
            }
        }
        ws_store<T0, DV>(a0, ws_out, lane);
        ws_store<T1, DV>(a1, ws_out, lane);
    }
}

template <int T, int DV>
__device__ __forceinline__ void init_tile(const float* Sh, const float* zh, int ldv, int use_init, float* ws_out) {
    constexpr int kNCT = DV / 16 + 1;
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    f32x4 acc[kNCT];
#pragma unroll
    for (int ct = 0; ct < kNCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (use_init) load_initial<T, DV>(acc, Sh, zh, ldv, g, r);
    ws_store<T, DV>(acc, ws_out, lane);
}

// Workgroup (head, segment s, column group), mapped as the prefill's: for
// s < nseg - 1 the increment of segment s into slot s + 1; for s = nseg - 1
// the caller's initial state (or zeros) into slot 0.
template <int DV>
__global__ __launch_bounds__(64 * kStateWaves) void segment_state_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int L, int ldv, int ncg, int seg_len, int nseg,
    const float* __restrict__ S, const float* __restrict__ z, int use_init, float* __restrict__ ws) {
    static_assert(sizeof(StateRingT<DV>) >= 5 * 2 * (DV / 16 + 1) * 64 * 16, "exchange area");
    __shared__ StateRingT<DV> rg;
    const int total = gridDim.x;
    int b = blockIdx.x;
    if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);
    const int cg = b % ncg;
    const int hs = b / ncg;
    const int seg = hs % nseg;
    const int head = hs / nseg;
    const int BH = total / (ncg * nseg);
    const int col0 = cg * DV;
    float* ws_out = ws + (((size_t)((seg + 1) % nseg) * BH + head) * ncg + cg) * ws_slot_floats<DV>();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (seg == nseg - 1) {
        const float* Sh = S + (size_t)head * kNumFeat * ldv + col0;
        const float* zh = z + (size_t)head * kNumFeat;
        switch (w) {
            case 0: init_tile<0, DV>(Sh, zh, ldv, use_init, ws_out); break;
            case 1: init_tile<1, DV>(Sh, zh, ldv, use_init, ws_out); break;
            case 2: init_tile<2, DV>(Sh, zh, ldv, use_init, ws_out); break;
            case 3: init_tile<3, DV>(Sh, zh, ldv, use_init, ws_out); break;
            case 4: init_tile<4, DV>(Sh, zh, ldv, use_init, ws_out); break;
            case 5: init_tile<5, DV>(Sh, zh, ldv, use_init, ws_out); break;
            case 6: init_tile<6, DV>(Sh, zh, ldv, use_init, ws_out); break;
            case 7: init_tile<7, DV>(Sh, zh, ldv, use_init, ws_out); break;
            case 8: init_tile<8, DV>(Sh, zh, ldv, use_init, ws_out); break;
            default: init_tile<9, DV>(Sh, zh, ldv, use_init, ws_out); break;
        }
        return;
    }
    const int tb = seg * seg_len;
    const uint16_t* kh = k + ((size_t)head * L + tb) * kDFeat;
    const uint16_t* vh = v + ((size_t)head * L + tb) * ldv + col0;
    const int nch = seg_len / kC;
    switch (w) {
        case 0: state_pair<0, 0, DV>(kh, vh, ldv, nch, rg, ws_out); break;
        case 1: state_pair<1, 0, DV>(kh, vh, ldv, nch, rg, ws_out); break;
        case 2: state_pair<2, 0, DV>(kh, vh, ldv, nch, rg, ws_out); break;
        case 3: state_pair<3, 0, DV>(kh, vh, ldv, nch, rg, ws_out); break;
        case 4: state_pair<4, 0, DV>(kh, vh, ldv, nch, rg, ws_out); break;
        case 5: state_pair<0, 1, DV>(kh, vh, ldv, nch, rg, ws_out); break;
        case 6: state_pair<1, 1, DV>(kh, vh, ldv, nch, rg, ws_out); break;
        case 7: state_pair<2, 1, DV>(kh, vh, ldv, nch, rg, ws_out); break;
        case 8: state_pair<3, 1, DV>(kh, vh, ldv, nch, rg, ws_out); break;
        default: state_pair<4, 1, DV>(kh, vh, ldv, nch, rg, ws_out); break;
    }
}

}  // namespace

// The instances compiled in prefill_mfma_ilp.hip: prefill_mfma_kernel<32,
// kModeFull> (dvl == 32, whole sequences) and <64, kModeSegment> (dvl == 64,
// the segment pass), launched on `st` with the kernel's own arguments.
// Any other (dvl, mode) returns hipErrorInvalidValue and launches nothing.
hipError_t launch_prefill_ilp_instance(int dvl, int mode, dim3 grid, hipStream_t st, const uint16_t* q,
                                       const uint16_t* k, const uint16_t* v, int L, int ldv, int ncg, int seg_len,
                                       int nseg, float eps, float* y, float* S, float* z, int use_init, float* ws);

}  // namespace based

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
// Every product is a 16x16 MFMA tile per wave (16 rows of its own, 16 of the
// other side at a time).  The operand layouts line up without register
// transposes: a score tile computed as K Q^T (keys x queries) leaves lane
// (g, r) with query r and keys 4g..4g+3, which is the A operand of a product
// over those keys for query row r; the staged tiles supply the other operand
// (K^T, V^T and G^T copies in LDS where a column of a row-major matrix is
// needed).  q, k, v are exact in bf16; the weights a, g and e are used as
// hi/lo bf16 pairs (about 16 significant bits), accumulation is fp32.
//
// Query side (one workgroup per 64 queries, wave w: queries 16w..16w+15):
//   pass 1 over the key tiles at or before the queries: N and D, then g, h
//   (to the workspace and, as bf16 hi/lo, to this wave's LDS);
//   pass 2: ga^T = V g^T, e, dq += e K.
// Key side (one workgroup per 64 keys): over the query tiles at or after the
// keys: s = Q K^T, dv += a^T g, ga = g V^T, e, dk += e^T Q.
#include "common.hpp"
#include "kernels.hpp"

namespace based {
namespace {

constexpr int kT = 64;         // rows per tile (queries or keys)
constexpr int kD = 16;         // feature dim of this path
constexpr int kRowQK = 24;     // LDS row stride (bf16) of Q and K tiles
constexpr int kRowT = 72;      // LDS row stride (bf16) of transposed tiles [dim][64]
constexpr float kInvSqrtD = 0.25f;

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
__device__ __forceinline__ bf16x8 join44(const uint16_t* p0, const uint16_t* p1) {
    const uint2 a = *reinterpret_cast<const uint2*>(p0);
    const uint2 b = *reinterpret_cast<const uint2*>(p1);
    const u32x4 u = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, u);
}
// hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void hilo4(const float (&x)[4], bf16x4& hi, bf16x4& lo) {
    const uint32_t h0 = pack_bf16x2(x[0], x[1]), h1 = pack_bf16x2(x[2], x[3]);
    const uint32_t l0 = pack_bf16x2(x[0] - bf16lo_f32(h0), x[1] - bf16hi_f32(h0));
    const uint32_t l1 = pack_bf16x2(x[2] - bf16lo_f32(h1), x[3] - bf16hi_f32(h1));
    hi = __builtin_bit_cast(bf16x4, make_uint2(h0, h1));
    lo = __builtin_bit_cast(bf16x4, make_uint2(l0, l1));
}
__device__ __forceinline__ void hilo8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        l[i] = pack_bf16x2(x[2 * i] - bf16lo_f32(h[i]), x[2 * i + 1] - bf16hi_f32(h[i]));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Stages a [64][W] bf16 tile (rows row0.. of a [L][W] matrix, rows past L
// zero) row-major into `rm` (row stride W + 8) and, if `tr`, transposed into
// `tr` ([W][kRowT]).
template <int W>
__device__ __forceinline__ void stage_tile(const uint16_t* mat, int L, int row0, uint16_t* rm, uint16_t* tr) {
    constexpr int kU = W / 8;  // 16-byte units per row
    for (int e = threadIdx.x; e < kT * kU; e += 256) {
        const int row = e / kU, u = e % kU;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row0 + row < L) x = *reinterpret_cast<const u32x4*>(mat + (size_t)(row0 + row) * W + 8 * u);
        *reinterpret_cast<u32x4*>(rm + row * (W + 8) + 8 * u) = x;
        if (tr) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tr[(8 * u + 2 * i) * kRowT + row] = (uint16_t)(x[i] & 0xffffu);
                tr[(8 * u + 2 * i + 1) * kRowT + row] = (uint16_t)(x[i] >> 16);
            }
        }
    }
}

template <int DV>
struct BwdQSmem {
    alignas(16) uint16_t q[kT * (kD + 8)];
    alignas(16) uint16_t k[kT * (kD + 8)];
    alignas(16) uint16_t kt[kD * kRowT];
    alignas(16) uint16_t v[kT * (DV + 8)];
    alignas(16) uint16_t vt[DV * kRowT];
    alignas(16) uint16_t ghi[4][16 * (DV + 8)];  // per wave: g of its 16 queries
    alignas(16) uint16_t glo[4][16 * (DV + 8)];
    float h[4][16];
};

// ---- query side
template <int DV>
__global__ __launch_bounds__(256) void bwd_query_mfma_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             const float* __restrict__ dy, int L, int ntiles,
                                                             float eps, float* __restrict__ dq,
                                                             float* __restrict__ g_ws, float* __restrict__ h_ws) {
    constexpr int kNV = DV / 16;  // column tiles
    __shared__ BwdQSmem<DV> sm;
    const int BH = gridDim.x / ntiles;
    const int head = blockIdx.x % BH;
    const int ti = ntiles - 1 - (int)(blockIdx.x / BH);  // the longest rows first, every head
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const uint16_t* qh = q + (size_t)head * L * kD;
    const uint16_t* kh = k + (size_t)head * L * kD;
    const uint16_t* vh = v + (size_t)head * L * DV;
    const int qw0 = ti * kT + 16 * w;  // first query of this wave
    const int qr = qw0 + r;            // this lane's query in score tiles

    stage_tile<kD>(qh, L, ti * kT, sm.q, nullptr);
    // ---- pass 1: N (yacc, rows = queries 4g+m, columns 16ct + r) and D
    f32x4 yacc[kNV];
#pragma unroll
    for (int ct = 0; ct < kNV; ++ct) yacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    for (int tj = 0; tj <= ti; ++tj) {
        __syncthreads();
        stage_tile<kD>(kh, L, tj * kT, sm.k, nullptr);
        stage_tile<DV>(vh, L, tj * kT, sm.v, sm.vt);
        __syncthreads();
        const bf16x4 qb = ld4(&sm.q[(16 * w + r) * (kD + 8) + 4 * g]);
        float a[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const f32x4 st = mfma16(ld4(&sm.k[(16 * kt + r) * (kD + 8) + 4 * g]), qb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int kg = tj * kT + 16 * kt + 4 * g + m;
                const float s = st[m] * kInvSqrtD;
                const float w8 = fmaf(s, fmaf(s, 0.5f, 1.f), 1.f);
                a[kt][m] = (kg <= qr && kg < L) ? w8 : 0.f;
                lsum += a[kt][m];
            }
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const float x[8] = {a[2 * p][0],     a[2 * p][1],     a[2 * p][2],     a[2 * p][3],
                                a[2 * p + 1][0], a[2 * p + 1][1], a[2 * p + 1][2], a[2 * p + 1][3]};
            bf16x8 ahi, alo;
            hilo8(x, ahi, alo);
#pragma unroll
            for (int ct = 0; ct < kNV; ++ct) {
                const uint16_t* row = &sm.vt[(16 * ct + r) * kRowT + 32 * p + 4 * g];
                const bf16x8 vb = join44(row, row + 16);
                yacc[ct] = mfma32(ahi, vb, yacc[ct]);
                yacc[ct] = mfma32(alo, vb, yacc[ct]);
            }
        }
    }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);  // D - eps of query qr, on every lane group

    // ---- g = dy/D, h = -(dy.y)/D for queries qw0 + 4g + m, columns 16ct + r
    float gv[kNV][4], hq[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int qi = qw0 + 4 * g + m;
        const float inv = 1.f / (__shfl(lsum, 4 * g + m, 64) + eps);
        float dyy = 0.f;
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) {
            const float dyc = qi < L ? dy[((size_t)head * L + qi) * DV + 16 * ct + r] : 0.f;
            dyy = fmaf(dyc, yacc[ct][m] * inv, dyy);
            gv[ct][m] = dyc * inv;
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) dyy += __shfl_xor(dyy, off, 64);
        hq[m] = -dyy * inv;
        if (qi < L) {
#pragma unroll
            for (int ct = 0; ct < kNV; ++ct) g_ws[((size_t)head * L + qi) * DV + 16 * ct + r] = gv[ct][m];
            if (r == 0) h_ws[(size_t)head * L + qi] = hq[m];
        }
    }
    // this wave's g as bf16 hi/lo rows [16 queries][DV], h per query
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) {
            const float x = gv[ct][m];
            const uint32_t hb = pack_bf16x2(x, 0.f);
            const uint32_t lb = pack_bf16x2(x - bf16lo_f32(hb), 0.f);
            sm.ghi[w][(4 * g + m) * (DV + 8) + 16 * ct + r] = (uint16_t)(hb & 0xffffu);
            sm.glo[w][(4 * g + m) * (DV + 8) + 16 * ct + r] = (uint16_t)(lb & 0xffffu);
        }
        if (r == 0) sm.h[w][4 * g + m] = hq[m];
    }

    // ---- pass 2: dq (rows = queries 4g+m, columns = feature r)
    f32x4 dqacc = {0.f, 0.f, 0.f, 0.f};
    for (int tj = 0; tj <= ti; ++tj) {
        __syncthreads();  // also orders this wave's g/h writes before its reads
        stage_tile<kD>(kh, L, tj * kT, sm.k, sm.kt);
        stage_tile<DV>(vh, L, tj * kT, sm.v, nullptr);
        __syncthreads();
        const bf16x4 qb = ld4(&sm.q[(16 * w + r) * (kD + 8) + 4 * g]);
        const float hr = sm.h[w][r];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const f32x4 st = mfma16(ld4(&sm.k[(16 * kt + r) * (kD + 8) + 4 * g]), qb, f32x4{0.f, 0.f, 0.f, 0.f});
            // ga^T: rows = keys 16kt + 4g + m, columns = queries r
            f32x4 ga = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cs = 0; cs < DV / 32; ++cs) {
                const bf16x8 va = ld8(&sm.v[(16 * kt + r) * (DV + 8) + 32 * cs + 8 * g]);
                ga = mfma32(va, ld8(&sm.ghi[w][r * (DV + 8) + 32 * cs + 8 * g]), ga);
                ga = mfma32(va, ld8(&sm.glo[w][r * (DV + 8) + 32 * cs + 8 * g]), ga);
            }
            float e[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int kg = tj * kT + 16 * kt + 4 * g + m;
                const float s = st[m] * kInvSqrtD;
                e[m] = (kg <= qr && kg < L) ? (ga[m] + hr) * (1.f + s) * kInvSqrtD : 0.f;
            }
            bf16x4 ehi, elo;
            hilo4(e, ehi, elo);
            const bf16x4 kb = ld4(&sm.kt[r * kRowT + 16 * kt + 4 * g]);
            dqacc = mfma16(ehi, kb, dqacc);
            dqacc = mfma16(elo, kb, dqacc);
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int qi = qw0 + 4 * g + m;
        if (qi < L) dq[((size_t)head * L + qi) * kD + r] = dqacc[m];
    }
}


template <int DV>
struct BwdKSmem {
    alignas(16) uint16_t q[kT * (kD + 8)];
    alignas(16) uint16_t qt[kD * kRowT];
    alignas(16) uint16_t ghi[kT * (DV + 8)];  // g of the query tile, hi / lo, row-major
    alignas(16) uint16_t glo[kT * (DV + 8)];
    alignas(16) uint16_t gthi[DV * kRowT];    // and transposed
    alignas(16) uint16_t gtlo[DV * kRowT];
    float h[kT];
};

// Stages g (fp32 rows row0.. of a [L][DV] matrix, rows past L zero) as bf16
// hi/lo pairs, row-major and transposed, and h of those rows.
template <int DV>
__device__ __forceinline__ void stage_g(const float* gh, const float* hh, int L, int row0, BwdKSmem<DV>& sm) {
    constexpr int kU = DV / 4;  // float4 units per row
    for (int e = threadIdx.x; e < kT * kU; e += 256) {
        const int row = e / kU, u = e % kU;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (row0 + row < L) x = *reinterpret_cast<const f32x4*>(gh + (size_t)(row0 + row) * DV + 4 * u);
        const float xs[4] = {x[0], x[1], x[2], x[3]};
        bf16x4 hi, lo;
        hilo4(xs, hi, lo);
        const uint2 hu = __builtin_bit_cast(uint2, hi), lu = __builtin_bit_cast(uint2, lo);
        *reinterpret_cast<uint2*>(&sm.ghi[row * (DV + 8) + 4 * u]) = hu;
        *reinterpret_cast<uint2*>(&sm.glo[row * (DV + 8) + 4 * u]) = lu;
        const uint32_t hw[2] = {hu.x, hu.y}, lw[2] = {lu.x, lu.y};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sm.gthi[(4 * u + i) * kRowT + row] = (uint16_t)(hw[i >> 1] >> (16 * (i & 1)));
            sm.gtlo[(4 * u + i) * kRowT + row] = (uint16_t)(lw[i >> 1] >> (16 * (i & 1)));
        }
    }
    if (threadIdx.x < kT) sm.h[threadIdx.x] = row0 + (int)threadIdx.x < L ? hh[row0 + threadIdx.x] : 0.f;
}

// ---- key side
template <int DV>
__global__ __launch_bounds__(256) void bwd_key_mfma_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, int L, int ntiles,
                                                           const float* __restrict__ g_ws,
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
    const uint16_t* kh = k + (size_t)head * L * kD;
    const uint16_t* vh = v + (size_t)head * L * DV;
    const float* gh = g_ws + (size_t)head * L * DV;
    const float* hh = h_ws + (size_t)head * L;
    const int kw0 = tj * kT + 16 * w;  // first key of this wave
    const int kr = kw0 + r;            // this lane's key in score tiles

    // this lane's key and value row pieces: the B operands of Q K^T and g V^T
    bf16x4 kb = __builtin_bit_cast(bf16x4, make_uint2(0u, 0u));
    bf16x8 vb[DV / 32];
#pragma unroll
    for (int cs = 0; cs < DV / 32; ++cs) vb[cs] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    if (kr < L) {
        kb = ld4(kh + (size_t)kr * kD + 4 * g);
#pragma unroll
        for (int cs = 0; cs < DV / 32; ++cs) vb[cs] = ld8(vh + (size_t)kr * DV + 32 * cs + 8 * g);
    }
    f32x4 dvacc[kNV];
#pragma unroll
    for (int ct = 0; ct < kNV; ++ct) dvacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 dkacc = {0.f, 0.f, 0.f, 0.f};

    for (int ti = tj; ti < ntiles; ++ti) {
        __syncthreads();
        stage_tile<kD>(qh, L, ti * kT, sm.q, sm.qt);
        stage_g<DV>(gh, hh, L, ti * kT, sm);
        __syncthreads();
        // a and e for queries ti*64 + 16qt + 4g + m and key kr
        float a[4][4], e[4][4];
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
            const f32x4 st = mfma16(ld4(&sm.q[(16 * qt + r) * (kD + 8) + 4 * g]), kb, f32x4{0.f, 0.f, 0.f, 0.f});
            f32x4 ga = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cs = 0; cs < DV / 32; ++cs) {
                ga = mfma32(ld8(&sm.ghi[(16 * qt + r) * (DV + 8) + 32 * cs + 8 * g]), vb[cs], ga);
                ga = mfma32(ld8(&sm.glo[(16 * qt + r) * (DV + 8) + 32 * cs + 8 * g]), vb[cs], ga);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int qg = ti * kT + 16 * qt + 4 * g + m;
                const bool ok = qg >= kr && qg < L;
                const float s = st[m] * kInvSqrtD;
                a[qt][m] = ok ? fmaf(s, fmaf(s, 0.5f, 1.f), 1.f) : 0.f;
                e[qt][m] = ok ? (ga[m] + sm.h[16 * qt + 4 * g + m]) * (1.f + s) * kInvSqrtD : 0.f;
            }
        }
        // dv += a^T g and dk += e^T Q, 32 queries per product
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const float xa[8] = {a[2 * p][0],     a[2 * p][1],     a[2 * p][2],     a[2 * p][3],
                                 a[2 * p + 1][0], a[2 * p + 1][1], a[2 * p + 1][2], a[2 * p + 1][3]};
            const float xe[8] = {e[2 * p][0],     e[2 * p][1],     e[2 * p][2],     e[2 * p][3],
                                 e[2 * p + 1][0], e[2 * p + 1][1], e[2 * p + 1][2], e[2 * p + 1][3]};
            bf16x8 ahi, alo, ehi, elo;
            hilo8(xa, ahi, alo);
            hilo8(xe, ehi, elo);
#pragma unroll
            for (int ct = 0; ct < kNV; ++ct) {
                const uint16_t* rh = &sm.gthi[(16 * ct + r) * kRowT + 32 * p + 4 * g];
                const uint16_t* rl = &sm.gtlo[(16 * ct + r) * kRowT + 32 * p + 4 * g];
                const bf16x8 gbh = join44(rh, rh + 16), gbl = join44(rl, rl + 16);
                dvacc[ct] = mfma32(ahi, gbh, dvacc[ct]);
                dvacc[ct] = mfma32(alo, gbh, dvacc[ct]);
                dvacc[ct] = mfma32(ahi, gbl, dvacc[ct]);
            }
            const uint16_t* rq = &sm.qt[r * kRowT + 32 * p + 4 * g];
            const bf16x8 qb = join44(rq, rq + 16);
            dkacc = mfma32(ehi, qb, dkacc);
            dkacc = mfma32(elo, qb, dkacc);
        }
    }
    // rows = keys kw0 + 4g + m; dv columns 16ct + r, dk feature r
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int kj = kw0 + 4 * g + m;
        if (kj < L) {
#pragma unroll
            for (int ct = 0; ct < kNV; ++ct) dvo[((size_t)head * L + kj) * DV + 16 * ct + r] = dvacc[ct][m];
            dk[((size_t)head * L + kj) * kD + r] = dkacc[m];
        }
    }
}

}  // namespace

template <int DV>
static void launch_both(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* dy, int BH, int L,
                        float eps, float* dq, float* dk, float* dvo, float* g_ws, float* h_ws, hipStream_t st) {
    const int ntiles = (L + kT - 1) / kT;
    const dim3 grid((unsigned)(ntiles * BH));
    hipLaunchKernelGGL((bwd_query_mfma_kernel<DV>), grid, dim3(256), 0, st, q, k, v, dy, L, ntiles, eps, dq, g_ws,
                       h_ws);
    hipLaunchKernelGGL((bwd_key_mfma_kernel<DV>), grid, dim3(256), 0, st, q, k, v, L, ntiles, g_ws, h_ws, dk, dvo);
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

// swa_backward.hip -- gradients of the causal sliding-window softmax on the
// gfx950 matrix cores (bf16 operands, fp32 accumulation): d_qk = 64,
// d_v in {64, 128}, windows of 1..64 keys.
//
// Method: "Simple linear attention language models balance the
// recall-throughput tradeoff", s4 "Local Exact Attention" (query i attends
// to the keys j in (i - w, i] with exact softmax weights) and s5 (the
// prefill also serves training).  With P_ij the softmax weights of query
// i, l_ij = scale q_i . k_j and y_i = sum_j P_ij v_j:
//   dv_j = sum_i P_ij dy_i,   dP_ij = dy_i . v_j,   D_i = sum_j P_ij dP_ij,
//   dS_ij = P_ij (dP_ij - D_i),
//   dq_i = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i.
//
// MI355X design
//  * Two kernels, one workgroup of four waves per (head, 64-row tile), each
//    wave 16 rows: the query side (dq, and per query the row maximum, the
//    inverse row sum and D_i into the workspace) and the key side (dk, dv,
//    rebuilding P from those three numbers).  With w <= 64 the rows of one
//    wave meet the 80 rows of five 16-row tiles of the other side, all
//    inside the 128 rows staged in LDS (the previous and the current tile
//    on the query side, the current and the next on the key side).
//  * Every product is a 16x16x32 bf16 MFMA.  The score tiles come out with
//    lane (g, r) holding row r against the other side's rows 4g..4g+3 of a
//    tile, which is as it stands the A operand of the next product over
//    that side (two tiles per 32-wide k-step); the B operands that need a
//    column of a row-major LDS tile come from transposed reads
//    (ds_read_b64_tr_b16).
//  * Operands that are not bf16 inputs (P, dS, and dy, which is fp32) enter
//    as bf16 hi/lo pairs.
//  * LDS rows are cut into 16-byte units XOR-swizzled by the row's low
//    three bits, so 16 lanes reading one unit of 16 consecutive rows hit
//    distinct banks.

#include "common.hpp"
#include "kernels.hpp"

namespace based {
namespace {

constexpr int kT = 64;     // rows per tile
constexpr int kDQK = 64;   // d_qk
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Element offset of (row, col) in a row-major [rows][W] bf16 tile.
template <int W>
__device__ __forceinline__ int sw_idx(int row, int col) {
    return row * W + 8 * ((col >> 3) ^ (row & 7)) + (col & 7);
}
template <int W>
__device__ __forceinline__ bf16x8 row8(const uint16_t* t, int row, int col) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(t + sw_idx<W>(row, col)));
}
// Transposed read: lane c of each 16-lane group passes the address of row
// rb + c/4, columns col0 + 4(c%4) .. +3, and receives rows rb .. rb+3 of
// column col0 + c.
template <int W>
__device__ __forceinline__ uint2 col4(const uint16_t* t, int rb, int col0, int c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const uint16_t* p = t + sw_idx<W>(rb + (c >> 2), col0 + 4 * (c & 3));
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) s16x4*)(p)));
}
// B operand of one 32-wide k-step over the row pairs (tile a, tile b):
// rows 4g..4g+3 of each, column col0 + c.
template <int W>
__device__ __forceinline__ bf16x8 colpair(const uint16_t* t, int ra, int rb, int col0, int c) {
    const uint2 x = col4<W>(t, ra, col0, c), y = col4<W>(t, rb, col0, c);
    return __builtin_bit_cast(bf16x8, u32x4{x.x, x.y, y.x, y.y});
}

// hi = bf16(x), lo = bf16(x - hi) for 8 values.
__device__ __forceinline__ void hilo8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        l[i] = lo_pair_of(h[i], x[2 * i], x[2 * i + 1]);
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Stage rows row0 .. row0 + 127 (clamped into [0, L)) of a [L][W] bf16
// matrix into a swizzled LDS tile.
template <int W>
__device__ __forceinline__ void stage_bf16(uint16_t* t, const uint16_t* src, int row0, int L) {
    constexpr int kU = W / 8;
    for (int u = threadIdx.x; u < 2 * kT * kU; u += 256) {
        const int row = u / kU, cu = u % kU;
        const int sr = min(max(row0 + row, 0), L - 1);
        *reinterpret_cast<u32x4*>(t + sw_idx<W>(row, 8 * cu)) =
            *reinterpret_cast<const u32x4*>(src + (size_t)sr * W + 8 * cu);
    }
}

// Per query: the row maximum of scale*log2(e)*q.k over its window, the
// inverse of the row sum of exp2(. - max), and D.
struct RowStats {
    float mx, inv, D, pad;
};

// ---------------------------------------------------------------- query side
template <int DV>
__global__ __launch_bounds__(256) void swa_bwd_query_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const float* __restrict__ dy, int L, int ntiles,
                                                            int window, float sl2, float scale,
                                                            float* __restrict__ dq, RowStats* __restrict__ stats) {
    constexpr int kNS = DV / 32;  // k-steps of dy . v
    __shared__ alignas(16) uint16_t ks[2 * kT * kDQK];
    __shared__ alignas(16) uint16_t vs[2 * kT * DV];
    const int head = blockIdx.x / ntiles, q0 = (blockIdx.x % ntiles) * kT;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const uint16_t* qh = q + (size_t)head * L * kDQK;
    const uint16_t* kh = k + (size_t)head * L * kDQK;
    const uint16_t* vh = v + (size_t)head * L * DV;
    const float* dyh = dy + (size_t)head * L * DV;

    // keys q0 - 64 .. q0 + 63 (rows outside [0, L) only meet masked weights)
    stage_bf16<kDQK>(ks, kh, q0 - kT, L);
    stage_bf16<DV>(vs, vh, q0 - kT, L);

    // this lane's query row (B operand of the scores) and its dy row (B
    // operand of dy . v, as a hi/lo pair)
    const int qi = q0 + 16 * w + r;
    const int qc = min(qi, L - 1);
    bf16x8 qb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        qb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + (size_t)qc * kDQK + 32 * s + 8 * g));
    bf16x8 dyb_hi[kNS], dyb_lo[kNS];
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
        float x[8];
        const f32x4 a = *reinterpret_cast<const f32x4*>(dyh + (size_t)qc * DV + 32 * s + 8 * g);
        const f32x4 b = *reinterpret_cast<const f32x4*>(dyh + (size_t)qc * DV + 32 * s + 8 * g + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = a[i];
            x[4 + i] = b[i];
        }
        hilo8(x, dyb_hi[s], dyb_lo[s]);
    }
    __syncthreads();

    // scores of the five key tiles 16(w + i) .. +15 of the staged rows
    // (keys q0 - 64 + 16(w + i) + 4g + m for query qi)
    float p[5][4], dp[5][4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int row = 16 * (w + i) + r;
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
        sc = mfma32(row8<kDQK>(ks, row, 8 * g), qb[0], sc);
        sc = mfma32(row8<kDQK>(ks, row, 32 + 8 * g), qb[1], sc);
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kNS; ++s) {
            const bf16x8 vr = row8<DV>(vs, row, 32 * s + 8 * g);
            d = mfma32(vr, dyb_hi[s], d);
            d = mfma32(vr, dyb_lo[s], d);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int kap = q0 - kT + 16 * (w + i) + 4 * g + m;
            const bool ok = kap <= qi && kap > qi - window && kap >= 0;
            p[i][m] = ok ? sc[m] * sl2 : -INFINITY;
            dp[i][m] = d[m];
            mx = fmaxf(mx, p[i][m]);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));  // finite: the query's own key is in its window
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            p[i][m] = __builtin_amdgcn_exp2f(p[i][m] - mx);
            l += p[i][m];
        }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.f / l;
    float D = 0.f;
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            p[i][m] *= inv;
            D = fmaf(p[i][m], dp[i][m], D);
        }
    D += __shfl_xor(D, 16, 64);
    D += __shfl_xor(D, 32, 64);

    // dq = scale * dS K over the key pairs (0, 1), (2, 3), (4, -)
    f32x4 acc[kDQK / 16];
#pragma unroll
    for (int ct = 0; ct < kDQK / 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks2 = 0; ks2 < 3; ++ks2) {
        const bool two = 2 * ks2 + 1 < 5;
        float x[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            x[m] = p[2 * ks2][m] * (dp[2 * ks2][m] - D);
            x[4 + m] = two ? p[two ? 2 * ks2 + 1 : 0][m] * (dp[two ? 2 * ks2 + 1 : 0][m] - D) : 0.f;
        }
        bf16x8 xh, xl;
        hilo8(x, xh, xl);
        const int ra = 16 * (w + 2 * ks2) + 4 * g;
        const int rb = two ? ra + 16 : ra;  // (a zero operand half needs no particular rows)
#pragma unroll
        for (int ct = 0; ct < kDQK / 16; ++ct) {
            const bf16x8 kb = colpair<kDQK>(ks, ra, rb, 16 * ct, r);
            acc[ct] = mfma32(xh, kb, acc[ct]);
            acc[ct] = mfma32(xl, kb, acc[ct]);
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int row = q0 + 16 * w + 4 * g + m;
        if (row < L) {
#pragma unroll
            for (int ct = 0; ct < kDQK / 16; ++ct)
                dq[((size_t)head * L + row) * kDQK + 16 * ct + r] = scale * acc[ct][m];
        }
    }
    if (g == 0 && qi < L) stats[(size_t)head * L + qi] = RowStats{mx, inv, D, 0.f};
}

// ---------------------------------------------------------------- key side
template <int DV>
__global__ __launch_bounds__(256) void swa_bwd_key_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const float* __restrict__ dy, int L, int ntiles,
                                                          int window, float sl2, float scale,
                                                          const RowStats* __restrict__ stats,
                                                          float* __restrict__ dk, float* __restrict__ dvo) {
    constexpr int kNS = DV / 32;
    __shared__ alignas(16) uint16_t qs[2 * kT * kDQK];
    __shared__ alignas(16) uint16_t dyhi[2 * kT * DV];
    __shared__ alignas(16) uint16_t dylo[2 * kT * DV];
    __shared__ RowStats st[2 * kT];
    const int head = blockIdx.x / ntiles, k0 = (blockIdx.x % ntiles) * kT;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const uint16_t* qh = q + (size_t)head * L * kDQK;
    const uint16_t* kh = k + (size_t)head * L * kDQK;
    const uint16_t* vh = v + (size_t)head * L * DV;
    const float* dyh = dy + (size_t)head * L * DV;

    // queries k0 .. k0 + 127 (rows past L only meet masked weights)
    stage_bf16<kDQK>(qs, qh, k0, L);
    {
        constexpr int kU = DV / 8;
        for (int u = threadIdx.x; u < 2 * kT * kU; u += 256) {
            const int row = u / kU, cu = u % kU;
            const int sr = min(k0 + row, L - 1);
            const f32x4 a = *reinterpret_cast<const f32x4*>(dyh + (size_t)sr * DV + 8 * cu);
            const f32x4 b = *reinterpret_cast<const f32x4*>(dyh + (size_t)sr * DV + 8 * cu + 4);
            const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            bf16x8 hi, lo;
            hilo8(x, hi, lo);
            *reinterpret_cast<bf16x8*>(dyhi + sw_idx<DV>(row, 8 * cu)) = hi;
            *reinterpret_cast<bf16x8*>(dylo + sw_idx<DV>(row, 8 * cu)) = lo;
        }
        for (int u = threadIdx.x; u < 2 * kT; u += 256) st[u] = stats[(size_t)head * L + min(k0 + u, L - 1)];
    }

    // this lane's key row (B operand of the scores) and value row (B
    // operand of dy . v)
    const int kj = k0 + 16 * w + r;
    const int kc = min(kj, L - 1);
    bf16x8 kb[2], vb[kNS];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        kb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kh + (size_t)kc * kDQK + 32 * s + 8 * g));
#pragma unroll
    for (int s = 0; s < kNS; ++s)
        vb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vh + (size_t)kc * DV + 32 * s + 8 * g));
    __syncthreads();

    // the five query tiles 16(w + t) .. +15 of the staged rows (queries
    // k0 + 16(w + t) + 4g + m for key kj): P and dS
    float p[5][4], ds[5][4];
#pragma unroll
    for (int t = 0; t < 5; ++t) {
        const int row = 16 * (w + t) + r;
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
        sc = mfma32(row8<kDQK>(qs, row, 8 * g), kb[0], sc);
        sc = mfma32(row8<kDQK>(qs, row, 32 + 8 * g), kb[1], sc);
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kNS; ++s) {
            d = mfma32(row8<DV>(dyhi, row, 32 * s + 8 * g), vb[s], d);
            d = mfma32(row8<DV>(dylo, row, 32 * s + 8 * g), vb[s], d);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int srow = 16 * (w + t) + 4 * g + m;
            const int qa = k0 + srow;
            const bool ok = qa >= kj && qa < kj + window && qa < L;
            const RowStats rs = st[srow];
            const float pv = ok ? __builtin_amdgcn_exp2f(fmaf(sc[m], sl2, -rs.mx)) * rs.inv : 0.f;
            p[t][m] = pv;
            ds[t][m] = pv * (d[m] - rs.D);
        }
    }

    // dv = P^T dy and dk = scale * dS^T Q over the query pairs (0, 1), (2, 3), (4, -)
    f32x4 av[DV / 16], ak[kDQK / 16];
#pragma unroll
    for (int ct = 0; ct < DV / 16; ++ct) av[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < kDQK / 16; ++ct) ak[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks2 = 0; ks2 < 3; ++ks2) {
        const bool two = 2 * ks2 + 1 < 5;
        float xp[8], xs[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            xp[m] = p[2 * ks2][m];
            xs[m] = ds[2 * ks2][m];
            xp[4 + m] = two ? p[two ? 2 * ks2 + 1 : 0][m] : 0.f;
            xs[4 + m] = two ? ds[two ? 2 * ks2 + 1 : 0][m] : 0.f;
        }
        bf16x8 ph, pl, sh, sl;
        hilo8(xp, ph, pl);
        hilo8(xs, sh, sl);
        const int ra = 16 * (w + 2 * ks2) + 4 * g;
        const int rb = two ? ra + 16 : ra;
#pragma unroll
        for (int ct = 0; ct < DV / 16; ++ct) {
            const bf16x8 bh = colpair<DV>(dyhi, ra, rb, 16 * ct, r);
            const bf16x8 bl = colpair<DV>(dylo, ra, rb, 16 * ct, r);
            av[ct] = mfma32(ph, bh, av[ct]);
            av[ct] = mfma32(pl, bh, av[ct]);
            av[ct] = mfma32(ph, bl, av[ct]);
        }
#pragma unroll
        for (int ct = 0; ct < kDQK / 16; ++ct) {
            const bf16x8 qbt = colpair<kDQK>(qs, ra, rb, 16 * ct, r);
            ak[ct] = mfma32(sh, qbt, ak[ct]);
            ak[ct] = mfma32(sl, qbt, ak[ct]);
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int row = k0 + 16 * w + 4 * g + m;
        if (row < L) {
#pragma unroll
            for (int ct = 0; ct < DV / 16; ++ct) dvo[((size_t)head * L + row) * DV + 16 * ct + r] = av[ct][m];
#pragma unroll
            for (int ct = 0; ct < kDQK / 16; ++ct)
                dk[((size_t)head * L + row) * kDQK + 16 * ct + r] = scale * ak[ct][m];
        }
    }
}

}  // namespace

size_t swa_backward_workspace_bytes(int BH, int L) { return (size_t)BH * L * sizeof(RowStats); }

hipError_t launch_swa_backward(const void* q, const void* k, const void* v, const float* dy, int BH, int L, int dv,
                               int window, float scale, float* dq, float* dk, float* dvo, void* workspace,
                               hipStream_t st) {
    const int ntiles = (L + kT - 1) / kT;
    const dim3 grid((unsigned)(BH * ntiles));
    const float sl2 = scale * kLog2e;
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* vv = static_cast<const uint16_t*>(v);
    RowStats* rs = static_cast<RowStats*>(workspace);
    if (dv == 64) {
        hipLaunchKernelGGL(swa_bwd_query_kernel<64>, grid, dim3(256), 0, st, qq, kk, vv, dy, L, ntiles, window, sl2,
                           scale, dq, rs);
        hipLaunchKernelGGL(swa_bwd_key_kernel<64>, grid, dim3(256), 0, st, qq, kk, vv, dy, L, ntiles, window, sl2,
                           scale, rs, dk, dvo);
    } else {
        hipLaunchKernelGGL(swa_bwd_query_kernel<128>, grid, dim3(256), 0, st, qq, kk, vv, dy, L, ntiles, window, sl2,
                           scale, dq, rs);
        hipLaunchKernelGGL(swa_bwd_key_kernel<128>, grid, dim3(256), 0, st, qq, kk, vv, dy, L, ntiles, window, sl2,
                           scale, rs, dk, dvo);
    }
    return hipGetLastError();
}

}  // namespace based

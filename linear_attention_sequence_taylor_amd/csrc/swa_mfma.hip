// swa_mfma.hip -- causal sliding-window softmax attention on the gfx950
// matrix cores (bf16 operands, fp32 softmax and accumulation).
//
// "Simple linear attention language models balance the recall-throughput
// tradeoff", s4 "Local Exact Attention": each query attends with exact
// softmax to the preceding `window` keys (its own included), O(L*window)
// work; BASED adds it to the linear-attention output of the same layer, so
// the kernel fuses y = add + softmax-window(q, k, v).
//
// MI355X design
//  * One workgroup (4 waves) per (batch*head, 64-query tile); wave w owns
//    queries i0+16w .. i0+16w+15, whose keys lie in 80 rows
//    [i0+16w-64, i0+16w+16) = 5 key tiles of 16.
//  * Q, K rows and V^T (transposed for the P.V operand) of the tile and its
//    64-row halo are staged in LDS once; the workgroup's halo is the
//    previous tile, which the block order keeps on the same XCD (its L2).
//  * Scores are computed transposed, S^T = K Q^T (16x16xK MFMA), so each
//    lane holds one query and 4 keys per tile: the probabilities are already
//    in the A-operand layout of P.V (keys of two tiles form one 32-deep
//    k-step).  Softmax runs in fp32 (exp2, max-subtracted); P enters the
//    MFMA as a hi/lo bf16 pair so the weights carry ~16 bits.
//  * The normaliser is the fp32 sum of the same probabilities; output is
//    fp32 with the optional fused add.
#include "common.hpp"
#include "kernels.hpp"

namespace based {
namespace {

constexpr int kQT = 64;        // queries per workgroup
constexpr int kKR = 128;       // key rows staged: 64-row halo + the tile
constexpr int kDV = 64;
constexpr int kVtRow = 136;    // LDS row stride (bf16) of V^T [col][key]
constexpr float kLog2e = 1.4426950408889634f;

template <int DQK>
struct SwaSmem {
    static constexpr int kRow = DQK + 8;  // padded row stride (bf16) of Q and K
    alignas(16) uint16_t q[kQT * kRow];
    alignas(16) uint16_t k[kKR * kRow];
    alignas(16) uint16_t vt[kDV * kVtRow];
};

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ __forceinline__ void pack8_hilo(const float (&a)[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = pack_bf16x2(a[2 * i], a[2 * i + 1]);
        l[i] = pack_bf16x2(a[2 * i] - bf16lo_f32(h[i]), a[2 * i + 1] - bf16hi_f32(h[i]));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Stage Q (64 rows), K (128 rows) row-major and V^T (64 x 128) into LDS.
// Rows outside [0, L) are zero.
template <int DQK>
__device__ __forceinline__ void swa_stage(const uint16_t* qh, const uint16_t* kh, const uint16_t* vh, int L,
                                          int i0, SwaSmem<DQK>& sm) {
    constexpr int kRow = SwaSmem<DQK>::kRow;
    constexpr int kVec = DQK / 8;  // 16-byte vectors per q/k row
    const int tid = threadIdx.x;
    const int kbase = i0 - 64;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // Q rows
    for (int e = tid; e < kQT * kVec; e += 256) {
        const int row = e / kVec, c8 = e % kVec, qi = i0 + row;
        const u32x4 x = qi < L ? *reinterpret_cast<const u32x4*>(qh + (size_t)qi * DQK + 8 * c8) : zero;
        uint2* d = reinterpret_cast<uint2*>(&sm.q[row * kRow + 8 * c8]);
        d[0] = make_uint2(x[0], x[1]);
        d[1] = make_uint2(x[2], x[3]);
    }
    // K rows
    for (int e = tid; e < kKR * kVec; e += 256) {
        const int row = e / kVec, c8 = e % kVec, kj = kbase + row;
        const u32x4 x =
            (kj >= 0 && kj < L) ? *reinterpret_cast<const u32x4*>(kh + (size_t)kj * DQK + 8 * c8) : zero;
        uint2* d = reinterpret_cast<uint2*>(&sm.k[row * kRow + 8 * c8]);
        d[0] = make_uint2(x[0], x[1]);
        d[1] = make_uint2(x[2], x[3]);
    }
    // V^T: each thread takes a pair of key rows and 8 columns.
    for (int e = tid; e < (kKR / 2) * (kDV / 8); e += 256) {
        const int p = e % (kKR / 2), cb = e / (kKR / 2);
        const int ka = kbase + 2 * p, kb = ka + 1;
        const u32x4 a = (ka >= 0 && ka < L) ? *reinterpret_cast<const u32x4*>(vh + (size_t)ka * kDV + 8 * cb) : zero;
        const u32x4 b = (kb >= 0 && kb < L) ? *reinterpret_cast<const u32x4*>(vh + (size_t)kb * kDV + 8 * cb) : zero;
        uint32_t* vt = reinterpret_cast<uint32_t*>(&sm.vt[0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vt[((8 * cb + 2 * i) * kVtRow + 2 * p) >> 1] = lo_pair(a[i], b[i]);
            vt[((8 * cb + 2 * i + 1) * kVtRow + 2 * p) >> 1] = hi_pair(a[i], b[i]);
        }
    }
}

// S^T tile: rows = 16 keys (LDS rows kr0..kr0+15), cols = the wave's 16
// queries (LDS rows qr0..qr0+15).  Lane (g, r): query r, keys 4g..4g+3.
template <int DQK>
__device__ __forceinline__ f32x4 score_tile(const SwaSmem<DQK>& sm, int kr0, int qr0, int g, int r) {
    constexpr int kRow = SwaSmem<DQK>::kRow;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DQK == 16) {
        const bf16x4 a = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(&sm.k[(kr0 + r) * kRow + 4 * g]));
        const bf16x4 b = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(&sm.q[(qr0 + r) * kRow + 4 * g]));
        acc = mfma16(a, b, acc);
    } else {
#pragma unroll
        for (int kk = 0; kk < DQK / 32; ++kk) {
            const uint16_t* ka = &sm.k[(kr0 + r) * kRow + 32 * kk + 8 * g];
            const uint16_t* qb = &sm.q[(qr0 + r) * kRow + 32 * kk + 8 * g];
            const uint2 a0 = reinterpret_cast<const uint2*>(ka)[0], a1 = reinterpret_cast<const uint2*>(ka)[1];
            const uint2 b0 = reinterpret_cast<const uint2*>(qb)[0], b1 = reinterpret_cast<const uint2*>(qb)[1];
            const u32x4 au = {a0.x, a0.y, a1.x, a1.y}, bu = {b0.x, b0.y, b1.x, b1.y};
            acc = mfma32(__builtin_bit_cast(bf16x8, au), __builtin_bit_cast(bf16x8, bu), acc);
        }
    }
    return acc;
}

template <int DQK>
__global__ __launch_bounds__(256) void swa_mfma_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, int L, int ntiles,
                                                       int total, int window, float scale, const float* add,
                                                       float* y) {
    __shared__ SwaSmem<DQK> sm;
    // Block order: the 8 XCDs take blocks round-robin, so give XCD x a
    // contiguous run of tiles (each tile's halo is its predecessor, already
    // in that XCD's L2).
    int b = blockIdx.x;
    if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);
    const int head = b / ntiles;
    const int i0 = (b % ntiles) * kQT;
    const uint16_t* qh = q + (size_t)head * L * DQK;
    const uint16_t* kh = k + (size_t)head * L * DQK;
    const uint16_t* vh = v + (size_t)head * L * kDV;
    swa_stage<DQK>(qh, kh, vh, L, i0, sm);
    __syncthreads();

    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const int q0 = i0 + 16 * w;           // first query of the wave
    const int qi = q0 + r;                // this lane's query
    const float sl2 = scale * kLog2e;

    // Scores for key tiles t = 0..4: keys q0 - 64 + 16t + 4g + m.
    float s[5][4];
#pragma unroll
    for (int t = 0; t < 5; ++t) {
        const f32x4 st = score_tile<DQK>(sm, 16 * w + 16 * t, 16 * w, g, r);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int kj = q0 - 64 + 16 * t + 4 * g + m;
            const bool ok = kj >= 0 && kj <= qi && kj > qi - window;
            s[t][m] = ok ? st[m] * sl2 : -INFINITY;
        }
    }
    // Row max over all 80 keys: this lane's 20, then across the 4 lane groups.
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 5; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m) mx = fmaxf(mx, s[t][m]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float l = 0.f;
#pragma unroll
    for (int t = 0; t < 5; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float p = exp2f(s[t][m] - mx);  // masked keys: exp2(-inf) = 0
            s[t][m] = p;
            l += p;
        }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);

    // Y = P V over 3 k-steps of 32 keys (tiles 2p, 2p+1; tile 5 is empty).
    f32x4 yacc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) yacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        float a[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            a[m] = s[2 * p][m];
            a[4 + m] = 2 * p + 1 < 5 ? s[(2 * p + 1 < 5) ? 2 * p + 1 : 0][m] : 0.f;
        }
        bf16x8 ahi, alo;
        pack8_hilo(a, ahi, alo);
        bf16x8 vb[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            // keys (LDS rows) 16w + 32p + 4g .. +3 and 16w + 32p + 16 + 4g .. +3
            const uint16_t* vr = &sm.vt[(16 * ct + r) * kVtRow + 16 * w + 32 * p + 4 * g];
            const uint2 x0 = *reinterpret_cast<const uint2*>(vr);
            // k-step 2 has no second key tile: its half of the operand is zero
            // (and must not be read: it would run past the staged keys).
            const uint2 x1 = 2 * p + 1 < 5 ? *reinterpret_cast<const uint2*>(vr + 16) : make_uint2(0u, 0u);
            const u32x4 u = {x0.x, x0.y, x1.x, x1.y};
            vb[ct] = __builtin_bit_cast(bf16x8, u);
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) yacc[ct] = mfma32(ahi, vb[ct], yacc[ct]);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) yacc[ct] = mfma32(alo, vb[ct], yacc[ct]);
    }

    // Rows of yacc are queries q0 + 4g + m; the normaliser of query q0+j
    // lives in lane group (j >> 2)... every lane of row group j holds it
    // for its own query r, so fetch l of query 4g + m from lane 4g + m.
    const size_t base = (size_t)head * L;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int qq = q0 + 4 * g + m;
        const float lq = __shfl(l, 4 * g + m, 64);
        if (qq < L) {
            const float inv = 1.f / lq;
            const size_t o = (base + qq) * kDV + r;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const float prev = add ? add[o + 16 * ct] : 0.f;
                y[o + 16 * ct] = prev + yacc[ct][m] * inv;
            }
        }
    }
}

}  // namespace

hipError_t launch_swa_mfma(const void* q, const void* k, const void* v, int BH, int L, int dqk, int window,
                           float scale, const float* add, float* y, hipStream_t st) {
    const int ntiles = (L + kQT - 1) / kQT;
    const int total = BH * ntiles;
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* vv = static_cast<const uint16_t*>(v);
    if (dqk == 16)
        hipLaunchKernelGGL((swa_mfma_kernel<16>), dim3(total), dim3(256), 0, st, qq, kk, vv, L, ntiles, total,
                           window, scale, add, y);
    else
        hipLaunchKernelGGL((swa_mfma_kernel<64>), dim3(total), dim3(256), 0, st, qq, kk, vv, L, ntiles, total,
                           window, scale, add, y);
    return hipGetLastError();
}

}  // namespace based

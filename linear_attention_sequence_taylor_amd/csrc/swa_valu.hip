// swa_valu.hip -- causal sliding-window softmax attention on the vector ALUs
// in fp32 (gfx950): the exact-precision path for fp32 inputs, and for bf16
// heads too long for the 32-bit offsets of the MFMA kernels in swa_mfma.hip.
// Windows up to 128 keys with 64 value columns stage every key row a tile
// can see at once; other windows and widths go through 64-row key blocks.
//
// "Simple linear attention language models balance the recall-throughput
// tradeoff", s4 "Local Exact Attention": each query attends with exact
// softmax to the preceding `window` keys (its own included); O(L*window).
//
// One workgroup per (batch*head, 32-query tile).  The tile's queries and the
// keys/values they can see (32 + window - 1 rows) are staged in LDS; eight
// threads share a query, each producing 8 of the 64 output columns with a
// one-pass (running max) softmax in fp32.
#include "common.hpp"
#include "kernels.hpp"

namespace based {

constexpr int kSwaValuQ = 32;

// MAXW: the largest window the staged key rows cover (64 or 128).
template <typename T, int DQK, int MAXW>
__global__ __launch_bounds__(256) void swa_valu_kernel(const T* __restrict__ q,
                                                       const T* __restrict__ k,
                                                       const T* __restrict__ v, int L, int window,
                                                       float scale, const float* add,
                                                       float* y) {
    constexpr int DV = 64;
    constexpr int KR = kSwaValuQ + MAXW - 1;  // key rows staged
    __shared__ float s_q[kSwaValuQ][DQK];
    __shared__ float s_k[KR][DQK];
    __shared__ float s_v[KR][DV];

    const int ntiles = (L + kSwaValuQ - 1) / kSwaValuQ;
    const int head = blockIdx.x / ntiles;
    const int i0 = (blockIdx.x % ntiles) * kSwaValuQ;
    const int tid = threadIdx.x;
    const int jbase = i0 - (MAXW - 1);  // key row of s_k[0]

    const T* qh = q + (size_t)head * L * DQK;
    const T* kh = k + (size_t)head * L * DQK;
    const T* vh = v + (size_t)head * L * DV;
    for (int e = tid; e < kSwaValuQ * DQK; e += 256) {
        const int t = e / DQK, a = e % DQK;
        s_q[t][a] = (i0 + t < L) ? load_elem(qh, (size_t)(i0 + t) * DQK + a) : 0.f;
    }
    for (int e = tid; e < KR * DQK; e += 256) {
        const int t = e / DQK, a = e % DQK, j = jbase + t;
        s_k[t][a] = (j >= 0 && j < L) ? load_elem(kh, (size_t)j * DQK + a) : 0.f;
    }
    for (int e = tid; e < KR * DV; e += 256) {
        const int t = e / DV, c = e % DV, j = jbase + t;
        s_v[t][c] = (j >= 0 && j < L) ? load_elem(vh, (size_t)j * DV + c) : 0.f;
    }
    __syncthreads();

    const int qi = tid / 8;
    const int cb = (tid % 8) * 8;
    const int i = i0 + qi;
    if (i >= L) return;
    const int jlo = max(0, i - window + 1);
    float m = -INFINITY, l = 0.f;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
    for (int j = jlo; j <= i; ++j) {
        const int r = j - jbase;
        float dot = 0.f;
#pragma unroll
        for (int a = 0; a < DQK; ++a) dot = fmaf(s_q[qi][a], s_k[r][a], dot);
        const float logit = scale * dot;
        if (logit > m) {
            const float corr = expf(m - logit);  // 0 on the first key
            l *= corr;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] *= corr;
            m = logit;
        }
        const float p = expf(logit - m);
        l += p;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(p, s_v[r][cb + c], acc[c]);
    }
    const float inv = 1.0f / l;
    const size_t o = ((size_t)head * L + i) * DV + cb;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float base = add ? add[o + c] : 0.f;
        y[o + c] = base + acc[c] * inv;
    }
}

// Any window and value width DV (64 or 128): the keys a 32-query tile can
// see are staged in LDS 64 rows at a time, and every query keeps a running
// maximum, normaliser and DV/8-column numerator (one-pass softmax) across
// the blocks.  Eight threads share a query.
template <typename T, int DQK, int DV>
__global__ __launch_bounds__(256) void swa_valu_blocked_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                               const T* __restrict__ v, int L, int window,
                                                               float scale, const float* add, float* y) {
    constexpr int kKB = 64;       // key rows per staged block
    constexpr int kCPT = DV / 8;  // output columns per thread
    __shared__ float s_q[kSwaValuQ][DQK];
    __shared__ float s_k[kKB][DQK];
    __shared__ float s_v[kKB][DV];

    const int ntiles = (L + kSwaValuQ - 1) / kSwaValuQ;
    const int head = blockIdx.x / ntiles;
    const int i0 = (blockIdx.x % ntiles) * kSwaValuQ;
    const int tid = threadIdx.x;
    const T* qh = q + (size_t)head * L * DQK;
    const T* kh = k + (size_t)head * L * DQK;
    const T* vh = v + (size_t)head * L * DV;
    for (int e = tid; e < kSwaValuQ * DQK; e += 256) {
        const int t = e / DQK, a = e % DQK;
        s_q[t][a] = (i0 + t < L) ? load_elem(qh, (size_t)(i0 + t) * DQK + a) : 0.f;
    }
    const int qi = tid / 8;
    const int cb = (tid % 8) * kCPT;
    const int i = i0 + qi;
    const int jlo = max(0, i - window + 1);
    float m = -INFINITY, l = 0.f;
    float acc[kCPT];
#pragma unroll
    for (int c = 0; c < kCPT; ++c) acc[c] = 0.f;
    const int jfirst = max(0, i0 - window + 1);
    const int jlast = min(L - 1, i0 + kSwaValuQ - 1);
    for (int jb = jfirst; jb <= jlast; jb += kKB) {
        __syncthreads();  // the previous block is no longer read
        for (int e = tid; e < kKB * DQK; e += 256) {
            const int t = e / DQK, a = e % DQK, j = jb + t;
            s_k[t][a] = j < L ? load_elem(kh, (size_t)j * DQK + a) : 0.f;
        }
        for (int e = tid; e < kKB * DV; e += 256) {
            const int t = e / DV, c = e % DV, j = jb + t;
            s_v[t][c] = j < L ? load_elem(vh, (size_t)j * DV + c) : 0.f;
        }
        __syncthreads();
        const int ja = max(jb, jlo), je = min(jb + kKB - 1, i);
        for (int j = ja; j <= je; ++j) {
            const int rr = j - jb;
            float dot = 0.f;
#pragma unroll
            for (int a = 0; a < DQK; ++a) dot = fmaf(s_q[qi][a], s_k[rr][a], dot);
            const float logit = scale * dot;
            if (logit > m) {
                const float corr = expf(m - logit);  // 0 on the first key
                l *= corr;
#pragma unroll
                for (int c = 0; c < kCPT; ++c) acc[c] *= corr;
                m = logit;
            }
            const float p = expf(logit - m);
            l += p;
#pragma unroll
            for (int c = 0; c < kCPT; ++c) acc[c] = fmaf(p, s_v[rr][cb + c], acc[c]);
        }
    }
    if (i >= L) return;
    const float inv = 1.0f / l;
    const size_t o = ((size_t)head * L + i) * DV + cb;
#pragma unroll
    for (int c = 0; c < kCPT; ++c) {
        const float base = add ? add[o + c] : 0.f;
        y[o + c] = base + acc[c] * inv;
    }
}

template <typename T, int DV>
static void launch_blocked(dim3 grid, hipStream_t st, const T* q, const T* k, const T* v, int L, int dqk, int window,
                           float scale, const float* add, float* y) {
    if (dqk == 16)
        hipLaunchKernelGGL((swa_valu_blocked_kernel<T, 16, DV>), grid, dim3(256), 0, st, q, k, v, L, window, scale,
                           add, y);
    else
        hipLaunchKernelGGL((swa_valu_blocked_kernel<T, 64, DV>), grid, dim3(256), 0, st, q, k, v, L, window, scale,
                           add, y);
}

template <typename T>
static hipError_t launch_swa_valu_t(const void* q, const void* k, const void* v, int BH, int L,
                                    int dqk, int dv, int window, float scale, const float* add, float* y,
                                    hipStream_t st) {
    const int ntiles = (L + kSwaValuQ - 1) / kSwaValuQ;
    const dim3 grid((unsigned)BH * ntiles);
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    if (dv != 64 || window > 128) {
        if (dv == 64) launch_blocked<T, 64>(grid, st, qq, kk, vv, L, dqk, window, scale, add, y);
        else launch_blocked<T, 128>(grid, st, qq, kk, vv, L, dqk, window, scale, add, y);
    } else if (window <= 64) {
        if (dqk == 16)
            hipLaunchKernelGGL((swa_valu_kernel<T, 16, 64>), grid, dim3(256), 0, st, qq, kk, vv, L, window,
                               scale, add, y);
        else
            hipLaunchKernelGGL((swa_valu_kernel<T, 64, 64>), grid, dim3(256), 0, st, qq, kk, vv, L, window,
                               scale, add, y);
    } else {
        if (dqk == 16)
            hipLaunchKernelGGL((swa_valu_kernel<T, 16, 128>), grid, dim3(256), 0, st, qq, kk, vv, L, window,
                               scale, add, y);
        else
            hipLaunchKernelGGL((swa_valu_kernel<T, 64, 128>), grid, dim3(256), 0, st, qq, kk, vv, L, window,
                               scale, add, y);
    }
    return hipGetLastError();
}

hipError_t launch_swa_valu(const void* q, const void* k, const void* v, bool bf16, int BH, int L,
                           int dqk, int dv, int window, float scale, const float* add, float* y,
                           hipStream_t st) {
    return bf16 ? launch_swa_valu_t<uint16_t>(q, k, v, BH, L, dqk, dv, window, scale, add, y, st)
                : launch_swa_valu_t<float>(q, k, v, BH, L, dqk, dv, window, scale, add, y, st);
}

}  // namespace based

// prefill_backward.hip -- gradients of causal Taylor linear attention for
// training-mode prefill (gfx950), fp32 on the vector ALUs.
//
// "Simple linear attention language models balance the recall-throughput
// tradeoff", s5 (prefill also serves training) and s4 "Taylor Linear
// Attention": with s_ij = q_i.k_j/sqrt(d'), a_ij = 1 + s_ij + s_ij^2/2,
// y_i = N_i / D_i, N_i = sum_{j<=i} a_ij v_j, D_i = sum_{j<=i} a_ij + eps,
// the chain rule for an upstream gradient dy gives
//   g_i = dy_i / D_i,  h_i = -(dy_i . y_i) / D_i,
//   e_ij = (g_i . v_j + h_i) (1 + s_ij) / sqrt(d'),
//   dq_i = sum_{j<=i} e_ij k_j,  dk_j = sum_{i>=j} e_ij q_i,
//   dv_j = sum_{i>=j} a_ij g_i.
//
// Two kernels, one thread per row, tiles of the other side staged in LDS
// (every lane of a wave reads the same staged row, a broadcast):
//   query side: N_i and D_i, then g_i and h_i (to the workspace) and dq_i;
//   key side:   dk_j and dv_j from the queries at or after j.
// This is the direct (quadratic) form: O(L^2) work per head.  bf16 inputs
// with feature dim 16 take the matrix-core kernels of
// prefill_backward_mfma.hip instead (same workspace layout).
#include "common.hpp"
#include "kernels.hpp"

namespace based {
namespace {

constexpr int kRows = 128;  // rows (threads) per workgroup
constexpr int kTile = 32;   // staged rows of the other side

template <typename T, int D, int DV>
__global__ __launch_bounds__(kRows) void bwd_query_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ v, const float* __restrict__ dy,
                                                          int L, float eps, float* __restrict__ dq,
                                                          float* __restrict__ g_ws, float* __restrict__ h_ws) {
    __shared__ float s_k[kTile][D];
    __shared__ float s_v[kTile][DV];
    const int nb = (L + kRows - 1) / kRows;
    const int head = blockIdx.x / nb;
    const int i0 = (blockIdx.x % nb) * kRows;
    const int i = i0 + threadIdx.x;
    const bool live = i < L;
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const T* qh = q + (size_t)head * L * D;
    const T* kh = k + (size_t)head * L * D;
    const T* vh = v + (size_t)head * L * DV;

    float qi[D];
#pragma unroll
    for (int e = 0; e < D; ++e) qi[e] = live ? load_elem(qh, (size_t)i * D + e) : 0.f;
    float acc[DV];
#pragma unroll
    for (int c = 0; c < DV; ++c) acc[c] = 0.f;
    float den = eps;
    const int jend = min(L, i0 + kRows);  // keys any row of this block can see

    auto stage = [&](int j0) {
        __syncthreads();
        for (int e = threadIdx.x; e < kTile * D; e += kRows) {
            const int r = e / D, a = e % D;
            s_k[r][a] = j0 + r < L ? load_elem(kh, (size_t)(j0 + r) * D + a) : 0.f;
        }
        for (int e = threadIdx.x; e < kTile * DV; e += kRows) {
            const int r = e / DV, c = e % DV;
            s_v[r][c] = j0 + r < L ? load_elem(vh, (size_t)(j0 + r) * DV + c) : 0.f;
        }
        __syncthreads();
    };
    // ---- N_i and D_i
    for (int j0 = 0; j0 < jend; j0 += kTile) {
        stage(j0);
        const int n = min(kTile, i - j0 + 1);  // keys j0 .. i of this tile
        for (int r = 0; r < n; ++r) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) s = fmaf(qi[e], s_k[r][e], s);
            s *= inv_sqrt_d;
            const float a = fmaf(s, fmaf(s, 0.5f, 1.f), 1.f);
            den += a;
#pragma unroll
            for (int c = 0; c < DV; ++c) acc[c] = fmaf(a, s_v[r][c], acc[c]);
        }
    }
    // ---- g_i (in acc) and h_i
    float h = 0.f;
    if (live) {
        const float inv = 1.f / den;
        const float* dyi = dy + ((size_t)head * L + i) * DV;
        float* gi = g_ws + ((size_t)head * L + i) * DV;
        float dyy = 0.f;
#pragma unroll
        for (int c = 0; c < DV; ++c) {
            const float dyc = dyi[c];
            dyy = fmaf(dyc, acc[c] * inv, dyy);
            acc[c] = dyc * inv;
            gi[c] = acc[c];
        }
        h = -dyy * inv;
        h_ws[(size_t)head * L + i] = h;
    }
    // ---- dq_i
    float dqi[D];
#pragma unroll
    for (int e = 0; e < D; ++e) dqi[e] = 0.f;
    for (int j0 = 0; j0 < jend; j0 += kTile) {
        stage(j0);
        const int n = min(kTile, i - j0 + 1);
        for (int r = 0; r < n; ++r) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) s = fmaf(qi[e], s_k[r][e], s);
            s *= inv_sqrt_d;
            float ga = h;
#pragma unroll
            for (int c = 0; c < DV; ++c) ga = fmaf(acc[c], s_v[r][c], ga);
            const float w = ga * (1.f + s) * inv_sqrt_d;
#pragma unroll
            for (int e = 0; e < D; ++e) dqi[e] = fmaf(w, s_k[r][e], dqi[e]);
        }
    }
    if (live) {
        float* dqo = dq + ((size_t)head * L + i) * D;
#pragma unroll
        for (int e = 0; e < D; ++e) dqo[e] = dqi[e];
    }
}

template <typename T, int D, int DV>
__global__ __launch_bounds__(kRows) void bwd_key_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                        const T* __restrict__ v, int L,
                                                        const float* __restrict__ g_ws, const float* __restrict__ h_ws,
                                                        float* __restrict__ dk, float* __restrict__ dvo) {
    __shared__ float s_q[kTile][D];
    __shared__ float s_g[kTile][DV];
    __shared__ float s_h[kTile];
    const int nb = (L + kRows - 1) / kRows;
    const int head = blockIdx.x / nb;
    const int j0b = (blockIdx.x % nb) * kRows;
    const int j = j0b + threadIdx.x;
    const bool live = j < L;
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const T* qh = q + (size_t)head * L * D;
    const T* kh = k + (size_t)head * L * D;
    const T* vh = v + (size_t)head * L * DV;

    float kj[D], vj[DV], dkj[D], dvj[DV];
#pragma unroll
    for (int e = 0; e < D; ++e) {
        kj[e] = live ? load_elem(kh, (size_t)j * D + e) : 0.f;
        dkj[e] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < DV; ++c) {
        vj[c] = live ? load_elem(vh, (size_t)j * DV + c) : 0.f;
        dvj[c] = 0.f;
    }
    // queries from the block's first key on; each thread uses i >= j
    for (int i0 = (j0b / kTile) * kTile; i0 < L; i0 += kTile) {
        __syncthreads();
        for (int e = threadIdx.x; e < kTile * D; e += kRows) {
            const int r = e / D, a = e % D;
            s_q[r][a] = i0 + r < L ? load_elem(qh, (size_t)(i0 + r) * D + a) : 0.f;
        }
        for (int e = threadIdx.x; e < kTile * DV; e += kRows) {
            const int r = e / DV, c = e % DV;
            s_g[r][c] = i0 + r < L ? g_ws[((size_t)head * L + i0 + r) * DV + c] : 0.f;
        }
        for (int r = threadIdx.x; r < kTile; r += kRows) s_h[r] = i0 + r < L ? h_ws[(size_t)head * L + i0 + r] : 0.f;
        __syncthreads();
        const int rb = max(0, j - i0), re = min(kTile, L - i0);  // queries max(i0, j) .. of this tile
        for (int r = rb; r < re; ++r) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) s = fmaf(s_q[r][e], kj[e], s);
            s *= inv_sqrt_d;
            const float a = fmaf(s, fmaf(s, 0.5f, 1.f), 1.f);
            float ga = s_h[r];
#pragma unroll
            for (int c = 0; c < DV; ++c) {
                ga = fmaf(s_g[r][c], vj[c], ga);
                dvj[c] = fmaf(a, s_g[r][c], dvj[c]);
            }
            const float w = ga * (1.f + s) * inv_sqrt_d;
#pragma unroll
            for (int e = 0; e < D; ++e) dkj[e] = fmaf(w, s_q[r][e], dkj[e]);
        }
    }
    if (live) {
        float* dko = dk + ((size_t)head * L + j) * D;
        float* dvo_j = dvo + ((size_t)head * L + j) * DV;
#pragma unroll
        for (int e = 0; e < D; ++e) dko[e] = dkj[e];
#pragma unroll
        for (int c = 0; c < DV; ++c) dvo_j[c] = dvj[c];
    }
}

template <typename T, int D, int DV>
hipError_t launch_bwd(const void* q, const void* k, const void* v, const float* dy, int BH, int L, float eps,
                      float* dq, float* dk, float* dv, float* g_ws, float* h_ws, hipStream_t st) {
    const dim3 grid((unsigned)(((L + kRows - 1) / kRows) * BH));
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    // bf16 with feature dim 16 runs on the matrix cores
    if (sizeof(T) == 2 && D == kDFeat) return launch_prefill_backward_mfma(q, k, v, dy, BH, L, DV, eps, dq, dk, dv,
                                                                          g_ws, h_ws, st);
    hipLaunchKernelGGL((bwd_query_kernel<T, D, DV>), grid, dim3(kRows), 0, st, qq, kk, vv, dy, L, eps, dq, g_ws, h_ws);
    hipLaunchKernelGGL((bwd_key_kernel<T, D, DV>), grid, dim3(kRows), 0, st, qq, kk, vv, L, g_ws, h_ws, dk, dv);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_dv(const void* q, const void* k, const void* v, const float* dy, int BH, int L, int dv_dim,
                         float eps, float* dq, float* dk, float* dv, float* g_ws, float* h_ws, hipStream_t st) {
    return dv_dim == 64 ? launch_bwd<T, D, 64>(q, k, v, dy, BH, L, eps, dq, dk, dv, g_ws, h_ws, st)
                        : launch_bwd<T, D, 128>(q, k, v, dy, BH, L, eps, dq, dk, dv, g_ws, h_ws, st);
}

template <typename T>
hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const float* dy, int BH, int L, int d, int dv_dim,
                        float eps, float* dq, float* dk, float* dv, float* g_ws, float* h_ws, hipStream_t st) {
    switch (d) {
        case 8: return launch_bwd_dv<T, 8>(q, k, v, dy, BH, L, dv_dim, eps, dq, dk, dv, g_ws, h_ws, st);
        case 24: return launch_bwd_dv<T, 24>(q, k, v, dy, BH, L, dv_dim, eps, dq, dk, dv, g_ws, h_ws, st);
        case 32: return launch_bwd_dv<T, 32>(q, k, v, dy, BH, L, dv_dim, eps, dq, dk, dv, g_ws, h_ws, st);
        default: return launch_bwd_dv<T, 16>(q, k, v, dy, BH, L, dv_dim, eps, dq, dk, dv, g_ws, h_ws, st);
    }
}

}  // namespace

size_t prefill_backward_workspace_bytes(int BH, int L, int dv) {
    return (size_t)BH * L * (dv + 1) * sizeof(float);
}

hipError_t launch_prefill_backward(const void* q, const void* k, const void* v, const float* dy, bool bf16, int BH,
                                   int L, int d, int dv_dim, float eps, float* dq, float* dk, float* dv,
                                   void* workspace, hipStream_t st) {
    float* g_ws = static_cast<float*>(workspace);
    float* h_ws = g_ws + (size_t)BH * L * dv_dim;
    return bf16 ? launch_bwd_t<uint16_t>(q, k, v, dy, BH, L, d, dv_dim, eps, dq, dk, dv, g_ws, h_ws, st)
                : launch_bwd_t<float>(q, k, v, dy, BH, L, d, dv_dim, eps, dq, dk, dv, g_ws, h_ws, st);
}

}  // namespace based

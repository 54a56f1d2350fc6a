// prefill_valu.hip -- chunked causal Taylor linear attention on the vector
// ALUs in fp32 (gfx950).  This is the exact-precision path: fp32 inputs and
// every chunk length 16/32/64 (bf16 inputs with chunk 64 take the MFMA
// kernel in prefill_mfma.hip).
//
// "Simple linear attention language models balance the recall-throughput
// tradeoff", App. B "Forward / Generation Prefill": the sequence is tiled;
// inside a tile the causally masked pairwise weights give the on-diagonal
// term, earlier tiles enter through the cumulative Taylor-order state (the
// off-diagonal term), and the state is carried to the next tile.  The
// pairwise weight is the closed form phi(q).phi(k) = 1 + s + s^2/2 with
// s = q.k/sqrt(d') (s4 "Taylor Linear Attention").
//
// One workgroup per (batch, head).  The caller's S and z buffers are the
// working state (updated in place, L2-resident); this path is sized for
// exactness, not speed.
#include "common.hpp"
#include "kernels.hpp"

namespace based {

template <typename T, int C, int DV, int D>
__global__ __launch_bounds__(256) void prefill_valu_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ k,
                                                           const T* __restrict__ v, int L,
                                                           float eps, float* __restrict__ y,
                                                           float* __restrict__ S,
                                                           float* __restrict__ z, int use_init) {
    constexpr int kTPT = 256 / C;   // threads per token
    constexpr int kCPT = DV / kTPT; // columns per thread
    constexpr int kF = Feat<D>::kF;
    __shared__ float s_q[C][D];
    __shared__ float s_k[C][D];
    __shared__ float s_v[C][DV];

    const int head = blockIdx.x;
    const int tid = threadIdx.x;
    const T* qh = q + (size_t)head * L * D;
    const T* kh = k + (size_t)head * L * D;
    const T* vh = v + (size_t)head * L * DV;
    float* yh = y + (size_t)head * L * DV;
    float* Sh = S + (size_t)head * kF * DV;
    float* zh = z + (size_t)head * kF;

    if (!use_init) {
        for (int e = tid; e < kF * DV; e += 256) Sh[e] = 0.f;
        for (int f = tid; f < kF; f += 256) zh[f] = 0.f;
    }

    const int ti = tid / kTPT;           // token within the chunk
    const int cb = (tid % kTPT) * kCPT;  // first column of this thread

    for (int t0 = 0; t0 < L; t0 += C) {
        const int n = min(C, L - t0);
        __syncthreads();  // state writes of the previous chunk are visible
        for (int e = tid; e < C * D; e += 256) {
            const int t = e / D, a = e % D;
            const bool ok = t < n;
            s_q[t][a] = ok ? load_elem(qh, (size_t)(t0 + t) * D + a) * Feat<D>::kPre : 0.f;
            s_k[t][a] = ok ? load_elem(kh, (size_t)(t0 + t) * D + a) * Feat<D>::kPre : 0.f;
        }
        for (int e = tid; e < C * DV; e += 256) {
            const int t = e / DV, c = e % DV;
            s_v[t][c] = t < n ? load_elem(vh, (size_t)(t0 + t) * DV + c) : 0.f;
        }
        __syncthreads();

        // Output of token ti: on-diagonal (masked closed-form weights) plus
        // off-diagonal (phi(q) against the state of the earlier chunks).
        float num[kCPT];
#pragma unroll
        for (int c = 0; c < kCPT; ++c) num[c] = 0.f;
        float den = 0.f;
        for (int j = 0; j <= ti; ++j) {
            float s = 0.f;
#pragma unroll
            for (int a = 0; a < D; ++a) s = fmaf(s_q[ti][a], s_k[j][a], s);
            const float w = 1.0f + s + 0.5f * s * s;
            den += w;
#pragma unroll
            for (int c = 0; c < kCPT; ++c) num[c] = fmaf(w, s_v[j][cb + c], num[c]);
        }
        for (int f = 0; f < kF; ++f) {
            const float pf = taylor_feature<D>(s_q[ti], f);
            den = fmaf(pf, zh[f], den);
#pragma unroll
            for (int c = 0; c < kCPT; ++c) num[c] = fmaf(pf, Sh[(size_t)f * DV + cb + c], num[c]);
        }
        if (ti < n) {
#pragma unroll
            for (int c = 0; c < kCPT; ++c) yh[(size_t)(t0 + ti) * DV + cb + c] = num[c] / (den + eps);
        }
        __syncthreads();  // every readout used the state before this chunk

        // State update with this chunk: S += phi(K)^T V, z += sum phi(K).
        for (int e = tid; e < kF * DV; e += 256) {
            const int f = e / DV, c = e % DV;
            float acc = 0.f;
            for (int t = 0; t < n; ++t) acc = fmaf(taylor_feature<D>(s_k[t], f), s_v[t][c], acc);
            Sh[e] += acc;
        }
        for (int f = tid; f < kF; f += 256) {
            float acc = 0.f;
            for (int t = 0; t < n; ++t) acc += taylor_feature<D>(s_k[t], f);
            zh[f] += acc;
        }
    }
}

template <typename T, int DV, int D>
static void launch_valu_dv(const T* q, const T* k, const T* v, int BH, int L, int chunk, float eps,
                           float* y, float* S, float* z, int use_init, hipStream_t st) {
    switch (chunk) {
        case 16:
            hipLaunchKernelGGL((prefill_valu_kernel<T, 16, DV, D>), dim3(BH), dim3(256), 0, st, q, k, v, L,
                               eps, y, S, z, use_init);
            break;
        case 32:
            hipLaunchKernelGGL((prefill_valu_kernel<T, 32, DV, D>), dim3(BH), dim3(256), 0, st, q, k, v, L,
                               eps, y, S, z, use_init);
            break;
        default:
            hipLaunchKernelGGL((prefill_valu_kernel<T, 64, DV, D>), dim3(BH), dim3(256), 0, st, q, k, v, L,
                               eps, y, S, z, use_init);
            break;
    }
}

template <typename T, int D>
static void launch_valu_d(const T* q, const T* k, const T* v, int BH, int L, int dv, int chunk, float eps,
                          float* y, float* S, float* z, int use_init, hipStream_t st) {
    if (dv == 64)
        launch_valu_dv<T, 64, D>(q, k, v, BH, L, chunk, eps, y, S, z, use_init, st);
    else
        launch_valu_dv<T, 128, D>(q, k, v, BH, L, chunk, eps, y, S, z, use_init, st);
}

template <typename T>
static hipError_t launch_valu_t(const void* q, const void* k, const void* v, int BH, int L, int d, int dv,
                                int chunk, float eps, float* y, float* S, float* z, int use_init,
                                hipStream_t st) {
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    switch (d) {
        case 8: launch_valu_d<T, 8>(qq, kk, vv, BH, L, dv, chunk, eps, y, S, z, use_init, st); break;
        case 24: launch_valu_d<T, 24>(qq, kk, vv, BH, L, dv, chunk, eps, y, S, z, use_init, st); break;
        case 32: launch_valu_d<T, 32>(qq, kk, vv, BH, L, dv, chunk, eps, y, S, z, use_init, st); break;
        default: launch_valu_d<T, 16>(qq, kk, vv, BH, L, dv, chunk, eps, y, S, z, use_init, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_prefill_valu(const void* q, const void* k, const void* v, bool bf16, int BH, int L, int d,
                               int dv, int chunk, float eps, float* y, float* S, float* z,
                               int use_init, hipStream_t st) {
    return bf16 ? launch_valu_t<uint16_t>(q, k, v, BH, L, d, dv, chunk, eps, y, S, z, use_init, st)
                : launch_valu_t<float>(q, k, v, BH, L, d, dv, chunk, eps, y, S, z, use_init, st);
}

}  // namespace based

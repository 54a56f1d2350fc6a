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
// One workgroup per (batch, head, group of 16 value columns), 256 threads.
// The caller's S (those 16 columns) is the working state; z lives in LDS for
// the whole sequence (each column group keeps its own copy) and a second
// kernel writes the final z.  Per chunk, the state goes through LDS in blocks of 32 feature
// rows: each block is read once, the chunk's readout uses it first (the
// state before the chunk), then its update is written back.  The features
// of the block's rows are formed once per block for every token of the
// chunk (queries and keys) and shared through LDS.  Every feature dim of
// the pages (8, 16, 24, 32) and every chunk (16, 32, 64) runs here.
#include "common.hpp"
#include "kernels.hpp"

namespace based {

constexpr int kCW = 16;  // value columns per workgroup
constexpr int kFB = 32;  // feature rows per state block

template <typename T, int C, int D>
__global__ __launch_bounds__(256) void prefill_valu_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, int L, int DV, float eps,
                                                           float* __restrict__ y, float* __restrict__ S,
                                                           float* __restrict__ z, int use_init) {
    constexpr int kF = Feat<D>::kF;
    constexpr int kTPT = 256 / C;     // threads per token
    constexpr int kCPT = kCW / kTPT;  // value columns per thread
    __shared__ float s_q[C][D];
    __shared__ float s_k[C][D];
    __shared__ float s_v[C][kCW];
    __shared__ float s_z[kF];
    __shared__ float s_phq[C][kFB + 1];  // features of the block's rows, per query
    __shared__ float s_phk[kFB][C + 1];  // and per key
    __shared__ float s_S[kFB][kCW];

    const int ncg = DV / kCW;
    const int cg = blockIdx.x % ncg, head = blockIdx.x / ncg;
    const int tid = threadIdx.x;
    const int c0 = cg * kCW;
    const T* qh = q + (size_t)head * L * D;
    const T* kh = k + (size_t)head * L * D;
    const T* vh = v + (size_t)head * L * DV + c0;
    float* yh = y + (size_t)head * L * DV + c0;
    float* Sh = S + (size_t)head * kF * DV + c0;
    float* zh = z + (size_t)head * kF;

    for (int f = tid; f < kF; f += 256) s_z[f] = use_init ? zh[f] : 0.f;
    if (!use_init)
        for (int e = tid; e < kF * kCW; e += 256) Sh[(size_t)(e / kCW) * DV + e % kCW] = 0.f;

    const int ti = tid / kTPT;                 // token of this thread in readouts
    const int cb = (tid % kTPT) * kCPT;        // its first column (of the 16)
    for (int t0 = 0; t0 < L; t0 += C) {
        const int n = min(C, L - t0);
        __syncthreads();  // previous chunk (and the state zeroing) done
        for (int e = tid; e < C * D; e += 256) {
            const int t = e / D, a = e % D;
            const bool ok = t < n;
            s_q[t][a] = ok ? load_elem(qh, (size_t)(t0 + t) * D + a) * Feat<D>::kPre : 0.f;
            s_k[t][a] = ok ? load_elem(kh, (size_t)(t0 + t) * D + a) * Feat<D>::kPre : 0.f;
        }
        for (int e = tid; e < C * kCW; e += 256) {
            const int t = e / kCW, c = e % kCW;
            s_v[t][c] = t < n ? load_elem(vh, (size_t)(t0 + t) * DV + c) : 0.f;
        }
        __syncthreads();

        // On-diagonal term: masked closed-form weights.
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

        // Off-diagonal term and state update, one block of feature rows at a
        // time; the next block's state is loaded into registers while this
        // one is processed (element e = tid + 256 i of a block: row e / 16,
        // column e % 16).
        constexpr int kSPer = kFB * kCW / 256;
        float nxt[kSPer];
#pragma unroll
        for (int i = 0; i < kSPer; ++i) {
            const int e = tid + 256 * i, f = e / kCW, c = e % kCW;
            nxt[i] = f < kF ? Sh[(size_t)f * DV + c] : 0.f;
        }
        for (int f0 = 0; f0 < kF; f0 += kFB) {
            for (int e = tid; e < C * kFB; e += 256) {
                const int t = e / kFB, f = e % kFB;
                const bool ok = f0 + f < kF;
                s_phq[t][f] = ok ? taylor_feature<D>(s_q[t], f0 + f) : 0.f;
                s_phk[f][t] = ok && t < n ? taylor_feature<D>(s_k[t], f0 + f) : 0.f;
            }
#pragma unroll
            for (int i = 0; i < kSPer; ++i) {
                const int e = tid + 256 * i;
                s_S[e / kCW][e % kCW] = nxt[i];
                const int fn = f0 + kFB + e / kCW;  // the same element of the next block
                nxt[i] = fn < kF ? Sh[(size_t)fn * DV + e % kCW] : 0.f;
            }
            __syncthreads();
            // readout with the state before this chunk
#pragma unroll 4
            for (int f = 0; f < kFB; ++f) {
                const float pf = s_phq[ti][f];
                den = fmaf(pf, f0 + f < kF ? s_z[f0 + f] : 0.f, den);
#pragma unroll
                for (int c = 0; c < kCPT; ++c) num[c] = fmaf(pf, s_S[f][cb + c], num[c]);
            }
            __syncthreads();
            // update with this chunk's keys (t < n)
            for (int e = tid; e < kFB * kCW; e += 256) {
                const int f = e / kCW, c = e % kCW;
                if (f0 + f < kF) {
                    float acc = 0.f;
                    for (int t = 0; t < n; ++t) acc = fmaf(s_phk[f][t], s_v[t][c], acc);
                    Sh[(size_t)(f0 + f) * DV + c] = s_S[f][c] + acc;
                }
            }
            if (tid < kFB && f0 + tid < kF) {
                float acc = 0.f;
                for (int t = 0; t < n; ++t) acc += s_phk[tid][t];
                s_z[f0 + tid] += acc;
            }
            __syncthreads();
        }
        if (ti < n) {
#pragma unroll
            for (int c = 0; c < kCPT; ++c) yh[(size_t)(t0 + ti) * DV + cb + c] = num[c] / (den + eps);
        }
    }
}

// Final normaliser state z = z_init + sum_t phi(k_t), one workgroup per
// head, launched after the main kernel: the column groups there only read
// the caller's z (a group that starts late must still see the initial one).
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_valu_z_kernel(const T* __restrict__ k, int L, float* __restrict__ z,
                                                             int use_init) {
    constexpr int kF = Feat<D>::kF;
    constexpr int kPer = (kF + 255) / 256;
    __shared__ float s_k[64][D];
    const int head = blockIdx.x, tid = threadIdx.x;
    const T* kh = k + (size_t)head * L * D;
    float* zh = z + (size_t)head * kF;
    float acc[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
    for (int t0 = 0; t0 < L; t0 += 64) {
        const int n = min(64, L - t0);
        __syncthreads();
        for (int e = tid; e < 64 * D; e += 256) {
            const int t = e / D, a = e % D;
            s_k[t][a] = t < n ? load_elem(kh, (size_t)(t0 + t) * D + a) * Feat<D>::kPre : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int f = tid + 256 * i;
            if (f < kF)
                for (int t = 0; t < n; ++t) acc[i] += taylor_feature<D>(s_k[t], f);
        }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int f = tid + 256 * i;
        if (f < kF) zh[f] = (use_init ? zh[f] : 0.f) + acc[i];
    }
}

template <typename T>
static void launch_z_t(const void* k, int BH, int L, int d, float* z, int use_init, hipStream_t st) {
    const T* kk = static_cast<const T*>(k);
    switch (d) {
        case 8: hipLaunchKernelGGL((prefill_valu_z_kernel<T, 8>), dim3(BH), dim3(256), 0, st, kk, L, z, use_init); break;
        case 24: hipLaunchKernelGGL((prefill_valu_z_kernel<T, 24>), dim3(BH), dim3(256), 0, st, kk, L, z, use_init); break;
        case 32: hipLaunchKernelGGL((prefill_valu_z_kernel<T, 32>), dim3(BH), dim3(256), 0, st, kk, L, z, use_init); break;
        default: hipLaunchKernelGGL((prefill_valu_z_kernel<T, 16>), dim3(BH), dim3(256), 0, st, kk, L, z, use_init); break;
    }
}

template <typename T, int D>
static void launch_valu_d(const T* q, const T* k, const T* v, int BH, int L, int dv, int chunk, float eps,
                          float* y, float* S, float* z, int use_init, hipStream_t st) {
    const dim3 grid((unsigned)(dv / kCW * BH));
    switch (chunk) {
        case 16:
            hipLaunchKernelGGL((prefill_valu_kernel<T, 16, D>), grid, dim3(256), 0, st, q, k, v, L, dv, eps, y, S, z,
                               use_init);
            break;
        case 32:
            hipLaunchKernelGGL((prefill_valu_kernel<T, 32, D>), grid, dim3(256), 0, st, q, k, v, L, dv, eps, y, S, z,
                               use_init);
            break;
        default:
            hipLaunchKernelGGL((prefill_valu_kernel<T, 64, D>), grid, dim3(256), 0, st, q, k, v, L, dv, eps, y, S, z,
                               use_init);
            break;
    }
    hipLaunchKernelGGL((prefill_valu_z_kernel<T, D>), dim3(BH), dim3(256), 0, st, k, L, z, use_init);
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

hipError_t launch_prefill_z(const void* k, bool bf16, int BH, int L, int d, float* z, int use_init,
                            hipStream_t st) {
    if (bf16) launch_z_t<uint16_t>(k, BH, L, d, z, use_init, st);
    else launch_z_t<float>(k, BH, L, d, z, use_init, st);
    return hipGetLastError();
}

}  // namespace based

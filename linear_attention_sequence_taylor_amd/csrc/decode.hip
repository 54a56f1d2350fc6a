// decode.hip -- fused next-token step of Taylor linear attention (gfx950).
//
// "Simple linear attention language models balance the recall-throughput
// tradeoff", App. B "Next Token Prediction" (KV-state update kernels) and
// s2 (constant-memory, O(1)-per-token generation):
//   S' = S + phi(k) v^T,  z' = z + phi(k),  y = phi(q)^T S' / (phi(q).z' + eps)
//
// The step is bound by HBM: the fp32 state (273 x d_v per head) is read once
// and written once, 0.5 flop per byte.  One workgroup per (batch, head),
// 256 threads; each thread owns one float4 column slice of the state and a
// strided set of rows, so every wave touches whole 512/256-byte rows with
// 16-byte accesses.  All loads of a batch of rows are issued before any
// arithmetic so that many 16-byte requests per thread are in flight.  The
// readout phi(q).S' is accumulated from the freshly updated registers and
// reduced through LDS; no state element is read twice.
#include "common.hpp"
#include "kernels.hpp"

namespace based {

template <int DV, int D>
struct DecodeShape {
    static constexpr int kF = Feat<D>::kF;             // state rows
    static constexpr int kC4 = DV / 4;                 // float4 slots per state row
    static constexpr int kRowStep = 256 / kC4;         // rows covered per sweep
    static constexpr int kIters = (kF + kRowStep - 1) / kRowStep;
    static constexpr int kBatch = 6;                   // rows in flight per thread
};

template <typename T>
__device__ __forceinline__ f32x4 load_v4(const T* v, size_t off);
template <>
__device__ __forceinline__ f32x4 load_v4<float>(const float* v, size_t off) {
    return *reinterpret_cast<const f32x4*>(v + off);
}
template <>
__device__ __forceinline__ f32x4 load_v4<uint16_t>(const uint16_t* v, size_t off) {
    const uint2 p = *reinterpret_cast<const uint2*>(v + off);
    f32x4 r = {bf16lo_f32(p.x), bf16hi_f32(p.x), bf16lo_f32(p.y), bf16hi_f32(p.y)};
    return r;
}

template <typename T, int DV, int D>
__global__ __launch_bounds__(256) void decode_step_kernel(const T* __restrict__ q,
                                                          const T* __restrict__ k,
                                                          const T* __restrict__ v, float eps,
                                                          float* __restrict__ S,
                                                          float* __restrict__ z,
                                                          float* __restrict__ y) {
    using Sh = DecodeShape<DV, D>;
    constexpr int kF = Sh::kF;
    __shared__ float s_q[D];
    __shared__ float s_k[D];
    __shared__ float s_part[Sh::kRowStep][DV];
    __shared__ float s_den[4];

    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid < D) {
        s_q[tid] = load_elem(q, (size_t)h * D + tid) * Feat<D>::kPre;
    } else if (tid < 2 * D) {
        s_k[tid - D] = load_elem(k, (size_t)h * D + tid - D) * Feat<D>::kPre;
    }
    __syncthreads();

    const int c4 = tid % Sh::kC4;
    const int r0 = tid / Sh::kC4;
    const f32x4 vv = load_v4<T>(v, (size_t)h * DV + c4 * 4);
    f32x4* Sh4 = reinterpret_cast<f32x4*>(S + (size_t)h * kF * DV) + c4;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // Fully unrolled for d' = 16 (at most 6 batches); capped for the larger
    // feature maps so the batches in flight fit the register file.
#pragma unroll 8
    for (int it0 = 0; it0 < Sh::kIters; it0 += Sh::kBatch) {
        f32x4 st[Sh::kBatch];
#pragma unroll
        for (int b = 0; b < Sh::kBatch; ++b) {
            const int r = r0 + (it0 + b) * Sh::kRowStep;
            if (it0 + b < Sh::kIters && r < kF)
                st[b] = __builtin_nontemporal_load(Sh4 + (size_t)r * Sh::kC4);
        }
#pragma unroll
        for (int b = 0; b < Sh::kBatch; ++b) {
            const int r = r0 + (it0 + b) * Sh::kRowStep;
            if (it0 + b < Sh::kIters && r < kF) {
                const float fk = taylor_feature<D>(s_k, r);
                const float fq = taylor_feature<D>(s_q, r);
                f32x4 s = st[b];
                s.x = fmaf(fk, vv.x, s.x);
                s.y = fmaf(fk, vv.y, s.y);
                s.z = fmaf(fk, vv.z, s.z);
                s.w = fmaf(fk, vv.w, s.w);
                __builtin_nontemporal_store(s, Sh4 + (size_t)r * Sh::kC4);
                acc.x = fmaf(fq, s.x, acc.x);
                acc.y = fmaf(fq, s.y, acc.y);
                acc.z = fmaf(fq, s.z, acc.z);
                acc.w = fmaf(fq, s.w, acc.w);
            }
        }
    }

    // Normaliser: z rows tid and tid + 256.
    float den = 0.f;
    float* zh = z + (size_t)h * kF;
    for (int r = tid; r < kF; r += 256) {
        const float zn = zh[r] + taylor_feature<D>(s_k, r);
        zh[r] = zn;
        den = fmaf(taylor_feature<D>(s_q, r), zn, den);
    }
    den = wave_sum(den);
    if ((tid & 63) == 0) s_den[tid >> 6] = den;
    s_part[r0][c4 * 4 + 0] = acc.x;
    s_part[r0][c4 * 4 + 1] = acc.y;
    s_part[r0][c4 * 4 + 2] = acc.z;
    s_part[r0][c4 * 4 + 3] = acc.w;
    __syncthreads();
    if (tid < DV) {
        float num = 0.f;
#pragma unroll
        for (int r = 0; r < Sh::kRowStep; ++r) num += s_part[r][tid];
        const float dsum = (s_den[0] + s_den[1]) + (s_den[2] + s_den[3]);
        y[(size_t)h * DV + tid] = num / (dsum + eps);
    }
}

template <typename T, int D>
static void launch_decode_d(const T* q, const T* k, const T* v, int BH, int dv, float eps, float* S, float* z,
                            float* y, hipStream_t st) {
    if (dv == 64)
        hipLaunchKernelGGL((decode_step_kernel<T, 64, D>), dim3(BH), dim3(256), 0, st, q, k, v, eps, S, z, y);
    else
        hipLaunchKernelGGL((decode_step_kernel<T, 128, D>), dim3(BH), dim3(256), 0, st, q, k, v, eps, S, z, y);
}

template <typename T>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, int BH, int d, int dv,
                                  float eps, float* S, float* z, float* y, hipStream_t st) {
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    switch (d) {
        case 8: launch_decode_d<T, 8>(qq, kk, vv, BH, dv, eps, S, z, y, st); break;
        case 24: launch_decode_d<T, 24>(qq, kk, vv, BH, dv, eps, S, z, y, st); break;
        case 32: launch_decode_d<T, 32>(qq, kk, vv, BH, dv, eps, S, z, y, st); break;
        default: launch_decode_d<T, 16>(qq, kk, vv, BH, dv, eps, S, z, y, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_decode_step(const void* q, const void* k, const void* v, bool bf16, int BH, int d,
                              int dv, float eps, float* S, float* z, float* y, hipStream_t st) {
    return bf16 ? launch_decode_t<uint16_t>(q, k, v, BH, d, dv, eps, S, z, y, st)
                : launch_decode_t<float>(q, k, v, BH, d, dv, eps, S, z, y, st);
}

}  // namespace based

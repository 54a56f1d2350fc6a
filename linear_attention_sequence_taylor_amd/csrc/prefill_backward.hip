// prefill_backward.hip -- gradients of causal Taylor linear attention for
// training-mode prefill (gfx950): fp32 inputs and every feature dim, in fp32
// on the fp32 matrix cores (v_mfma_f32_16x16x4_f32).  bf16 inputs with
// feature dim 16 take the bf16 matrix-core kernels of
// prefill_backward_mfma.hip (same workspace layout).
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
// This is the direct (quadratic) form: O(L^2) work per head.
//
// Two kernels, one workgroup of 4 waves per 64 rows, wave w owning rows
// 16w..16w+15; the other side goes through LDS in 64-row fp32 tiles (row
// stride width + 4: the row reads and the column reads below then hit 64
// distinct banks) while the wave's own rows sit in registers:
//   query side: pass 1 over the key tiles at or before the queries gives N
//     and D, then g and h (to the workspace); pass 2 gives dq;
//   key side: over the query tiles at or after the keys, dk and dv.
// A score tile computed as K Q^T (or Q K^T) leaves lane (g, r) = (lane/16,
// lane%16) with row r of its own side against rows 4g..4g+3 of the other;
// a product over those rows then takes its k-step m from lane group g's row
// 4g + m, so the weights enter the next product without moving between
// lanes.  Only the diagonal tile is masked; rows past L are staged as zeros
// (their weights meet zero g rows or are masked) and never stored.
#include "common.hpp"
#include "kernels.hpp"

namespace based {
namespace {

constexpr int kT = 64;  // rows per tile

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Feature width padded to whole 16-column output tiles.
template <int D>
constexpr int feat_pad() {
    return D <= 16 ? 16 : 32;
}

// Rows row0.. of a [L][W] matrix as fp32 into columns 0..W-1 of a
// [64][WP + 4] LDS tile, rows past L as zeros, in two phases: load issues
// every 16-byte load of the tile (rows past L read row L-1), store writes
// them to LDS.  Loading all tiles of an interval before storing any lets
// their loads overlap instead of each waiting for the one before.  Columns
// W..WP-1 are left alone: zero_pad zeroes them once.
template <typename T, int W>
struct TileStage {
    static constexpr int kVec = 16 / (int)sizeof(T);  // elements per 16-byte piece
    static constexpr int kPer = W / kVec;             // pieces per row
    static constexpr int kN = kT * kPer;
    static constexpr int kIt = (kN + 255) / 256;
    u32x4 raw[kIt];

    __device__ __forceinline__ void load(const T* mat, int L, int row0) {
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int e = threadIdx.x + 256 * i;
            if (kN % 256 == 0 || e < kN) {
                const int row = e / kPer, c = (e % kPer) * kVec;
                raw[i] = *reinterpret_cast<const u32x4*>(mat + (size_t)min(row0 + row, L - 1) * W + c);
            }
        }
    }
    template <int WP>
    __device__ __forceinline__ void store(int L, int row0, float* dst) const {
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int e = threadIdx.x + 256 * i;
            if (kN % 256 == 0 || e < kN) {
                const int row = e / kPer, c = (e % kPer) * kVec;
                const bool live = row0 + row < L;
                f32x4* d = reinterpret_cast<f32x4*>(dst + row * (WP + 4) + c);
                if constexpr (sizeof(T) == 4) {
                    d[0] = live ? __builtin_bit_cast(f32x4, raw[i]) : f32x4{0.f, 0.f, 0.f, 0.f};
                } else {
                    const uint32_t a0 = raw[i][0], a1 = raw[i][1], a2 = raw[i][2], a3 = raw[i][3];
                    const f32x4 x0 = {bf16lo_f32(a0), bf16hi_f32(a0), bf16lo_f32(a1), bf16hi_f32(a1)};
                    const f32x4 x1 = {bf16lo_f32(a2), bf16hi_f32(a2), bf16lo_f32(a3), bf16hi_f32(a3)};
                    d[0] = live ? x0 : f32x4{0.f, 0.f, 0.f, 0.f};
                    d[1] = live ? x1 : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    }
};
// Zeroes columns W..WP-1 of a [64][WP + 4] LDS tile (the feature padding,
// which staging never writes).
template <int W, int WP>
__device__ __forceinline__ void zero_pad(float* dst) {
    if constexpr (WP > W) {
        constexpr int kP = WP - W;
        for (int e = threadIdx.x; e < kT * kP; e += 256) dst[(e / kP) * (WP + 4) + W + e % kP] = 0.f;
    }
}

template <int D, int DV>
struct BwdQSmemF {
    static constexpr int kLdK = feat_pad<D>() + 4, kLdV = DV + 4;
    float k[kT * kLdK];
    float v[kT * kLdV];
    float g[4][16 * kLdV];  // per wave: g of its 16 queries
    float h[4][16];
};

template <typename T, int D, int DV>
__global__ __launch_bounds__(256) void bwd_query_f32_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                            const T* __restrict__ v, const float* __restrict__ dy,
                                                            int L, int ntiles, float eps, float* __restrict__ dq,
                                                            float* __restrict__ g_ws, float* __restrict__ h_ws) {
    using SM = BwdQSmemF<D, DV>;
    constexpr int kKW = feat_pad<D>(), kLdK = SM::kLdK, kLdV = SM::kLdV;
    constexpr int kNV = DV / 16, kNK = kKW / 16;
    __shared__ SM sm;
    const float isd = 1.f / sqrtf((float)D);
    const int BH = gridDim.x / ntiles;
    const int head = blockIdx.x % BH;
    const int ti = ntiles - 1 - (int)(blockIdx.x / BH);  // the longest rows first, every head
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const T* kh = k + (size_t)head * L * D;
    const T* vh = v + (size_t)head * L * DV;
    const int qw0 = ti * kT + 16 * w;  // first query of this wave
    const int qr = qw0 + r;            // this lane's query in the score tiles

    // B operand of the scores: this lane's query, dims 4j + g, / sqrt(d')
    // (all loads first, from row L-1 past the end, then zeroed there)
    float qb[D / 4];
    const T* qrow = q + ((size_t)head * L + min(qr, L - 1)) * D + g;
    T qraw[D / 4];
#pragma unroll
    for (int j = 0; j < D / 4; ++j) qraw[j] = qrow[4 * j];
#pragma unroll
    for (int j = 0; j < D / 4; ++j) qb[j] = qr < L ? load_elem(qraw, j) * isd : 0.f;

    // scores of key tile kt: st[m] = s(key 16kt + 4g + m, query r)
    auto scores = [&](int kt) {
        f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < D / 4; ++j) st = mfma_f32(sm.k[(16 * kt + r) * kLdK + 4 * j + g], qb[j], st);
        return st;
    };

    // ---- pass 1: N (rows = queries 4g+m, columns 16ct + r), and D - eps of
    // query r over this lane's keys
    f32x4 yacc[kNV];
#pragma unroll
    for (int ct = 0; ct < kNV; ++ct) yacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    zero_pad<D, kKW>(sm.k);
    TileStage<T, D> kst;
    TileStage<T, DV> vst;
    for (int tj = 0; tj <= ti; ++tj) {
        __syncthreads();
        kst.load(kh, L, tj * kT);
        vst.load(vh, L, tj * kT);
        kst.template store<kKW>(L, tj * kT, sm.k);
        vst.template store<DV>(L, tj * kT, sm.v);
        __syncthreads();
        const bool diag = tj == ti;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const f32x4 st = scores(kt);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float s = st[m];
                float a = fmaf(s, fmaf(s, 0.5f, 1.f), 1.f);
                if (diag && 16 * kt + 4 * g + m > 16 * w + r) a = 0.f;
                lsum += a;
#pragma unroll
                for (int ct = 0; ct < kNV; ++ct)
                    yacc[ct] = mfma_f32(a, sm.v[(16 * kt + 4 * g + m) * kLdV + 16 * ct + r], yacc[ct]);
            }
        }
    }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);  // D - eps of query qr, on every lane group

    // ---- g = dy/D and h = -(dy.y)/D of queries qw0 + 4g + m (columns 16ct + r);
    // the dy loads all go out at once (rows past L read row L-1, zeroed)
    float dyv[4][kNV];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float* dyr = dy + ((size_t)head * L + min(qw0 + 4 * g + m, L - 1)) * DV + r;
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) dyv[m][ct] = dyr[16 * ct];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int qi = qw0 + 4 * g + m;
        const float inv = 1.f / (__shfl(lsum, 4 * g + m, 64) + eps);
        float dyy = 0.f;
#pragma unroll
        for (int ct = 0; ct < kNV; ++ct) {
            const float dyc = qi < L ? dyv[m][ct] : 0.f;
            dyy = fmaf(dyc, yacc[ct][m], dyy);
            const float gv = dyc * inv;
            sm.g[w][(4 * g + m) * kLdV + 16 * ct + r] = gv;
            if (qi < L) g_ws[((size_t)head * L + qi) * DV + 16 * ct + r] = gv;
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) dyy += __shfl_xor(dyy, off, 64);
        const float hq = -dyy * inv * inv;
        if (r == 0) {
            sm.h[w][4 * g + m] = hq;
            if (qi < L) h_ws[(size_t)head * L + qi] = hq;
        }
    }

    // ---- pass 2: dq (rows = queries 4g+m, columns = features 16ct + r),
    // from the diagonal tile (still staged) back to the first
    f32x4 dqacc[kNK];
#pragma unroll
    for (int ct = 0; ct < kNK; ++ct) dqacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int tj = ti; tj >= 0; --tj) {
        __syncthreads();  // also orders the g/h writes above before their reads
        if (tj != ti) {
            kst.load(kh, L, tj * kT);
            vst.load(vh, L, tj * kT);
            kst.template store<kKW>(L, tj * kT, sm.k);
            vst.template store<DV>(L, tj * kT, sm.v);
            __syncthreads();
        }
        const bool diag = tj == ti;
        const float hr = sm.h[w][r];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const f32x4 st = scores(kt);
            // (g . v): rows = keys 16kt + 4g + m, columns = queries r
            f32x4 ga = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < DV / 4; ++j)
                ga = mfma_f32(sm.v[(16 * kt + r) * kLdV + 4 * j + g], sm.g[w][r * kLdV + 4 * j + g], ga);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                float e = (ga[m] + hr) * (1.f + st[m]) * isd;
                if (diag && 16 * kt + 4 * g + m > 16 * w + r) e = 0.f;
#pragma unroll
                for (int ct = 0; ct < kNK; ++ct)
                    dqacc[ct] = mfma_f32(e, sm.k[(16 * kt + 4 * g + m) * kLdK + 16 * ct + r], dqacc[ct]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int qi = qw0 + 4 * g + m;
#pragma unroll
        for (int ct = 0; ct < kNK; ++ct)
            if (qi < L && 16 * ct + r < D) dq[((size_t)head * L + qi) * D + 16 * ct + r] = dqacc[ct][m];
    }
}

template <int D, int DV>
struct BwdKSmemF {
    static constexpr int kLdQ = feat_pad<D>() + 4, kLdG = DV + 4;
    float q[kT * kLdQ];
    float g[kT * kLdG];
    float h[kT];
};

template <typename T, int D, int DV>
__global__ __launch_bounds__(256) void bwd_key_f32_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ v, int L, int ntiles,
                                                          const float* __restrict__ g_ws,
                                                          const float* __restrict__ h_ws, float* __restrict__ dk,
                                                          float* __restrict__ dvo) {
    using SM = BwdKSmemF<D, DV>;
    constexpr int kKW = feat_pad<D>(), kLdQ = SM::kLdQ, kLdG = SM::kLdG;
    constexpr int kNV = DV / 16, kNK = kKW / 16;
    __shared__ SM sm;
    const float isd = 1.f / sqrtf((float)D);
    const int BH = gridDim.x / ntiles;
    const int head = blockIdx.x % BH;
    const int tj = blockIdx.x / BH;  // the first keys (the longest loops) first, every head
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const T* qh = q + (size_t)head * L * D;
    const float* gh = g_ws + (size_t)head * L * DV;
    const float* hh = h_ws + (size_t)head * L;
    const int kw0 = tj * kT + 16 * w;  // first key of this wave
    const int kr = kw0 + r;            // this lane's key in the score tiles

    // this lane's key (/ sqrt(d')) and value: the B operands of Q K^T and
    // g V^T (dims / columns 4j + g)
    // (all loads first, from row L-1 past the end, then zeroed there)
    float kb[D / 4], vb[DV / 4];
    const T* krow = k + ((size_t)head * L + min(kr, L - 1)) * D + g;
    const T* vrow = v + ((size_t)head * L + min(kr, L - 1)) * DV + g;
    T kraw[D / 4], vraw[DV / 4];
#pragma unroll
    for (int j = 0; j < D / 4; ++j) kraw[j] = krow[4 * j];
#pragma unroll
    for (int j = 0; j < DV / 4; ++j) vraw[j] = vrow[4 * j];
#pragma unroll
    for (int j = 0; j < D / 4; ++j) kb[j] = kr < L ? load_elem(kraw, j) * isd : 0.f;
#pragma unroll
    for (int j = 0; j < DV / 4; ++j) vb[j] = kr < L ? load_elem(vraw, j) : 0.f;
    f32x4 dvacc[kNV], dkacc[kNK];
#pragma unroll
    for (int ct = 0; ct < kNV; ++ct) dvacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < kNK; ++ct) dkacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    zero_pad<D, kKW>(sm.q);
    TileStage<T, D> qst;
    TileStage<float, DV> gst;
    for (int ti = tj; ti < ntiles; ++ti) {
        __syncthreads();
        float hq = 0.f;
        if (threadIdx.x < kT) hq = hh[min(ti * kT + (int)threadIdx.x, L - 1)];
        qst.load(qh, L, ti * kT);
        gst.load(gh, L, ti * kT);
        qst.template store<kKW>(L, ti * kT, sm.q);
        gst.template store<DV>(L, ti * kT, sm.g);
        if (threadIdx.x < kT) sm.h[threadIdx.x] = ti * kT + (int)threadIdx.x < L ? hq : 0.f;
        __syncthreads();
        const bool diag = ti == tj;
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
            // scores and (g . v): rows = queries 16qt + 4g + m, columns = keys r
            f32x4 st = {0.f, 0.f, 0.f, 0.f}, ga = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < D / 4; ++j) st = mfma_f32(sm.q[(16 * qt + r) * kLdQ + 4 * j + g], kb[j], st);
#pragma unroll
            for (int j = 0; j < DV / 4; ++j) ga = mfma_f32(sm.g[(16 * qt + r) * kLdG + 4 * j + g], vb[j], ga);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int qrow = 16 * qt + 4 * g + m;
                const float s = st[m];
                float a = fmaf(s, fmaf(s, 0.5f, 1.f), 1.f);
                float e = (ga[m] + sm.h[qrow]) * (1.f + s) * isd;
                if (diag && qrow < 16 * w + r) a = e = 0.f;
                // dv += a^T g and dk += e^T q (rows = keys 4g+m', columns
                // 16ct + r): k-step m, lane group g brings query qrow
#pragma unroll
                for (int ct = 0; ct < kNV; ++ct) dvacc[ct] = mfma_f32(a, sm.g[qrow * kLdG + 16 * ct + r], dvacc[ct]);
#pragma unroll
                for (int ct = 0; ct < kNK; ++ct) dkacc[ct] = mfma_f32(e, sm.q[qrow * kLdQ + 16 * ct + r], dkacc[ct]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int kj = kw0 + 4 * g + m;
        if (kj < L) {
#pragma unroll
            for (int ct = 0; ct < kNV; ++ct) dvo[((size_t)head * L + kj) * DV + 16 * ct + r] = dvacc[ct][m];
#pragma unroll
            for (int ct = 0; ct < kNK; ++ct)
                if (16 * ct + r < D) dk[((size_t)head * L + kj) * D + 16 * ct + r] = dkacc[ct][m];
        }
    }
}

template <typename T, int D, int DV>
hipError_t launch_bwd(const void* q, const void* k, const void* v, const float* dy, int BH, int L, float eps,
                      float* dq, float* dk, float* dv, float* g_ws, float* h_ws, hipStream_t st) {
    // bf16 with feature dim 16 runs on the bf16 matrix cores
    if constexpr (sizeof(T) == 2 && D == kDFeat) {
        return launch_prefill_backward_mfma(q, k, v, dy, BH, L, DV, eps, dq, dk, dv, g_ws, h_ws, st);
    } else {
    const int ntiles = (L + kT - 1) / kT;
    const dim3 grid((unsigned)(ntiles * BH));
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    hipLaunchKernelGGL((bwd_query_f32_kernel<T, D, DV>), grid, dim3(256), 0, st, qq, kk, vv, dy, L, ntiles, eps, dq,
                       g_ws, h_ws);
    hipLaunchKernelGGL((bwd_key_f32_kernel<T, D, DV>), grid, dim3(256), 0, st, qq, kk, vv, L, ntiles, g_ws, h_ws, dk,
                       dv);
    return hipGetLastError();
    }
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

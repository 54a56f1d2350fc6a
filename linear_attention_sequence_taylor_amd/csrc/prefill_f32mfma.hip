// prefill_f32mfma.hip -- chunked causal Taylor linear attention for every
// feature dim (8, 16, 24, 32) in fp32 on the gfx950 fp32 matrix cores
// (v_mfma_f32_16x16x4_f32), chunk 64, bf16 or fp32 inputs (bf16 widened
// exactly).
//
// "Simple linear attention language models balance the recall-throughput
// tradeoff", App. B "Forward / Generation Prefill": per chunk, the causally
// masked pairwise weights give the on-diagonal term, earlier chunks enter
// through the cumulative Taylor-order state (off-diagonal term) and the
// state is carried to the next chunk; s4 "Taylor Linear Attention": the
// pairwise weight is 1 + s + s^2/2 with s = q.k/sqrt(d'), and the state
// rows are the features phi(x~) = [1, x~, vec(x~ (x) x~)/sqrt2] of
// x~ = x d'^(-1/4) (App. D.4: F = 1 + d' + d'^2 rows).
//
// One workgroup of 8 waves per (batch, head, 16 value columns) walks the
// chunks in order.  Internally the feature rows are ordered [1, x~_0 ..
// x~_(d'-1), 0, 0, 0, x~_a x~_b / sqrt2 (a-major)]: with d' a multiple of 4
// every 4-row k-step of the quadratic block stays inside one row a.  The
// rows come in 16-row tiles; per chunk:
//   * scores s = Q~ K~^T for the 10 lower-triangle 16x16 tiles (fp32 MFMA
//     over d'), masked weights into LDS;
//   * readout: wave w takes query tile w % 4 and every other feature tile
//     (w / 4 picks which): phi(Q~) S and phi(Q~).z with the state before
//     the chunk, read from LDS; the feature values are formed per lane;
//   * update: wave w owns feature tiles w, w + 8, ...: S += phi(K~)^T V in
//     MFMA accumulators, z in per-lane partial sums;
//   * after a barrier: waves 0..3 add A V (and the row sums of A) for their
//     query tile to the two readout halves, normalise and store y; every
//     wave publishes its state tiles to LDS for the next chunk.
// Q~, K~ and V of the next chunk are loaded into registers at the start of
// a chunk and stored to the other LDS buffer before its end.
#include "common.hpp"
#include "kernels.hpp"

namespace based {
namespace {

constexpr int kC = 64;      // chunk
constexpr int kCW = 16;     // value columns per workgroup
constexpr int kWaves = 8;   // waves per workgroup
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Internal feature order (see above) for feature dim D.
template <int D>
struct FMap {
    static_assert(D % 4 == 0, "feature dim a multiple of 4");
    static constexpr int kLin = D + 4;  // rows before the quadratic block
    static constexpr int kRows = kLin + D * D;
    static constexpr int kTiles = (kRows + 15) / 16;
    static constexpr int kRowsPad = 16 * kTiles;
    static constexpr int kOwn = (kTiles + kWaves - 1) / kWaves;  // update tiles per wave
    static constexpr int kF = 1 + D + D * D;                     // the caller's rows
    // The caller's row of internal row f, or -1 (padding).
    __device__ static int caller_row(int f) {
        if (f <= D) return f;
        if (f < kLin || f >= kRows) return -1;
        return 1 + D + (f - kLin);
    }
};

// phi_f(x) = x[a] x[b] mul for internal row f, where column D of every
// staged row holds 1: the constant row is x[D] x[D], a linear row
// x[f-1] x[D], a quadratic row x[a] x[b] / sqrt2, padding rows have mul 0.
struct FeatIdx {
    int a, b;
    float mul;
};
template <int D>
__device__ __forceinline__ FeatIdx feat_idx(int f) {
    constexpr int kLin = FMap<D>::kLin, kRows = FMap<D>::kRows;
    FeatIdx r;
    if (f >= kLin && f < kRows) {
        const int e = f - kLin;
        r.a = e / D;
        r.b = e - r.a * D;
        r.mul = kInvSqrt2;
    } else {
        r.a = (f >= 1 && f <= D) ? f - 1 : D;
        r.b = D;
        r.mul = f <= D ? 1.f : 0.f;
    }
    return r;
}

template <int D>
struct F32Smem {
    static constexpr int kLd = D + 1;  // odd row stride: conflict-free column reads
    float q[2][kC * kLd];              // Q~ (pre-scaled), double-buffered
    float k[2][kC * kLd];
    float v[2][kC * kCW];
    float s[FMap<D>::kRowsPad * kCW];  // state before the current chunk (internal rows)
    float z[FMap<D>::kRowsPad];
    float a[kC * (kC + 1)];            // masked intra-chunk weights
    float rnum[2][kC * kCW];           // readout halves
    float rden[2][kC];
};

// Staging of one chunk: q~, k~ (pre-scaled) and the workgroup's v columns.
template <typename T, int D>
struct Stage {
    static constexpr int kQK = kC * D;  // elements of q (and of k)
    static constexpr int kV = kC * kCW;
    static constexpr int kPer = (2 * kQK + kV + kThreads - 1) / kThreads;
    float x[kPer];

    __device__ __forceinline__ void load(const T* qh, const T* kh, const T* vh, int ldv, int t0, int L) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = threadIdx.x + kThreads * i;
            float val = 0.f;
            if (e < 2 * kQK) {
                const int w = e % kQK, t = w / D, c = w % D;
                const T* src = e < kQK ? qh : kh;
                if (t0 + t < L) val = load_elem(src, (size_t)(t0 + t) * D + c) * Feat<D>::kPre;
            } else if (e < 2 * kQK + kV) {
                const int w = e - 2 * kQK, t = w / kCW, c = w % kCW;
                if (t0 + t < L) val = load_elem(vh, (size_t)(t0 + t) * ldv + c);
            }
            x[i] = val;
        }
    }
    __device__ __forceinline__ void store(F32Smem<D>& sm, int buf) const {
        constexpr int kLd = F32Smem<D>::kLd;
        if (threadIdx.x < 2 * kC) (threadIdx.x < kC ? sm.q[buf] : sm.k[buf])[(threadIdx.x % kC) * kLd + D] = 1.f;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = threadIdx.x + kThreads * i;
            if (e < 2 * kQK) {
                const int w = e % kQK, t = w / D, c = w % D;
                (e < kQK ? sm.q[buf] : sm.k[buf])[t * kLd + c] = x[i];
            } else if (e < 2 * kQK + kV) {
                sm.v[buf][e - 2 * kQK] = x[i];
            }
        }
    }
};

// Lower-triangle score tiles of the chunk: index -> (query tile, key tile).
__device__ __forceinline__ void tri_tile(int idx, int& ti, int& tj) {
    ti = idx >= 6 ? 3 : (idx >= 3 ? 2 : (idx >= 1 ? 1 : 0));
    tj = idx - ti * (ti + 1) / 2;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 1) void prefill_f32mfma_kernel(const T* __restrict__ q,
                                                                      const T* __restrict__ k,
                                                                      const T* __restrict__ v, int L, int dv,
                                                                      float eps, float* __restrict__ y,
                                                                      float* __restrict__ S, float* __restrict__ z,
                                                                      int use_init) {
    using M = FMap<D>;
    constexpr int kLd = F32Smem<D>::kLd;
    __shared__ F32Smem<D> sm;
    const int ncg = dv / kCW;
    const int cg = blockIdx.x % ncg, head = blockIdx.x / ncg;
    const int col0 = cg * kCW;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const T* qh = q + (size_t)head * L * D;
    const T* kh = k + (size_t)head * L * D;
    const T* vh = v + (size_t)head * L * dv + col0;
    float* yh = y + (size_t)head * L * dv + col0;
    float* Sh = S + (size_t)head * M::kF * dv + col0;
    float* zh = z + (size_t)head * M::kF;
    const int nchunks = (L + kC - 1) / kC;

    // ---- state: this wave's tiles w + 8u in accumulators (rows 16rt + 4g + m,
    // column r), z as per-lane partial sums (row 16rt + r, this lane group's
    // tokens; the caller's initial z sits in lane group 0)
    f32x4 sacc[M::kOwn];
    float zp[M::kOwn];
#pragma unroll
    for (int u = 0; u < M::kOwn; ++u) {
        const int rt = w + kWaves * u;
        sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        zp[u] = 0.f;
        if (use_init && rt < M::kTiles) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int cr = M::caller_row(16 * rt + 4 * g + m);
                if (cr >= 0) sacc[u][m] = Sh[(size_t)cr * dv + r];
            }
            const int cr = M::caller_row(16 * rt + r);
            if (g == 0 && cr >= 0) zp[u] = zh[cr];
        }
    }
    // feature indices of this lane's update row (16rt + r) of every own tile
    int ua[M::kOwn], ub[M::kOwn];
    float um[M::kOwn];
#pragma unroll
    for (int u = 0; u < M::kOwn; ++u) {
        const FeatIdx fi = feat_idx<D>(16 * (w + kWaves * u) + r);
        ua[u] = fi.a;
        ub[u] = fi.b;
        um[u] = (w + kWaves * u) < M::kTiles ? fi.mul : 0.f;
    }
    // publish the initial state (the state before chunk 0)
    auto publish = [&]() {
#pragma unroll
        for (int u = 0; u < M::kOwn; ++u) {
            const int rt = w + kWaves * u;
            if (rt < M::kTiles) {
#pragma unroll
                for (int m = 0; m < 4; ++m) sm.s[(16 * rt + 4 * g + m) * kCW + r] = sacc[u][m];
                float zs = zp[u];
                zs += __shfl_xor(zs, 16, 64);
                zs += __shfl_xor(zs, 32, 64);
                if (g == 0) sm.z[16 * rt + r] = zs;
            }
        }
    };
    publish();
    Stage<T, D> st;
    st.load(qh, kh, vh, dv, 0, L);
    st.store(sm, 0);
    __syncthreads();

    const int tt = w & 3, half = w >> 2;  // readout: query tile, feature half
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1, t0 = c * kC;
        const float* qs = sm.q[buf];
        const float* ks = sm.k[buf];
        const float* vs = sm.v[buf];
        const bool more = c + 1 < nchunks;
        if (more) st.load(qh, kh, vh, dv, t0 + kC, L);

        // ---- intra-chunk scores: tiles w and w + 8 of the lower triangle
#pragma unroll
        for (int rep = 0; rep < 2; ++rep) {
            const int idx = w + kWaves * rep;
            if (idx < 10) {
                int ti, tj;
                tri_tile(idx, ti, tj);
                f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < D / 4; ++j)
                    sc = mfma_f32(qs[(16 * ti + r) * kLd + 4 * j + g], ks[(16 * tj + r) * kLd + 4 * j + g], sc);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int qi = 16 * ti + 4 * g + m, kj = 16 * tj + r;
                    const float s = sc[m];
                    sm.a[qi * (kC + 1) + kj] = kj <= qi ? fmaf(s, fmaf(s, 0.5f, 1.f), 1.f) : 0.f;
                }
            }
        }

        // ---- readout with the state before this chunk: query tile tt,
        // feature tiles half, half + 2, ...
        {
            f32x4 num = {0.f, 0.f, 0.f, 0.f};
            float den = 0.f;
            const float* qrow = qs + (16 * tt + r) * kLd;
            for (int rt = half; rt < M::kTiles; rt += 2) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // rows f0 .. f0+3 (this lane: f0 + g); inside the quadratic
                    // block they share row a of the outer product
                    const int f0 = 16 * rt + 4 * j, f = f0 + g;
                    float phi;
                    if (f0 >= M::kLin && f0 + 4 <= M::kRows) {
                        const int e0 = f0 - M::kLin, a = e0 / D;
                        phi = qrow[a] * qrow[e0 - a * D + g] * kInvSqrt2;
                    } else {
                        const FeatIdx fi = feat_idx<D>(f);
                        phi = qrow[fi.a] * qrow[fi.b] * fi.mul;
                    }
                    num = mfma_f32(phi, sm.s[f * kCW + r], num);
                    den = fmaf(phi, sm.z[f], den);
                }
            }
            den += __shfl_xor(den, 16, 64);
            den += __shfl_xor(den, 32, 64);  // token 16tt + r, this half's features
#pragma unroll
            for (int m = 0; m < 4; ++m) sm.rnum[half][(16 * tt + 4 * g + m) * kCW + r] = num[m];
            if (g == 0) sm.rden[half][16 * tt + r] = den;
        }

        // ---- update with this chunk's keys: tiles w + 8u
        {
            const int nvalid = min(kC, L - t0);
#pragma unroll 4
            for (int j = 0; j < kC / 4; ++j) {
                const int t = 4 * j + g;  // this lane group's token
                const float vb = vs[t * kCW + r];
                const float* krow = ks + t * kLd;
                const float tok_ok = t < nvalid ? 1.f : 0.f;
#pragma unroll
                for (int u = 0; u < M::kOwn; ++u) {
                    const int rt = w + kWaves * u;
                    if (rt < M::kTiles) {
                        const float phi = krow[ua[u]] * krow[ub[u]] * (um[u] * tok_ok);
                        sacc[u] = mfma_f32(phi, vb, sacc[u]);
                        zp[u] += phi;
                    }
                }
            }
        }
        __syncthreads();  // weights, readout halves done; no more reads of the state

        // ---- A V, normalisation and the stores (query tile w, waves 0..3)
        if (w < 4) {
            f32x4 nacc = {0.f, 0.f, 0.f, 0.f}, dacc = {0.f, 0.f, 0.f, 0.f};
            for (int j = 0; j < 4 * (w + 1); ++j) {
                const float av = sm.a[(16 * w + r) * (kC + 1) + 4 * j + g];
                nacc = mfma_f32(av, vs[(4 * j + g) * kCW + r], nacc);
                dacc = mfma_f32(av, 1.f, dacc);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int row = 16 * w + 4 * g + m;
                if (t0 + row < L) {
                    const float numv = nacc[m] + sm.rnum[0][row * kCW + r] + sm.rnum[1][row * kCW + r];
                    const float denv = dacc[m] + sm.rden[0][row] + sm.rden[1][row];
                    yh[(size_t)(t0 + row) * dv + r] = numv / (denv + eps);
                }
            }
        }
        publish();
        if (more) st.store(sm, buf ^ 1);
        __syncthreads();
    }

    // ---- final state in the caller's row order (z from column group 0)
#pragma unroll
    for (int u = 0; u < M::kOwn; ++u) {
        const int rt = w + kWaves * u;
        if (rt < M::kTiles) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int cr = M::caller_row(16 * rt + 4 * g + m);
                if (cr >= 0) Sh[(size_t)cr * dv + r] = sacc[u][m];
            }
            float zs = zp[u];
            zs += __shfl_xor(zs, 16, 64);
            zs += __shfl_xor(zs, 32, 64);
            const int cr = M::caller_row(16 * rt + r);
            if (cg == 0 && g == 0 && cr >= 0) zh[cr] = zs;
        }
    }
}

template <typename T, int D>
void launch_d(const void* q, const void* k, const void* v, int BH, int L, int dv, float eps, float* y, float* S,
              float* z, int use_init, hipStream_t st) {
    hipLaunchKernelGGL((prefill_f32mfma_kernel<T, D>), dim3((unsigned)(BH * (dv / kCW))), dim3(kThreads), 0, st,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), L, dv, eps, y,
                       S, z, use_init);
}

template <typename T>
void launch_t(const void* q, const void* k, const void* v, int BH, int L, int d, int dv, float eps, float* y,
              float* S, float* z, int use_init, hipStream_t st) {
    switch (d) {
        case 8: launch_d<T, 8>(q, k, v, BH, L, dv, eps, y, S, z, use_init, st); break;
        case 24: launch_d<T, 24>(q, k, v, BH, L, dv, eps, y, S, z, use_init, st); break;
        case 32: launch_d<T, 32>(q, k, v, BH, L, dv, eps, y, S, z, use_init, st); break;
        default: launch_d<T, 16>(q, k, v, BH, L, dv, eps, y, S, z, use_init, st); break;
    }
}

}  // namespace

hipError_t launch_prefill_f32mfma(const void* q, const void* k, const void* v, bool bf16, int BH, int L, int d,
                                  int dv, float eps, float* y, float* S, float* z, int use_init, hipStream_t st) {
    if (bf16) launch_t<uint16_t>(q, k, v, BH, L, d, dv, eps, y, S, z, use_init, st);
    else launch_t<float>(q, k, v, BH, L, d, dv, eps, y, S, z, use_init, st);
    return hipGetLastError();
}

}  // namespace based

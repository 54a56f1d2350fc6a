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
// chunks in order.  The quadratic part of phi(q).phi(k) is symmetric in the
// pair (a, b), so the state keeps one internal row per unordered pair:
// internal rows [1, x~_0 .. x~_(d'-1), 0, 0, 0, pairs a <= b (a-major)],
// T_ab = sum_t k~_a k~_b v_t (update features k~_a k~_b), read out with
// q~_a q~_b for a < b and q~_a^2 / 2 on the diagonal.  The caller's rows
// (a, b) and (b, a) are both T_ab / sqrt2; a carried state enters as
// T_ab = (S_ab + S_ba) / sqrt2 (T_aa = sqrt2 S_aa) and each mirror row gets
// the same increment back, so its antisymmetric part (which no readout
// sees) is kept.  F = 1 + d' + d'(d'+1)/2 internal rows instead of 1 + d' +
// d'^2.  The rows come in 16-row tiles; per chunk:
//   * scores s = Q~ K~^T for the 10 lower-triangle 16x16 tiles (fp32 MFMA
//     over d'), masked weights into LDS;
//   * readout: wave w takes query tile w % 4 and every other feature tile
//     (w / 4 picks which): phi(Q~) S and phi(Q~).z with the state before
//     the chunk, read from LDS; the feature values are formed per lane
//     from a table of (a, b, weight) per internal row;
//   * update: wave w owns feature tiles w, w + 8, ...: S += phi(K~)^T V in
//     MFMA accumulators, z in per-lane partial sums;
//   * after a barrier: waves 0..3 add A V (and the row sums of A) for their
//     query tile to the two readout halves, normalise and store y; every
//     wave publishes its state tiles to LDS for the next chunk.
// Q~, K~ and V of the next chunk are loaded into registers at the start of
// a chunk and stored to the other LDS buffer before its end.
//
// Few heads (fewer than 256 workgroups) and long sequences: each head is cut
// into segments of at least 8 chunks.  A state-only pass (update alone)
// writes every segment's increment but the last one's to a workspace slot in
// the caller's row layout, a prefix over segments turns the slots into the
// states before each segment (from the caller's initial state), and the
// output pass runs every (head, segment, column group) from its slot; the
// last segment writes the caller's S and z.
#include "common.hpp"
#include "kernels.hpp"

namespace based {
namespace {

constexpr int kC = 64;      // chunk
constexpr int kCW = 16;     // value columns per workgroup
constexpr int kWaves = 8;   // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr float kSqrt2 = 1.41421356237309504880f;

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Internal feature order (see above) for feature dim D.
template <int D>
struct FMap {
    static_assert(D % 4 == 0, "feature dim a multiple of 4");
    static constexpr int kLin = D + 4;           // rows before the pair block
    static constexpr int kPairs = D * (D + 1) / 2;
    static constexpr int kRows = kLin + kPairs;
    static constexpr int kTiles = (kRows + 15) / 16;
    static constexpr int kRowsPad = 16 * kTiles;
    static constexpr int kOwn = (kTiles + kWaves - 1) / kWaves;  // update tiles per wave
    static constexpr int kF = 1 + D + D * D;                     // the caller's rows
};

// Internal row f: phi_f(x) = x[a] x[b] w, where column D of every staged
// row holds 1 (the constant row is x[D] x[D], a linear row x[f-1] x[D]).
// wq / wk are the readout / update weights (0 on padding rows), pair = 1
// for the pair rows (then a <= b).
struct RowInfo {
    int a, b;
    float wq, wk;
    bool pair;
};
template <int D>
__device__ __forceinline__ RowInfo row_info(int f) {
    using M = FMap<D>;
    RowInfo ri;
    ri.pair = f >= M::kLin && f < M::kRows;
    if (ri.pair) {
        int p = f - M::kLin, a = 0;
        while (p >= D - a) {  // row a holds pairs (a, a) .. (a, D-1)
            p -= D - a;
            ++a;
        }
        ri.a = a;
        ri.b = a + p;
        ri.wq = p == 0 ? 0.5f : 1.f;
        ri.wk = 1.f;
    } else {
        ri.a = (f >= 1 && f <= D) ? f - 1 : D;
        ri.b = D;
        ri.wq = ri.wk = f <= D ? 1.f : 0.f;
    }
    return ri;
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
    int2 tab[FMap<D>::kRowsPad];       // per internal row: a | b << 8, readout weight bits
};

// Staging of one chunk: q~, k~ (pre-scaled) and the workgroup's v columns.
// load issues every element's load unconditionally (the source is selected,
// tokens past L read token L-1, and the slots past the chunk's elements
// read a valid element they never store), so all of them are in flight
// together; the zeroing of tokens past L and the bf16 widening wait for
// store.
__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t x) { return bf16_bits_to_f32(x); }

// WITH_Q = false stages k and v only (the state-only pass).
template <typename T, int D, bool WITH_Q = true>
struct Stage {
    static constexpr int kQK = kC * D;          // elements of q (and of k)
    static constexpr int kNM = WITH_Q ? 2 : 1;  // staged [kC][D] matrices: q, k or k
    static constexpr int kV = kC * kCW;
    static constexpr int kPer = (kNM * kQK + kV + kThreads - 1) / kThreads;
    T x[kPer];

    __device__ __forceinline__ void load(const T* qh, const T* kh, const T* vh, int ldv, int t0, int L) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = threadIdx.x + kThreads * i;
            const bool qk = e < kNM * kQK;
            const int w = qk ? e % kQK : e - kNM * kQK;
            const int tok = min(t0 + (qk ? w / D : w / kCW), L - 1);
            const T* src = qk ? (WITH_Q && e < kQK ? qh : kh) + (size_t)tok * D + w % D
                              : vh + (size_t)tok * ldv + w % kCW;
            x[i] = *src;
        }
    }
    __device__ __forceinline__ void store(F32Smem<D>& sm, int buf, int t0, int L) const {
        constexpr int kLd = F32Smem<D>::kLd;
        if (WITH_Q) {
            if (threadIdx.x < 2 * kC) (threadIdx.x < kC ? sm.q[buf] : sm.k[buf])[(threadIdx.x % kC) * kLd + D] = 1.f;
        } else if (threadIdx.x < kC) {
            sm.k[buf][threadIdx.x * kLd + D] = 1.f;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = threadIdx.x + kThreads * i;
            if (e < kNM * kQK) {
                const int w = e % kQK, t = w / D, c = w % D;
                (WITH_Q && e < kQK ? sm.q[buf] : sm.k[buf])[t * kLd + c] =
                    t0 + t < L ? widen(x[i]) * Feat<D>::kPre : 0.f;
            } else if (e < kNM * kQK + kV) {
                const int w = e - kNM * kQK;
                sm.v[buf][w] = t0 + w / kCW < L ? widen(x[i]) : 0.f;
            }
        }
    }
};

// Where a workgroup's carried-in state comes from and where its final state
// goes, in the caller's row layout: bases with element strides per head and
// per segment (the caller's S and z, or workspace slots).  A null Sin means
// a zero initial state.
struct StateIO {
    const float* Sin;
    const float* zin;
    int in_h, in_s, in_hz, in_sz;
    float* Sout;
    float* zout;
    int out_h, out_s, out_hz, out_sz;
    int out_last_only;  // only the last segment of the grid writes its final state
    int write_z;        // column group 0 writes z (0: a later launch does)
};

// Lower-triangle score tiles of the chunk: index -> (query tile, key tile).
__device__ __forceinline__ void tri_tile(int idx, int& ti, int& tj) {
    ti = idx >= 6 ? 3 : (idx >= 3 ? 2 : (idx >= 1 ? 1 : 0));
    tj = idx - ti * (ti + 1) / 2;
}

// One workgroup per (head, segment, 16 value columns); a segment is the
// chunks [seg cps, (seg + 1) cps).  STATE_ONLY: the state increment alone
// (no scores, readout or output), by two workgroups per (head, segment,
// columns) that take the even and the odd update tiles u of every wave
// (where a wave owns two or more).
template <typename T, int D, bool STATE_ONLY>
__global__ __launch_bounds__(kThreads, 1) void prefill_f32mfma_kernel(const T* __restrict__ q,
                                                                      const T* __restrict__ k,
                                                                      const T* __restrict__ v, int L, int dv,
                                                                      float eps, float* __restrict__ y,
                                                                      StateIO io, int nseg, int cps) {
    using M = FMap<D>;
    constexpr int kLd = F32Smem<D>::kLd;
    __shared__ F32Smem<D> sm;
    const int ncg = dv / kCW;
    constexpr int kSplit = (STATE_ONLY && M::kOwn >= 2) ? 2 : 1;
    const int part = kSplit == 2 ? (int)(blockIdx.x & 1) : 0;  // update tiles u with u % 2 == part
    const int bid = (int)blockIdx.x / kSplit;
    const int cg = bid % ncg, hs = bid / ncg;
    const int seg = hs % nseg, head = hs / nseg;
    const int col0 = cg * kCW;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const T* qh = q + (size_t)head * L * D;
    const T* kh = k + (size_t)head * L * D;
    const T* vh = v + (size_t)head * L * dv + col0;
    float* yh = STATE_ONLY ? nullptr : y + (size_t)head * L * dv + col0;
    const bool use_init = io.Sin != nullptr;
    const float* Sin = use_init ? io.Sin + (size_t)head * io.in_h + (size_t)seg * io.in_s + col0 : nullptr;
    const float* zin = use_init ? io.zin + (size_t)head * io.in_hz + (size_t)seg * io.in_sz : nullptr;
    float* Sout = io.Sout + (size_t)head * io.out_h + (size_t)seg * io.out_s + col0;
    float* zout = io.zout + (size_t)head * io.out_hz + (size_t)seg * io.out_sz;
    const int c_begin = seg * cps;
    const int c_end = min((L + kC - 1) / kC, c_begin + cps);

    // feature table of the readout
    for (int f = threadIdx.x; f < M::kRowsPad; f += kThreads) {
        const RowInfo ri = row_info<D>(f);
        sm.tab[f] = make_int2(ri.a | (ri.b << 8), __float_as_int(ri.wq));
    }
    // ---- state: this wave's tiles w + 8u in accumulators (rows 16rt + 4g + m,
    // column r), z as per-lane partial sums (row 16rt + r, this lane group's
    // tokens; the initial z sits in lane group 0).  A carried state enters
    // folded onto the pair rows.
    auto init_row = [&](int f, int col, const float* base, size_t stride) -> float {
        const RowInfo ri = row_info<D>(f);
        if (ri.wk == 0.f) return 0.f;
        if (!ri.pair) return base[(size_t)f * stride + col];
        const float x = base[(size_t)(1 + D + D * ri.a + ri.b) * stride + col];
        const float y = base[(size_t)(1 + D + D * ri.b + ri.a) * stride + col];
        return ri.a == ri.b ? kSqrt2 * x : (x + y) * kInvSqrt2;
    };
    f32x4 sacc[M::kOwn];
    float zp[M::kOwn];
#pragma unroll
    for (int u = 0; u < M::kOwn; ++u) {
        const int rt = w + kWaves * u;
        sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        zp[u] = 0.f;
        if (use_init && rt < M::kTiles) {
#pragma unroll
            for (int m = 0; m < 4; ++m) sacc[u][m] = init_row(16 * rt + 4 * g + m, r, Sin, dv);
            if (g == 0) zp[u] = init_row(16 * rt + r, 0, zin, 1);
        }
    }
    // feature indices of this lane's update row (16rt + r) of every own tile
    int ua[M::kOwn], ub[M::kOwn];
    float um[M::kOwn];
#pragma unroll
    for (int u = 0; u < M::kOwn; ++u) {
        const RowInfo ri = row_info<D>(16 * (w + kWaves * u) + r);
        ua[u] = ri.a;
        ub[u] = ri.b;
        um[u] = (w + kWaves * u) < M::kTiles ? ri.wk : 0.f;
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
    // ---- update with chunk c's keys (staged in buffer buf): tiles w + 8u
    auto update = [&](int c, int buf) {
        const float* ks = sm.k[buf];
        const float* vs = sm.v[buf];
        const int nvalid = min(kC, L - c * kC);
#pragma unroll 4
        for (int j = 0; j < kC / 4; ++j) {
            const int t = 4 * j + g;  // this lane group's token
            const float vb = vs[t * kCW + r];
            const float* krow = ks + t * kLd;
            const float tok_ok = t < nvalid ? 1.f : 0.f;
#pragma unroll
            for (int u = 0; u < M::kOwn; ++u) {
                const int rt = w + kWaves * u;
                if (rt < M::kTiles && (kSplit == 1 || (u & 1) == part)) {
                    const float phi = krow[ua[u]] * krow[ub[u]] * (um[u] * tok_ok);
                    sacc[u] = mfma_f32(phi, vb, sacc[u]);
                    zp[u] += phi;
                }
            }
        }
    };

    if constexpr (STATE_ONLY) {
        // Update alone is short per chunk, so two chunks' loads are kept in
        // flight: at chunk c, registers hold chunk c+1 and take chunk c+2's
        // loads; chunk c+1 goes to the other LDS buffer at the end of c.
        Stage<T, D, false> sa, sb;
        sa.load(qh, kh, vh, dv, c_begin * kC, L);
        sa.store(sm, 0, c_begin * kC, L);
        if (c_begin + 1 < c_end) sb.load(qh, kh, vh, dv, (c_begin + 1) * kC, L);
        __syncthreads();
        auto step = [&](int c, Stage<T, D, false>& nxt, Stage<T, D, false>& fre) {
            const int buf = (c - c_begin) & 1;
            if (c + 2 < c_end) fre.load(qh, kh, vh, dv, (c + 2) * kC, L);
            update(c, buf);
            if (c + 1 < c_end) nxt.store(sm, buf ^ 1, (c + 1) * kC, L);
            __syncthreads();
        };
        for (int c = c_begin; c < c_end; c += 2) {
            step(c, sb, sa);
            if (c + 1 < c_end) step(c + 1, sa, sb);
        }
    }
    if constexpr (!STATE_ONLY) {
    publish();
    Stage<T, D> st;
    st.load(qh, kh, vh, dv, c_begin * kC, L);
    st.store(sm, 0, c_begin * kC, L);
    __syncthreads();

    const int tt = w & 3, half = w >> 2;  // readout: query tile, feature half
    for (int c = c_begin; c < c_end; ++c) {
        const int buf = (c - c_begin) & 1, t0 = c * kC;
        const float* qs = sm.q[buf];
        const float* ks = sm.k[buf];
        const float* vs = sm.v[buf];
        const bool more = c + 1 < c_end;
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
                    const int f = 16 * rt + 4 * j + g;
                    const int2 te = sm.tab[f];
                    const float phi = qrow[te.x & 255] * qrow[te.x >> 8] * __int_as_float(te.y);
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

        update(c, buf);
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
        if (more) st.store(sm, buf ^ 1, t0 + kC, L);
        __syncthreads();
    }
    }  // !STATE_ONLY

    // ---- final state in the caller's rows (z from column group 0, unless a
    // carried z is shared by several groups and read from the same array:
    // then every group must read the caller's z however late it starts, and
    // a later launch writes it): a pair row goes to both mirror rows, as
    // T / sqrt2 or, after a carried state, as that state plus this call's
    // increment
    if (io.out_last_only && seg != nseg - 1) return;
    auto store_row = [&](int f, int col, float tv, const float* in, float* out, size_t stride) {
        const RowInfo ri = row_info<D>(f);
        if (ri.wk == 0.f) return;
        if (!ri.pair) {
            out[(size_t)f * stride + col] = tv;
            return;
        }
        const size_t ab = (size_t)(1 + D + D * ri.a + ri.b) * stride + col;
        const size_t ba = (size_t)(1 + D + D * ri.b + ri.a) * stride + col;
        if (!use_init) {
            out[ab] = tv * kInvSqrt2;
            out[ba] = tv * kInvSqrt2;
        } else {
            const float x = in[ab], y = in[ba];
            const float t_init = ri.a == ri.b ? kSqrt2 * x : (x + y) * kInvSqrt2;
            const float inc = (tv - t_init) * kInvSqrt2;
            out[ab] = x + inc;
            if (ri.a != ri.b) out[ba] = y + inc;
        }
    };
#pragma unroll
    for (int u = 0; u < M::kOwn; ++u) {
        const int rt = w + kWaves * u;
        if (rt < M::kTiles && (kSplit == 1 || (u & 1) == part)) {
#pragma unroll
            for (int m = 0; m < 4; ++m) store_row(16 * rt + 4 * g + m, r, sacc[u][m], Sin, Sout, dv);
            float zs = zp[u];
            zs += __shfl_xor(zs, 16, 64);
            zs += __shfl_xor(zs, 32, 64);
            if (io.write_z && cg == 0 && g == 0) store_row(16 * rt + r, 0, zs, zin, zout, 1);
        }
    }
}

// Prefix over segments of the workspace slots, per (head, element): slot 0
// becomes the caller's initial state (or zero) and slot s (holding segment
// s-1's increment) the state before segment s.
__global__ __launch_bounds__(256) void f32_segment_prefix_kernel(float* __restrict__ ws, const float* __restrict__ S0,
                                                                 const float* __restrict__ z0, int BH, int nseg,
                                                                 int F, int dv, size_t slot) {
    const size_t per = (size_t)F * dv + F;
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (size_t)BH * per) return;
    const size_t head = e / per, i = e % per;
    float acc = 0.f;
    if (S0) acc = i < (size_t)F * dv ? S0[head * F * dv + i] : z0[head * F + (i - (size_t)F * dv)];
    float* p = ws + head * nseg * slot + i;
    p[0] = acc;
    for (int s = 1; s < nseg; ++s) {
        acc += p[s * slot];
        p[s * slot] = acc;
    }
}

template <typename T, int D>
void launch_d(const void* q, const void* k, const void* v, int BH, int L, int dv, float eps, float* y,
              const StateIO& io, int nseg_grid, int cps, int state_only, hipStream_t st) {
    const int split = state_only && FMap<D>::kOwn >= 2 ? 2 : 1;  // the kernel's kSplit
    const dim3 grid((unsigned)(BH * nseg_grid * (dv / kCW) * split));
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    if (state_only)
        hipLaunchKernelGGL((prefill_f32mfma_kernel<T, D, true>), grid, dim3(kThreads), 0, st, qq, kk, vv, L, dv, eps,
                           y, io, nseg_grid, cps);
    else
        hipLaunchKernelGGL((prefill_f32mfma_kernel<T, D, false>), grid, dim3(kThreads), 0, st, qq, kk, vv, L, dv,
                           eps, y, io, nseg_grid, cps);
}

template <typename T>
void launch_t(const void* q, const void* k, const void* v, int BH, int L, int d, int dv, float eps, float* y,
              const StateIO& io, int nseg_grid, int cps, int state_only, hipStream_t st) {
    switch (d) {
        case 8: launch_d<T, 8>(q, k, v, BH, L, dv, eps, y, io, nseg_grid, cps, state_only, st); break;
        case 24: launch_d<T, 24>(q, k, v, BH, L, dv, eps, y, io, nseg_grid, cps, state_only, st); break;
        case 32: launch_d<T, 32>(q, k, v, BH, L, dv, eps, y, io, nseg_grid, cps, state_only, st); break;
        default: launch_d<T, 16>(q, k, v, BH, L, dv, eps, y, io, nseg_grid, cps, state_only, st); break;
    }
}

// Segments per head: one workgroup per (head, 16 columns) fills fewer than
// the 256 compute units when B*H*d_v/16 < 256; then each head is cut into
// segments of at least 8 chunks, up to one launch's worth of 256
// workgroups.  The segments' increments come from a state-only pass (every
// segment but the last), a prefix over segments adds them up, and the
// output pass runs every segment from its carried-in state.
int f32_segments(int BH, int L, int dv) {
    const long long groups = (long long)BH * (dv / kCW);
    const int nch = (L + kC - 1) / kC;
    if (groups >= 256) return 1;
    const int by_chip = (int)(256 / groups);
    const int by_len = nch / 8;
    const int n = by_chip < by_len ? by_chip : by_len;
    return n > 1 ? n : 1;
}

size_t f32_slot_floats(int d, int dv) {
    const size_t F = (size_t)1 + d + (size_t)d * d;
    return (F * dv + F + 63) & ~(size_t)63;
}

}  // namespace

size_t prefill_f32mfma_workspace_bytes(int BH, int L, int d, int dv) {
    const int nseg = f32_segments(BH, L, dv);
    return nseg > 1 ? (size_t)BH * nseg * f32_slot_floats(d, dv) * sizeof(float) : 0;
}

hipError_t launch_prefill_f32mfma(const void* q, const void* k, const void* v, bool bf16, int BH, int L, int d,
                                  int dv, float eps, float* y, float* S, float* z, int use_init, void* workspace,
                                  size_t workspace_bytes, hipStream_t st) {
    const size_t F = (size_t)1 + d + (size_t)d * d;
    const int nch = (L + kC - 1) / kC;
    const int nseg = f32_segments(BH, L, dv);
    auto run = [&](const StateIO& io, int nseg_grid, int cps, int state_only) {
        if (bf16) launch_t<uint16_t>(q, k, v, BH, L, d, dv, eps, y, io, nseg_grid, cps, state_only, st);
        else launch_t<float>(q, k, v, BH, L, d, dv, eps, y, io, nseg_grid, cps, state_only, st);
    };
    if (nseg > 1 && workspace && workspace_bytes >= prefill_f32mfma_workspace_bytes(BH, L, d, dv)) {
        const int cps = (nch + nseg - 1) / nseg;
        const int nseg_used = (nch + cps - 1) / cps;
        float* ws = static_cast<float*>(workspace);
        const size_t slot = f32_slot_floats(d, dv);
        const size_t hstride = (size_t)nseg_used * slot;
        // 1. increments of segments 0 .. n-2 into slots 1 .. n-1
        const int hs = (int)hstride, sl = (int)slot, fdv = (int)(F * dv), f = (int)F;
        StateIO inc{nullptr, nullptr, 0, 0, 0, 0, ws + slot, ws + slot + F * dv, hs, sl, hs, sl, 0, 1};
        run(inc, nseg_used - 1, cps, 1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // 2. prefix over segments, from the caller's initial state
        const size_t total = (size_t)BH * (F * dv + F);
        hipLaunchKernelGGL(f32_segment_prefix_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, ws,
                           use_init ? S : nullptr, use_init ? z : nullptr, BH, nseg_used, (int)F, dv, slot);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // 3. every segment from its carried-in state; the last one writes the
        // caller's S and z (nothing reads them meanwhile)
        StateIO out{ws, ws + F * dv, hs, sl, hs, sl, S, z, fdv, 0, f, 0, 1, 1};
        run(out, nseg_used, cps, 0);
        return hipGetLastError();
    }
    // One segment per head.  With a carried z and several column groups, no
    // group may overwrite z while another may still read it: the groups
    // leave z alone and a stream-ordered launch adds this call's increment
    // afterwards.
    const bool z_after = use_init && dv / kCW > 1;
    const int fdv = (int)(F * dv), f = (int)F;
    StateIO io{use_init ? S : nullptr, use_init ? z : nullptr, fdv, 0, f, 0, S, z, fdv, 0, f, 0, 0, z_after ? 0 : 1};
    run(io, 1, nch, 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !z_after) return e;
    return launch_prefill_z(k, bf16, BH, L, d, z, use_init, st);
}

}  // namespace based

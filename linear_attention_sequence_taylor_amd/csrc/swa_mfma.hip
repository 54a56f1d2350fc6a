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
//  * A workgroup (4 waves) walks a run of 64-query tiles of one head.  K and
//    V tiles live in a 3-slot LDS ring (the previous tile is the current
//    tile's halo, so every K/V row is fetched from HBM once), Q in 2 slots.
//    Tile t+1 is copied global -> LDS with asynchronous 16-byte LDS-DMA
//    loads while tile t is computed; the fused-add input of tile t+1 is
//    prefetched into registers at the same time.
//  * LDS rows are 16-byte units XOR-swizzled by row, which makes the
//    score-operand reads and the transposed V reads conflict-free.
//  * Wave w owns queries i0+16w .. +15, whose keys lie in the 80 rows
//    [i0+16w-64, i0+16w+16) = 5 key tiles of 16.  Scores are computed
//    transposed, S^T = K Q^T, so each lane holds one query and 4 keys per
//    tile: the probabilities are already in the A-operand layout of P.V
//    (two key tiles form one 32-deep k-step).  The V operand comes from
//    row-major V through transposed LDS reads (ds_read_b64_tr_b16).
//  * Softmax runs in fp32 (exp2, max-subtracted); P enters the MFMA as a
//    hi/lo bf16 pair so the weights carry ~16 bits; the normaliser is the
//    fp32 sum of the same probabilities.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace based {
namespace {

constexpr int kQT = 64;  // queries per tile = key rows per ring slot
constexpr int kDV = 64;
constexpr float kLog2e = 1.4426950408889634f;

#define BASED_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// LDS slots of one step: K/V of the HALO tiles before the current one and of
// the current tile (oldest first), Q of the current tile, and the slots that
// receive tile t+1.  Each slot is its own __shared__ array, so the compiler
// can tell the copies in flight from the data being read.
template <int HALO>
struct SwaSlots {
    const uint16_t* k[HALO + 1];
    const uint16_t* v[HALO + 1];
    const uint16_t* qc;
    uint16_t *kn, *vn, *qn;
};

// a[(16w + 16j) / 64] for the wave index w (0..3) and a tile offset j that
// is a constant once the caller's loop is unrolled: one of the two
// neighbouring entries a[j/4] and a[j/4 + 1], chosen by one scalar compare
// (a longer select chain is turned into an indexed stack array).
template <int N>
__device__ __forceinline__ const uint16_t* slot_of(const uint16_t* const (&a)[N], int w, int j) {
    const int b = j >> 2;
    if (b + 1 >= N) return a[N - 1];
    return w + (j & 3) >= 4 ? a[b + 1] : a[b];
}

// Element offset of (row, col) in a [64][D] bf16 tile whose 16-byte units
// are XOR-swizzled by row bits.
template <int D>
__device__ __forceinline__ int tile_idx(int row, int col) {
    const int sw = D == 64 ? (row & 7) : ((row >> 3) & 1);
    return row * D + 8 * ((col >> 3) ^ sw) + (col & 7);
}

// Asynchronous copy of block b (1 KB = 64 lanes x 16 B) of a [64][D] tile:
// rows row0.. of a [L][D] matrix (clamped into [0, L)) into an LDS tile.
// The DMA puts lane l's 16 bytes at byte 16*l of the block, so each lane
// fetches the source unit that the swizzle stores there.
// ld is the source's row stride in elements (D for q and k; the value head
// dim for a 64-column slice of v).
template <int D>
__device__ __forceinline__ void dma_block(const uint16_t* mat, int ld, int L, int row0, uint16_t* tile, int b,
                                          int lane) {
    constexpr int kUnits = D / 8;       // 16-byte units per row
    constexpr int kRows = 64 / kUnits;  // rows per 1 KB block
    const int row = kRows * b + lane / kUnits;
    const int su = lane % kUnits;
    const int sw = D == 64 ? (row & 7) : ((row >> 3) & 1);
    const int gu = su ^ sw;
    const int src = min(max(row0 + row, 0), L - 1);
    __builtin_amdgcn_global_load_lds(mat + (size_t)src * ld + 8 * gu, BASED_LDS(void, tile + 512 * b), 16, 0, 0);
}

// Copies of tile t into slots ks, vs (and qs), split over the four waves.
// with_q = false for the halo before the run.
template <int DQK>
__device__ __forceinline__ void dma_tile(const uint16_t* qh, const uint16_t* kh, const uint16_t* vh, int ldv, int L,
                                         int t, uint16_t* ks, uint16_t* vs, uint16_t* qs, bool with_q, int w,
                                         int lane) {
    const int row0 = t * kQT;
    dma_block<kDV>(vh, ldv, L, row0, vs, 2 * w, lane);
    dma_block<kDV>(vh, ldv, L, row0, vs, 2 * w + 1, lane);
    if constexpr (DQK == 64) {
        dma_block<64>(kh, 64, L, row0, ks, 2 * w, lane);
        dma_block<64>(kh, 64, L, row0, ks, 2 * w + 1, lane);
        if (with_q) {
            dma_block<64>(qh, 64, L, row0, qs, 2 * w, lane);
            dma_block<64>(qh, 64, L, row0, qs, 2 * w + 1, lane);
        }
    } else {
        if (w < 2) dma_block<16>(kh, 16, L, row0, ks, w, lane);
        else if (with_q) dma_block<16>(qh, 16, L, row0, qs, w - 2, lane);
    }
}

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void pack8_hilo(const float (&a)[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = pack_bf16x2(a[2 * i], a[2 * i + 1]);
        l[i] = lo_pair_of(h[i], a[2 * i], a[2 * i + 1]);
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// S^T tile: rows = 16 keys (rows kr0.. of key slot ks), cols = the wave's 16
// queries (rows qr0.. of q slot qs).  Lane (g, r): query r, keys 4g..4g+3.
template <int DQK>
__device__ __forceinline__ f32x4 score_tile(const uint16_t* ks, int kr0, const uint16_t* qs, int qr0, int g, int r) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DQK == 16) {
        const bf16x4 a = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(ks + tile_idx<16>(kr0 + r, 4 * g)));
        const bf16x4 b = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(qs + tile_idx<16>(qr0 + r, 4 * g)));
        acc = mfma16(a, b, acc);
    } else {
#pragma unroll
        for (int kk = 0; kk < DQK / 32; ++kk) {
            const bf16x8 a =
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ks + tile_idx<64>(kr0 + r, 32 * kk + 8 * g)));
            const bf16x8 b =
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qs + tile_idx<64>(qr0 + r, 32 * kk + 8 * g)));
            acc = mfma32(a, b, acc);
        }
    }
    return acc;
}

// LDS byte address of the 8 bytes that lane c of a 16-lane group supplies
// to a transposed 16-bit read of value rows rb..rb+3, column tile ct: row
// rb + (c >> 2), columns 16ct + 4(c & 3) .. +3.  The read returns to lane c
// the 4 rows of column 16ct + c.
__device__ __forceinline__ uint32_t v_tr_addr(const uint16_t* vs, int rb, int ct, int c) {
    const uint16_t* p = vs + tile_idx<64>(rb + (c >> 2), 16 * ct + 4 * (c & 3));
    return (uint32_t)(uintptr_t)BASED_LDS(void, p);
}

// B operands of one P.V k-step for the 4 column tiles: keys (rows) r1..r1+3
// of slot v1 (first half) and r2..r2+3 of slot v2 (second half, zero when
// TWO is false).  Written as one asm block (with its own wait) because the
// compiler, unable to tell these reads from the LDS copies in flight,
// would otherwise wait for every outstanding memory operation first.  The
// outputs are early-clobber: a read's data may land while later reads of
// the block have not issued yet, so no output may share a register with an
// address.
template <bool TWO>
__device__ __forceinline__ void v_kstep(const uint16_t* v1, int r1, const uint16_t* v2, int r2, int c,
                                        bf16x8 (&vb)[4]) {
    uint2 x[8];
    if constexpr (TWO) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\t"
            "ds_read_b64_tr_b16 %1, %9\n\t"
            "ds_read_b64_tr_b16 %2, %10\n\t"
            "ds_read_b64_tr_b16 %3, %11\n\t"
            "ds_read_b64_tr_b16 %4, %12\n\t"
            "ds_read_b64_tr_b16 %5, %13\n\t"
            "ds_read_b64_tr_b16 %6, %14\n\t"
            "ds_read_b64_tr_b16 %7, %15\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
            : "v"(v_tr_addr(v1, r1, 0, c)), "v"(v_tr_addr(v1, r1, 1, c)), "v"(v_tr_addr(v1, r1, 2, c)),
              "v"(v_tr_addr(v1, r1, 3, c)), "v"(v_tr_addr(v2, r2, 0, c)), "v"(v_tr_addr(v2, r2, 1, c)),
              "v"(v_tr_addr(v2, r2, 2, c)), "v"(v_tr_addr(v2, r2, 3, c))
            : "memory");
    } else {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %4\n\t"
            "ds_read_b64_tr_b16 %1, %5\n\t"
            "ds_read_b64_tr_b16 %2, %6\n\t"
            "ds_read_b64_tr_b16 %3, %7\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
            : "v"(v_tr_addr(v1, r1, 0, c)), "v"(v_tr_addr(v1, r1, 1, c)), "v"(v_tr_addr(v1, r1, 2, c)),
              "v"(v_tr_addr(v1, r1, 3, c))
            : "memory");
        x[4] = x[5] = x[6] = x[7] = make_uint2(0u, 0u);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const u32x4 u = {x[ct].x, x[ct].y, x[4 + ct].x, x[4 + ct].y};
        vb[ct] = __builtin_bit_cast(bf16x8, u);
    }
}

// One 64-query tile for wave w: y rows in yacc (P.V, unnormalised) and the
// normaliser l of this lane's query.  Keys: the 64*HALO before the wave's
// first query and the wave's 16, i.e. 4*HALO + 1 key tiles of 16.
template <int DQK, int HALO>
__device__ __forceinline__ void swa_tile(const SwaSlots<HALO>& sl, int t, int window, float sl2, int w, int g,
                                         int r, f32x4 (&yacc)[4], float& l) {
    constexpr int kKT = 4 * HALO + 1;  // key tiles
    constexpr int kHR = kQT * HALO;    // halo rows
    const uint16_t* qs = sl.qc;
    const int q0 = t * kQT + 16 * w;  // first query of the wave
    const int qi = q0 + r;            // this lane's query

    // Scores for key tiles j: keys q0 - 64*HALO + 16j + 4g + m, which sit in
    // row 16w + 16j of the window [tile t-HALO | ... | tile t].
    float s[kKT][4];
#pragma unroll
    for (int j = 0; j < kKT; ++j) {
        const int R = 16 * w + 16 * j;
        const f32x4 st = score_tile<DQK>(slot_of(sl.k, w, j), R & 63, qs, 16 * w, g, r);
        if (window == kHR && q0 >= kHR) {
            // Full window, no key before the sequence start: key 16j + 4g + m
            // is in the window of query r iff it lies in (r, r + 64*HALO], so
            // only the first and last key tiles are cut.
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int d = 16 * j + 4 * g + m;
                const bool ok = j == 0 ? d > r : (j == kKT - 1 ? d <= r + kHR : true);
                s[j][m] = ok ? st[m] * sl2 : -INFINITY;
            }
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int kj = q0 - kHR + 16 * j + 4 * g + m;
                const bool ok = kj >= 0 && kj <= qi && kj > qi - window;
                s[j][m] = ok ? st[m] * sl2 : -INFINITY;
            }
        }
    }
    // Row max over all keys: this lane's, then across the 4 lane groups.
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKT; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) mx = fmaxf(mx, s[j][m]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    l = 0.f;
#pragma unroll
    for (int j = 0; j < kKT; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // hardware 2^x: masked keys give 2^-inf = 0; arguments below -126
            // (weights under 2^-126 of the row maximum) may flush to 0
            const float p = __builtin_amdgcn_exp2f(s[j][m] - mx);
            s[j][m] = p;
            l += p;
        }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);

    // Y = P V over 2*HALO + 1 k-steps of 32 keys (tiles 2p, 2p+1; the last
    // k-step has only tile 4*HALO).
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) yacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p <= 2 * HALO; ++p) {
        float a[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            a[m] = s[2 * p][m];
            a[4 + m] = 2 * p + 1 < kKT ? s[(2 * p + 1 < kKT) ? 2 * p + 1 : 0][m] : 0.f;
        }
        bf16x8 ahi, alo;
        pack8_hilo(a, ahi, alo);
        // key rows of this lane group: R1 + 4g .. +3 (tile 2p), R2 + 4g .. +3 (tile 2p+1)
        const int R1 = 16 * w + 32 * p, R2 = R1 + 16;
        const uint16_t* v1 = slot_of(sl.v, w, 2 * p);
        const uint16_t* v2 = slot_of(sl.v, w, 2 * p + 1);
        const int r1 = (R1 & 63) + 4 * g, r2 = (R2 & 63) + 4 * g;
        bf16x8 vb[4];
        // the last k-step has no second key tile: that half of the operand is zero
        if (p < 2 * HALO) v_kstep<true>(v1, r1, v2, r2, r, vb);
        else v_kstep<false>(v1, r1, v2, r2, r, vb);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) yacc[ct] = mfma32(ahi, vb[ct], yacc[ct]);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) yacc[ct] = mfma32(alo, vb[ct], yacc[ct]);
    }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8; the other counters left at "no wait").  Issued
// through the builtin so that the compiler's own wait insertion knows
// which memory operations have completed.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// Byte offset of (query row, column) in a head's [L][ldv] fp32 array
// (relative to the workgroup's first column).
__device__ __forceinline__ int out_off(int row, int col, int ldv) { return (row * ldv + col) * 4; }
constexpr int kNT = 2;  // buffer access: streaming (nontemporal)

// Fused-add input of one tile for this lane: rows q0 + 4g + m, columns
// 16ct + r.  Buffer loads: rows past the end read as 0 (range-checked by
// the resource), so the access needs no branch.
__device__ __forceinline__ void load_add(__amdgpu_buffer_rsrc_t ra, int q0, int g, int r, int ldv, float (&a)[16]) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
            a[4 * m + ct] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(ra, out_off(q0 + 4 * g + m, 16 * ct + r, ldv), 0, kNT));
}

// Barrier without the compiler's release/acquire fences (which would wait
// for every outstanding copy); the waits are explicit in the pipeline.
__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int DQK, bool ADD, int HALO, int NCS>
__global__ __launch_bounds__(256) void swa_mfma_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, int L, int ntiles,
                                                       int tiles_per_wg, int wg_per_head, int window, float scale,
                                                       const float* add, float* y) {
    constexpr int ldv = kDV * NCS;  // row stride of v, y and add: NCS slices of 64 columns
    // K/V ring of HALO + 2 slots: tile tb - HALO + j lives in slot j mod
    // (HALO + 2); Q of tile tb + j in slot j mod 2.  (The fourth slot is a
    // placeholder when HALO = 1.)
    constexpr int kNS = HALO + 2;
    constexpr int kS3K = HALO == 2 ? kQT * DQK : 8, kS3V = HALO == 2 ? kQT * kDV : 8;
    __shared__ alignas(16) uint16_t k0[kQT * DQK], k1[kQT * DQK], k2[kQT * DQK], k3[kS3K];
    __shared__ alignas(16) uint16_t v0[kQT * kDV], v1[kQT * kDV], v2[kQT * kDV], v3[kS3V];
    __shared__ alignas(16) uint16_t q0s[kQT * DQK], q1s[kQT * DQK];
    uint16_t* const ks[4] = {k0, k1, k2, k3};
    uint16_t* const vs[4] = {v0, v1, v2, v3};
    uint16_t* const qs[2] = {q0s, q1s};

    // Workgroup -> (head, run, 64-column slice), slice fastest.
    int bid = blockIdx.x;
    const int col0 = (bid % NCS) * kDV;
    bid /= NCS;
    const int head = bid / wg_per_head;
    const int tb = (bid % wg_per_head) * tiles_per_wg;
    const int te = min(tb + tiles_per_wg, ntiles);
    // The wave index is uniform across the wave: held in a scalar register,
    // the slot choices below are scalar branches, not per-lane selects.
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const uint16_t* qh = q + (size_t)head * L * DQK;
    const uint16_t* kh = k + (size_t)head * L * DQK;
    const uint16_t* vh = v + (size_t)head * L * ldv + col0;
    // Outputs (and the fused-add input) through buffer resources covering
    // exactly this head from the slice's first column: rows past L are
    // dropped (stores) or read as 0, so every step issues the same memory
    // instructions, with no branches.
    const int head_bytes = (L * ldv - col0) * 4;
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(y + (size_t)head * L * ldv + col0, (short)0, head_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        ADD ? (void*)(add + (size_t)head * L * ldv + col0) : (void*)y, (short)0, ADD ? head_bytes : 0, 0x00020000);
    const float sl2 = scale * kLog2e;

    // Prologue: halo tiles tb-HALO .. tb-1 (K, V) into slots 0 .. HALO-1 and
    // tile tb into slot HALO; add of tile tb.  The vector-memory counter
    // retires in issue order, so waiting until only the 16 add loads remain
    // means every copy landed.
    float adda[16], addb[16];
#pragma unroll
    for (int h = 0; h < HALO; ++h)
        dma_tile<DQK>(qh, kh, vh, ldv, L, tb - HALO + h, ks[h], vs[h], nullptr, false, w, lane);
    dma_tile<DQK>(qh, kh, vh, ldv, L, tb, ks[HALO], vs[HALO], q0s, true, w, lane);
    // The counted waits below need the copies issued before every other
    // vector-memory access that follows them in the source: nothing may be
    // scheduled across this point (the add loads would otherwise be free to
    // move above the copies, and the wait would then let copies still be in
    // flight at the barrier).
    __builtin_amdgcn_sched_barrier(0);
    if (ADD) {
        load_add(ra, tb * kQT + 16 * w, g, r, ldv, adda);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(16));
    } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    raw_barrier();

    // Step j of the run (tile t = tb + j): start the copies (and the add
    // loads) of tile t+1 unless t is the run's last tile, compute and store
    // tile t, then wait for tile t+1's copies -- the 16 add loads and 16
    // stores issued after them may stay in flight -- before the barrier.
    auto step = [&](auto J, int t, const float (&cur_add)[16], float (&next_add)[16]) {
        constexpr int j = decltype(J)::value;
        SwaSlots<HALO> sl;
#pragma unroll
        for (int h = 0; h <= HALO; ++h) {
            sl.k[h] = ks[(j + h) % kNS];
            sl.v[h] = vs[(j + h) % kNS];
        }
        sl.qc = qs[j % 2];
        sl.kn = ks[(j + HALO + 1) % kNS];
        sl.vn = vs[(j + HALO + 1) % kNS];
        sl.qn = qs[(j + 1) % 2];
        if (t + 1 < te) {
            dma_tile<DQK>(qh, kh, vh, ldv, L, t + 1, sl.kn, sl.vn, sl.qn, true, w, lane);
            __builtin_amdgcn_sched_barrier(0);  // the copies first (see the prologue)
            if (ADD) load_add(ra, (t + 1) * kQT + 16 * w, g, r, ldv, next_add);
        }
        f32x4 yacc[4];
        float l;
        swa_tile<DQK, HALO>(sl, t, window, sl2, w, g, r, yacc, l);
        const int q0 = t * kQT + 16 * w;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float inv = __builtin_amdgcn_rcpf(__shfl(l, 4 * g + m, 64));  // l >= 1: the max key has p = 1
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const float o = yacc[ct][m] * inv + (ADD ? cur_add[4 * m + ct] : 0.f);
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o), ry,
                                                      out_off(q0 + 4 * g + m, 16 * ct + r, ldv), 0, kNT);
            }
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(ADD ? 32 : 16));
        raw_barrier();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    // Slot indices repeat every lcm(HALO + 2, 2) tiles: 6 steps per
    // iteration for HALO = 1, 4 for HALO = 2, nested so that each step
    // follows exactly one other in the control flow.
    constexpr int kPeriod = HALO == 1 ? 6 : 4;
    for (int t = tb; t < te; t += kPeriod) {
        step(I0{}, t, adda, addb);
        if (t + 1 < te) {
            step(I1{}, t + 1, addb, adda);
            if (t + 2 < te) {
                step(I2{}, t + 2, adda, addb);
                if (t + 3 < te) {
                    step(I3{}, t + 3, addb, adda);
                    if constexpr (kPeriod == 6) {
                        if (t + 4 < te) {
                            step(I4{}, t + 4, adda, addb);
                            if (t + 5 < te) step(I5{}, t + 5, addb, adda);
                        }
                    }
                }
            }
        }
    }
}

// ---- windows over 128 keys (up to the whole causal prefix).  One workgroup
// per (head, 64-query tile, 64-column slice) walks the key tiles that meet
// any of its queries' windows, oldest first, with an online softmax: per
// key tile the running row maximum m is raised to cover the tile's scores,
// the probabilities are taken against it, and the partial sums of earlier
// tiles are scaled down by 2^(m_old - m_new).  K/V tiles alternate between
// two LDS slots; tile kt+1 is copied in (LDS-DMA) while tile kt is used.
// Same operand layouts as the run kernel above: S^T = K Q^T per 16-key
// sub-tile (lane: one query, 4 keys), P as a hi/lo bf16 pair, V through
// transposed LDS reads.
template <int DQK>
struct LongSlot {
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* kn;
    uint16_t* vn;
};

template <int DQK>
__device__ __forceinline__ void dma_kv(const uint16_t* kh, const uint16_t* vh, int ldv, int L, int t, uint16_t* ks,
                                       uint16_t* vs, int w, int lane) {
    const int row0 = t * kQT;
    dma_block<kDV>(vh, ldv, L, row0, vs, 2 * w, lane);
    dma_block<kDV>(vh, ldv, L, row0, vs, 2 * w + 1, lane);
    if constexpr (DQK == 64) {
        dma_block<64>(kh, 64, L, row0, ks, 2 * w, lane);
        dma_block<64>(kh, 64, L, row0, ks, 2 * w + 1, lane);
    } else {
        if (w < 2) dma_block<16>(kh, 16, L, row0, ks, w, lane);
    }
}

// Online-softmax update of this wave's 16 queries with key tile kt (keys
// 64kt .. 64kt+63 in slots ks, vs).  m: running maximum (log2 units) of this
// lane's query r; lp: this lane's partial sum of probabilities.
template <int DQK>
__device__ __forceinline__ void long_tile(const uint16_t* ks, const uint16_t* vs, const uint16_t* qs, int kt, int qi,
                                          int window, float sl2, int w, int g, int r, float& m, float& lp,
                                          f32x4 (&yacc)[4]) {
    float s[4][4];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x4 st = score_tile<DQK>(ks, 16 * j, qs, 16 * w, g, r);
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
            const int key = kt * kQT + 16 * j + 4 * g + mm;
            const bool ok = key <= qi && key > qi - window;
            s[j][mm] = ok ? st[mm] * sl2 : -INFINITY;
            mt = fmaxf(mt, s[j][mm]);
        }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m, mt);
    // no key of this query seen yet: keep every weight at 0 without NaN
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float corr = __builtin_amdgcn_exp2f(m - mu);  // m = -inf: 0
    m = mn;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
            s[j][mm] = __builtin_amdgcn_exp2f(s[j][mm] - mu);
            acc += s[j][mm];
        }
    lp = lp * corr + acc;
    // rows of yacc are the queries 4g + mm: their scale factors
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
        const float c = __shfl(corr, 4 * g + mm, 64);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) yacc[ct][mm] *= c;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        float a[8];
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
            a[mm] = s[2 * p][mm];
            a[4 + mm] = s[2 * p + 1][mm];
        }
        bf16x8 ahi, alo;
        pack8_hilo(a, ahi, alo);
        bf16x8 vb[4];
        v_kstep<true>(vs, 32 * p + 4 * g, vs, 32 * p + 16 + 4 * g, r, vb);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) yacc[ct] = mfma32(ahi, vb[ct], yacc[ct]);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) yacc[ct] = mfma32(alo, vb[ct], yacc[ct]);
    }
}

template <int DQK, bool ADD, int NCS>
__global__ __launch_bounds__(256) void swa_long_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, int L, int ntiles, int window,
                                                       float scale, const float* add, float* y) {
    constexpr int ldv = kDV * NCS;
    __shared__ alignas(16) uint16_t k0[kQT * DQK], k1[kQT * DQK];
    __shared__ alignas(16) uint16_t v0[kQT * kDV], v1[kQT * kDV];
    __shared__ alignas(16) uint16_t qs[kQT * DQK];

    int bid = blockIdx.x;
    const int total = gridDim.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int col0 = (bid % NCS) * kDV;
    bid /= NCS;
    const int head = bid / ntiles;
    const int qt = ntiles - 1 - bid % ntiles;  // the longest key ranges first
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const uint16_t* qh = q + (size_t)head * L * DQK;
    const uint16_t* kh = k + (size_t)head * L * DQK;
    const uint16_t* vh = v + (size_t)head * L * ldv + col0;
    const int head_bytes = (L * ldv - col0) * 4;
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(y + (size_t)head * L * ldv + col0, (short)0, head_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        ADD ? (void*)(add + (size_t)head * L * ldv + col0) : (void*)y, (short)0, ADD ? head_bytes : 0, 0x00020000);
    const float sl2 = scale * kLog2e;
    const int q0 = qt * kQT + 16 * w;  // first query of the wave
    const int qi = q0 + r;             // this lane's query
    const int kt_lo = max(0, qt * kQT - window + 1) / kQT;

    // prologue: Q of the tile, K/V of the first key tile into slot 0
    if constexpr (DQK == 64) {
        dma_block<64>(qh, 64, L, qt * kQT, qs, 2 * w, lane);
        dma_block<64>(qh, 64, L, qt * kQT, qs, 2 * w + 1, lane);
    } else {
        if (w >= 2) dma_block<16>(qh, 16, L, qt * kQT, qs, w - 2, lane);
    }
    dma_kv<DQK>(kh, vh, ldv, L, kt_lo, k0, v0, w, lane);
    float adda[16];
    if (ADD) load_add(ra, q0, g, r, ldv, adda);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    raw_barrier();

    f32x4 yacc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) yacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lp = 0.f;
    // Key tiles in pairs, so that each slot is a fixed array in each half.
    for (int kt = kt_lo; kt <= qt; kt += 2) {
        if (kt + 1 <= qt) dma_kv<DQK>(kh, vh, ldv, L, kt + 1, k1, v1, w, lane);
        long_tile<DQK>(k0, v0, qs, kt, qi, window, sl2, w, g, r, m, lp, yacc);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        raw_barrier();
        if (kt + 1 > qt) break;
        if (kt + 2 <= qt) dma_kv<DQK>(kh, vh, ldv, L, kt + 2, k0, v0, w, lane);
        long_tile<DQK>(k1, v1, qs, kt + 1, qi, window, sl2, w, g, r, m, lp, yacc);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        raw_barrier();
    }
    float l = lp;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
        const float inv = __builtin_amdgcn_rcpf(__shfl(l, 4 * g + mm, 64));  // l >= 1: the max key has p = 1
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const float o = yacc[ct][mm] * inv + (ADD ? adda[4 * mm + ct] : 0.f);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o), ry,
                                                  out_off(q0 + 4 * g + mm, 16 * ct + r, ldv), 0, kNT);
        }
    }
}

template <int DQK, bool ADD, int NCS>
void launch_ncs(int halo, bool long_window, dim3 grid, dim3 lgrid, hipStream_t st, const uint16_t* q,
                const uint16_t* k, const uint16_t* v, int L, int ntiles, int tpw, int wg_per_head, int window,
                float scale, const float* add, float* y) {
    if (long_window)
        hipLaunchKernelGGL((swa_long_kernel<DQK, ADD, NCS>), lgrid, dim3(256), 0, st, q, k, v, L, ntiles, window, scale,
                           add, y);
    else if (halo == 1)
        hipLaunchKernelGGL((swa_mfma_kernel<DQK, ADD, 1, NCS>), grid, dim3(256), 0, st, q, k, v, L, ntiles, tpw,
                           wg_per_head, window, scale, add, y);
    else
        hipLaunchKernelGGL((swa_mfma_kernel<DQK, ADD, 2, NCS>), grid, dim3(256), 0, st, q, k, v, L, ntiles, tpw,
                           wg_per_head, window, scale, add, y);
}

template <int DQK, bool ADD>
void launch_dqk(int ncs, int halo, bool long_window, dim3 grid, dim3 lgrid, hipStream_t st, const uint16_t* q,
                const uint16_t* k, const uint16_t* v, int L, int ntiles, int tpw, int wg_per_head, int window,
                float scale, const float* add, float* y) {
    if (ncs == 1)
        launch_ncs<DQK, ADD, 1>(halo, long_window, grid, lgrid, st, q, k, v, L, ntiles, tpw, wg_per_head, window,
                                scale, add, y);
    else
        launch_ncs<DQK, ADD, 2>(halo, long_window, grid, lgrid, st, q, k, v, L, ntiles, tpw, wg_per_head, window,
                                scale, add, y);
}

}  // namespace

hipError_t launch_swa_mfma(const void* q, const void* k, const void* v, int BH, int L, int dqk, int dv, int window,
                           float scale, const float* add, float* y, hipStream_t st) {
    const int ntiles = (L + kQT - 1) / kQT;
    const int ncs = dv / kDV;  // 64-column slices: each recomputes the scores of its tiles
    // Tiles per workgroup: long runs amortise the halo and the pipeline
    // fill; keep about two workgroups per compute unit.
    const int tpw = max(1, min(16, (BH * ncs * ntiles + 511) / 512));
    const int wg_per_head = (ntiles + tpw - 1) / tpw;
    const dim3 grid(BH * wg_per_head * ncs);
    const dim3 lgrid(BH * ntiles * ncs);
    const int halo = window > kQT ? 2 : 1;    // key tiles of 64 before the query tile
    const bool long_window = window > 2 * kQT;  // the online-softmax kernel over 64-key tiles
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* vv = static_cast<const uint16_t*>(v);
    if (dqk == 16) {
        if (add) launch_dqk<16, true>(ncs, halo, long_window, grid, lgrid, st, qq, kk, vv, L, ntiles, tpw, wg_per_head, window, scale, add, y);
        else launch_dqk<16, false>(ncs, halo, long_window, grid, lgrid, st, qq, kk, vv, L, ntiles, tpw, wg_per_head, window, scale, add, y);
    } else {
        if (add) launch_dqk<64, true>(ncs, halo, long_window, grid, lgrid, st, qq, kk, vv, L, ntiles, tpw, wg_per_head, window, scale, add, y);
        else launch_dqk<64, false>(ncs, halo, long_window, grid, lgrid, st, qq, kk, vv, L, ntiles, tpw, wg_per_head, window, scale, add, y);
    }
    return hipGetLastError();
}

}  // namespace based

// swa_decode.hip -- next-token step of the causal sliding window and the fill
// of its key/value ring cache (gfx950).
//
// "Simple linear attention language models balance the recall-throughput
// tradeoff", s4 "Local Exact Attention" (each query sees the preceding w
// keys, its own included, through a w-sized key/value cache) and App. B
// "Next Token Prediction" (the window's next-token kernel).
//
// Cache layout: per (batch, head) a ring of `window` slots, [B,H,window,d];
// the token at position p lives in slot p mod window.
//
// Decode step: HBM-bound (each cached key and value is read once per step).
// Windows up to 128: one wave per (batch, head), four per workgroup, no
// workgroup barrier (wider windows: swa_decode_long_kernel below).
// Lane j scores slot j (and j + 64 for windows over 64) from its key row
// (16-byte loads; bf16 rows through packed bf16 dot products with fp32
// sums); for P.V, lane
// (key group kg, column group cg) accumulates 8 columns over the keys kg,
// kg + KG, ... and the key groups are summed with lane shuffles.  Key and
// value loads are all issued before any arithmetic, so a wave waits for
// memory once.  The new token's key and value are taken from the inputs (and
// written to their slot).
// Loads do not wait for the position: every slot of the ring is loaded at
// once and slots that do not hold one of the last `window` tokens are then
// replaced by zeros or -inf through selects.
#include "common.hpp"
#include "kernels.hpp"

namespace based {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// 8 consecutive elements of a row: 16 bytes of bf16 or 32 of fp32, kept in
// their loaded form until used.
template <typename T>
struct Chunk8;
template <>
struct Chunk8<uint16_t> {
    u32x4 u;
    __device__ __forceinline__ void load(const uint16_t* p) { u = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<u32x4*>(p) = u; }
    __device__ __forceinline__ void zero() { u = u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ float get(int i) const {
        return (i & 1) ? bf16hi_f32(u[i >> 1]) : bf16lo_f32(u[i >> 1]);
    }
    // acc[i] += the two products of pair i (v_dot2_f32_bf16: bf16 products,
    // fp32 sum), with no widening of either operand.  Each element is copied
    // to a scalar before the bit cast: a bit cast of a vector element
    // expression reads the vector's first element instead.
    __device__ __forceinline__ void dot_into(const Chunk8& o, float (&acc)[4]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a = u[i], b = o.u[i];
            acc[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc[i],
                                                     false);
        }
    }
};
template <>
struct Chunk8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const f32x4*>(p);
        b = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ void store(float* p) const {
        *reinterpret_cast<f32x4*>(p) = a;
        *reinterpret_cast<f32x4*>(p + 4) = b;
    }
    __device__ __forceinline__ void zero() { a = b = f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ float get(int i) const { return i < 4 ? a[i] : b[i - 4]; }
    __device__ __forceinline__ void dot_into(const Chunk8& o, float (&acc)[4]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(b[i], o.b[i], fmaf(a[i], o.a[i], acc[i]));
    }
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

// Copies n 16-byte units from src to dst, one unit per lane.
__device__ __forceinline__ void copy_units(const void* src, void* dst, int n, int lane) {
    if (lane < n) reinterpret_cast<u32x4*>(dst)[lane] = reinterpret_cast<const u32x4*>(src)[lane];
}

template <typename T, int DQK, int DV, int R>
__global__ __launch_bounds__(256) void swa_decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                         const T* __restrict__ v,
                                                         const long long* __restrict__ pos, int H, int BH,
                                                         int window, float scale, T* __restrict__ kc,
                                                         T* __restrict__ vc, const float* add,
                                                         float* __restrict__ y) {
    // R rounds of 64 slots: window <= 64 R.  Lane `lane` scores slots
    // lane + 64 r; P.V lane (kg, cg) covers keys kg + KG i, i < KPL.
    constexpr int kQC = DQK / 8;               // chunks of 8 in a key row
    constexpr int kCG = DV / 8;                // column groups of 8
    constexpr int kKG = 64 / kCG;              // key groups in P.V
    constexpr int kKPL = 64 * R / kKG;         // keys per lane in P.V
    constexpr int kKU = DQK * sizeof(T) / 16;  // 16-byte units of a key row
    constexpr int kVU = DV * sizeof(T) / 16;   // and of a value row
    const int lane = threadIdx.x & 63;
    const int head = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (head >= BH) return;
    const int cg = lane % kCG, kg = lane / kCG;
    float* yh = y + (size_t)head * DV;
    const T* kn = k + (size_t)head * DQK;
    const T* vn = v + (size_t)head * DV;
    T* kch = kc + (size_t)head * window * DQK;
    T* vch = vc + (size_t)head * window * DV;

    // ---- loads, all issued before the position is known: the query, the
    // new key and value, the keys of this lane's slots and its value chunks
    // of every slot (the slot addresses do not depend on the position).
    const long long p = pos[head / H];
    Chunk8<T> qr[kQC], kr[R][kQC], knr[kQC], vr[kKPL], vnr;
#pragma unroll
    for (int c = 0; c < kQC; ++c) {
        qr[c].load(q + (size_t)head * DQK + 8 * c);
        knr[c].load(kn + 8 * c);
#pragma unroll
        for (int r = 0; r < R; ++r)  // slots past the ring: a row of it, discarded below
            kr[r][c].load(kch + (size_t)min(lane + 64 * r, window - 1) * DQK + 8 * c);
    }
    vnr.load(vn + 8 * cg);
#pragma unroll
    for (int i = 0; i < kKPL; ++i) vr[i].load(vch + (size_t)min(kg + kKG * i, window - 1) * DV + 8 * cg);
    float ad[8];
    if (add) {  // every key group loads it (the same 32 bytes); key group 0 uses it
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(add + (size_t)head * DV + 8 * cg);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(add + (size_t)head * DV + 8 * cg + 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            ad[c] = a0[c];
            ad[4 + c] = a1[c];
        }
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) ad[c] = 0.f;
    }
    if (p < 0) {  // no valid position: NaN outputs, cache untouched
        if (kg == 0) {
#pragma unroll
            for (int c = 0; c < 8; ++c) yh[8 * cg + c] = __builtin_nanf("");
        }
        return;
    }
    // Slots 0..nvalid-1 hold the last tokens; the new one goes to slot_new.
    // Data of other slots was loaded but is replaced by selects (never
    // multiplied), so whatever they hold cannot reach the result.
    const int slot_new = (int)(p % window);
    const int nvalid = p + 1 < window ? (int)p + 1 : window;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < kQC; ++c)
            if (lane + 64 * r == slot_new) kr[r][c] = knr[c];

    // ---- scores and softmax over the valid slots (fp32, base 2); they need
    // only the keys, so they run while the value rows are still arriving
    float s[R];
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kQC; ++c) qr[c].dot_into(kr[r][c], part);
        const float dot = (part[0] + part[1]) + (part[2] + part[3]);
        s[r] = lane + 64 * r < nvalid ? dot * (scale * kLog2e) : -INFINITY;
        m = fmaxf(m, s[r]);
    }
    m = wave_max(m);
    float pe[R], l = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        pe[r] = lane + 64 * r < nvalid ? __builtin_amdgcn_exp2f(s[r] - m) : 0.f;
        l += pe[r];
    }
    l = wave_sum(l);

    // ---- P.V: this lane's keys, then the sum over key groups
#pragma unroll
    for (int i = 0; i < kKPL; ++i) {
        const int j = kg + kKG * i;
        if (j == slot_new) vr[i] = vnr;
        else if (j >= nvalid) vr[i].zero();
    }
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
    for (int i = 0; i < kKPL; ++i) {
        const int j = kg + kKG * i;  // slot j's weight is on lane j % 64, round j / 64
        float pj = __shfl(pe[0], j & 63, 64);
        if constexpr (R == 2) {
            const float pj1 = __shfl(pe[R - 1], j & 63, 64);
            pj = j >= 64 ? pj1 : pj;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(pj, vr[i].get(c), acc[c]);
    }
#pragma unroll
    for (int off = kCG; off < 64; off <<= 1)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += __shfl_xor(acc[c], off, 64);
    if (kg == 0) {
        const float inv = 1.f / l;  // l >= 1: the maximum key has weight 1
        f32x4 o0, o1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            o0[c] = fmaf(acc[c], inv, ad[c]);
            o1[c] = fmaf(acc[4 + c], inv, ad[4 + c]);
        }
        *reinterpret_cast<f32x4*>(yh + 8 * cg) = o0;
        *reinterpret_cast<f32x4*>(yh + 8 * cg + 4) = o1;
    }

    // ---- the new token into its slot (no lane of this step reads that slot)
    copy_units(kn, kch + (size_t)slot_new * DQK, kKU, lane);
    copy_units(vn, vch + (size_t)slot_new * DV, kVU, lane);
}

// d_qk = 64 and windows up to 64 R slots: one workgroup of four waves per
// (batch, head), wave w taking the 16 R slots [16 R w, 16 R (w + 1)) of the
// ring, so each wave loads a quarter of the rows and more waves share a SIMD
// (the one-wave form above leaves each wave a long chain of dependent steps
// with few waves to hide it).  Scores: lane (s, p) takes slot s of the
// wave's block and the 8-dim pieces p, p + P, ... of its key row (P = 64 /
// (16 R) lanes per slot, so one load instruction of the P lanes of a slot
// reads 16 P contiguous bytes), the parts added across lanes.  P.V: lane (kg, cg) takes 8 columns
// of the keys kg, kg + KG, ... of the block.  Each wave's (max, sum, P.V)
// goes to LDS and one wave merges the four after a barrier; slots beyond
// the valid ones weigh zero through selects, as above.
template <typename T, int DV, int R>
__global__ __launch_bounds__(256) void swa_decode_split_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                               const T* __restrict__ v,
                                                               const long long* __restrict__ pos, int H,
                                                               int window, float scale, T* __restrict__ kc,
                                                               T* __restrict__ vc, const float* add,
                                                               float* __restrict__ y) {
    constexpr int DQK = 64;
    constexpr int kSPW = 16 * R;             // slots per wave
    constexpr int kP = 64 / kSPW;            // lanes per slot in the scores
    constexpr int kDPL = DQK / kP;           // dims per lane in the scores
    constexpr int kQC = kDPL / 8;            // chunks of 8 dims per lane
    constexpr int kCG = DV / 8, kKG = 64 / kCG, kKPL = kSPW / kKG;
    __shared__ float part_acc[4][DV];
    __shared__ float part_ml[4][2];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t head = blockIdx.x;
    const int sl = lane / kP, pp = lane % kP;
    const int cg = lane % kCG, kg = lane / kCG;
    const int base = kSPW * w;  // first slot of this wave's block
    float* yh = y + head * DV;
    const T* kn = k + head * DQK;
    const T* vn = v + head * DV;
    T* kch = kc + head * (size_t)window * DQK;
    T* vch = vc + head * (size_t)window * DV;

    // ---- loads, all issued before the position is known (slots past the
    // ring read its last row and are discarded below)
    const long long p = pos[blockIdx.x / (unsigned)H];  // 32-bit division: the grid is B * H < 2^31
    const int j = base + sl;  // this lane's slot in the scores
    Chunk8<T> qr[kQC], kr[kQC], knr[kQC], vr[kKPL], vnr;
#pragma unroll
    for (int c = 0; c < kQC; ++c) {
        qr[c].load(q + head * DQK + 8 * (pp + kP * c));
        knr[c].load(kn + 8 * (pp + kP * c));
        kr[c].load(kch + (size_t)min(j, window - 1) * DQK + 8 * (pp + kP * c));
    }
    vnr.load(vn + 8 * cg);
#pragma unroll
    for (int i = 0; i < kKPL; ++i) vr[i].load(vch + (size_t)min(base + kg + kKG * i, window - 1) * DV + 8 * cg);
    // the fused-add input of the lanes that write y, in flight with the rest
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
    if (add && w == 0 && kg == 0) {
        a0 = *reinterpret_cast<const f32x4*>(add + head * DV + 8 * cg);
        a1 = *reinterpret_cast<const f32x4*>(add + head * DV + 8 * cg + 4);
    }
    if (p < 0) {  // no valid position: NaN outputs, cache untouched
        if (w == 0 && kg == 0) {
#pragma unroll
            for (int c = 0; c < 8; ++c) yh[8 * cg + c] = __builtin_nanf("");
        }
        return;
    }
    const int slot_new = (int)(p % window);
    const int nvalid = p + 1 < window ? (int)p + 1 : window;
    if (j == slot_new) {
#pragma unroll
        for (int c = 0; c < kQC; ++c) kr[c] = knr[c];
    }

    // ---- scores and this wave's softmax statistics (a wave whose block
    // holds no valid slot ends with m = -inf, l = 0, P.V = 0)
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kQC; ++c) qr[c].dot_into(kr[c], part);
    float dot = (part[0] + part[1]) + (part[2] + part[3]);
#pragma unroll
    for (int off = 1; off < kP; off <<= 1) dot += __shfl_xor(dot, off, 64);
    const bool valid = j < nvalid;
    const float sc = valid ? dot * (scale * kLog2e) : -INFINITY;
    const float m = wave_max(sc);
    const float pe = valid ? __builtin_amdgcn_exp2f(sc - m) : 0.f;
    const float l = wave_sum(pp == 0 ? pe : 0.f);

    // ---- P.V over the block, then the sum over key groups
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
    for (int i = 0; i < kKPL; ++i) {
        const int jj = base + kg + kKG * i;
        if (jj == slot_new) vr[i] = vnr;
        else if (jj >= nvalid) vr[i].zero();
        const float pj = __shfl(pe, (kg + kKG * i) * kP, 64);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(pj, vr[i].get(c), acc[c]);
    }
#pragma unroll
    for (int off = kCG; off < 64; off <<= 1)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += __shfl_xor(acc[c], off, 64);
    if (kg == 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) part_acc[w][8 * cg + c] = acc[c];
    }
    if (lane == 0) {
        part_ml[w][0] = m;
        part_ml[w][1] = l;
    }
    __syncthreads();
    if (w == 0 && kg == 0) {
        // wave 0's block holds slot 0, which is always valid: mx is finite
        float mx = part_ml[0][0];
#pragma unroll
        for (int u = 1; u < 4; ++u) mx = fmaxf(mx, part_ml[u][0]);
        float den = 0.f, o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float e = __builtin_amdgcn_exp2f(part_ml[u][0] - mx);
            den = fmaf(e, part_ml[u][1], den);
#pragma unroll
            for (int c = 0; c < 8; ++c) o[c] = fmaf(e, part_acc[u][8 * cg + c], o[c]);
        }
        const float inv = 1.f / den;  // den >= 1: the maximum key has weight 1
        f32x4 o0, o1;  // a0, a1 are zero without add
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            o0[c] = fmaf(o[c], inv, a0[c]);
            o1[c] = fmaf(o[4 + c], inv, a1[c]);
        }
        *reinterpret_cast<f32x4*>(yh + 8 * cg) = o0;
        *reinterpret_cast<f32x4*>(yh + 8 * cg + 4) = o1;
    }
    // the new token into its slot, from the registers every wave loaded it
    // into (lanes s = 0 hold the key's pieces, lanes kg = 0 the value's), so
    // the last step of the workgroup waits on no load
    if (w == 1) {
        if (sl == 0) {
#pragma unroll
            for (int c = 0; c < kQC; ++c) knr[c].store(kch + (size_t)slot_new * DQK + 8 * (pp + kP * c));
        }
        if (kg == 0) vnr.store(vch + (size_t)slot_new * DV + 8 * cg);
    }
}

// Windows over 128 slots: one workgroup of four waves per (batch, head).
// The valid slots are taken in rounds of 64 (lane j scores slot 64 n + j of
// round n), wave w taking rounds w, w + 4, ...; each wave keeps an online
// softmax (running maximum m, sum l and the unnormalised P.V of its 8
// columns per lane, rescaled by exp2(m_old - m_new) when the maximum
// grows), and the four are merged through LDS after one barrier.  Slot
// loads do not depend on the position, as above; the new token's slot is
// written after the barrier, when every wave's loads have been consumed.
template <typename T, int DQK, int DV>
__global__ __launch_bounds__(256) void swa_decode_long_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                              const T* __restrict__ v,
                                                              const long long* __restrict__ pos, int H,
                                                              int window, float scale, T* __restrict__ kc,
                                                              T* __restrict__ vc, const float* add,
                                                              float* __restrict__ y) {
    constexpr int kQC = DQK / 8, kCG = DV / 8, kKG = 64 / kCG, kKPL = 64 / kKG;
    constexpr int kKU = DQK * sizeof(T) / 16, kVU = DV * sizeof(T) / 16;
    __shared__ float part_acc[4][DV];
    __shared__ float part_ml[4][2];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t head = blockIdx.x;
    const int cg = lane % kCG, kg = lane / kCG;
    float* yh = y + head * DV;
    const T* kn = k + head * DQK;
    const T* vn = v + head * DV;
    T* kch = kc + head * (size_t)window * DQK;
    T* vch = vc + head * (size_t)window * DV;
    const long long p = pos[head / H];
    if (p < 0) {  // no valid position: NaN outputs, cache untouched
        if (w == 0 && kg == 0) {
#pragma unroll
            for (int c = 0; c < 8; ++c) yh[8 * cg + c] = __builtin_nanf("");
        }
        return;
    }
    const int slot_new = (int)(p % window);
    const int nvalid = p + 1 < window ? (int)p + 1 : window;
    const int nround = (nvalid + 63) / 64;
    Chunk8<T> qr[kQC], knr[kQC], vnr;
#pragma unroll
    for (int c = 0; c < kQC; ++c) {
        qr[c].load(q + head * DQK + 8 * c);
        knr[c].load(kn + 8 * c);
    }
    vnr.load(vn + 8 * cg);
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;  // fused-add input of the lanes that write y
    if (add && w == 0 && kg == 0) {
        a0 = *reinterpret_cast<const f32x4*>(add + head * DV + 8 * cg);
        a1 = *reinterpret_cast<const f32x4*>(add + head * DV + 8 * cg + 4);
    }
    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
    for (int n = w; n < nround; n += 4) {
        const int j = 64 * n + lane;  // this lane's slot for the scores
        Chunk8<T> kr[kQC], vr[kKPL];
#pragma unroll
        for (int c = 0; c < kQC; ++c) kr[c].load(kch + (size_t)min(j, window - 1) * DQK + 8 * c);
#pragma unroll
        for (int i = 0; i < kKPL; ++i) vr[i].load(vch + (size_t)min(64 * n + kg + kKG * i, window - 1) * DV + 8 * cg);
        if (j == slot_new) {
#pragma unroll
            for (int c = 0; c < kQC; ++c) kr[c] = knr[c];
        }
        float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kQC; ++c) qr[c].dot_into(kr[c], part);
        const float dot = (part[0] + part[1]) + (part[2] + part[3]);
        const float sc = j < nvalid ? dot * (scale * kLog2e) : -INFINITY;
        const float mn = fmaxf(m, wave_max(sc));  // finite: slot 64 n is valid
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        const float pe = j < nvalid ? __builtin_amdgcn_exp2f(sc - mn) : 0.f;
        l = l * alpha + wave_sum(pe);
        m = mn;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] *= alpha;
#pragma unroll
        for (int i = 0; i < kKPL; ++i) {
            const int jj = 64 * n + kg + kKG * i;
            if (jj == slot_new) vr[i] = vnr;
            else if (jj >= nvalid) vr[i].zero();
            const float pj = __shfl(pe, kg + kKG * i, 64);
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = fmaf(pj, vr[i].get(c), acc[c]);
        }
    }
#pragma unroll
    for (int off = kCG; off < 64; off <<= 1)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += __shfl_xor(acc[c], off, 64);
    if (kg == 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) part_acc[w][8 * cg + c] = acc[c];
    }
    if (lane == 0) {
        part_ml[w][0] = m;
        part_ml[w][1] = l;
    }
    __syncthreads();
    if (w == 0 && kg == 0) {
        // waves without a round hold m = -inf, l = 0 and weigh exp2(-inf) = 0
        float mx = part_ml[0][0];
#pragma unroll
        for (int u = 1; u < 4; ++u) mx = fmaxf(mx, part_ml[u][0]);
        float den = 0.f, o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float e = __builtin_amdgcn_exp2f(part_ml[u][0] - mx);
            den = fmaf(e, part_ml[u][1], den);
#pragma unroll
            for (int c = 0; c < 8; ++c) o[c] = fmaf(e, part_acc[u][8 * cg + c], o[c]);
        }
        const float inv = 1.f / den;  // den >= 1: the maximum key has weight 1
        f32x4 o0, o1;  // a0, a1 are zero without add
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            o0[c] = fmaf(o[c], inv, a0[c]);
            o1[c] = fmaf(o[4 + c], inv, a1[c]);
        }
        *reinterpret_cast<f32x4*>(yh + 8 * cg) = o0;
        *reinterpret_cast<f32x4*>(yh + 8 * cg + 4) = o1;
    }
    if (w == 1) {
        copy_units(kn, kch + (size_t)slot_new * DQK, kKU, lane);
        copy_units(vn, vch + (size_t)slot_new * DV, kVU, lane);
    }
}

// The slots of the last min(L, window) tokens of a prefix, one workgroup per
// (batch, head).
template <typename T, int DQK, int DV>
__global__ __launch_bounds__(256) void swa_cache_fill_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                             int L, int window, T* __restrict__ kc,
                                                             T* __restrict__ vc) {
    constexpr int kKU = DQK * sizeof(T) / 16, kVU = DV * sizeof(T) / 16;
    const size_t head = blockIdx.x;
    const int n = L < window ? L : window, p0 = L - n;
    for (int e = threadIdx.x; e < n * (kKU + kVU); e += 256) {
        const int r = e / (kKU + kVU), u = e % (kKU + kVU);
        const int p = p0 + r, slot = p % window;
        if (u < kKU) {
            const u32x4* src = reinterpret_cast<const u32x4*>(k + (head * L + p) * DQK);
            reinterpret_cast<u32x4*>(kc + (head * window + slot) * DQK)[u] = src[u];
        } else {
            const u32x4* src = reinterpret_cast<const u32x4*>(v + (head * L + p) * DV);
            reinterpret_cast<u32x4*>(vc + (head * window + slot) * DV)[u - kKU] = src[u - kKU];
        }
    }
}

template <typename T, int DQK>
hipError_t decode_dv(const void* q, const void* k, const void* v, const long long* pos, int H, int BH, int dv,
                     int window, float scale, void* kc, void* vc, const float* add, float* y, hipStream_t st) {
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    T* kcc = static_cast<T*>(kc);
    T* vcc = static_cast<T*>(vc);
    // a workgroup per (batch, head), or (the wave form) four heads per workgroup
#define BASED_SWA_DEC(KERNEL, GRID) \
    hipLaunchKernelGGL((KERNEL), dim3(GRID), dim3(256), 0, st, qq, kk, vv, pos, H, window, scale, kcc, vcc, add, y)
#define BASED_SWA_DEC_WAVE(KERNEL) \
    hipLaunchKernelGGL((KERNEL), dim3((BH + 3) / 4), dim3(256), 0, st, qq, kk, vv, pos, H, BH, window, scale, kcc, \
                       vcc, add, y)
    if (window > 128) {
        if (dv == 64) BASED_SWA_DEC((swa_decode_long_kernel<T, DQK, 64>), BH);
        else BASED_SWA_DEC((swa_decode_long_kernel<T, DQK, 128>), BH);
    } else if constexpr (DQK == 64) {
        if (window <= 64) {
            if (dv == 64) BASED_SWA_DEC((swa_decode_split_kernel<T, 64, 1>), BH);
            else BASED_SWA_DEC((swa_decode_split_kernel<T, 128, 1>), BH);
        } else {
            if (dv == 64) BASED_SWA_DEC((swa_decode_split_kernel<T, 64, 2>), BH);
            else BASED_SWA_DEC((swa_decode_split_kernel<T, 128, 2>), BH);
        }
    } else {
        if (window <= 64) {
            if (dv == 64) BASED_SWA_DEC_WAVE((swa_decode_kernel<T, DQK, 64, 1>));
            else BASED_SWA_DEC_WAVE((swa_decode_kernel<T, DQK, 128, 1>));
        } else {
            if (dv == 64) BASED_SWA_DEC_WAVE((swa_decode_kernel<T, DQK, 64, 2>));
            else BASED_SWA_DEC_WAVE((swa_decode_kernel<T, DQK, 128, 2>));
        }
    }
#undef BASED_SWA_DEC
#undef BASED_SWA_DEC_WAVE
    return hipGetLastError();
}

template <typename T, int DQK>
hipError_t fill_dv(const void* k, const void* v, int BH, int L, int dv, int window, void* kc, void* vc,
                   hipStream_t st) {
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    T* kcc = static_cast<T*>(kc);
    T* vcc = static_cast<T*>(vc);
    if (dv == 64)
        hipLaunchKernelGGL((swa_cache_fill_kernel<T, DQK, 64>), dim3(BH), dim3(256), 0, st, kk, vv, L, window, kcc,
                           vcc);
    else
        hipLaunchKernelGGL((swa_cache_fill_kernel<T, DQK, 128>), dim3(BH), dim3(256), 0, st, kk, vv, L, window, kcc,
                           vcc);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_swa_decode_step(const void* q, const void* k, const void* v, bool bf16, const long long* pos,
                                  int H, int BH, int dqk, int dv, int window, float scale, void* kc, void* vc,
                                  const float* add, float* y, hipStream_t st) {
    if (bf16)
        return dqk == 16 ? decode_dv<uint16_t, 16>(q, k, v, pos, H, BH, dv, window, scale, kc, vc, add, y, st)
                         : decode_dv<uint16_t, 64>(q, k, v, pos, H, BH, dv, window, scale, kc, vc, add, y, st);
    return dqk == 16 ? decode_dv<float, 16>(q, k, v, pos, H, BH, dv, window, scale, kc, vc, add, y, st)
                     : decode_dv<float, 64>(q, k, v, pos, H, BH, dv, window, scale, kc, vc, add, y, st);
}

hipError_t launch_swa_cache_fill(const void* k, const void* v, bool bf16, int BH, int L, int dqk, int dv,
                                 int window, void* kc, void* vc, hipStream_t st) {
    if (bf16)
        return dqk == 16 ? fill_dv<uint16_t, 16>(k, v, BH, L, dv, window, kc, vc, st)
                         : fill_dv<uint16_t, 64>(k, v, BH, L, dv, window, kc, vc, st);
    return dqk == 16 ? fill_dv<float, 16>(k, v, BH, L, dv, window, kc, vc, st)
                     : fill_dv<float, 64>(k, v, BH, L, dv, window, kc, vc, st);
}

}  // namespace based

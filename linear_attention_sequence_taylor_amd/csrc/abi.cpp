// abi.cpp -- the C ABI of libbased.so (declared in include/based.h).
//
// Responsibilities: validate every argument before anything is launched
// (so a rejected call touches no memory), choose the kernel for the dtype
// and shape, launch it on the caller's stream, and map the HIP launch status
// to based_status_t.  No allocation, no synchronisation, no global state.
#include "based.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.hpp"

#define BASED_API extern "C" __attribute__((visibility("default")))

namespace {

// The feature dims every path supports.  The bf16 matrix-core prefill is
// built for 16 (its 16-row rotation tiles); other dims, and fp32 inputs, run
// in fp32 on the fp32 matrix cores (chunk 64) or the vector ALUs (chunks 16
// and 32).
constexpr int kDFeatMfma = 16;
bool feat_dim_ok(int d) { return d == 8 || d == 16 || d == 24 || d == 32; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Product of non-negative factors with overflow detection (false = overflow).
bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) {
    if (a != 0 && b > UINT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// Byte ranges [p, p + n) overlap?
bool overlaps(const void* p, uint64_t n, const void* q, uint64_t m) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + m && b < a + n;
}

size_t elem_size(based_dtype_t t) { return t == BASED_BF16 ? 2 : 4; }

based_status_t launch_status(hipError_t e) { return e == hipSuccess ? BASED_OK : BASED_E_LAUNCH; }

// Common shape checks; fills element counts.  Returns BASED_OK or an error.
based_status_t check_dims(int B, int H, int L, uint64_t* BH, uint64_t* BHL) {
    // L stays 1023 below INT32_MAX so that chunk and tile counts rounded up
    // in int arithmetic (L + 63) / 64 cannot overflow.
    if (B < 1 || H < 1 || L < 1 || L > INT32_MAX - 1023) return BASED_E_INVALID;
    // B*H <= 2^27 keeps every grid (at most 16 workgroups per head outside
    // the segment splits, which only run for few heads) inside 2^31.
    if (!mul_ok((uint64_t)B, (uint64_t)H, BH) || *BH > ((uint64_t)1 << 27)) return BASED_E_INVALID;
    if (!mul_ok(*BH, (uint64_t)L, BHL) || *BHL > ((uint64_t)1 << 40)) return BASED_E_INVALID;
    return BASED_OK;
}

}  // namespace

BASED_API int based_num_features(int d_feat) {
    if (d_feat < 1 || d_feat > 46340) return -1;
    return 1 + d_feat + d_feat * d_feat;
}

BASED_API const char* based_status_string(based_status_t s) {
    switch (s) {
        case BASED_OK: return "BASED_OK";
        case BASED_E_INVALID: return "BASED_E_INVALID: malformed argument (null/misaligned pointer, bad size, overlap)";
        case BASED_E_UNSUPPORTED: return "BASED_E_UNSUPPORTED: shape, dtype or chunk not implemented";
        case BASED_E_LAUNCH: return "BASED_E_LAUNCH: HIP kernel launch failed";
        case BASED_E_TOO_LARGE:
            return "BASED_E_TOO_LARGE: the call needs more scratch than the static buffer of based_prefill_noalloc "
                   "holds (BASED_PREFILL_NOALLOC_SCRATCH_BYTES); use based_prefill with a workspace";
    }
    return "BASED_E_UNKNOWN";
}

BASED_API size_t based_prefill_workspace_bytes(int B, int H, int L, int d_feat, int d_v) {
    uint64_t BH, BHL;
    if (check_dims(B, H, L, &BH, &BHL) != BASED_OK) return 0;
    if (!feat_dim_ok(d_feat) || (d_v != 64 && d_v != 128)) return 0;
    // the fp32 matrix-core path (fp32 inputs, or any d_feat != 16) and, for
    // d_feat = 16, the bf16 matrix-core plan: enough for whichever runs
    const size_t f32 = based::prefill_f32mfma_workspace_bytes((int)BH, L, d_feat, d_v);
    if (d_feat != kDFeatMfma) return f32;
    const size_t bf = based::prefill_mfma_workspace_bytes((int)BH, L, d_v);
    return bf > f32 ? bf : f32;
}

BASED_API based_status_t based_prefill(const void* q, const void* k, const void* v,
                                       based_dtype_t dtype, int B, int H, int L, int d_feat,
                                       int d_v, int chunk, float eps, float* y, float* S, float* z,
                                       int use_initial_state, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_E_INVALID;
    if (!q || !k || !v || !y || !S || !z) return BASED_E_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) || !aligned16(S) ||
        !aligned16(z))
        return BASED_E_INVALID;
    if (!isfinite(eps) || chunk < 1 || d_feat < 1 || d_v < 1) return BASED_E_INVALID;
    uint64_t BH, BHL;
    if (check_dims(B, H, L, &BH, &BHL) != BASED_OK) return BASED_E_INVALID;
    if (!feat_dim_ok(d_feat)) return BASED_E_UNSUPPORTED;
    if (d_v != 64 && d_v != 128) return BASED_E_UNSUPPORTED;
    const bool bf16 = dtype == BASED_BF16;
    const bool mfma = bf16 && d_feat == kDFeatMfma;
    if (chunk != 64 && (mfma || (chunk != 16 && chunk != 32))) return BASED_E_UNSUPPORTED;

    const uint64_t es = elem_size(dtype);
    const uint64_t F = (uint64_t)based_num_features(d_feat);
    const uint64_t qk_bytes = BHL * d_feat * es, v_bytes = BHL * d_v * es;
    const uint64_t y_bytes = BHL * d_v * 4, S_bytes = BH * F * d_v * 4, z_bytes = BH * F * 4;
    if (overlaps(y, y_bytes, q, qk_bytes) || overlaps(y, y_bytes, k, qk_bytes) ||
        overlaps(y, y_bytes, v, v_bytes) || overlaps(y, y_bytes, S, S_bytes) ||
        overlaps(y, y_bytes, z, z_bytes) || overlaps(S, S_bytes, z, z_bytes) ||
        overlaps(S, S_bytes, q, qk_bytes) || overlaps(S, S_bytes, k, qk_bytes) ||
        overlaps(S, S_bytes, v, v_bytes) || overlaps(z, z_bytes, q, qk_bytes) ||
        overlaps(z, z_bytes, k, qk_bytes) || overlaps(z, z_bytes, v, v_bytes))
        return BASED_E_INVALID;
    if (workspace && !aligned16(workspace)) return BASED_E_INVALID;
    // the part of the workspace a launch plan may use must not overlap
    // anything else
    if (workspace && workspace_bytes) {
        const uint64_t need = based_prefill_workspace_bytes(B, H, L, d_feat, d_v);
        const uint64_t used = need < workspace_bytes ? need : workspace_bytes;
        const void* other[6] = {y, S, z, q, k, v};
        const uint64_t other_bytes[6] = {y_bytes, S_bytes, z_bytes, qk_bytes, qk_bytes, v_bytes};
        for (int i = 0; i < 6; ++i)
            if (used && overlaps(workspace, used, other[i], other_bytes[i])) return BASED_E_INVALID;
    }

    hipStream_t st = static_cast<hipStream_t>(stream);
    const int init = use_initial_state ? 1 : 0;
    if (mfma)
        return launch_status(based::launch_prefill_mfma(q, k, v, (int)BH, L, d_v, eps, y, S, z, init,
                                                        workspace, workspace_bytes, st));
    // fp32 inputs or d_feat != 16: fp32 arithmetic throughout; chunk 64 on
    // the fp32 matrix cores, chunks 16 and 32 on the vector ALUs
    if (chunk == 64)
        return launch_status(
            based::launch_prefill_f32mfma(q, k, v, bf16, (int)BH, L, d_feat, d_v, eps, y, S, z, init, workspace,
                                          workspace_bytes, st));
    return launch_status(
        based::launch_prefill_valu(q, k, v, bf16, (int)BH, L, d_feat, d_v, chunk, eps, y, S, z, init, st));
}

BASED_API based_status_t based_decode_step(const void* q, const void* k, const void* v,
                                           based_dtype_t dtype, int B, int H, int d_feat, int d_v,
                                           float eps, float* S, float* z, float* y, void* stream) {
    if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_E_INVALID;
    if (!q || !k || !v || !y || !S || !z) return BASED_E_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) || !aligned16(S) ||
        !aligned16(z))
        return BASED_E_INVALID;
    if (!isfinite(eps) || d_feat < 1 || d_v < 1) return BASED_E_INVALID;
    uint64_t BH, BHL;
    if (check_dims(B, H, 1, &BH, &BHL) != BASED_OK) return BASED_E_INVALID;
    if (!feat_dim_ok(d_feat)) return BASED_E_UNSUPPORTED;
    if (d_v != 64 && d_v != 128) return BASED_E_UNSUPPORTED;
    const uint64_t F = (uint64_t)based_num_features(d_feat);
    const uint64_t S_bytes = BH * F * d_v * 4, z_bytes = BH * F * 4, y_bytes = BH * d_v * 4;
    if (overlaps(y, y_bytes, S, S_bytes) || overlaps(y, y_bytes, z, z_bytes) ||
        overlaps(S, S_bytes, z, z_bytes))
        return BASED_E_INVALID;
    return launch_status(based::launch_decode_step(q, k, v, dtype == BASED_BF16, (int)BH, d_feat, d_v, eps,
                                                   S, z, y, static_cast<hipStream_t>(stream)));
}

BASED_API based_status_t swa_forward(const void* q, const void* k, const void* v,
                                     based_dtype_t dtype, int B, int H, int L, int d_qk, int d_v,
                                     int window, float scale, const float* add, float* y,
                                     void* stream) {
    if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_E_INVALID;
    if (!q || !k || !v || !y) return BASED_E_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) ||
        (add && !aligned16(add)))
        return BASED_E_INVALID;
    if (!isfinite(scale) || window < 1 || d_qk < 1 || d_v < 1) return BASED_E_INVALID;
    uint64_t BH, BHL;
    if (check_dims(B, H, L, &BH, &BHL) != BASED_OK) return BASED_E_INVALID;
    if (d_qk != 16 && d_qk != 64) return BASED_E_UNSUPPORTED;
    if (d_v != 64 && d_v != 128) return BASED_E_UNSUPPORTED;
    const uint64_t es = elem_size(dtype);
    const uint64_t qk_bytes = BHL * d_qk * es, v_bytes = BHL * d_v * es, y_bytes = BHL * d_v * 4;
    if (overlaps(y, y_bytes, q, qk_bytes) || overlaps(y, y_bytes, k, qk_bytes) ||
        overlaps(y, y_bytes, v, v_bytes))
        return BASED_E_INVALID;
    if (add && add != y && overlaps(add, y_bytes, y, y_bytes)) return BASED_E_INVALID;
    const uint64_t tiles = ((uint64_t)L + 63) / 64;
    if (BH * tiles * (d_v / 64) > (uint64_t)INT32_MAX / 2) return BASED_E_INVALID;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // The matrix-core kernels address a head's fp32 rows with 32-bit byte
    // offsets (L * d_v * 4 bytes); longer heads take the fp32 kernels.
    const bool bf16 = dtype == BASED_BF16;
    if (bf16 && (uint64_t)L * d_v * 4 <= (uint64_t)INT32_MAX)
        return launch_status(
            based::launch_swa_mfma(q, k, v, (int)BH, L, d_qk, d_v, window, scale, add, y, st));
    return launch_status(
        based::launch_swa_valu(q, k, v, bf16, (int)BH, L, d_qk, d_v, window, scale, add, y, st));
}

BASED_API size_t based_hybrid_prefill_workspace_bytes(int B, int H, int L, int d_feat, int d_v) {
    uint64_t BH, BHL;
    if (check_dims(B, H, L, &BH, &BHL) != BASED_OK) return 0;
    if (!feat_dim_ok(d_feat) || (d_v != 64 && d_v != 128)) return 0;
    // the linear branch run alone (based_prefill's need) or the fused pass
    const size_t a = based_prefill_workspace_bytes(B, H, L, d_feat, d_v);
    const size_t b = d_feat == kDFeatMfma ? based::hybrid_mfma_workspace_bytes((int)BH, L, d_v) : 0;
    return a > b ? a : b;
}

BASED_API based_status_t based_hybrid_prefill(const void* q, const void* k, const void* q_win, const void* k_win,
                                              const void* v, based_dtype_t dtype, int B, int H, int L, int d_feat,
                                              int d_qk, int d_v, int chunk, float eps, int window, float scale,
                                              int path, float* y, float* S, float* z, int use_initial_state,
                                              void* workspace, size_t workspace_bytes, void* stream) {
    if (path != BASED_HYBRID_AUTO && path != BASED_HYBRID_FUSED && path != BASED_HYBRID_TWO_PASS)
        return BASED_E_INVALID;
    if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_E_INVALID;
    if (!q || !k || !q_win || !k_win || !v || !y || !S || !z) return BASED_E_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(q_win) || !aligned16(k_win) || !aligned16(v) ||
        !aligned16(y) || !aligned16(S) || !aligned16(z) || (workspace && !aligned16(workspace)))
        return BASED_E_INVALID;
    if (!isfinite(eps) || !isfinite(scale) || chunk < 1 || d_feat < 1 || d_qk < 1 || d_v < 1 || window < 1)
        return BASED_E_INVALID;
    uint64_t BH, BHL;
    if (check_dims(B, H, L, &BH, &BHL) != BASED_OK) return BASED_E_INVALID;
    if (!feat_dim_ok(d_feat) || (d_v != 64 && d_v != 128) || (d_qk != 16 && d_qk != 64))
        return BASED_E_UNSUPPORTED;
    const bool bf16 = dtype == BASED_BF16;
    const bool mfma = bf16 && d_feat == kDFeatMfma;
    if (chunk != 64 && (mfma || (chunk != 16 && chunk != 32))) return BASED_E_UNSUPPORTED;
    const uint64_t es = elem_size(dtype);
    const uint64_t F = (uint64_t)based_num_features(d_feat);
    const void* ins[5] = {q, k, q_win, k_win, v};
    const uint64_t in_bytes[5] = {BHL * d_feat * es, BHL * d_feat * es, BHL * d_qk * es, BHL * d_qk * es,
                                  BHL * d_v * es};
    const void* outs[3] = {y, S, z};
    const uint64_t out_bytes[3] = {BHL * d_v * 4, BH * F * d_v * 4, BH * F * 4};
    for (int a = 0; a < 3; ++a) {
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return BASED_E_INVALID;
        for (int b = 0; b < 5; ++b)
            if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b])) return BASED_E_INVALID;
    }
    if (BH * (((uint64_t)L + 63) / 64) * (d_v / 64) > (uint64_t)INT32_MAX / 2) return BASED_E_INVALID;
    if (workspace && workspace_bytes) {  // the part a plan may use overlaps nothing else
        const uint64_t need = based_hybrid_prefill_workspace_bytes(B, H, L, d_feat, d_v);
        const uint64_t used = need < workspace_bytes ? need : workspace_bytes;
        for (int a = 0; a < 3; ++a)
            if (used && overlaps(workspace, used, outs[a], out_bytes[a])) return BASED_E_INVALID;
        for (int b = 0; b < 5; ++b)
            if (used && overlaps(workspace, used, ins[b], in_bytes[b])) return BASED_E_INVALID;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    // The fused pass where it exists and is chosen; otherwise the two
    // branches in turn (the window adds into y in place).
    const bool fusable = mfma && d_qk == 64 && window <= 64;
    if (path == BASED_HYBRID_FUSED && !fusable) return BASED_E_UNSUPPORTED;
    if (path != BASED_HYBRID_TWO_PASS && fusable) {
        bool launched = false;
        const hipError_t e = based::launch_hybrid_mfma(q, k, q_win, k_win, v, (int)BH, L, d_v, eps, window, scale, y,
                                                       S, z, use_initial_state ? 1 : 0, workspace, workspace_bytes,
                                                       st, &launched);
        if (launched) return launch_status(e);
        if (path == BASED_HYBRID_FUSED) return BASED_E_UNSUPPORTED;
    }
    const based_status_t s = based_prefill(q, k, v, dtype, B, H, L, d_feat, d_v, chunk, eps, y, S, z,
                                           use_initial_state, workspace, workspace_bytes, stream);
    if (s != BASED_OK) return s;
    return swa_forward(q_win, k_win, v, dtype, B, H, L, d_qk, d_v, window, scale, y, y, stream);
}

namespace {

// Shared checks of the window cache entry points.
based_status_t check_window_cache(based_dtype_t dtype, int d_qk, int d_v, int window) {
    if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_E_INVALID;
    if (window < 1 || d_qk < 1 || d_v < 1) return BASED_E_INVALID;
    if (d_qk != 16 && d_qk != 64) return BASED_E_UNSUPPORTED;
    if (d_v != 64 && d_v != 128) return BASED_E_UNSUPPORTED;
    return BASED_OK;
}

}  // namespace

BASED_API based_status_t swa_cache_fill(const void* k, const void* v, based_dtype_t dtype, int B, int H, int L,
                                        int d_qk, int d_v, int window, void* k_cache, void* v_cache,
                                        void* stream) {
    if (!k || !v || !k_cache || !v_cache) return BASED_E_INVALID;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return BASED_E_INVALID;
    const based_status_t c = check_window_cache(dtype, d_qk, d_v, window);
    if (c != BASED_OK) return c;
    uint64_t BH, BHL;
    if (check_dims(B, H, L, &BH, &BHL) != BASED_OK) return BASED_E_INVALID;
    const uint64_t es = elem_size(dtype);
    const uint64_t kc_bytes = BH * window * d_qk * es, vc_bytes = BH * window * d_v * es;
    const uint64_t k_bytes = BHL * d_qk * es, v_bytes = BHL * d_v * es;
    if (overlaps(k_cache, kc_bytes, v_cache, vc_bytes) || overlaps(k_cache, kc_bytes, k, k_bytes) ||
        overlaps(k_cache, kc_bytes, v, v_bytes) || overlaps(v_cache, vc_bytes, k, k_bytes) ||
        overlaps(v_cache, vc_bytes, v, v_bytes))
        return BASED_E_INVALID;
    return launch_status(based::launch_swa_cache_fill(k, v, dtype == BASED_BF16, (int)BH, L, d_qk, d_v, window,
                                                      k_cache, v_cache, static_cast<hipStream_t>(stream)));
}

BASED_API based_status_t swa_decode_step(const void* q, const void* k, const void* v, based_dtype_t dtype, int B,
                                         int H, int d_qk, int d_v, int window, float scale, const long long* pos,
                                         void* k_cache, void* v_cache, const float* add, float* y,
                                         void* stream) {
    if (!q || !k || !v || !pos || !k_cache || !v_cache || !y) return BASED_E_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(y) || (add && !aligned16(add)) || (reinterpret_cast<uintptr_t>(pos) & 7u) != 0)
        return BASED_E_INVALID;
    if (!isfinite(scale)) return BASED_E_INVALID;
    const based_status_t c = check_window_cache(dtype, d_qk, d_v, window);
    if (c != BASED_OK) return c;
    uint64_t BH, BHL;
    if (check_dims(B, H, 1, &BH, &BHL) != BASED_OK) return BASED_E_INVALID;
    const uint64_t es = elem_size(dtype);
    const uint64_t kc_bytes = BH * window * d_qk * es, vc_bytes = BH * window * d_v * es;
    const uint64_t qk_bytes = BH * d_qk * es, v_bytes = BH * d_v * es, y_bytes = BH * d_v * 4;
    const uint64_t pos_bytes = (uint64_t)B * 8;
    const void* outs[3] = {k_cache, v_cache, y};
    const uint64_t out_bytes[3] = {kc_bytes, vc_bytes, y_bytes};
    const void* ins[4] = {q, k, v, pos};
    const uint64_t in_bytes[4] = {qk_bytes, qk_bytes, v_bytes, pos_bytes};
    for (int a = 0; a < 3; ++a) {
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return BASED_E_INVALID;
        for (int b = 0; b < 4; ++b)
            if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b])) return BASED_E_INVALID;
    }
    if (add && add != y && overlaps(add, y_bytes, y, y_bytes)) return BASED_E_INVALID;
    return launch_status(based::launch_swa_decode_step(q, k, v, dtype == BASED_BF16, pos, H, (int)BH, d_qk, d_v,
                                                       window, scale, k_cache, v_cache, add, y,
                                                       static_cast<hipStream_t>(stream)));
}

BASED_API size_t based_prefill_backward_workspace_bytes(int B, int H, int L, int d_feat, int d_v) {
    uint64_t BH, BHL;
    if (check_dims(B, H, L, &BH, &BHL) != BASED_OK) return 0;
    if (!feat_dim_ok(d_feat) || (d_v != 64 && d_v != 128)) return 0;
    const size_t direct = based::prefill_backward_workspace_bytes((int)BH, L, d_v);
    if (d_feat == 16) {
        const size_t chunked = based::prefill_backward_chunked_workspace_bytes((int)BH, L);
        return chunked > direct ? chunked : direct;
    }
    return direct;
}

// The automatic choice takes the chunked form from this length on (where it
// is the faster one).
static const int kBackwardChunkedMinL = 1024;

BASED_API based_status_t based_prefill_backward(const void* q, const void* k, const void* v, const float* dy,
                                                based_dtype_t dtype, int B, int H, int L, int d_feat, int d_v,
                                                float eps, int form, float* dq, float* dk, float* dv,
                                                void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_E_INVALID;
    if (form != BASED_BACKWARD_AUTO && form != BASED_BACKWARD_DIRECT && form != BASED_BACKWARD_CHUNKED)
        return BASED_E_INVALID;
    if (!q || !k || !v || !dy || !dq || !dk || !dv || !workspace) return BASED_E_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dy) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv) || !aligned16(workspace))
        return BASED_E_INVALID;
    if (!isfinite(eps) || d_feat < 1 || d_v < 1) return BASED_E_INVALID;
    uint64_t BH, BHL;
    if (check_dims(B, H, L, &BH, &BHL) != BASED_OK) return BASED_E_INVALID;
    if (!feat_dim_ok(d_feat) || (d_v != 64 && d_v != 128)) return BASED_E_UNSUPPORTED;
    // one workgroup of 256 threads per 64 rows of a head: the grid's thread
    // count must fit 32 bits
    if (BH * (((uint64_t)L + 63) / 64) * 256 > (uint64_t)INT32_MAX) return BASED_E_INVALID;
    const bool chunk_ok = dtype == BASED_BF16 && d_feat == 16;
    if (form == BASED_BACKWARD_CHUNKED && !chunk_ok) return BASED_E_UNSUPPORTED;
    const bool chunked = form == BASED_BACKWARD_CHUNKED || (form == BASED_BACKWARD_AUTO && chunk_ok &&
                                                            L >= kBackwardChunkedMinL);
    const uint64_t ws_need = chunked ? based::prefill_backward_chunked_workspace_bytes((int)BH, L)
                                     : based::prefill_backward_workspace_bytes((int)BH, L, d_v);
    if (workspace_bytes < ws_need) return BASED_E_INVALID;
    const uint64_t es = elem_size(dtype);
    const uint64_t qk_bytes = BHL * d_feat * es, v_bytes = BHL * d_v * es;
    const uint64_t dqk_bytes = BHL * d_feat * 4, dv_bytes = BHL * d_v * 4;
    const void* outs[4] = {dq, dk, dv, workspace};
    const uint64_t out_bytes[4] = {dqk_bytes, dqk_bytes, dv_bytes, ws_need};
    const void* ins[4] = {q, k, v, dy};
    const uint64_t in_bytes[4] = {qk_bytes, qk_bytes, v_bytes, dv_bytes};
    for (int a = 0; a < 4; ++a) {
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return BASED_E_INVALID;
        for (int b = 0; b < 4; ++b)
            if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b])) return BASED_E_INVALID;
    }
    if (chunked)
        return launch_status(based::launch_prefill_backward_chunked(q, k, v, dy, (int)BH, L, d_v, eps, dq, dk, dv,
                                                                    workspace, static_cast<hipStream_t>(stream)));
    return launch_status(based::launch_prefill_backward(q, k, v, dy, dtype == BASED_BF16, (int)BH, L, d_feat, d_v,
                                                        eps, dq, dk, dv, workspace,
                                                        static_cast<hipStream_t>(stream)));
}

BASED_API size_t based_swa_backward_workspace_bytes(int B, int H, int L) {
    uint64_t BH, BHL;
    if (check_dims(B, H, L, &BH, &BHL) != BASED_OK) return 0;
    return based::swa_backward_workspace_bytes((int)BH, L);
}

BASED_API based_status_t based_swa_backward(const void* q, const void* k, const void* v, const float* dy,
                                            based_dtype_t dtype, int B, int H, int L, int d_qk, int d_v,
                                            int window, float scale, float* dq, float* dk, float* dv,
                                            void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_E_INVALID;
    if (!q || !k || !v || !dy || !dq || !dk || !dv || !workspace) return BASED_E_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dy) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv) || !aligned16(workspace))
        return BASED_E_INVALID;
    if (!isfinite(scale) || window < 1 || d_qk < 1 || d_v < 1) return BASED_E_INVALID;
    uint64_t BH, BHL;
    if (check_dims(B, H, L, &BH, &BHL) != BASED_OK) return BASED_E_INVALID;
    if (dtype != BASED_BF16 || d_qk != 64 || (d_v != 64 && d_v != 128) || window > 64) return BASED_E_UNSUPPORTED;
    if (BH * (((uint64_t)L + 63) / 64) * 256 > (uint64_t)INT32_MAX) return BASED_E_INVALID;
    const uint64_t ws_need = based::swa_backward_workspace_bytes((int)BH, L);
    if (workspace_bytes < ws_need) return BASED_E_INVALID;
    const uint64_t qk_bytes = BHL * d_qk * 2, v_bytes = BHL * d_v * 2;
    const uint64_t dqk_bytes = BHL * d_qk * 4, dv_bytes = BHL * d_v * 4;
    const void* outs[4] = {dq, dk, dv, workspace};
    const uint64_t out_bytes[4] = {dqk_bytes, dqk_bytes, dv_bytes, ws_need};
    const void* ins[4] = {q, k, v, dy};
    const uint64_t in_bytes[4] = {qk_bytes, qk_bytes, v_bytes, dv_bytes};
    for (int a = 0; a < 4; ++a) {
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return BASED_E_INVALID;
        for (int b = 0; b < 4; ++b)
            if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b])) return BASED_E_INVALID;
    }
    return launch_status(based::launch_swa_backward(q, k, v, dy, (int)BH, L, d_v, window, scale, dq, dk, dv,
                                                    workspace, static_cast<hipStream_t>(stream)));
}

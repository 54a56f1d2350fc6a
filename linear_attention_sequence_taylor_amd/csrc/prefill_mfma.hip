// prefill_mfma.hip -- launch plans of the chunked prefill and of the fused
// hybrid layer on the gfx950 matrix cores (the kernels and their design
// are in prefill_mfma_kernels.hpp).  Two kernel instances are compiled
// in prefill_mfma_ilp.hip under another instruction scheduler and
// launched through launch_prefill_ilp_instance; the others here.

#include "prefill_mfma_kernels.hpp"
#include "kernels.hpp"

namespace based {
namespace {

// Inclusive prefix over segment slots, per head: slot s <- slot s-1 + slot s.
// After it, slot s holds the state entering segment s.  Each thread owns one
// 16-byte element of a slot and walks the segments eight at a time, all
// eight loads issued before the adds and stores.
__global__ __launch_bounds__(256) void segment_scan_kernel(float* __restrict__ ws, int nseg, int BH,
                                                           size_t slot_floats) {
    const size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const int head = blockIdx.y;
    if (e >= slot_floats) return;
    f32x4* p = reinterpret_cast<f32x4*>(ws + (size_t)head * slot_floats + e);
    const size_t stride = (size_t)BH * slot_floats / 4;  // in f32x4
    f32x4 run = p[0];
    for (int s0 = 1; s0 < nseg; s0 += 8) {
        f32x4 x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = s0 + i < nseg ? p[(size_t)(s0 + i) * stride] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            run += x[i];
            if (s0 + i < nseg) p[(size_t)(s0 + i) * stride] = run;
        }
    }
}

// Launch shape.  Value columns are split into groups of `dvl` (each group
// carries its own copy of the normaliser tile and recomputes the features),
// and long sequences into segments, until there are enough workgroups for
// one per compute unit (the LDS footprint allows one resident workgroup per
// CU).  Segments cost an extra state pass; 32-wide groups cost a second
// copy of all feature work.  So: 32-wide groups when they fill the chip
// without segments; otherwise, if the sequence is long enough for segments
// alone to fill it, 64-wide groups plus segments; otherwise 32-wide groups
// plus as many segments as the length allows.
constexpr int kTargetWorkgroups = 256;
struct PrefillPlan {
    int dvl, ncg, nseg;
};
PrefillPlan plan_prefill(int BH, int L, int dv, bool use_init, bool have_ws) {
    PrefillPlan pl;
    const int nchunks = (L + kC - 1) / kC;
    const int max_seg = nchunks / 2;  // segments of at least two chunks
    const int units32 = BH * (dv / 32), units64 = BH * (dv / 64);
    pl.dvl = (dv == 128 && BH * 4 > 1024) ? 64 : 32;
    if (units32 < kTargetWorkgroups && have_ws && max_seg * units64 >= kTargetWorkgroups) pl.dvl = 64;
    pl.ncg = dv / pl.dvl;
    const int units = BH * pl.ncg;
    pl.nseg = 1;
    if (units < kTargetWorkgroups && nchunks >= 4)
        pl.nseg = max(1, min((kTargetWorkgroups + units - 1) / units, max_seg));
    // With an initial state and several column groups, the carried state
    // goes through the workspace (no group may overwrite z while another
    // still reads it).  Without a workspace: one 64-wide group for d_v = 64;
    // d_v = 128 with an initial state has no MFMA plan (dvl = 0).
    const bool need_ws = pl.nseg > 1 || (use_init && pl.ncg > 1);
    if (need_ws && !have_ws) {
        pl.nseg = 1;
        if (use_init) {
            pl.dvl = dv == 64 ? 64 : 0;
            pl.ncg = 1;
        }
    }
    return pl;
}

template <int DVL>
size_t workspace_bytes_dvl(int BH, int ncg, int nseg) {
    return (size_t)nseg * BH * ncg * ws_slot_floats<DVL>() * sizeof(float);
}

size_t plan_workspace_bytes(const PrefillPlan& pl, int BH) {
    return pl.dvl == 32 ? workspace_bytes_dvl<32>(BH, pl.ncg, pl.nseg) : workspace_bytes_dvl<64>(BH, pl.ncg, pl.nseg);
}

template <int DVL>
hipError_t launch_plan(const PrefillPlan& pl, const uint16_t* q, const uint16_t* k, const uint16_t* v, int BH,
                       int L, int dv, float eps, float* y, float* S, float* z, int use_init, void* ws,
                       hipStream_t st) {
    const bool via_ws = pl.nseg > 1 || (use_init && pl.ncg > 1);
    if (!via_ws) {
        if constexpr (DVL == 32) {
            return launch_prefill_ilp_instance(DVL, kModeFull, dim3(BH * pl.ncg), st, q, k, v, L, dv, pl.ncg, L, 1,
                                               eps, y, S, z, use_init, nullptr);
        } else {
            hipLaunchKernelGGL((prefill_mfma_kernel<DVL, kModeFull>), dim3(BH * pl.ncg), dim3(768), 0, st, q, k, v, L,
                               dv, pl.ncg, L, 1, eps, y, S, z, use_init, nullptr, nullptr, nullptr, 0, 0.f);
            return hipGetLastError();
        }
    }
    const int nchunks = (L + kC - 1) / kC;
    const int seg_len = ((nchunks + pl.nseg - 1) / pl.nseg) * kC;
    const int nseg = (L + seg_len - 1) / seg_len;
    float* wsf = static_cast<float*>(ws);
    const dim3 grid(BH * pl.ncg * nseg);
    hipLaunchKernelGGL((segment_state_kernel<DVL>), grid, dim3(64 * kStateWaves), 0, st, k, v, L, dv, pl.ncg, seg_len,
                       nseg, S, z, use_init, wsf);
    // (one segment: the slot already holds the initial state; with several,
    // B*H*ncg is below the workgroup target, well inside the grid's y range)
    const size_t slot = ws_slot_floats<DVL>();
    if (nseg > 1)
        hipLaunchKernelGGL(segment_scan_kernel, dim3((unsigned)((slot / 4 + 255) / 256), BH * pl.ncg), dim3(256), 0,
                           st, wsf, nseg, BH * pl.ncg, slot);
    if constexpr (DVL == 64) {
        return launch_prefill_ilp_instance(DVL, kModeSegment, grid, st, q, k, v, L, dv, pl.ncg, seg_len, nseg, eps, y,
                                           S, z, use_init, wsf);
    } else {
        hipLaunchKernelGGL((prefill_mfma_kernel<DVL, kModeSegment>), grid, dim3(768), 0, st, q, k, v, L, dv, pl.ncg,
                           seg_len, nseg, eps, y, S, z, use_init, wsf, nullptr, nullptr, 0, 0.f);
        return hipGetLastError();
    }
}

}  // namespace

size_t prefill_mfma_workspace_bytes(int BH, int L, int dv) {
    // Enough for any plan this shape can take (an initial state may need it).
    const PrefillPlan pl = plan_prefill(BH, L, dv, true, true);
    const bool via_ws = pl.nseg > 1 || pl.ncg > 1;
    return via_ws ? plan_workspace_bytes(pl, BH) : 0;
}

size_t prefill_mfma_plan_bytes(int BH, int L, int dv, int use_init) {
    const PrefillPlan pl = plan_prefill(BH, L, dv, use_init != 0, true);
    const bool via_ws = pl.nseg > 1 || (use_init && pl.ncg > 1);
    return via_ws ? plan_workspace_bytes(pl, BH) : 0;
}

hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, int BH, int L, int dv,
                               float eps, float* y, float* S, float* z, int use_init, void* ws,
                               size_t ws_bytes, hipStream_t st) {
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* vv = static_cast<const uint16_t*>(v);
    PrefillPlan pl = plan_prefill(BH, L, dv, use_init != 0, ws != nullptr);
    const bool via_ws = pl.nseg > 1 || (use_init && pl.ncg > 1);
    if (via_ws && ws_bytes < plan_workspace_bytes(pl, BH)) pl = plan_prefill(BH, L, dv, use_init != 0, false);
    switch (pl.dvl) {
        case 32: return launch_plan<32>(pl, qq, kk, vv, BH, L, dv, eps, y, S, z, use_init, ws, st);
        case 64: return launch_plan<64>(pl, qq, kk, vv, BH, L, dv, eps, y, S, z, use_init, ws, st);
        default:  // no workspace for a carried d_v = 128 state: the fp32 chunked kernel
            return launch_prefill_f32mfma(q, k, v, true, BH, L, kDFeat, dv, eps, y, S, z, use_init, nullptr, 0, st);
    }
}

// ---- fused hybrid layer: 32-column groups (the window waves' LDS fits
// next to that plan).  Long sequences with few heads split into segments as
// the plain prefill would at 64 columns: a 64-column state pass and scan
// (cheaper than two 32-column ones), then the fused 32-column segment pass
// (two workgroups per head and segment) reads its columns of each slot.
static PrefillPlan plan_hybrid(int BH, int L, int dv, bool use_init, bool have_ws) {
    PrefillPlan pl;
    const int nchunks = (L + kC - 1) / kC;
    pl.dvl = kWinCols;
    pl.ncg = dv / kWinCols;
    pl.nseg = 1;
    if (BH * pl.ncg < kTargetWorkgroups && nchunks >= 4)
        pl.nseg = max(1, min((kTargetWorkgroups + BH - 1) / BH, nchunks / 2));
    const bool need_ws = pl.nseg > 1 || (use_init && pl.ncg > 1);
    if (need_ws && !have_ws) {
        pl.nseg = 1;
        if (use_init && pl.ncg > 1) pl.dvl = 0;  // no plan: the caller runs the two branches in turn
    }
    return pl;
}

static size_t hybrid_ws_bytes(const PrefillPlan& pl, int BH, int dv) {
    return (size_t)pl.nseg * BH * (dv / 64) * ws_slot_floats<64>() * sizeof(float);
}

size_t hybrid_mfma_workspace_bytes(int BH, int L, int dv) {
    const PrefillPlan pl = plan_hybrid(BH, L, dv, true, true);
    const bool via_ws = pl.nseg > 1 || pl.ncg > 1;
    return via_ws ? hybrid_ws_bytes(pl, BH, dv) : 0;
}

static hipError_t launch_hybrid_plan(const PrefillPlan& pl, const uint16_t* q, const uint16_t* k,
                                     const uint16_t* v, int BH, int L, int dv, float eps, float* y, float* S,
                                     float* z, int use_init, void* ws, hipStream_t st, const uint16_t* q2,
                                     const uint16_t* k2, int window, float win_scale) {
    const bool via_ws = pl.nseg > 1 || (use_init && pl.ncg > 1);
    if (!via_ws) {
        hipLaunchKernelGGL((prefill_mfma_kernel<kWinCols, kModeFull, true>), dim3(BH * pl.ncg), dim3(1024), 0, st, q,
                           k, v, L, dv, pl.ncg, L, 1, eps, y, S, z, use_init, nullptr, q2, k2, window, win_scale);
        return hipGetLastError();
    }
    const int nchunks = (L + kC - 1) / kC;
    const int seg_len = ((nchunks + pl.nseg - 1) / pl.nseg) * kC;
    const int nseg = (L + seg_len - 1) / seg_len;
    float* wsf = static_cast<float*>(ws);
    // state pass and scan at 64 columns (one group per 64 value columns)
    const int ncg64 = dv / 64;
    hipLaunchKernelGGL((segment_state_kernel<64>), dim3(BH * ncg64 * nseg), dim3(64 * kStateWaves), 0, st, k, v, L,
                       dv, ncg64, seg_len, nseg, S, z, use_init, wsf);
    const size_t slot = ws_slot_floats<64>();
    if (nseg > 1)
        hipLaunchKernelGGL(segment_scan_kernel, dim3((unsigned)((slot / 4 + 255) / 256), BH * ncg64), dim3(256), 0, st,
                           wsf, nseg, BH * ncg64, slot);
    hipLaunchKernelGGL((prefill_mfma_kernel<kWinCols, kModeSegment, true>), dim3(BH * pl.ncg * nseg), dim3(1024), 0,
                       st, q, k, v, L, dv, pl.ncg, seg_len, nseg, eps, y, S, z, use_init, wsf, q2, k2, window,
                       win_scale);
    return hipGetLastError();
}

hipError_t launch_hybrid_mfma(const void* q, const void* k, const void* q2, const void* k2, const void* v, int BH,
                              int L, int dv, float eps, int window, float scale, float* y, float* S, float* z,
                              int use_init, void* ws, size_t ws_bytes, hipStream_t st, bool* launched) {
    PrefillPlan pl = plan_hybrid(BH, L, dv, use_init != 0, ws != nullptr);
    const bool via_ws = pl.nseg > 1 || (use_init && pl.ncg > 1);
    if (via_ws && ws_bytes < hybrid_ws_bytes(pl, BH, dv)) pl = plan_hybrid(BH, L, dv, use_init != 0, false);
    *launched = pl.dvl == kWinCols && (dv == 64 || dv == 128);
    if (!*launched) return hipSuccess;
    return launch_hybrid_plan(pl, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                              static_cast<const uint16_t*>(v), BH, L, dv, eps, y, S, z, use_init, ws, st,
                              static_cast<const uint16_t*>(q2), static_cast<const uint16_t*>(k2), window, scale);
}

}  // namespace based

// prefill_mfma_ilp.hip -- the prefill kernel instances that run faster
// under the compiler's instruction-level-parallelism scheduler (this unit
// is built with -mllvm -amdgpu-sched-strategy=iterative-ilp):
// prefill_mfma_kernel<32, kModeFull> (32-column groups over whole
// sequences) and <64, kModeSegment> (the segment pass of 64-column
// groups).  Measured on MI355X, both ran 5-7% shorter than under the
// default scheduler, with bit-identical results.  The other instances
// (the 64-column whole-sequence kernel, the fused hybrid layer) spill
// registers under that scheduler and stay in prefill_mfma.hip.
#include "prefill_mfma_kernels.hpp"

namespace based {

hipError_t launch_prefill_ilp_instance(int dvl, int mode, dim3 grid, hipStream_t st, const uint16_t* q,
                                       const uint16_t* k, const uint16_t* v, int L, int ldv, int ncg, int seg_len,
                                       int nseg, float eps, float* y, float* S, float* z, int use_init, float* ws) {
    if (dvl == 32 && mode == kModeFull)
        hipLaunchKernelGGL((prefill_mfma_kernel<32, kModeFull>), grid, dim3(768), 0, st, q, k, v, L, ldv, ncg, seg_len,
                           nseg, eps, y, S, z, use_init, ws, nullptr, nullptr, 0, 0.f);
    else if (dvl == 64 && mode == kModeSegment)
        hipLaunchKernelGGL((prefill_mfma_kernel<64, kModeSegment>), grid, dim3(768), 0, st, q, k, v, L, ldv, ncg,
                           seg_len, nseg, eps, y, S, z, use_init, ws, nullptr, nullptr, 0, 0.f);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace based

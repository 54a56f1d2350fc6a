// prefill_mfma.hip -- placeholder while the MFMA kernel is written: forwards
// to the vector-ALU path.
#include "common.hpp"
#include "kernels.hpp"
namespace based {
size_t prefill_mfma_workspace_bytes(int, int, int) { return 0; }
hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, int BH, int L, int dv,
                               float eps, float* y, float* S, float* z, int use_init, void*, size_t,
                               hipStream_t st) {
    return launch_prefill_valu(q, k, v, true, BH, L, dv, 64, eps, y, S, z, use_init, st);
}
}  // namespace based

// swa_mfma.hip -- placeholder while the MFMA kernel is written.
#include "common.hpp"
#include "kernels.hpp"
namespace based {
hipError_t launch_swa_mfma(const void* q, const void* k, const void* v, int BH, int L, int dqk,
                           int window, float scale, const float* add, float* y, hipStream_t st) {
    return launch_swa_valu(q, k, v, true, BH, L, dqk, window, scale, add, y, st);
}
}  // namespace based

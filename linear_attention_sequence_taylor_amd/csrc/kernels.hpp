// kernels.hpp -- host-side launchers of the gfx950 kernels.  Every launcher
// enqueues on `st` and returns the launch status (hipGetLastError); shapes
// and pointers are validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace based {

// Fused next-token step (decode.hip).  dv in {64, 128}.
hipError_t launch_decode_step(const void* q, const void* k, const void* v, bool bf16, int BH,
                              int dv, float eps, float* S, float* z, float* y, hipStream_t st);

// fp32 vector-ALU chunked prefill (prefill_valu.hip).  chunk in {16,32,64}.
hipError_t launch_prefill_valu(const void* q, const void* k, const void* v, bool bf16, int BH, int L,
                               int dv, int chunk, float eps, float* y, float* S, float* z,
                               int use_init, hipStream_t st);

// bf16 MFMA chunked prefill (prefill_mfma.hip), chunk 64.  `seg_len` > 0
// splits each head into segments of seg_len tokens (a multiple of 64); the
// workspace then holds one carried state per segment.
size_t prefill_mfma_workspace_bytes(int BH, int L, int dv);
hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, int BH, int L, int dv,
                               float eps, float* y, float* S, float* z, int use_init,
                               void* workspace, size_t workspace_bytes, hipStream_t st);

// fp32 vector-ALU sliding-window softmax (swa_valu.hip).  dqk in {16, 64}.
hipError_t launch_swa_valu(const void* q, const void* k, const void* v, bool bf16, int BH, int L,
                           int dqk, int window, float scale, const float* add, float* y,
                           hipStream_t st);

// bf16 MFMA sliding-window softmax (swa_mfma.hip).  dqk in {16, 64}.
hipError_t launch_swa_mfma(const void* q, const void* k, const void* v, int BH, int L, int dqk,
                           int window, float scale, const float* add, float* y, hipStream_t st);

}  // namespace based

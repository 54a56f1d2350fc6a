// kernels.hpp -- host-side launchers of the gfx950 kernels.  Every launcher
// enqueues on `st` and returns the launch status (hipGetLastError); shapes
// and pointers are validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace based {

// Fused next-token step (decode.hip).  d (feature dim) in {8, 16, 24, 32},
// dv in {64, 128}.
hipError_t launch_decode_step(const void* q, const void* k, const void* v, bool bf16, int BH, int d,
                              int dv, float eps, float* S, float* z, float* y, hipStream_t st);

// Chunk-64 prefill for every feature dim in fp32 on the fp32 matrix cores
// (prefill_f32mfma.hip); bf16 inputs are widened exactly.  With a workspace
// of prefill_f32mfma_workspace_bytes (0: the shape is never split) few
// heads are split into sequence segments; without one, or with too small a
// one, each head runs as one segment.
size_t prefill_f32mfma_workspace_bytes(int BH, int L, int d, int dv);
hipError_t launch_prefill_f32mfma(const void* q, const void* k, const void* v, bool bf16, int BH, int L, int d,
                                  int dv, float eps, float* y, float* S, float* z, int use_init, void* workspace,
                                  size_t workspace_bytes, hipStream_t st);
// Final normaliser state z = z_init + sum_t phi(k_t) (prefill_valu.hip), one
// workgroup per head; launched after a prefill whose column groups only
// read the caller's initial z.
hipError_t launch_prefill_z(const void* k, bool bf16, int BH, int L, int d, float* z, int use_init,
                            hipStream_t st);
// fp32 vector-ALU chunked prefill (prefill_valu.hip).  d in {8, 16, 24, 32},
// chunk in {16, 32, 64}.
hipError_t launch_prefill_valu(const void* q, const void* k, const void* v, bool bf16, int BH, int L, int d,
                               int dv, int chunk, float eps, float* y, float* S, float* z,
                               int use_init, hipStream_t st);

// bf16 MFMA chunked prefill (prefill_mfma.hip), chunk 64.  `seg_len` > 0
// splits each head into segments of seg_len tokens (a multiple of 64); the
// workspace then holds one carried state per segment.
size_t prefill_mfma_workspace_bytes(int BH, int L, int dv);
// Workspace bytes the launch plan of this shape uses when one is available
// (0: the plan needs none), for a call with or without an initial state.
size_t prefill_mfma_plan_bytes(int BH, int L, int dv, int use_init);
// Fused hybrid layer (prefill_mfma.hip): y = linear attention (q, k, v) +
// the w <= 64 window (q2, k2 of dim 64, the same v), bf16, d' = 16; final
// state into S, z.  *launched is false when no fused plan fits the
// arguments (then nothing ran).
size_t hybrid_mfma_workspace_bytes(int BH, int L, int dv);
hipError_t launch_hybrid_mfma(const void* q, const void* k, const void* q2, const void* k2, const void* v, int BH,
                              int L, int dv, float eps, int window, float scale, float* y, float* S, float* z,
                              int use_init, void* ws, size_t ws_bytes, hipStream_t st, bool* launched);
hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, int BH, int L, int dv,
                               float eps, float* y, float* S, float* z, int use_init,
                               void* workspace, size_t workspace_bytes, hipStream_t st);

// fp32 vector-ALU sliding-window softmax (swa_valu.hip).  dqk in {16, 64},
// dv in {64, 128}, any window >= 1.
hipError_t launch_swa_valu(const void* q, const void* k, const void* v, bool bf16, int BH, int L,
                           int dqk, int dv, int window, float scale, const float* add, float* y,
                           hipStream_t st);

// bf16 MFMA sliding-window softmax (swa_mfma.hip).  dqk in {16, 64}, dv in
// {64, 128} (64-column slices), any window >= 1 (over 128 keys: the
// online-softmax kernel); L * dv * 4 must fit in 31 bits.
hipError_t launch_swa_mfma(const void* q, const void* k, const void* v, int BH, int L, int dqk, int dv,
                           int window, float scale, const float* add, float* y, hipStream_t st);

// Next-token step of the sliding window on its key/value ring cache, and the
// fill of that cache from a prefix (swa_decode.hip).  dqk in {16, 64}, dv in
// {64, 128}, any window >= 1; pos is a device array [B].
hipError_t launch_swa_decode_step(const void* q, const void* k, const void* v, bool bf16, const long long* pos,
                                  int H, int BH, int dqk, int dv, int window, float scale, void* kc, void* vc,
                                  const float* add, float* y, hipStream_t st);
hipError_t launch_swa_cache_fill(const void* k, const void* v, bool bf16, int BH, int L, int dqk, int dv,
                                 int window, void* kc, void* vc, hipStream_t st);

// Gradients of the prefill output, direct (quadratic) form
// (prefill_backward.hip: fp32 inputs or feature dims other than 16, on the
// fp32 matrix cores); the workspace holds BH*L*(dv+1) floats.
size_t prefill_backward_workspace_bytes(int BH, int L, int dv);
// The same on the matrix cores for bf16 inputs with feature dim 16
// (prefill_backward_mfma.hip); g_ws / h_ws as above.
hipError_t launch_prefill_backward_mfma(const void* q, const void* k, const void* v, const float* dy, int BH, int L,
                                        int dv, float eps, float* dq, float* dk, float* dvo, float* g_ws,
                                        float* h_ws, hipStream_t st);
hipError_t launch_prefill_backward(const void* q, const void* k, const void* v, const float* dy, bool bf16, int BH,
                                   int L, int d, int dv_dim, float eps, float* dq, float* dk, float* dv,
                                   void* workspace, hipStream_t st);
// The same gradients in linear time through the carried state
// (prefill_backward_mfma.hip, chunked form): bf16 inputs, feature dim 16,
// dv 64 or 128 (128 as two passes over the column halves).  The workspace
// holds g and h of one 64-column pass and adds two sets of per-segment
// states when a head is split into segments; it does not depend on dv.
size_t prefill_backward_chunked_workspace_bytes(int BH, int L);
hipError_t launch_prefill_backward_chunked(const void* q, const void* k, const void* v, const float* dy, int BH,
                                           int L, int dv, float eps, float* dq, float* dk, float* dvo,
                                           void* workspace, hipStream_t st);

// Gradients of the sliding-window softmax (swa_backward.hip): bf16 inputs,
// d_qk = 64, dv in {64, 128}, windows 1..64; dy fp32, outputs fp32.  The
// workspace holds 16 bytes per (head, query) for the row statistics the key
// side reads.
size_t swa_backward_workspace_bytes(int BH, int L);
hipError_t launch_swa_backward(const void* q, const void* k, const void* v, const float* dy, int BH, int L, int dv,
                               int window, float scale, float* dq, float* dk, float* dvo, void* workspace,
                               hipStream_t st);

}  // namespace based

/*
 * based.h -- C ABI of the MI355X (gfx950) Taylor linear attention library.
 *
 * The operations, as the BASED paper frames inference [1]:
 *   based_prefill      "prompt processing": causal Taylor linear attention
 *                      over a whole sequence, returning the outputs and the
 *                      recurrent state ([1] s5 "Execution stages";
 *                      App. B "Forward / Generation Prefill").
 *   based_decode_step  "next-token prediction": one recurrent KV-state update
 *                      plus readout per head ([1] App. B "Next Token
 *                      Prediction"; s2 constant-memory, O(1)-per-token
 *                      generation).
 *   swa_forward        causal sliding-window softmax attention, each query
 *                      seeing the preceding `window` keys ([1] s4 "Local
 *                      Exact Attention"), with an optional fused add of the
 *                      linear-attention output (BASED pairs the two).
 *   based_hybrid_prefill  both branches of a BASED layer over one sequence
 *                      (linear attention + the window, summed) in one pass
 *                      where a fused kernel exists ([1] s4; s5 fusion).
 *   swa_cache_fill,    the window's next-token step on a w-sized key/value
 *   swa_decode_step    ring cache (same section; App. B "Next Token
 *                      Prediction").
 *   based_prefill_backward  gradients of the prefill output (training-mode
 *                      prefill, s5).
 *   swa_backward       gradients of the window's output (s4 "Local Exact
 *                      Attention"; training-mode prefill, s5).
 *
 * [1] "Simple linear attention language models balance the recall-throughput
 *     tradeoff" (arXiv 2402.18668v2).
 *
 * Definitions (every routine computes exactly these, up to rounding):
 *   d' = d_feat (16 in BASED layers; 8, 24 and 32 are the pages' ablation
 *   sizes, [1] App. D.4).  x~ = x * d'^(-1/4) (the library applies this
 *   itself to raw q and k).  Taylor features ([1] s4 "Taylor Linear
 *   Attention", 2nd order), F = 1 + d' + d'^2 rows (273 for 16) in this
 *   order:
 *       row 0                     1
 *       row 1 + a                 x~_a                    a = 0..d'-1
 *       row 1 + d' + a*d' + b     x~_a * x~_b / sqrt(2)   a-major
 *   so phi(q).phi(k) = 1 + s + s^2/2 with s = q.k / sqrt(d').
 *   Linear attention ([1] s2): y_i = sum_{j<=i} phi(q_i).phi(k_j) v_j /
 *   (sum_{j<=i} phi(q_i).phi(k_j) + eps); the sum of phi(k_j) is the extra
 *   K-state that gives the denominator ([1] App. D.4 "State size").
 *   State per (batch, head): S = sum_j phi(k_j) v_j^T  [F x d_v] and
 *   z = sum_j phi(k_j) [F], both fp32.
 *
 * Memory, layout, ownership (all entry points):
 *   - Every pointer argument is a DEVICE pointer (HIP global memory) unless
 *     stated otherwise.  The caller allocates, owns and frees every buffer;
 *     the library never allocates or frees device memory and keeps no
 *     pointer after a call returns.  Calls are reentrant; the one exception
 *     is based_prefill_noalloc, whose static scratch buffer (one per GPU) is
 *     shared by all its calls on that GPU.
 *   - Tensors are dense and row-major: [B, H, L, dim] (prefill, window) or
 *     [B, H, dim] (decode).  Element type of q, k, v is `dtype`; outputs and
 *     state are always fp32.  Pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued on it asynchronously; no call synchronises the stream.
 *
 * Sizes: B, H, L >= 1 with B*H <= 2^27, L <= 2^31 - 1024 and
 * B*H*L <= 2^40; anything larger returns BASED_E_INVALID.
 *
 * Errors: arguments are checked before anything is launched; a bad argument
 * returns BASED_E_INVALID (malformed) or BASED_E_UNSUPPORTED (well formed
 * but outside what the kernels implement) and touches no memory.  A failed
 * kernel launch returns BASED_E_LAUNCH.  Faults during execution surface at
 * the caller's next synchronisation of `stream`.  NaN/Inf inputs are not
 * checked; they propagate to the outputs.
 */
#ifndef BASED_H
#define BASED_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BASED_OK = 0,
    BASED_E_INVALID = 1,     /* null/misaligned pointer, non-positive size, overflow */
    BASED_E_UNSUPPORTED = 2, /* d_feat, d_v, d_qk, chunk or dtype not implemented */
    BASED_E_LAUNCH = 3,      /* the HIP runtime rejected a kernel launch */
    BASED_E_TOO_LARGE = 4    /* needs more scratch than based_prefill_noalloc's
                                static buffer holds */
} based_status_t;

typedef enum { BASED_F32 = 0, BASED_BF16 = 1 } based_dtype_t;

/* Number of Taylor features for feature dim d_feat: 1 + d + d*d (273 for
 * 16), i.e. the row count of the state S and z.  Returns -1 if d_feat < 1. */
int based_num_features(int d_feat);

/* Human-readable name of a status code (static string, never NULL). */
const char *based_status_string(based_status_t s);

/* Size in bytes of the optional workspace that lets based_prefill split
 * long sequences into segments processed in parallel (carried states are
 * combined by a prefix sum over segments), enough for whichever path the
 * call takes (the bf16 matrix cores for d_feat 16, the fp32 matrix cores
 * for every other input at chunk 64).  0 means the call never uses a
 * workspace for this shape.  Host-only; launches nothing. */
size_t based_prefill_workspace_bytes(int B, int H, int L, int d_feat, int d_v);

/*
 * based_prefill -- causal Taylor linear attention over a full sequence.
 * [1] App. B "Forward / Generation Prefill": the sequence is processed in
 * chunks; within a chunk the masked pairwise weights 1 + s + s^2/2 are used
 * directly (on-diagonal term), earlier chunks enter through the cumulative
 * state (off-diagonal term), and the state is carried to the next chunk.
 *
 *   q, k   [B,H,L,d_feat] dtype       raw (not pre-scaled) queries/keys
 *   v      [B,H,L,d_v]    dtype
 *   chunk  chunk length: 64; 16 or 32 too except for bf16 with d_feat = 16
 *          (that case runs on the matrix cores, chunk 64)
 *   eps    denominator guard (1e-6 in BASED layers)
 *   y      [B,H,L,d_v]    fp32, written
 *   S      [B,H,F,d_v]    fp32 state; read as the initial state when
 *   z      [B,H,F]        fp32  use_initial_state != 0 (else zero), and
 *                               always overwritten with the state after the
 *                               last token (the handoff to based_decode_step)
 *   workspace, workspace_bytes  optional scratch (may be NULL/0); see
 *          based_prefill_workspace_bytes.  With too small a workspace the
 *          call still runs, without the segment split.  Its first
 *          min(workspace_bytes, based_prefill_workspace_bytes) bytes must
 *          not overlap q, k, v, y, S or z (else BASED_E_INVALID).
 * Supported: d_feat in {8, 16, 24, 32}; d_v in {64, 128}; L >= 1 (any, not
 * only multiples of chunk).  bf16 inputs with d_feat = 16 run on the bf16
 * matrix cores (fp32 accumulation and state); every other input runs in
 * fp32 throughout: chunk 64 on the fp32 matrix cores, chunks 16 and 32 on
 * the vector ALUs.  y must not alias q, k, v, S or z.
 */
based_status_t based_prefill(const void *q, const void *k, const void *v,
                             based_dtype_t dtype, int B, int H, int L,
                             int d_feat, int d_v, int chunk, float eps,
                             float *y, float *S, float *z,
                             int use_initial_state,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * based_prefill_noalloc -- based_prefill for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, semantics and errors as
 * based_prefill, without the workspace: the segment split (and an initial
 * state shared by several column groups) uses a static device buffer of
 * BASED_PREFILL_NOALLOC_SCRATCH_BYTES inside this library instead.  The call
 * allocates nothing.  Each GPU holds its own buffer from the first call on
 * it until the process ends; its device address is taken on that first call
 * (the stream's device).
 *   - A call whose launch plan needs more scratch than the buffer holds
 *     returns BASED_E_TOO_LARGE before anything is launched (every call
 *     without an initial state fits; with one, the need grows with B*H).
 *   - All calls on one GPU share that GPU's buffer: calls that overlap in
 *     time on one GPU (other streams, other threads) race, and the caller
 *     must order them.  Consecutive calls on one stream are safe; no call
 *     needs the buffer's previous contents.
 */
#define BASED_PREFILL_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
based_status_t based_prefill_noalloc(const void *q, const void *k, const void *v,
                                     based_dtype_t dtype, int B, int H, int L,
                                     int d_feat, int d_v, int chunk, float eps,
                                     float *y, float *S, float *z,
                                     int use_initial_state, void *stream);

/*
 * based_decode_step -- one next-token step for every (batch, head), in
 * place on the state ([1] App. B "Next Token Prediction"):
 *   S' = S + phi(k) v^T,  z' = z + phi(k),
 *   y  = phi(q)^T S' / (phi(q).z' + eps)
 * (update first, so the current token attends to itself, as in prefill).
 * Each state element is read once and written once.
 *
 *   q, k [B,H,d_feat] dtype;  v [B,H,d_v] dtype
 *   S    [B,H,F,d_v] fp32 in/out;  z [B,H,F] fp32 in/out
 *   y    [B,H,d_v]   fp32 out (must not alias the state)
 * Supported: d_feat in {8, 16, 24, 32}; d_v in {64, 128}.
 */
based_status_t based_decode_step(const void *q, const void *k, const void *v,
                                 based_dtype_t dtype, int B, int H,
                                 int d_feat, int d_v, float eps,
                                 float *S, float *z, float *y,
                                 void *stream);

/*
 * swa_forward -- causal sliding-window softmax attention ([1] s4 "Local
 * Exact Attention"; O(L*window) work):
 *   y_i = add_i + sum_{j=max(0,i-window+1)}^{i} e_ij v_j / sum_j e_ij,
 *   e_ij = exp(scale * q_i.k_j - m_i),  m_i = max_j scale * q_i.k_j.
 * The window holds `window` keys including the query's own.
 *
 *   q, k   [B,H,L,d_qk] dtype;  v [B,H,L,d_v] dtype
 *   window >= 1 (64 in BASED layers)
 *   scale  logit scale (1/sqrt(d_qk) for standard attention)
 *   add    optional [B,H,L,d_v] fp32 added to the output (e.g. the linear
 *          attention output of the same layer); NULL for none; may equal y
 *          for an in-place accumulate
 *   y      [B,H,L,d_v] fp32 out
 * Supported: d_qk in {16, 64}; d_v in {64, 128}; any window >= 1 (a
 * window of L or more keys is plain causal softmax attention).  bf16 inputs
 * run on the matrix cores (windows up to 128 keys in one pass over a tile's
 * keys, longer windows with a running-maximum softmax over 64-key tiles);
 * fp32 inputs, and bf16 heads with L * d_v * 4 >= 2^31, run in fp32 on the
 * vector ALUs.
 */
based_status_t swa_forward(const void *q, const void *k, const void *v,
                           based_dtype_t dtype, int B, int H, int L,
                           int d_qk, int d_v, int window, float scale,
                           const float *add, float *y, void *stream);

/*
 * based_hybrid_prefill -- a BASED layer's two mixers over one sequence,
 * summed ([1] s4: Taylor linear attention paired with "Local Exact
 * Attention"; s5: fuse work and avoid extra passes over HBM):
 *   y = based_prefill(q, k, v).y + swa_forward(q_win, k_win, v).y
 * with the final linear-attention state in S, z exactly as based_prefill
 * (each branch normalised on its own; v is shared).
 *
 *   q, k          [B,H,L,d_feat] dtype (the linear branch)
 *   q_win, k_win  [B,H,L,d_qk] dtype (the window branch)
 *   v             [B,H,L,d_v] dtype
 *   chunk, eps, S, z, use_initial_state, workspace: as based_prefill, with
 *                 the workspace size from
 *                 based_hybrid_prefill_workspace_bytes
 *   window, scale: as swa_forward;  y [B,H,L,d_v] fp32 out
 *   path          BASED_HYBRID_AUTO, _FUSED or _TWO_PASS (below);
 *                 anything else is BASED_E_INVALID
 * Supported: what both based_prefill and swa_forward support (d_v in
 * {64, 128}, any window >= 1).  A fused kernel exists for bf16 with
 * d_feat = 16, d_qk = 64 and window <= 64 (q, k, q_win, k_win and v read
 * once, y written once); an initial state with no large enough workspace
 * has none.  The two-pass
 * form runs the branches in turn on the stream (the window adds into y in
 * place).  AUTO fuses wherever a fused kernel exists; FUSED returns
 * BASED_E_UNSUPPORTED where none does; TWO_PASS always runs the branches
 * in turn.
 * Outputs must not overlap each other or any input (BASED_E_INVALID).
 */
enum { BASED_HYBRID_AUTO = 0, BASED_HYBRID_FUSED = 1, BASED_HYBRID_TWO_PASS = 2 };
size_t based_hybrid_prefill_workspace_bytes(int B, int H, int L, int d_feat, int d_v);

based_status_t based_hybrid_prefill(const void *q, const void *k, const void *q_win,
                                    const void *k_win, const void *v, based_dtype_t dtype,
                                    int B, int H, int L, int d_feat, int d_qk, int d_v,
                                    int chunk, float eps, int window, float scale, int path,
                                    float *y, float *S, float *z, int use_initial_state,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * swa_cache_fill / swa_decode_step -- next-token generation for the
 * sliding window ([1] s4 "Local Exact Attention": each query sees the
 * preceding `window` keys through a w-sized key/value cache; App. B "Next
 * Token Prediction").
 *
 * Cache: per (batch, head) a ring of `window` slots, k_cache
 * [B,H,window,d_qk] and v_cache [B,H,window,d_v] in `dtype`, caller-owned.
 * The token at position p (0-based) lives in slot p mod window.
 *
 * swa_cache_fill writes the slots of the last min(L, window) tokens of a
 * prefix k [B,H,L,d_qk], v [B,H,L,d_v]; other slots are left untouched.
 *
 * swa_decode_step handles the token at position pos[b] of each sequence b:
 *   1. k, v [B,H,d_qk] / [B,H,d_v] go into slot pos[b] mod window;
 *   2. y = add + sum_{t=max(0,pos-window+1)}^{pos} e_t v_t / sum_t e_t,
 *      e_t = exp(scale * q.k_t - m), m = max_t scale * q.k_t,
 *      over the tokens t held in their slots (the new token included) --
 *      exactly row pos of swa_forward on the whole sequence.
 * What a slot holds that is not one of those tokens never reaches y (it may
 * be loaded and is then discarded), so a cache only needs the fill (or
 * nothing, when decoding starts at position 0).
 *   q     [B,H,d_qk] dtype;  pos [B] int64 device array, not modified
 *         (the caller advances it); pos[b] < 0 gives NaN outputs for b and
 *         leaves its cache untouched
 *   add   optional [B,H,d_v] fp32 added to y (e.g. the linear-attention
 *         decode output); NULL or equal to y for in place
 *   y     [B,H,d_v] fp32 out
 * Supported: d_qk in {16, 64}; d_v in {64, 128}; any window >= 1 (up to
 * 128 one wave per (batch, head); wider, one workgroup of four waves per
 * (batch, head), an online softmax over rounds of 64 slots).  The caches,
 * y and the inputs must not overlap (add may equal y).
 */
based_status_t swa_cache_fill(const void *k, const void *v, based_dtype_t dtype,
                              int B, int H, int L, int d_qk, int d_v, int window,
                              void *k_cache, void *v_cache, void *stream);

based_status_t swa_decode_step(const void *q, const void *k, const void *v,
                               based_dtype_t dtype, int B, int H, int d_qk, int d_v,
                               int window, float scale, const long long *pos,
                               void *k_cache, void *v_cache, const float *add,
                               float *y, void *stream);

/*
 * based_prefill_backward -- gradients of based_prefill's output y for an
 * upstream gradient dy (training-mode prefill; [1] s5).  With
 * s_ij = q_i.k_j/sqrt(d'), a_ij = 1 + s_ij + s_ij^2/2, y_i = N_i / D_i,
 * N_i = sum_{j<=i} a_ij v_j, D_i = sum_{j<=i} a_ij + eps:
 *   g_i = dy_i / D_i,  h_i = -(dy_i . y_i) / D_i,
 *   e_ij = (g_i . v_j + h_i)(1 + s_ij) / sqrt(d'),
 *   dq_i = sum_{j<=i} e_ij k_j,  dk_j = sum_{i>=j} e_ij q_i,
 *   dv_j = sum_{i>=j} a_ij g_i
 * (starting from a zero state; no gradient of an initial state).
 *
 *   q, k  [B,H,L,d_feat] dtype;  v [B,H,L,d_v] dtype
 *   dy    [B,H,L,d_v] fp32
 *   dq, dk [B,H,L,d_feat] fp32 out;  dv [B,H,L,d_v] fp32 out
 *   workspace  required, at least based_prefill_backward_workspace_bytes
 *          (else BASED_E_INVALID); must not overlap anything else
 *   form   BASED_BACKWARD_AUTO, _DIRECT or _CHUNKED (below); anything else
 *          is BASED_E_INVALID
 * Supported: d_feat in {8, 16, 24, 32}; d_v in {64, 128}; B*H*ceil(L/64)*256
 * must not exceed INT32_MAX (else BASED_E_INVALID).  Two forms, both on the
 * matrix cores with fp32 accumulation:
 *   DIRECT   the sums above pair by pair, O(L^2) work per head; bf16 inputs
 *            with d_feat 16 take bf16 products with the weights split into
 *            bf16 hi/lo pairs, every other input fp32 products;
 *   CHUNKED  linear in L through the recurrent form ([1] s2): with the
 *            prefix state S_i, z_i and the suffix sums
 *            R_j = sum_{i>=j} phi(q_i) g_i^T, r_j = sum_{i>=j} phi(q_i) h_i,
 *            dq_i = J(q_i)^T (S_i g_i + h_i z_i), dk_j = J(k_j)^T (R_j v_j + r_j),
 *            dv_j = R_j^T phi(k_j) (J: the Jacobian of phi), pairs within a
 *            64-token chunk taken directly; bf16 inputs with d_feat 16 only
 *            (else BASED_E_UNSUPPORTED), every non-input operand a bf16
 *            hi/lo pair.  d_v 128 runs once per 64-column half of v, dy
 *            and dv (each half with its own h, the sums of which are the
 *            full h), the second run adding into dq and dk.
 * AUTO takes CHUNKED where it is supported and L >= 1024, else DIRECT.  The
 * workspace size covers either form.
 */
enum { BASED_BACKWARD_AUTO = 0, BASED_BACKWARD_DIRECT = 1, BASED_BACKWARD_CHUNKED = 2 };
size_t based_prefill_backward_workspace_bytes(int B, int H, int L, int d_feat, int d_v);

based_status_t based_prefill_backward(const void *q, const void *k, const void *v,
                                      const float *dy, based_dtype_t dtype, int B, int H,
                                      int L, int d_feat, int d_v, float eps, int form,
                                      float *dq, float *dk, float *dv, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * based_swa_backward -- gradients of swa_forward's output y (without the
 * fused add, whose gradient is dy itself) for an upstream gradient dy
 * (training-mode prefill; [1] s4 "Local Exact Attention", s5).  With
 * P_ij = softmax_j(scale q_i.k_j) over j in (i - window, i], y_i =
 * sum_j P_ij v_j:
 *   dv_j = sum_i P_ij dy_i,   dP_ij = dy_i . v_j,   D_i = sum_j P_ij dP_ij,
 *   dS_ij = P_ij (dP_ij - D_i),
 *   dq_i = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i.
 *
 *   q, k  [B,H,L,d_qk] dtype;  v [B,H,L,d_v] dtype
 *   dy    [B,H,L,d_v] fp32
 *   dq, dk [B,H,L,d_qk] fp32 out;  dv [B,H,L,d_v] fp32 out
 *   workspace  required, at least based_swa_backward_workspace_bytes (16
 *          bytes per (batch, head, query): the row statistics the key side
 *          reads), else BASED_E_INVALID; must not overlap anything else
 * Supported: bf16 inputs, d_qk 64, d_v in {64, 128}, window 1..64 (else
 * BASED_E_UNSUPPORTED); B*H*ceil(L/64)*256 must not exceed INT32_MAX (else
 * BASED_E_INVALID).  Two launches on the bf16 matrix cores with fp32
 * accumulation (the query side, then the key side); P, dS and dy enter the
 * products as bf16 hi/lo pairs.
 */
size_t based_swa_backward_workspace_bytes(int B, int H, int L);

based_status_t based_swa_backward(const void *q, const void *k, const void *v, const float *dy,
                                  based_dtype_t dtype, int B, int H, int L, int d_qk, int d_v,
                                  int window, float scale, float *dq, float *dk, float *dv,
                                  void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BASED_H */

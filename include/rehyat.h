/*
 * rehyat.h - C ABI of librehyat: ReHyAt temporally chunked hybrid attention on MI355X (gfx950).
 *
 * The method (papernotes.org note "ReHyAt: Recurrent Hybrid Attention for Video Diffusion
 * Transformers", section "method details"):
 *   - N = T*HW tokens, time-major: token f*HW + s is spatial position s of latent frame f.
 *   - Chunks of Tc frames (N' = Tc*HW tokens). The queries of chunk t are the rows
 *     [t*N', min((t+1)*N', N)) (key design 1).
 *   - Softmax keys of chunk t: [lo_t, hi_t), lo_t = max(t*N' - To*HW, 0),
 *     hi_t = min((t+1)*N', N): the chunk plus the To frames before it (key design 2).
 *   - Linear keys: causal [0, lo_t) (key design 4); bidirectional [0, lo_t) U [hi_t, N),
 *     the complement of the overlapped window (key design 1).
 *   - y = (a^S + a^L) / (n^S + n^L) with a^S = sum_S exp(q.k/sqrt(D)) v,
 *     a^L = phi(q) (sum_L phi(k) v^T), n^S, n^L the matching weight sums (key design 1).
 *     No stabiliser enters the result: running maxima inside the kernels are compensated
 *     exactly.
 *   - Feature map phi, chosen by desc->phi_kind (key design 3):
 *       REHYAT_PHI_POLY2 (0): phi(x)_i = 1 + u_i + u_i^2/2, u = x W / sqrt(D); W is a D x F
 *         matrix ([D, F], or [H, D, F] with w_per_head).
 *       REHYAT_PHI_ELU (1): phi(x) = 1 + elu(x) elementwise (x + 1 for x > 0, exp(x)
 *         otherwise), the linear-attention baseline the note compares with. F = D; W is
 *         unused and may be NULL.
 *       REHYAT_PHI_MLP (2): the learned polynomial map: psi = relu(x W1 + b1) W2 + b2 (one
 *         hidden layer of h = phi_hidden units), split into P = phi_parts equal parts of
 *         F/P features, part i (i = 1..P) raised elementwise to the power i. W points to the
 *         parameter block, bf16, row-major, concatenated: W1 [D, h], b1 [h], W2 [h, F],
 *         b2 [F] (D*h + h + h*F + F elements); with w_per_head, H such blocks back to back.
 *         The note fixes neither the activation nor P: ReLU and the block layout are this
 *         library's choice, P is a parameter (the plainest reading is P = 2).
 *       Maps 1 and 2 can give phi(q).phi(k) of either sign; n^L then enters the joint
 *       normalisation with its sign.
 *   - Causal form as a chunk-wise RNN (key design 4): state S = sum phi(k) v^T (F x D) and
 *     z = sum phi(k) (F) over the keys already out of reach of the softmax window.
 *
 * Conventions for every entry point
 *   - All tensors are dense, row-major, head-major: [B, H, rows, cols]. Device pointers
 *     must be 16-byte aligned. The caller owns every buffer; the library allocates no
 *     device memory, keeps no state between calls (apart from the static scratch array of
 *     rehyat_recurrent_step_fused_noalloc) and never synchronises the stream.
 *   - dtype REHYAT_BF16: q, k, v, W (and tails) are bf16; products run on bf16 MFMA with
 *     fp32 accumulation; phi(q), phi(k), the softmax weights and the state are rounded to
 *     bf16 where they enter an MFMA. dtype REHYAT_F32: everything in fp32.
 *     S and z are always fp32. y has dtype y_dtype (fp32 or bf16).
 *   - `stream` is a hipStream_t (NULL: the null stream). Work is enqueued asynchronously.
 *   - Argument checks run on the host before anything is enqueued; on failure nothing is
 *     launched, outputs are untouched and a status != REHYAT_OK is returned (details in
 *     rehyat_last_error()). No C++ exception crosses this boundary and nothing aborts.
 *   - Outputs must not overlap inputs.
 *   - Supported sizes: bf16: D = 128, F in {64, 128, 256}. fp32: D in {64, 128},
 *     F in {16, 32, ..., 256} (a multiple of 16). B, H >= 1; T, HW, Tc >= 1; To >= 0;
 *     B*H*T*HW*max(D,F) < 2^31 elements per tensor. phi_kind 1 and 2 need dtype bf16;
 *     phi_kind 2 needs phi_hidden in {64, 128, 256} and F a multiple of phi_parts >= 1
 *     with parts of at least 8 features (phi_parts <= F/8).
 *   - phi_kind 1 and 2 evaluate phi(q) and phi(k) into the workspace ahead of the attention
 *     and state kernels (bf16 rows); their *_workspace() sizes include those rows.
 */
#ifndef REHYAT_H
#define REHYAT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  REHYAT_OK = 0,
  REHYAT_ERR_NULL = 1,        /* a required pointer is NULL */
  REHYAT_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  REHYAT_ERR_DTYPE = 3,       /* unknown dtype or mode value */
  REHYAT_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
  REHYAT_ERR_UNSUPPORTED = 5, /* valid, but outside the supported sizes listed above */
  REHYAT_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the *_workspace() size */
  REHYAT_ERR_HIP = 7,         /* the HIP runtime reported an error at launch */
  REHYAT_ERR_ALIAS = 8        /* an output overlaps an input */
} rehyat_status;

typedef enum { REHYAT_F32 = 0, REHYAT_BF16 = 1 } rehyat_dtype;
typedef enum { REHYAT_CAUSAL = 0, REHYAT_BIDIR = 1 } rehyat_mode;
typedef enum { REHYAT_PHI_POLY2 = 0, REHYAT_PHI_ELU = 1, REHYAT_PHI_MLP = 2 } rehyat_phi_kind;

/* Problem description shared by all entry points. */
typedef struct {
  int32_t B, H;       /* batch, heads */
  int32_t T, HW;      /* latent frames of the whole video, tokens per frame (N = T*HW) */
  int32_t D, F;       /* head dimension, feature dimension of phi */
  int32_t Tc, To;     /* frames per chunk, overlap frames (softmax window reach-back) */
  int32_t dtype;      /* rehyat_dtype of q, k, v, W, k_tail, v_tail */
  int32_t y_dtype;    /* rehyat_dtype of y */
  int32_t mode;       /* rehyat_mode (rehyat_hybrid_fwd only; the step path is causal) */
  int32_t w_per_head; /* 0: Wq and Wk are shared by all heads; 1: one per head (H of them) */
  int32_t phi_kind;   /* rehyat_phi_kind of the feature map (0: the fixed polynomial) */
  int32_t phi_hidden; /* REHYAT_PHI_MLP: hidden units h; ignored otherwise */
  int32_t phi_parts;  /* REHYAT_PHI_MLP: number of parts P; ignored otherwise */
} rehyat_desc;

/*
 * Feature map phi of key design 3, of the kind desc->phi_kind names (see above).
 *   x   [B, H, n, D]  dtype     (device)
 *   W   the map's parameters, as described above for each phi_kind (device)
 *   phi [B, H, n, F]  dtype     (device, written)
 * n >= 0 rows per (b, h); n = 0 is a no-op.
 */
rehyat_status rehyat_phi(const rehyat_desc* desc, const void* x, int64_t n, const void* W,
                         void* phi, void* stream);

/*
 * Recurrent-state update (key design 4, the sums s and z of the chunk-wise RNN):
 *   S[b,h] += sum_{rows r} phi(k_r) v_r^T,   z[b,h] += sum_r phi(k_r)
 *   k, v  [B, H, n, D]  dtype   (device)
 *   Wk    parameters of phi (see phi_kind above) (device)
 *   S     [B, H, F, D]  fp32    (device, read and written)
 *   z     [B, H, F]     fp32    (device, read and written)
 *   ws    device scratch of at least rehyat_state_update_workspace(desc, n) bytes.
 * The reduction order is fixed: results are bitwise reproducible.
 */
size_t rehyat_state_update_workspace(const rehyat_desc* desc, int64_t n);
rehyat_status rehyat_state_update(const rehyat_desc* desc, const void* k, const void* v,
                                  int64_t n, const void* Wk, float* S, float* z,
                                  void* ws, size_t ws_bytes, void* stream);

/*
 * Whole-sequence hybrid attention (key designs 1, 2 and 4): causal (mode REHYAT_CAUSAL,
 * the non-recursive form of the chunk-wise RNN) or bidirectional (REHYAT_BIDIR).
 *   q, k, v [B, H, N, D] dtype  (device), N = T*HW; T need not be a multiple of Tc (the
 *                                last chunk is then shorter)
 *   Wq, Wk  parameters of the maps applied to q and to k (see phi_kind above; device; may
 *           be the same buffer)
 *   y       [B, H, N, D] y_dtype (device, written)
 *   ws      device scratch of at least rehyat_hybrid_fwd_workspace(desc) bytes (per-frame
 *           partial states, the per-chunk linear-branch states and, for bf16, the work
 *           counters of the attention launch, reset by the call itself); no contents are
 *           required on entry. Two calls must not use one workspace at the same time.
 */
size_t rehyat_hybrid_fwd_workspace(const rehyat_desc* desc);
rehyat_status rehyat_hybrid_fwd(const rehyat_desc* desc, const void* q, const void* k,
                                const void* v, const void* Wq, const void* Wk, void* y,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * rehyat_hybrid_fwd that also writes, for every query row, the log2 of its joint
 * normaliser (key design 1): lse[b,h,i] = log2(n^S_i + n^L_i), the softmax weights taken
 * as exp(q.k/sqrt(D)) without any stabiliser. The backward (rehyat_hybrid_bwd) takes it.
 *   lse [B, H, N] fp32 (device, written); other arguments as for rehyat_hybrid_fwd.
 */
rehyat_status rehyat_hybrid_fwd_stats(const rehyat_desc* desc, const void* q, const void* k,
                                      const void* v, const void* Wq, const void* Wk, void* y,
                                      float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * One chunk of the causal form run as the chunk-wise RNN (key design 4), the sampling-time
 * use in which one chunk of Tc frames is produced at a time with the state carried.
 *   chunk_index t >= 0; the chunk holds frames [t*Tc, min((t+1)*Tc, T)), c_f of them.
 *   q_c, k_c, v_c [B, H, c_f*HW, D] dtype (device)
 *   S [B,H,F,D], z [B,H,F] fp32 (device, read and written): on entry the sums over all
 *           keys before lo_t; on exit the sums over all keys before lo_{t+1}. For t = 0 the
 *           entry values are ignored (the state starts empty).
 *   k_tail, v_tail [B, H, To*HW, D] dtype (device, read and written): on entry the K and V
 *           rows of the To frames before the chunk (ignored for t = 0); on exit those of
 *           the chunk's last To frames. May be NULL when To = 0.
 *   y_c  [B, H, c_f*HW, D] y_dtype (device, written)
 *   ws   device scratch of at least rehyat_recurrent_step_workspace(desc) bytes.
 * Requirements: To <= Tc; c_f >= To (a short final chunk must still cover the tail).
 * Memory use is independent of t: calling it for t = 0, 1, 2, ... reproduces
 * rehyat_hybrid_fwd(mode = REHYAT_CAUSAL) chunk by chunk (up to rounding order).
 */
size_t rehyat_recurrent_step_workspace(const rehyat_desc* desc);
rehyat_status rehyat_recurrent_step(const rehyat_desc* desc, int32_t chunk_index,
                                    const void* q_c, const void* k_c, const void* v_c,
                                    const void* Wq, const void* Wk, float* S, float* z,
                                    void* k_tail, void* v_tail, void* y_c,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * rehyat_recurrent_step as one kernel launch (key design 4's chunk-wise RNN, for streaming
 * where a step is short and launch gaps would show): the chunk's attention, the per-frame
 * sums of the window rows no later window reaches, their fold into S and z and the new
 * tail come from a single launch. Arguments, requirements and results as for
 * rehyat_recurrent_step, bit for bit, except that the tail has separate input and output
 * buffers (a caller alternates two):
 *   k_tail, v_tail [B, H, To*HW, D] dtype (device, read): the K and V rows of the To frames
 *           before the chunk (ignored for t = 0). May be NULL when To = 0.
 *   k_tail_out, v_tail_out [B, H, To*HW, D] dtype (device, written): those of the chunk's
 *           last To frames; they must not overlap any other buffer of the call. May be NULL
 *           when To = 0.
 *   ws   device scratch of at least rehyat_recurrent_step_fused_workspace(desc) bytes.
 *        Its first B*H*4 bytes are per-head completion counters: they must be zero before
 *        the first call (zero the whole workspace once when allocating it); every call
 *        leaves them zero. Two calls must not use one workspace at the same time.
 * Supported: dtype bf16 (D = 128, F in {64, 128, 256}) with phi_kind REHYAT_PHI_POLY2;
 * other descriptors return REHYAT_ERR_UNSUPPORTED (use rehyat_recurrent_step).
 */
size_t rehyat_recurrent_step_fused_workspace(const rehyat_desc* desc);
rehyat_status rehyat_recurrent_step_fused(const rehyat_desc* desc, int32_t chunk_index,
                                          const void* q_c, const void* k_c, const void* v_c,
                                          const void* Wq, const void* Wk, float* S, float* z,
                                          const void* k_tail, const void* v_tail,
                                          void* k_tail_out, void* v_tail_out, void* y_c,
                                          void* ws, size_t ws_bytes, void* stream);

/*
 * rehyat_recurrent_step_fused for callers that cannot allocate device memory or take a
 * workspace: code under HIP graph capture, tight serving loops and harnesses that forbid
 * allocation. The same kernel and results, bit for bit; the scratch (per-head completion
 * counters, the new state, the fold's partials) comes from a static device array of
 * REHYAT_STATIC_SCRATCH_BYTES bytes that every device the library runs on holds until the
 * process ends. The call allocates nothing. Arguments, requirements and results as for
 * rehyat_recurrent_step_fused, without ws and ws_bytes.
 *   Limit: rehyat_recurrent_step_fused_workspace(desc) must not exceed
 *          REHYAT_STATIC_SCRATCH_BYTES (it is 256*ceil(B*H/64) + 12*B*H*(F*D + F) bytes,
 *          e.g. 2.4 MB for B*H = 12, F = 128); larger descriptors return
 *          REHYAT_ERR_WORKSPACE before anything is enqueued.
 *   Device: the array of the calling thread's current device is used; `stream` must belong
 *          to that device. The first call on a device looks the array up and enqueues a fill
 *          kernel on `stream` that zeroes it (make that call outside stream capture); every
 *          call leaves the counters zero again.
 *   Concurrency: all calls on one device share its array, which keeps the last call's
 *          contents; calls that overlap in time on one device (other streams, other
 *          threads) race and must not be issued.
 */
#define REHYAT_STATIC_SCRATCH_BYTES (16 * 1024 * 1024)
rehyat_status rehyat_recurrent_step_fused_noalloc(const rehyat_desc* desc, int32_t chunk_index,
                                                  const void* q_c, const void* k_c,
                                                  const void* v_c, const void* Wq,
                                                  const void* Wk, float* S, float* z,
                                                  const void* k_tail, const void* v_tail,
                                                  void* k_tail_out, void* v_tail_out,
                                                  void* y_c, void* stream);

/*
 * Backward of the non-recursive causal form (key designs 1 and 4: the form the method is
 * trained and its feature maps distilled with): the gradients of sum(dy * y) for
 * y = rehyat_hybrid_fwd(q, k, v, Wq, Wk), the fixed feature map.
 *   q, k, v [B, H, N, D] bf16, Wq, Wk as for the forward (device)
 *   y    [B, H, N, D] y_dtype: the forward's output (device)
 *   lse  [B, H, N] fp32: from rehyat_hybrid_fwd_stats (device)
 *   dy   [B, H, N, D] y_dtype (device)
 *   dq, dk, dv [B, H, N, D] fp32 (device, written)
 *   dWq, dWk   [D, F] or [H, D, F] fp32 (device, written): summed over the batch (and over
 *              the heads for a shared W). When Wq and Wk are one tensor, its gradient is
 *              dWq + dWk.
 *   ws   device scratch of at least rehyat_hybrid_bwd_workspace(desc) bytes.
 * Supported: dtype bf16 (D = 128, F in {64, 128, 256}), phi_kind REHYAT_PHI_POLY2, mode
 * REHYAT_CAUSAL; other descriptors return REHYAT_ERR_UNSUPPORTED. The window products run
 * on bf16 MFMA with fp32 accumulation; dy, dy/den, the softmax weights and their gradients,
 * phi and the feature gradients are rounded to bf16 where they enter an MFMA.
 */
size_t rehyat_hybrid_bwd_workspace(const rehyat_desc* desc);
rehyat_status rehyat_hybrid_bwd(const rehyat_desc* desc, const void* q, const void* k,
                                const void* v, const void* Wq, const void* Wk, const void* y,
                                const float* lse, const void* dy, float* dq, float* dk,
                                float* dv, float* dWq, float* dWk, void* ws, size_t ws_bytes,
                                void* stream);

/* Human-readable name of a status code (static string). */
const char* rehyat_status_str(rehyat_status status);

/* Detail message of the last failed call on the calling host thread ("" if none). */
const char* rehyat_last_error(void);

/*
 * Kernel timing (measurement aid). While enabled, every launch of one kernel is bracketed
 * by HIP events recorded on the launch stream (events are created once, at most 4096
 * launches are recorded). The argument selects it: 1 the hybrid-attention kernel of the
 * forward and of rehyat_recurrent_step, 2 the dk/dv kernel and 3 the dq kernel of
 * rehyat_hybrid_bwd, 4 the kernel of rehyat_recurrent_step_fused; 0 disables.
 * rehyat_timing_read synchronises on the last recorded event and returns the summed kernel
 * time in milliseconds and the launch count, then clears the record. Enabling clears the
 * record too. Not thread-safe.
 */
rehyat_status rehyat_timing_enable(int32_t enable);
rehyat_status rehyat_timing_read(double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* REHYAT_H */

/*
 * lr_block.h -- C ABI of the fused low-rank bottleneck block for AMD MI355X (gfx950).
 *
 * The operation is the low-rank layer of BOOST ("BOOST: BOttleneck-Optimized
 * Scalable Training Framework for Low-Rank Large Language Models"): a d x d
 * weight replaced by a d x r "down" factor and an r x d "up" factor with a
 * pointwise operation between them (technical summary, §1 and §2.1), preceded by
 * RMSNorm whose statistic is computed locally and applied late (§2.2,
 * Online-RMSNorm), with the down-projections that share one input concatenated
 * into one weight and the up-projections run as a batch (§2.2, linear layer
 * grouping), and a backward pass that keeps only the rank-r pre-activation and
 * recomputes the pointwise operation from it (§2.2, low-rank activation
 * checkpointing).
 *
 * Forward, for tokens t < T, hidden index j < d, rank index c < r:
 *   rstd_t = (sum_j x_tj^2 / D + eps)^(-1/2)          D = d_norm, or d when d_norm == 0
 *   h      = diag(rstd) . x . diag(gamma) . A          A = [A_0 | ... | A_{g-1}], [d, g*r]
 *   z_i    = sigma(h_i)                                h_i = columns [i*r, (i+1)*r) of h
 *            identity: z_i = h_i ; SiLU: z_i = h_i * sigmoid(h_i)
 *            SwiGLU (g == 2): z_0 = SiLU(h_0) * h_1
 *   y_i    = z_i . B_i                                 n_up = 1 for SwiGLU, else g
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, row-major, dense, 16-byte aligned.
 *     Arrays of pointers (B, y, dy, dB) are HOST arrays of n_up device pointers.
 *     Pointers to [T, ...] buffers may be NULL when T == 0.
 *   - The element type of x, gamma, A, B_i, y_i, h, dy_i and dx is dims->dtype
 *     (LR_BF16: bfloat16 storage, fp32 accumulation; LR_F32: fp32).  sumsq,
 *     rstd, the shard partial and all weight gradients are fp32.
 *   - The caller owns every buffer.  The library allocates no device memory,
 *     keeps no pointer after a call returns and holds no mutable global state,
 *     except lr_block_fwd_noalloc's per-GPU device scratch (below).  Scratch
 *     space is the caller's workspace `ws` of at least lr_block_workspace_size()
 *     bytes (256-byte aligned).
 *   - All work is enqueued on `stream`; nothing synchronises.  Buffers must stay
 *     alive until the stream has passed the call.
 *   - Outputs must not alias inputs.  Gradients are overwritten, not accumulated.
 *   - Shape and argument checks run on the host before any launch: a bad call
 *     returns LR_EINVAL / LR_EUNSUPPORTED / LR_EWORKSPACE and launches nothing.
 *     A failed launch returns LR_EHIP.  After an error the outputs are
 *     undefined.  Nothing else crosses the ABI (no exceptions, no aborts).
 *   - Supported shapes: T >= 0 (any value, ragged tails included); d and r
 *     positive multiples of 64; 1 <= g <= 8; SwiGLU needs g == 2.
 *   - Results are deterministic for a given device, shape and input (no
 *     floating-point atomics).
 */
#ifndef LR_BLOCK_H
#define LR_BLOCK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LR_OK = 0,
  LR_EINVAL = 1,        /* null / misaligned pointer, negative size, bad enum */
  LR_EUNSUPPORTED = 2,  /* valid but unsupported shape or combination        */
  LR_EWORKSPACE = 3,    /* workspace missing or smaller than required        */
  LR_EHIP = 4           /* a HIP launch failed                               */
} lr_status;

typedef enum { LR_F32 = 0, LR_BF16 = 1 } lr_dtype;

typedef enum { LR_ACT_IDENTITY = 0, LR_ACT_SILU = 1, LR_ACT_SWIGLU = 2 } lr_act;

typedef struct {
  int64_t T;        /* tokens (b*s)                                              */
  int64_t d;        /* hidden width held by this call (a shard's slice under TP) */
  int64_t r;        /* rank                                                      */
  int64_t g;        /* grouped down-projection branches                          */
  int64_t d_norm;   /* width the RMS mean is taken over; 0 -> d                  */
  float eps;        /* RMSNorm epsilon, inside the square root                   */
  int32_t dtype;    /* lr_dtype                                                  */
  int32_t act;      /* lr_act                                                    */
} lr_dims;

/* RMSNorm with the statistic computed in one pass (Online-RMSNorm, §2.2).
 *   x [T, d], gamma [d] (dtype).  Each output may be NULL:
 *   y [T, d] (dtype)  = x_tj * rstd_t * gamma_j
 *   sumsq [T] (fp32)  = sum_j x_tj^2      (the additive local statistic)
 *   rstd [T] (fp32)   = (sumsq_t / D + eps)^(-1/2)
 * gamma may be NULL when y is NULL.  d must be a multiple of 8. */
lr_status rmsnorm_online(const lr_dims* dims, const void* x, const void* gamma, void* y,
                         float* sumsq, float* rstd, hipStream_t stream);

/* Forward of the block.
 *   x [T, d], gamma [d], A [d, g*r], B[i] [r, d]            (dtype)
 *   y[i] [T, d]  for i < n_up                                (dtype)
 *   h_save [T, g*r] (dtype): the rank-r pre-activation h, the only activation the
 *   backward needs besides x (low-rank activation checkpointing, §2.2).  NULL for
 *   inference.
 * For bf16 with small g*r (r = 64 and g <= 4, r = 128 and g <= 2, r = 256 and
 * g == 1, identity or SiLU; SwiGLU's pair at r = 64 or 128) the forward is one
 * kernel and z never reaches device memory; otherwise z is written once to the
 * workspace between the two projections. */
lr_status lr_block_fwd(const lr_dims* dims, const void* x, const void* gamma, const void* A,
                       const void* const* B, void* const* y, void* h_save,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* lr_block_fwd that also keeps the RMSNorm statistic beside the checkpoint
 * (Online-RMSNorm and low-rank activation checkpointing, §2.2: the statistic is
 * 4 bytes a token against 2*g*r for h, and lets the backward skip a pass over x).
 *   rstd_save [T] (fp32): rstd_t = (sum_j x_tj^2 / D + eps)^(-1/2), the factor
 *   that scaled row t of h; NULL behaves as lr_block_fwd.
 * Other arguments, workspace and errors as lr_block_fwd. */
lr_status lr_block_fwd_rstd(const lr_dims* dims, const void* x, const void* gamma, const void* A,
                            const void* const* B, void* const* y, void* h_save, float* rstd_save,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of the block from the saved pre-activation.
 *   inputs : x, gamma, A, B[i] as in the forward; h_saved [T, g*r] (dtype), the
 *            forward's h_save; dy[i] [T, d] (dtype), the upstream gradients.
 *   outputs: dx [T, d] (dtype); dgamma [d], dA [d, g*r], dB[i] [r, d] (fp32).
 * sigma is recomputed from h_saved (low-rank activation checkpointing, §2.2);
 * rstd is recomputed from x (one pass over x). */
lr_status lr_block_bwd(const lr_dims* dims, const void* x, const void* gamma, const void* A,
                       const void* const* B, const void* h_saved,
                       const void* const* dy, void* dx, float* dgamma, float* dA, float* const* dB,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* lr_block_bwd that takes the forward's RMSNorm statistic instead of recomputing
 * it from x (§2.2, as lr_block_fwd_rstd).
 *   rstd_saved [T] (fp32): lr_block_fwd_rstd's rstd_save for the same x; NULL
 *   behaves as lr_block_bwd.
 * Other arguments, workspace and errors as lr_block_bwd. */
lr_status lr_block_bwd_rstd(const lr_dims* dims, const void* x, const void* gamma, const void* A,
                            const void* const* B, const void* h_saved, const float* rstd_saved,
                            const void* const* dy, void* dx, float* dgamma, float* dA, float* const* dB,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Residual variant.  The block is the body of a pre-norm transformer sublayer
 * (the low-rank layers the pages train sit in LLaMA-2 models, technical summary
 * §4), whose output adds the sublayer's input back.  The add is fused into the
 * up-projection's epilogue, so y never makes a second pass through HBM:
 *   y[i] = residual[i] + z_i . B[i]
 *   residual: HOST array of n_up device pointers, residual[i] [T, d] (dtype);
 *   residual[i] may equal y[i] (in-place accumulation into the residual
 *   stream), otherwise it must not overlap any output.
 * rstd_save as lr_block_fwd_rstd (may be NULL).  With a residual the
 * small-rank shapes do not use the one-kernel forward: they run the
 * down-projection and the up-projection kernels (same workspace size).
 * LR_EINVAL when residual is NULL.  Other arguments and errors as lr_block_fwd. */
lr_status lr_block_fwd_residual(const lr_dims* dims, const void* x, const void* gamma, const void* A,
                                const void* const* B, const void* const* residual, void* const* y,
                                void* h_save, float* rstd_save, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* Backward of the residual variant: the residual path's gradient is added to
 * the block's dx in the dx epilogue.
 *   dx = (the block's dx) + dx_residual         dx_residual [T, d] (dtype)
 * For out = x + block(x) (residual[0] = x, one up-projection) pass
 * dx_residual = dy[0].  dx_residual may equal dx; it may be NULL only when T == 0
 * (LR_EINVAL otherwise).  rstd_saved as lr_block_bwd_rstd (may be NULL).  The
 * weight gradients do not depend on the residual.  Other arguments and errors
 * as lr_block_bwd. */
lr_status lr_block_bwd_residual(const lr_dims* dims, const void* x, const void* gamma, const void* A,
                                const void* const* B, const void* h_saved, const float* rstd_saved,
                                const void* const* dy, const void* dx_residual, void* dx, float* dgamma,
                                float* dA, float* const* dB, void* ws, size_t ws_bytes, hipStream_t stream);

/* Device scratch of lr_block_fwd_noalloc, per GPU: 128 MiB. */
#define LR_NOALLOC_SCRATCH_BYTES (128u << 20)

/* lr_block_fwd_rstd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a file-scope device
 * array of LR_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds
 * until the process ends; the call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).
 *   - Arguments, outputs and errors as lr_block_fwd_rstd (rstd_save may be NULL).
 *   - LR_EWORKSPACE when these dims need more than LR_NOALLOC_SCRATCH_BYTES
 *     (lr_block_workspace_size(dims, 0) > LR_NOALLOC_SCRATCH_BYTES); checked on
 *     the host, nothing launched.
 *   - `stream` must belong to the current device (LR_EINVAL otherwise).  The
 *     first call on a device looks the array's address up once (LR_EHIP if that
 *     fails).
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's
 *     contents (the forward writes every scratch byte it reads, so nothing needs
 *     clearing): calls that overlap on one GPU (two streams, or two host
 *     threads) race and must be serialised by the caller. */
lr_status lr_block_fwd_noalloc(const lr_dims* dims, const void* x, const void* gamma, const void* A,
                               const void* const* B, void* const* y, void* h_save, float* rstd_save,
                               hipStream_t stream);

/* Shard seam of bottleneck-aware tensor parallelism (§2.1: the d x r factor runs
 * row-parallel over this call's slice of d; §2.2: Online-RMSNorm keeps the local
 * statistic and defers normalisation).  On one GPU the all-reduce of the partial
 * and of sumsq that would sit between the two calls is the identity.
 *   x [T, d] (this shard's columns), gamma [d], A [d, g*r] (this shard's rows)
 *   partial [T, g*r] (fp32) = (x . diag(gamma)) . A        -- not normalised
 *   sumsq [T] (fp32)        = sum_j x_tj^2 over this shard's columns */
lr_status lr_down_partial(const lr_dims* dims, const void* x, const void* gamma, const void* A,
                          float* partial, float* sumsq, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Second half of the seam: h = partial * (sumsq / D + eps)^(-1/2) with D =
 * d_norm (the unsharded width), z = sigma(h), y[i] = z_i . B[i].
 *   partial [T, g*r], sumsq [T] (fp32); B[i] [r, d] (this shard's columns);
 *   y[i] [T, d]; h_save [T, g*r] or NULL (dtype). */
lr_status lr_up_finish(const lr_dims* dims, const float* partial, const float* sumsq,
                       const void* const* B, void* const* y, void* h_save,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes the calls above need for these dims:
 *   backward == 0: lr_block_fwd, lr_down_partial and lr_up_finish;
 *   backward != 0: lr_block_bwd.
 * Returns 0 for dims that the calls would reject. */
size_t lr_block_workspace_size(const lr_dims* dims, int backward);

/* Per-projection low-rank SwiGLU MLP: the other reading of how the block's
 * SwiGLU is wired.  The MLP sublayer of the LLaMA-2 models the pages pre-train
 * (technical summary §4) keeps SwiGLU at its full width f, and each of its
 * three linear maps is a low-rank layer of rank r with nothing between its two
 * factors (§1, §2.1).  The two input-side down factors read the same normalised
 * input and are concatenated, their up factors run as a batch (§2.2, linear
 * layer grouping); the checkpoint is the two narrow tensors h_in and h_out
 * (§2.2, low-rank activation checkpointing), from which the backward
 * recomputes gate, up and s.
 *   rstd_t = (sum_j x_tj^2 / d + eps)^(-1/2)
 *   h_in   = diag(rstd) . x . diag(gamma) . A_in         A_in = [A_g | A_u], [d, 2r]
 *   gate   = h_in[:, :r] . B_g,  up = h_in[:, r:] . B_u   B_g, B_u [r, f]
 *   s      = SiLU(gate) * up                               [T, f]
 *   h_out  = s . A_o                                       A_o [f, r]
 *   out    = h_out . B_o  (+ residual)                     B_o [r, d]
 * Element types as for the block (dims->dtype; weight gradients fp32).
 * Supported: T >= 0; d, f and r positive multiples of 64. */
typedef struct {
  int64_t T, d, f, r;   /* tokens, model width, MLP width, rank of every factorised linear */
  float eps;
  lr_dtype dtype;
} lr_mlp_dims;

/* Workspace bytes of lr_mlp_fwd (backward == 0) or lr_mlp_bwd (backward != 0);
 * 0 for dims the calls would reject.  The forward holds gate and s, the
 * backward gate, up and s ([T, f] each). */
size_t lr_mlp_workspace_size(const lr_mlp_dims* dims, int backward);

/* Forward.  x [T, d], gamma [d], A_in [d, 2r], B_g and B_u [r, f], A_o [f, r],
 * B_o [r, d]; out [T, d].  residual [T, d] or NULL (none), may equal out.
 * h_in_save [T, 2r], h_out_save [T, r] (the checkpoint) and rstd_save [T] (fp32)
 * may each be NULL (inference).  Errors as lr_block_fwd. */
lr_status lr_mlp_fwd(const lr_mlp_dims* dims, const void* x, const void* gamma, const void* A_in,
                     const void* B_g, const void* B_u, const void* A_o, const void* B_o,
                     const void* residual, void* out, void* h_in_save, void* h_out_save, float* rstd_save,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward for the upstream gradient dout [T, d].  h_in_saved and h_out_saved
 * are the forward's checkpoint; rstd_saved [T] or NULL (recomputed from x).
 * dx [T, d] (dtype) = the MLP's input gradient (+ dx_residual [T, d] when
 * non-NULL; for out = x + mlp(x) pass dout, and dx_residual may equal dx).
 * Weight gradients (fp32, overwritten): dgamma [d], dA_in [d, 2r], dB_g and
 * dB_u [r, f], dA_o [f, r], dB_o [r, d].  Errors as lr_block_bwd. */
lr_status lr_mlp_bwd(const lr_mlp_dims* dims, const void* x, const void* gamma, const void* A_in,
                     const void* B_g, const void* B_u, const void* A_o, const void* B_o,
                     const void* h_in_saved, const void* h_out_saved, const float* rstd_saved,
                     const void* dout, const void* dx_residual, void* dx, float* dgamma, float* dA_in,
                     float* dB_g, float* dB_u, float* dA_o, float* dB_o, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Kernel timing for benchmarks (not part of the block's arithmetic).
 * Between lr_trace_begin and lr_trace_end, every kernel that an entry point
 * launches from the CALLING THREAD whose name matches `kernel` (NULL: all) is
 * bracketed by two hipEvents recorded on the launch stream, up to
 * `max_launches` launches.  Kernel names: "fold_gamma" (every weight fold),
 * "down", "up", "fused" (the one-kernel forward), "finish", "rms_stats", "dz",
 * "wgrad", "wgrad_reduce", "sum_parts", "dx".  This
 * per-thread trace is the only state the library keeps between calls; it owns
 * its events.
 *   lr_trace_begin: LR_EINVAL if max_launches is outside [1, 65536], a trace is
 *                   already active or its host arrays cannot be allocated;
 *                   LR_EHIP if events cannot be created.
 *   lr_trace_count: launches recorded so far (0 when no trace is active).
 *   lr_trace_elapsed: waits for launch i's end event; writes its kernel name
 *                   (static string) and duration in milliseconds.
 *   lr_trace_end:   destroys the events (the stream must have passed them). */
lr_status lr_trace_begin(const char* kernel, int max_launches);
int lr_trace_count(void);
lr_status lr_trace_elapsed(int i, const char** kernel, float* ms);
lr_status lr_trace_end(void);

/* Static, NUL-terminated name of a status code. */
const char* lr_status_str(lr_status status);

#ifdef __cplusplus
}
#endif

#endif /* LR_BLOCK_H */

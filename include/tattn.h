/*
 * tattn -- tiled fused attention forward for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libtattn.so. Every entry point is asynchronous: it validates its
 * arguments on the host, enqueues kernels on `stream` and returns. Nothing is
 * launched and nothing is written when validation fails. Errors raised by the
 * device while the kernels run surface at the caller's next synchronisation
 * on that stream. No entry point synchronises the device.
 *
 * Pointers named as device pointers must point to device memory (for example
 * from hipMalloc or torch on a ROCm device); `stream` is a hipStream_t passed
 * as void* (NULL selects the default stream of the current device). Kernels
 * run on the calling thread's current device: the pointers and the stream
 * must belong to it (the library cannot check that). The
 * library never frees, retains or reallocates caller memory; outputs are
 * fully overwritten (never accumulated into). Calls are reentrant and may be
 * issued concurrently on different streams. attn_fwd, attn_fwd_ex,
 * attn_fwd_f32 and ssd_scan allocate nothing and issue only kernel launches,
 * so they may be captured into a HIP graph, and so does mla_decode_noalloc;
 * mla_decode keeps device workspaces per stream (see its description).
 *
 * bf16 tensors are raw IEEE bfloat16 bit patterns (uint16 storage). All
 * tensors are dense, row-major (last index fastest), with no padding.
 *
 * Source of the method: the four TileLang web pages this library is based
 * on. "TileLang study notes" (section "FlashAttention implementation") gives
 * the attention definition S = Q*K^T, P = softmax(S), O = P*V and the
 * online-softmax recurrence; "TileLang programming model and FlashMLA"
 * (sections 2.1-2.2, 3.1) gives the MLA decode kernel with its exp2 softmax
 * and running log-sum. The state-space scan (ssd_scan) is the Mamba-2
 * chunk-state / chunk-scan workload named in "TileLang paper summary"
 * (appendix A.4) and sketched as a tiled scan in "From FlashAttention to
 * general kernels" (section 4).
 */
#ifndef TATTN_H
#define TATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define TATTN_OK               0   /* enqueued (or nothing to do)                       */
#define TATTN_ERR_INVALID_ARG (-1) /* null pointer, negative size, non-finite scale ... */
#define TATTN_ERR_UNSUPPORTED (-2) /* valid request outside the supported shapes        */
#define TATTN_ERR_ALIGN       (-3) /* a pointer misses its required alignment           */
#define TATTN_ERR_OOM         (-4) /* device workspace could not be allocated           */
#define TATTN_ERR_HIP         (-5) /* no usable HIP device, or a launch failed           */
#define TATTN_ERR_SCRATCH     (-6) /* mla_decode_noalloc: workspace above its static cap */

/*
 * attn_fwd -- multi-head attention forward, bf16 in, fp32 accumulate.
 *
 * Computes, for every batch b < B, head h < H and query row i < Sq,
 *   O[b,h,i,:]  = sum_j P_ij * V[b,h,j,:],  P_ij = exp(s_ij) / sum_j' exp(s_ij'),
 *   LSE[b,h,i]  = ln sum_j exp(s_ij),       s_ij = scale * Q[b,h,i,:] . K[b,h,j,:],
 * over the keys j the row may see: all j < Skv, or with causal != 0 the keys
 * j <= i + (Skv - Sq) (the mask is aligned to the bottom-right corner; for
 * Sq == Skv this is j <= i). This is the attention definition and the online
 * softmax recurrence of "TileLang study notes", section "FlashAttention
 * implementation"; LSE is the running log-sum ("logsum") of "TileLang
 * programming model and FlashMLA", section 3.1, in natural-log units.
 * The score matrix never reaches memory.
 *
 *   q   device, bf16 [B, H, Sq,  D], 16-byte aligned, read only
 *   k   device, bf16 [B, H, Skv, D], 16-byte aligned, read only
 *   v   device, bf16 [B, H, Skv, D], 16-byte aligned, read only
 *   o   device, bf16 [B, H, Sq,  D], 16-byte aligned, written (RNE from fp32)
 *   lse device, fp32 [B, H, Sq],      4-byte aligned, written
 *   B, H, Sq >= 0 (any of them 0: nothing to do, TATTN_OK); Skv >= 0
 *   D   head dimension: 64 or 128 (else TATTN_ERR_UNSUPPORTED)
 *   causal 0 or 1; scale finite and > 0 (typically 1/sqrt(D)), else
 *   TATTN_ERR_INVALID_ARG
 *
 * A row that sees no key (Skv == 0, or causal rows with i + Skv - Sq < 0)
 * gets O = 0 and LSE = -inf. q/k/v may overlap each other; o and lse must
 * not overlap any input or each other.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Sq, int Skv, int D, int causal, float scale,
             void* stream);

/*
 * attn_fwd_ex -- attn_fwd with the attention variants of "TileLang
 * programming model and FlashMLA", section 5.1 (other attention variants):
 * grouped or single KV heads (multi-query), a sliding key window (local
 * attention) and a block mask (sparse attention). With Hkv == H, window == 0 and block_mask == NULL it
 * computes exactly what attn_fwd computes.
 *
 *   k, v       device, bf16 [B, Hkv, Skv, D]; query head h reads KV head
 *              h / (H / Hkv). Hkv >= 1 and H a multiple of Hkv, else
 *              TATTN_ERR_INVALID_ARG.
 *   window     0: no window. W > 0: row i sees only keys j with
 *              pos - W <= j < pos + W, pos = i + (Skv - Sq) (the key loop of
 *              the local-attention example runs from the query position minus
 *              the window size to the query position plus it), intersected
 *              with the causal rule when causal != 0. Negative: INVALID_ARG;
 *              above 2^30: UNSUPPORTED.
 *   block_mask NULL, or device uint8 [B, H, ceil(Sq/64), ceil(Skv/64)],
 *              read only: the (64-row query block, 64-key block) pairs whose
 *              byte is 0 are not computed (their scores count as -inf).
 *              Any alignment.
 *   everything else as attn_fwd (same layouts of q, o, lse; D 64 or 128).
 *
 * A row that sees no key (window, causal rule and mask together) gets O = 0
 * and LSE = -inf. Grouped heads run at the speed of attn_fwd; with a window
 * or a mask the kernel visits only the 32-key tiles some row of a 128-row
 * query tile (two 64-row mask blocks) can see.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int Hkv, int Sq, int Skv, int D, int causal, int window,
                const uint8_t* block_mask, float scale, void* stream);

/*
 * attn_fwd_f32 -- the same operation as attn_fwd with fp32 q, k, v and o
 * (fp32 arithmetic throughout). Same arguments, layouts, masking, edge
 * cases and status codes; q, k, v, o are fp32 and 16-byte aligned.
 * D is 64 or 128.
 */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                 int B, int H, int Sq, int Skv, int D, int causal, float scale,
                 void* stream);

/*
 * mla_decode -- multi-head latent attention decode (one query position per
 * batch), bf16 in, fp32 accumulate.
 *
 * "TileLang programming model and FlashMLA" (sections 2.1-2.2, 3.1): the H
 * query heads of a batch share one KV head made of a 512-wide latent part
 * KV and a 64-wide rotary part K_pe. For batch b, head h and key j of that
 * batch, s_hj = scale * (Q[b,h,:] . KV[j,:] + Q_pe[b,h,:] . K_pe[j,:]);
 * the values are the latent rows themselves, so
 *   O[b,h,:]  = sum_j P_hj * KV[j,:],  LSE[b,h] = ln sum_j exp(s_hj).
 *
 * Keys of all batches are packed back to back: batch b owns rows
 * kv_indptr[b] <= j < kv_indptr[b+1] of kv and k_pe.
 *
 *   q         device, bf16 [B, H, 512], 16-byte aligned
 *   q_pe      device, bf16 [B, H, 64],  16-byte aligned
 *   kv        device, bf16 [N, 512],    16-byte aligned, N = kv_indptr[B]
 *   k_pe      device, bf16 [N, 64],     16-byte aligned
 *             (kv and k_pe may be NULL when N = 0: no batch has keys)
 *   o         device, bf16 [B, H, 512], 16-byte aligned, written
 *   lse       device, fp32 [B, H],      4-byte aligned, written
 *   B >= 0 (0: nothing to do); 1 <= H <= 128 (else TATTN_ERR_UNSUPPORTED)
 *   kv_indptr device, int32 [B+1], 4-byte aligned, read on the device only:
 *             kv_indptr[0] >= 0 and non-decreasing; the caller guarantees
 *             that rows up to kv_indptr[B] exist. A decreasing pair is
 *             treated as an empty batch.
 *   scale     finite and > 0 (typically 1/sqrt(576)), else TATTN_ERR_INVALID_ARG
 *
 * A batch with no keys gets O = 0 and LSE = -inf. Work is split along the
 * packed key axis over the GPU's compute units; each piece writes a
 * normalised partial output and its log-sum-exp into a device workspace
 * ((CUs + B) * H * (512 * 2 + 4) bytes plus the split plan), and a second
 * kernel merges the pieces of each batch. The library keeps one such
 * workspace per (device, stream) for the life of the process, for up to 8
 * streams per device: a call that needs more than its stream's workspace
 * holds allocates a larger one with hipMalloc (TATTN_ERR_OOM if that fails)
 * and frees the old one at a later call, once that buffer's last kernels
 * have finished (the host never waits for them); any other call allocates
 * nothing. Calls on different streams use different workspaces and do not
 * wait for each other; a ninth stream takes over the least recently used
 * stream's workspace and first waits for that stream's last call: on the
 * device, or, if that call came while its stream was the only one with a
 * workspace on the device, on the host until the device has finished its
 * work: the one case in which this call blocks the host, and at most once
 * per device (only a device's first workspace can be left in that state).
 */
int mla_decode(const void* q, const void* q_pe, const void* kv, const void* k_pe,
               void* o, float* lse, int B, int H, const int32_t* kv_indptr,
               float scale, void* stream);

/*
 * mla_decode_noalloc -- mla_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, layouts, results and status codes as
 * mla_decode (same kernels, bit-identical output); it allocates nothing,
 * creates no event and only enqueues kernel launches on `stream`.
 *
 * Its workspace (the split plan and the per-piece partial outputs, the
 * same (CUs + B) * H * (512 * 2 + 4) bytes plus the plan that mla_decode
 * needs) is a static array of 64 MiB inside the library, one per GPU the
 * library runs on, held until the process ends. A request whose workspace
 * exceeds 64 MiB returns TATTN_ERR_SCRATCH before any launch (on a 256-CU
 * MI355X at H = 128 that is more than about 250 batches). Every call on one
 * GPU uses that GPU's array and leaves its contents behind: calls whose
 * kernels overlap on one GPU (different streams without ordering between
 * them) race and give wrong results; calls ordered on one stream are safe.
 */
int mla_decode_noalloc(const void* q, const void* q_pe, const void* kv, const void* k_pe,
                       void* o, float* lse, int B, int H, const int32_t* kv_indptr,
                       float scale, void* stream);

/*
 * ssd_scan -- Mamba-2 state-space scan (chunk state, state passing and chunk
 * scan fused into one pass), bf16 in and out, fp32 state.
 *
 * The linear-attention workload of "TileLang paper summary" (appendix A.4:
 * Mamba-2's chunk-scan and chunk-state functions), walked in chunks of 64
 * steps like the tiled Mamba scan of "From FlashAttention to general
 * kernels" (section 4). For every batch b < batch and head h < heads, with
 * group g = h / (heads / groups) and state S (headdim x dstate, fp32):
 *   S_t = exp(dt[b,t,h] * A[h]) * S_{t-1} + dt[b,t,h] * x[b,t,h,:] (outer) B[b,t,g,:]
 *   y[b,t,h,:] = S_t * C[b,t,g,:]
 * for t = 0 .. seqlen-1, starting from S_{-1} = init_state[b,h] (zero when
 * init_state is NULL). The scan runs chunk by chunk: inside a chunk the
 * outputs come from one causal, decay-weighted product against the chunk's
 * own steps plus the decayed entering state; the state then advances by the
 * chunk's contribution. The state never leaves the GPU between chunks.
 *
 *   x           device bf16 [batch, seqlen, heads, headdim]
 *   dt          device fp32 [batch, seqlen, heads], step sizes (> 0 in
 *               Mamba-2; any finite value is accepted and used as given)
 *   A           device fp32 [heads], decay rates (< 0 in Mamba-2)
 *   B, C        device bf16 [batch, seqlen, groups, dstate]
 *   y           device bf16 [batch, seqlen, heads, headdim], written
 *   init_state  device fp32 [batch, heads, headdim, dstate] or NULL
 *   final_state device fp32 [batch, heads, headdim, dstate] or NULL; when
 *               given, receives S_{seqlen-1} (init_state, or zero, when
 *               seqlen == 0). It must not overlap init_state.
 *   batch, seqlen, heads >= 0; groups >= 1 dividing heads (else
 *               TATTN_ERR_INVALID_ARG)
 *   headdim     64, dstate 128 (else TATTN_ERR_UNSUPPORTED)
 * Alignment: x, B, C, y, init_state and final_state 16 bytes, dt and A 4
 * bytes (else TATTN_ERR_ALIGN). batch * seqlen * heads * headdim must stay
 * below 2^62 elements and batch * heads below 2^31 (else
 * TATTN_ERR_UNSUPPORTED). y is rounded to bf16 once, at the end; the state
 * enters the products with C as bf16, and the decay-weighted B of a chunk
 * enters the state update as bf16, like the reference Mamba-2 kernels.
 */
int ssd_scan(const void* x, const float* dt, const float* A, const void* B, const void* C, void* y,
             const float* init_state, float* final_state, int batch, int seqlen, int heads,
             int groups, int headdim, int dstate, void* stream);

/* Static, NUL-terminated description of a status code ("unknown status"
 * for a value that is not one of the codes above). Never returns NULL. */
const char* tattn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* TATTN_H */

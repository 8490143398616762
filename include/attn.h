/*
 * attn.h — C ABI of libattn.so, a fused scaled dot-product attention forward
 * pass (and its backward pass, attn_bwd) for AMD Instinct MI355X (gfx950).
 *
 * Operation. For every batch b, query head h and query row i:
 *
 *     out[b,i,h,:] = sum_j softmax_j( scale * <q[b,i,h,:], k[b,j,g,:]> ) * v[b,j,g,:]
 *
 * with g = h / (Hq / Hkv), the formula softmax(Q K^T / sqrt(d_k)) V of the
 * codelab "Accelerate attention on GPU with cuDNN and TransformerEngine",
 * §1 "How attention works", computed in the four steps listed there (score,
 * scale + softmax over keys, weighted sum of V, output shaped like Q).
 *   - causal = 1 applies the lower-triangular mask of §7 "Add a causal
 *     mask": key j is visible to query i iff j <= i (top-left alignment when
 *     Sq != Skv; every row sees key 0, so no row is ever fully masked).
 *   - causal = 2 is the same mask aligned to the bottom-right corner, the
 *     key-value-cache form of the inference use §9 motivates GQA / MQA with:
 *     the Sq queries are the last Sq of Skv tokens, so key j is visible to
 *     query i iff j <= i + Skv - Sq. It needs Sq <= Skv. With Sq == Skv it
 *     is the causal = 1 mask.
 *   - Hkv < Hq is the MHA / GQA / MQA broadcast of §9 "Compare MHA, GQA and
 *     MQA": contiguous groups of Hq / Hkv query heads share one K/V head.
 *   - The kernel is fused in the sense of §5-§6 of the codelab: one launch,
 *     the (Sq x Skv) score and weight matrices never reach device memory.
 *
 * Layout. Contiguous (B, S, H, D) as in §3 "Create Q, K, V test arrays":
 *   q, out : [B][Sq][Hq][D]        element (b,i,h,d) at ((b*Sq+i)*Hq+h)*D+d
 *   k, v   : [B][Skv][Hkv][D]
 * All four pointers are device pointers, 16-byte aligned.
 *
 * Arithmetic. Inputs are read in their own type; scores, softmax statistics
 * and the output accumulator are float32; the attention weights enter the
 * second product in the input type (bf16 / f16; bf16 on the FP8 path); the
 * output is rounded to nearest even once at the end.
 *
 * Ownership and synchronisation. The caller allocates and owns every buffer,
 * including the workspace of attn_fwd_split. The library allocates nothing,
 * keeps no pointer after it returns and never synchronises: a call validates
 * its arguments on the host, enqueues its kernel(s) on `stream` and returns.
 * ATTN_OK means "enqueued". Calls are stateless and may be made from several
 * host threads at once (two calls sharing one workspace must be ordered, as
 * for any buffer).
 *
 * Errors. Every entry point returns 0 or a negative attn_status. Arguments are
 * validated before any HIP call, so a rejected call launches nothing and
 * touches no device state. There is no fallback path: unsupported input is an
 * error, never a slower route (the codelab's §6 notes that a forced fused
 * backend raises rather than silently falling back; this library does the
 * same).
 */
#ifndef ATTN_MI355X_ATTN_H
#define ATTN_MI355X_ATTN_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. ATTN_FP8_E4M3 is the OCP 8-bit E4M3 format ("E4M3FN":
 * bias 7, no infinities, largest finite 448), the forward-pass FP8 format of
 * the codelab's §10. */
enum attn_dtype {
    ATTN_F32 = 0,      /* q, k, v, out: float32                    */
    ATTN_BF16 = 1,     /* q, k, v, out: bfloat16                   */
    ATTN_F16 = 2,      /* q, k, v, out: IEEE binary16              */
    ATTN_FP8_E4M3 = 3, /* q, k, v: E4M3 codes; out: bfloat16       */
    ATTN_FP8_E5M2 = 4  /* OCP E5M2 codes (gradients; see attn_bwd_fp8
                          and the FP8 scaling state)                 */
};

enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,       /* a pointer argument is NULL                     */
    ATTN_ERR_SHAPE = -2,      /* B < 0, Sq < 0, Hq/Hkv/D <= 0, or Skv < 1 with
                                 B*Sq > 0, or a tensor exceeds 2^31 elements     */
    ATTN_ERR_GROUP = -3,      /* Hq is not a multiple of Hkv                    */
    ATTN_ERR_HEAD_DIM = -4,   /* D is not 32, 64 or 128 (E4M3: not 64 or 128)  */
    ATTN_ERR_DTYPE = -5,      /* unknown dtype, or ATTN_FP8_E4M3 given to
                                 attn_fwd (FP8 needs attn_fwd_fp8's descales)   */
    ATTN_ERR_ALIGN = -6,      /* a pointer is not 16-byte aligned               */
    ATTN_ERR_ALIAS = -7,      /* an output (out, lse, a gradient) overlaps an
                                 input or another output                        */
    ATTN_ERR_SCALE = -8,      /* scale or a descale is NaN or infinite          */
    ATTN_ERR_HIP = -9,        /* the kernel launch failed (hipGetLastError)     */
    ATTN_ERR_CAUSAL = -10,    /* causal is not 0, 1 or 2, or causal = 2 with
                                 Sq > Skv                                       */
    ATTN_ERR_SPLIT = -11,     /* n_split outside 1 .. ATTN_MAX_SPLIT            */
    ATTN_ERR_WORKSPACE = -12, /* workspace NULL, misaligned, too small, or
                                 overlapping an input or an output              */
    ATTN_ERR_STRIDE = -13,    /* a stride is negative or above 2^40, or out's
                                 strides map two elements to one address        */
    ATTN_ERR_SCRATCH = -14    /* attn_fwd_split_noalloc: the call needs more
                                 than ATTN_NOALLOC_SCRATCH_BYTES of scratch     */
};

/* Largest number of key ranges attn_fwd_split accepts. */
#define ATTN_MAX_SPLIT 256

/*
 * attn_fwd — out = softmax(scale * q k^T [+ causal mask]) v.
 *
 *   q, k, v  device pointers to the inputs, element type `dtype`, layout above
 *   out      device pointer to the output, element type `dtype`; must not
 *            overlap any input
 *   B        batch size (>= 0)
 *   Hq, Hkv  query heads and K/V heads (> 0, Hq % Hkv == 0)
 *   Sq, Skv  query and key/value sequence lengths (Sq >= 0; Skv >= 1 unless
 *            B * Sq == 0)
 *   D        head dimension: 32, 64 or 128 (attn_fwd_fp8: 64 or 128)
 *   scale    any finite float; the codelab uses 1 / sqrt(D) (§4)
 *   causal   0 = full attention, 1 = lower-triangular mask (§7), 2 = the same
 *            mask aligned bottom-right (Sq <= Skv; see above)
 *   dtype    ATTN_F32, ATTN_BF16 or ATTN_F16
 *   stream   HIP stream the kernel is enqueued on (0 = null stream)
 *
 * B * Sq == 0 is a successful no-op that launches nothing.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out,
             int B, int Hq, int Hkv, int Sq, int Skv, int D,
             float scale, int causal, int dtype, hipStream_t stream);

/*
 * attn_fwd_lse — attn_fwd that also stores, for every row, the natural-log
 * log-sum-exp of its visible scaled scores:
 *
 *     lse[b,h,i] = log( sum_j exp( scale * <q[b,i,h,:], k[b,j,g,:]> ) )
 *
 * over the keys j the mask leaves visible. It is the normaliser of the
 * softmax (weights = exp(score - lse)), kept so that a backward pass can
 * rebuild the weights without another pass over the keys; the codelab's §1
 * motivates the scale by the softmax's gradients.
 *
 *   lse      device pointer to float32 [B][Hq][Sq], 4-byte aligned, not
 *            overlapping q, k, v or out
 *   dtype    ATTN_F32, ATTN_BF16 or ATTN_F16
 *
 * Other arguments and errors as attn_fwd (ATTN_ERR_NULL for a NULL lse).
 * The output equals attn_fwd's bit for bit.
 */
int attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int Hq, int Hkv, int Sq, int Skv, int D,
                 float scale, int causal, int dtype, hipStream_t stream);

/*
 * attn_fwd_fp8 — the same operation on E4M3 inputs, bfloat16 output.
 *
 * q, k and v hold E4M3 codes with per-tensor dequantisation factors
 * (the codelab's §10 recipe with margin 0 gives x ~ code * (amax / 448)):
 * the operation is computed on q_descale * q, k_descale * k and
 * v_descale * v. The products q.k run on FP8 matrix cores with
 * scale * q_descale * k_descale folded into the softmax; v is widened to
 * bfloat16 exactly and v_descale is folded into the final normalisation.
 * Descales must be finite. Arguments and errors are otherwise those of
 * attn_fwd; out is bfloat16, [B][Sq][Hq][D].
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* out,
                 int B, int Hq, int Hkv, int Sq, int Skv, int D,
                 float scale, int causal,
                 float q_descale, float k_descale, float v_descale,
                 hipStream_t stream);

/*
 * attn_fwd_fp8_lse — attn_fwd_fp8 that also stores the row log-sum-exp of
 * the scaled scores on the dequantised inputs (scale * q_descale * k_descale
 * * q.k), as attn_fwd_lse does: float32 [B][Hq][Sq], 4-byte aligned, not
 * overlapping q, k, v or out. Arguments and errors otherwise as
 * attn_fwd_fp8; the output equals attn_fwd_fp8's bit for bit.
 */
int attn_fwd_fp8_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Skv, int D,
                     float scale, int causal,
                     float q_descale, float k_descale, float v_descale,
                     hipStream_t stream);

/*
 * attn_fwd_split — attn_fwd with the keys of every query row cut into
 * n_split contiguous ranges that separate workgroups process, followed by a
 * combine kernel (split-key or "flash-decoding" form). For grids too small
 * to fill the GPU: few query rows against many keys, as in key-value-cache
 * inference (§9). The result is the same softmax over all keys (each
 * range's partial sums are rescaled to a common maximum before the one
 * division), up to float rounding.
 *
 *   n_split    number of key ranges, 1 .. ATTN_MAX_SPLIT (attn_split_suggest
 *              gives a value for the shape); 1 is exactly attn_fwd and needs
 *              no workspace
 *   workspace  device buffer of at least attn_split_workspace(...) bytes,
 *              16-byte aligned, not overlapping q, k, v or out; its contents
 *              on entry do not matter and are undefined after the call
 *   workspace_bytes  its size
 *   dtype      ATTN_BF16 or ATTN_F16
 *
 * Other arguments and errors as attn_fwd. Two kernels are enqueued on
 * `stream` (the ranges, then the combine).
 */
int attn_fwd_split(const void* q, const void* k, const void* v, void* out,
                   int B, int Hq, int Hkv, int Sq, int Skv, int D,
                   float scale, int causal, int dtype, int n_split,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* attn_split_workspace — bytes of workspace attn_fwd_split needs:
 * n_split * B * Sq * Hq * (D + 2) * 4 (float32 partial outputs, maxima and
 * weight sums); 0 for n_split <= 1 or an empty problem. */
size_t attn_split_workspace(int B, int Hq, int Sq, int D, int n_split);

/* Bytes of the device array that attn_fwd_split_noalloc uses in place of a
 * workspace (32 MiB per GPU the library runs on). */
#define ATTN_NOALLOC_SCRATCH_BYTES (32 << 20)

/*
 * attn_fwd_split_noalloc — attn_fwd_split for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc. It takes no workspace: the key ranges'
 * partial results go to a file-scope device array of
 * ATTN_NOALLOC_SCRATCH_BYTES, which each GPU holds from the library's first
 * use on it until the process ends. The call allocates and frees nothing.
 *
 * Arguments as attn_fwd_split without workspace and workspace_bytes; the
 * device is the current one (the stream must belong to it). The result
 * equals attn_fwd_split's bit for bit (same kernels). Errors as
 * attn_fwd_split, plus ATTN_ERR_SCRATCH when attn_split_workspace(B, Hq, Sq,
 * D, n_split) exceeds ATTN_NOALLOC_SCRATCH_BYTES (checked before anything
 * else, on the host), and ATTN_ERR_HIP if the array's address cannot be
 * obtained. All calls on one GPU share its array: calls that overlap in time
 * on one GPU (e.g. on two streams) race and must be ordered by the caller.
 */
int attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* out,
                           int B, int Hq, int Hkv, int Sq, int Skv, int D,
                           float scale, int causal, int dtype, int n_split, hipStream_t stream);

/* attn_split_suggest — a key-range count for attn_fwd_split that fills the
 * GPU for this shape (1 when attn_fwd alone already does). Arguments as
 * attn_fwd; returns 1 for shapes attn_fwd would reject. */
int attn_split_suggest(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal);

/*
 * attn_fwd_strided — attn_fwd on tensors with arbitrary batch, sequence and
 * head strides (the head dimension D must be contiguous): e.g. (B, H, S, D)
 * tensors seen as (B, S, H, D), slices of a packed QKV buffer, or K and V
 * shared by every batch (batch stride 0). The layout sensitivity of fused
 * kernels is noted in §3 of the codelab.
 *
 *   q_strides, k_strides, v_strides, out_strides
 *            host pointers to 3 element strides each: batch, sequence, head
 *            (element (b, i, h, d) of q is q[b*s0 + i*s1 + h*s2 + d]); each
 *            stride in [0, 2^40], times the element size a multiple of 16
 *            bytes; out's strides must give every output element its own
 *            address, and out's span must not overlap any input's span
 *   dtype    ATTN_F32, ATTN_BF16 or ATTN_F16
 *
 * Other arguments and errors as attn_fwd; additionally ATTN_ERR_STRIDE, and
 * ATTN_ERR_SHAPE when (Skv - 1) * key stride + D elements of one head span
 * 2^32 bytes or more.
 */
int attn_fwd_strided(const void* q, const void* k, const void* v, void* out,
                     int B, int Hq, int Hkv, int Sq, int Skv, int D,
                     const int64_t* q_strides, const int64_t* k_strides,
                     const int64_t* v_strides, const int64_t* out_strides,
                     float scale, int causal, int dtype, hipStream_t stream);

/*
 * attn_bwd — gradients of the forward pass: with L = sum(dout * out) for
 * out = attn_fwd(q, k, v) (same scale, causal mask and head grouping),
 *
 *     dq = dL/dq,  dk = dL/dk,  dv = dL/dv.
 *
 * The codelab's §1 motivates the scale by the softmax's gradients, which
 * vanish when the scores saturate it. Writing S = scale q k^T (masked
 * entries -inf), P = softmax(S) = exp(S - lse), dP = dout v^T and
 * Delta_i = rowsum(dout_i * out_i) (equal to rowsum(P_i * dP_i)):
 *
 *     dS = P * (dP - Delta),  dv = P^T dout,  dk = scale dS^T q,  dq = scale dS k,
 *
 * with dk and dv of a K/V head summed over the query heads that share it
 * (§9). Products run on matrix cores in the input type with float32
 * accumulation; P and dS enter them rounded to the input type; the
 * gradients are rounded once at the end. The result is deterministic (no
 * atomics).
 *
 *   q, k, v   the forward's inputs (device, layout above)
 *   out       the forward's output, [B][Sq][Hq][D]
 *   dout      gradient of the loss with respect to out, [B][Sq][Hq][D]
 *   lse       the forward's row log-sum-exp from attn_fwd_lse, float32
 *             [B][Hq][Sq], 4-byte aligned
 *   dq        output, [B][Sq][Hq][D]
 *   dk, dv    outputs, [B][Skv][Hkv][D] (written in full: keys no query
 *             sees get 0)
 *   dtype     ATTN_BF16 or ATTN_F16 (every tensor above but lse)
 *   workspace device buffer of at least attn_bwd_workspace(B, Hq, Sq)
 *             bytes, 16-byte aligned; holds per-row values between the
 *             two kernels; contents on entry do not matter
 *   workspace_bytes  its size
 *
 * The outputs and the workspace must not overlap an input or each other
 * (ATTN_ERR_ALIAS; ATTN_ERR_WORKSPACE for the workspace). Other arguments
 * and errors as attn_fwd. B * (Sq + Skv) == 0 is a no-op; Sq == 0 with
 * Skv > 0 writes zero dk and dv. Pointers to empty tensors may be NULL (q,
 * out, dout, lse, dq when B * Sq == 0; k, v, dk, dv when B * Skv == 0).
 * Two kernels are enqueued on `stream`.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Sq, int Skv, int D,
             float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
             hipStream_t stream);

/* attn_bwd_workspace — bytes of workspace attn_bwd needs: 2 * B * Hq * Sq * 4
 * (per query row, float32 Delta and lse * log2(e)); 0 for an empty problem. */
size_t attn_bwd_workspace(int B, int Hq, int Sq);

/*
 * attn_bwd_fp8 — attn_bwd for the FP8 forward: q, k, v are the E4M3 codes
 * attn_fwd_fp8 took, and the incoming gradient dout is in E5M2, the FP8
 * format the codelab's §10 names for the backward pass (gradients): OCP
 * E5M2, bias 15, largest finite 57344, with infinities and NaNs. Each has a
 * per-tensor dequantisation factor (real value = code * descale), so the
 * gradients are those of attn_bwd on q_descale * q, k_descale * k,
 * v_descale * v and do_descale * dout.
 *
 *   out       attn_fwd_fp8's output (bfloat16), [B][Sq][Hq][D]
 *   lse       attn_fwd_fp8_lse's row log-sum-exp, float32 [B][Hq][Sq]
 *   dq, dk, dv  outputs, bfloat16, shapes of q, k, v
 *   *_descale finite float32 factors
 *   workspace at least attn_bwd_fp8_workspace(...) bytes, 16-byte aligned
 *
 * Every code is first widened to bfloat16 (exactly: both formats' values
 * are bfloat16 values) into the workspace; the products then run as in
 * attn_bwd on the codes, with the descales folded into the score scale, into
 * dP and Delta, and into the final factors of dq, dk and dv. D is 64 or
 * 128, as for attn_fwd_fp8. Other arguments and errors as attn_bwd.
 */
int attn_bwd_fp8(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal,
                 float q_descale, float k_descale, float v_descale, float do_descale,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* attn_bwd_fp8_workspace — bytes of workspace attn_bwd_fp8 needs: bfloat16
 * copies of q, k, v and dout (each padded to a multiple of 256 bytes) and
 * attn_bwd_workspace(B, Hq, Sq); 0 for an empty problem. */
size_t attn_bwd_fp8_workspace(int B, int Hq, int Hkv, int Sq, int Skv, int D);

/*
 * attn_bwd_fp8_dev — attn_bwd_fp8 with the four dequantisation factors read
 * on the device, from float32 device pointers (4-byte aligned), when the
 * kernels start: e.g. the scale_inv words of FP8 scaling states, so that no
 * factor travels through the host. The factors must be finite, and so must
 * their products with scale. Arguments and errors otherwise as
 * attn_bwd_fp8 (ATTN_ERR_NULL for a NULL factor pointer). The result
 * equals attn_bwd_fp8's with the same factor values, bit for bit.
 */
int attn_bwd_fp8_dev(const void* q, const void* k, const void* v, const void* out, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal,
                     const float* q_descale, const float* k_descale, const float* v_descale,
                     const float* do_descale, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * FP8 delayed scaling, kept on the device.
 *
 * The codelab's §10 runs FP8 attention under TransformerEngine's delayed
 * scaling recipe: per tensor, a history of the last 1024 absolute maxima,
 * reduced with max, margin 0, E4M3 for the forward pass and E5M2 for the
 * backward pass. One state per tensor lives in caller-owned device memory,
 * ATTN_FP8_STATE_BYTES bytes, 16-byte aligned, as 32-bit words:
 *
 *     [0] scale       (float32) the factor a cast multiplies by
 *     [1] scale_inv   (float32) 1 / scale: the dequantisation factor
 *     [2] step        (uint32)  steps completed
 *     [3] format      (uint32)  0 = E4M3, 1 = E5M2
 *     [4 .. 4 + 1024) amax history (float32), slot = step mod 1024
 *
 * A step: attn_fp8_quantize for each tensor (cast with the current scale,
 * i.e. the one derived from earlier steps; record this step's amax), the
 * attention call with the scale_inv words as device factors
 * (attn_fwd_fp8_dev / attn_bwd_fp8_dev, pointer = state + 4 bytes), then
 * attn_fp8_update. Nothing is read back by the host.
 */
#define ATTN_AMAX_HISTORY 1024
#define ATTN_FP8_STATE_BYTES (16 + 4 * ATTN_AMAX_HISTORY)

/* attn_fp8_state_bytes — ATTN_FP8_STATE_BYTES, for bindings. */
size_t attn_fp8_state_bytes(void);

/* attn_fp8_state_init — n_states consecutive states (ATTN_FP8_STATE_BYTES
 * apart) set to scale = scale_inv = 1, step 0, an all-zero history, and
 * format ATTN_FP8_E4M3 or ATTN_FP8_E5M2 (else ATTN_ERR_DTYPE). One kernel,
 * no memset (safe inside captured graphs). */
int attn_fp8_state_init(void* states, int n_states, int format, hipStream_t stream);

/* attn_fp8_quantize — codes[i] = FP8 code (the state's format) of
 * float32(x[i] * scale), nearest-even, saturating at the largest finite
 * value (448 or 57344; NaN stays NaN), for n elements of x (x_dtype
 * ATTN_F32, ATTN_BF16 or ATTN_F16), and amax(|x|) of the call folded (max)
 * into the history slot of the state's current step. x, codes and state
 * 16-byte aligned and mutually disjoint. Several calls may share a step
 * (their amaxes combine). */
int attn_fp8_quantize(const void* x, int x_dtype, void* codes, int64_t n, void* state, hipStream_t stream);

/* attn_fp8_update — for n_states consecutive states: amax = max of the
 * history; if finite and positive, scale = fmax / amax and scale_inv =
 * 1 / scale (binary32, correctly rounded); then step + 1 and the history
 * slot of the new step cleared. */
int attn_fp8_update(void* states, int n_states, hipStream_t stream);

/*
 * attn_fwd_fp8_dev — attn_fwd_fp8 (with an optional row log-sum-exp output,
 * as attn_fwd_fp8_lse; lse may be NULL) whose three dequantisation factors
 * are read on the device from float32 device pointers (4-byte aligned):
 * e.g. the scale_inv words of the q, k and v FP8 scaling states. The factors
 * must be finite, and so must scale times the q and k factors. Arguments and
 * errors otherwise as attn_fwd_fp8 (ATTN_ERR_NULL for a NULL factor
 * pointer). The output equals attn_fwd_fp8's with the same factor values,
 * bit for bit.
 */
int attn_fwd_fp8_dev(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal,
                     const float* q_descale, const float* k_descale, const float* v_descale,
                     hipStream_t stream);

/* attn_strerror — a static, human-readable description of a status code. */
const char* attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_ATTN_H */

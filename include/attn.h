/*
 * attn.h — C ABI of libattn.so, a fused scaled dot-product attention forward
 * pass for AMD Instinct MI355X (gfx950).
 *
 * Operation. For every batch b, query head h and query row i:
 *
 *     out[b,i,h,:] = sum_j softmax_j( scale * <q[b,i,h,:], k[b,j,g,:]> ) * v[b,j,g,:]
 *
 * with g = h / (Hq / Hkv), the formula softmax(Q K^T / sqrt(d_k)) V of the
 * codelab "Accelerate attention on GPU with cuDNN and TransformerEngine",
 * §1 "How attention works", computed in the four steps listed there (score,
 * scale + softmax over keys, weighted sum of V, output shaped like Q).
 *   - causal != 0 applies the lower-triangular mask of §7 "Add a causal
 *     mask": key j is visible to query i iff j <= i (top-left alignment when
 *     Sq != Skv; every row sees key 0, so no row is ever fully masked).
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
 * Ownership and synchronisation. The caller allocates and owns every buffer.
 * The library allocates nothing, keeps no pointer after it returns and never
 * synchronises: a call validates its arguments on the host, enqueues one
 * kernel on `stream` and returns. ATTN_OK means "enqueued". Calls are
 * stateless and may be made from several host threads at once.
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
    ATTN_FP8_E4M3 = 3  /* q, k, v: E4M3 codes; out: bfloat16       */
};

enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,       /* a pointer argument is NULL                     */
    ATTN_ERR_SHAPE = -2,      /* B < 0, Sq < 0, Hq/Hkv/D <= 0, or Skv < 1 with
                                 B*Sq > 0, or a tensor exceeds 2^31 elements     */
    ATTN_ERR_GROUP = -3,      /* Hq is not a multiple of Hkv                    */
    ATTN_ERR_HEAD_DIM = -4,   /* D is not 64 or 128                             */
    ATTN_ERR_DTYPE = -5,      /* unknown dtype, or ATTN_FP8_E4M3 given to
                                 attn_fwd (FP8 needs attn_fwd_fp8's descales)   */
    ATTN_ERR_ALIGN = -6,      /* a pointer is not 16-byte aligned               */
    ATTN_ERR_ALIAS = -7,      /* out overlaps q, k or v                         */
    ATTN_ERR_SCALE = -8,      /* scale or a descale is NaN or infinite          */
    ATTN_ERR_HIP = -9         /* the kernel launch failed (hipGetLastError)     */
};

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
 *   D        head dimension, 64 or 128
 *   scale    any finite float; the codelab uses 1 / sqrt(D) (§4)
 *   causal   0 = full attention, nonzero = lower-triangular mask (§7)
 *   dtype    ATTN_F32, ATTN_BF16 or ATTN_F16
 *   stream   HIP stream the kernel is enqueued on (0 = null stream)
 *
 * B * Sq == 0 is a successful no-op that launches nothing.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out,
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

/* attn_strerror — a static, human-readable description of a status code. */
const char* attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_ATTN_H */

// attn_api.cpp — the C ABI of libattn.so (declared in include/attn.h).
//
// Host side only: validates arguments without touching HIP, fills the kernel
// parameter block, picks the kernel for (dtype, D, causal) and enqueues it on
// the caller's stream. There is exactly one kernel per dtype family and no
// fallback route: anything unsupported is an error code.

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/attn.h"
#include "kernel_common.h"

namespace attn {
hipError_t launch_fwd_mfma(const FwdParams& p, int D, bool is_bf16, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int D, bool causal, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdParams& p, int D, bool causal, hipStream_t stream);
hipError_t launch_fwd_rb2(const FwdParams& p, int D, int dtype, bool causal, hipStream_t stream);
}

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;

bool ranges_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t a0 = (uintptr_t)a, a1 = a0 + (uintptr_t)na;
    const uintptr_t b0 = (uintptr_t)b, b1 = b0 + (uintptr_t)nb;
    return na > 0 && nb > 0 && a0 < b1 && b0 < a1;
}

// Shared validation of both entry points. Returns ATTN_OK or an error code;
// sets *noop when the call has nothing to compute.
int validate(const void* q, const void* k, const void* v, const void* out,
             int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
             int in_bytes, int out_bytes, bool* noop) {
    *noop = false;
    if (!q || !k || !v || !out) return ATTN_ERR_NULL;
    if (B < 0 || Sq < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Skv < 0) return ATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATTN_ERR_GROUP;
    if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if ((int64_t)B * Sq == 0) { *noop = true; return ATTN_OK; }
    if (Skv < 1) return ATTN_ERR_SHAPE;
    const int64_t nq = (int64_t)B * Sq * Hq * D;
    const int64_t nk = (int64_t)B * Skv * Hkv * D;
    if (nq >= kMaxElems || nk >= kMaxElems) return ATTN_ERR_SHAPE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return ATTN_ERR_ALIGN;
    const int64_t ob = nq * out_bytes;
    if (ranges_overlap(out, ob, q, nq * in_bytes) || ranges_overlap(out, ob, k, nk * in_bytes) ||
        ranges_overlap(out, ob, v, nk * in_bytes))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

attn::FwdParams make_params(const void* q, const void* k, const void* v, void* out,
                            int B, int Hq, int Hkv, int Sq, int Skv, float scale_log2, float out_mul,
                            bool mfma, int rows_per_wave) {
    attn::FwdParams p;
    p.q = q; p.k = k; p.v = v; p.out = out;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Skv = Skv;
    p.G = Hq / Hkv;
    // A workgroup of four waves shares one KV head between gpack query heads
    // (the largest of 4, 2, 1 dividing G) and 4 / gpack row blocks of
    // rows_per_wave rows each.
    p.gpack = mfma ? ((p.G % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1) : 1;
    p.rows_per_wg = rows_per_wave * (4 / p.gpack);
    p.n_row_blocks = (Sq + p.rows_per_wg - 1) / p.rows_per_wg;
    p.n_units = B * Hkv * (p.G / p.gpack);
    p.xcd_remap = (p.n_units % 8 == 0) ? 1 : 0;
    p.scale_log2 = scale_log2;
    p.out_mul = out_mul;
    return p;
}

const float kLog2e = 1.4426950408889634f;

// The kernels never see a zero score multiplier: scale 0 (every visible key
// weighted equally) is run with multiplier 2^-100 instead. For any score
// |s| < 2^35, exp2(s * 2^-100) rounds to exactly 1.0f, so the weights, and
// the result, are those of scale 0; and masked scores (+-inf) still map to
// -inf, which lets the kernels mask with a single select.
float nonzero_multiplier(float c) { return c == 0.0f ? 0x1p-100f : c; }

// Matrix-core kernel choice: 32 query rows per wave (two waves per SIMD) by
// default; 64 rows per wave (one wave per SIMD, half the LDS traffic per
// flop) only on request, since it measures slower on every shape so far.
// ATTN_ROWS_PER_WAVE=32 or 64 in the environment selects one explicitly
// (the tests use it to cover both kernels on every shape).
int rows_per_wave() {
    const char* e = getenv("ATTN_ROWS_PER_WAVE");
    if (e && strcmp(e, "64") == 0) return 64;
    return 32;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out,
                        int B, int Hq, int Hkv, int Sq, int Skv, int D,
                        float scale, int causal, int dtype, hipStream_t stream) {
    int eb;
    switch (dtype) {
        case ATTN_F32: eb = 4; break;
        case ATTN_BF16: case ATTN_F16: eb = 2; break;
        default: return ATTN_ERR_DTYPE;   // includes ATTN_FP8_E4M3: use attn_fwd_fp8
    }
    bool noop;
    const int st = validate(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, eb, eb, &noop);
    if (st != ATTN_OK || noop) return st;
    hipError_t e;
    if (dtype == ATTN_F32) {
        const attn::FwdParams p = make_params(q, k, v, out, B, Hq, Hkv, Sq, Skv,
                                              nonzero_multiplier(scale * kLog2e), 1.0f, false, 32);
        e = attn::launch_fwd_f32(p, D, causal != 0, stream);
    } else {
        const int rpw = rows_per_wave();
        const attn::FwdParams p = make_params(q, k, v, out, B, Hq, Hkv, Sq, Skv,
                                              nonzero_multiplier(scale * kLog2e), 1.0f, true, rpw);
        e = rpw == 64 ? attn::launch_fwd_rb2(p, D, dtype, causal != 0, stream)
                      : attn::launch_fwd_mfma(p, D, dtype == ATTN_BF16, causal != 0, stream);
    }
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fwd_fp8(const void* q, const void* k, const void* v, void* out,
                            int B, int Hq, int Hkv, int Sq, int Skv, int D,
                            float scale, int causal,
                            float q_descale, float k_descale, float v_descale,
                            hipStream_t stream) {
    bool noop;
    const int st = validate(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, 1, 2, &noop);
    if (st != ATTN_OK) return st;
    if (!isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale)) return ATTN_ERR_SCALE;
    if (noop) return ATTN_OK;
    const float sl2 = scale * q_descale * k_descale * kLog2e;
    if (!isfinite(sl2)) return ATTN_ERR_SCALE;
    const int rpw = rows_per_wave();
    const attn::FwdParams p = make_params(q, k, v, out, B, Hq, Hkv, Sq, Skv, nonzero_multiplier(sl2),
                                          v_descale, true, rpw);
    const hipError_t e = rpw == 64 ? attn::launch_fwd_rb2(p, D, ATTN_FP8_E4M3, causal != 0, stream)
                                   : attn::launch_fwd_fp8(p, D, causal != 0, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" const char* attn_strerror(int status) {
    switch (status) {
        case ATTN_OK: return "success";
        case ATTN_ERR_NULL: return "a pointer argument is NULL";
        case ATTN_ERR_SHAPE: return "invalid shape (B, Sq >= 0; Hq, Hkv, D > 0; Skv >= 1 unless B*Sq == 0; < 2^31 elements per tensor)";
        case ATTN_ERR_GROUP: return "Hq is not a multiple of Hkv";
        case ATTN_ERR_HEAD_DIM: return "head dimension D must be 64 or 128";
        case ATTN_ERR_DTYPE: return "unsupported dtype (attn_fwd takes F32, BF16, F16; E4M3 goes through attn_fwd_fp8)";
        case ATTN_ERR_ALIGN: return "q, k, v and out must be 16-byte aligned";
        case ATTN_ERR_ALIAS: return "out overlaps an input";
        case ATTN_ERR_SCALE: return "scale or a descale is not finite";
        case ATTN_ERR_HIP: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

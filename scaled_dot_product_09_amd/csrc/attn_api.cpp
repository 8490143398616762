// attn_api.cpp — the C ABI of libattn.so (declared in include/attn.h).
//
// Host side only: validates arguments without touching HIP, fills the kernel
// parameter block, picks the kernel for (dtype, D, causal) and enqueues it on
// the caller's stream. There is exactly one kernel per dtype family and no
// fallback route: anything unsupported is an error code.

#include <math.h>
#include <stdint.h>

#include "../../include/attn.h"
#include "kernel_common.h"

namespace attn {
hipError_t launch_fwd_mfma(const FwdParams& p, int D, bool is_bf16, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int D, bool causal, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdParams& p, int D, bool causal, hipStream_t stream);
hipError_t launch_combine(const FwdParams& p, int D, bool is_bf16, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& bp, int D, bool is_bf16, bool causal, hipStream_t stream);
hipError_t launch_widen_fp8(const void* in, void* out, int64_t n, bool e5m2, hipStream_t stream);
hipError_t launch_fp8_state_init(void* states, int n_states, int fmt, hipStream_t stream);
hipError_t launch_fp8_quantize(const void* x, int dtype, void* codes, int64_t n, void* state, hipStream_t stream);
hipError_t launch_fp8_update(void* states, int n_states, hipStream_t stream);
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
             int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal,
             int in_bytes, int out_bytes, bool* noop) {
    *noop = false;
    if (!q || !k || !v || !out) return ATTN_ERR_NULL;
    if (B < 0 || Sq < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Skv < 0) return ATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATTN_ERR_GROUP;
    if (D != 32 && D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
    if (D == 32 && in_bytes == 1) return ATTN_ERR_HEAD_DIM;   // one FP8 score MFMA spans 64 of D
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (causal < 0 || causal > 2) return ATTN_ERR_CAUSAL;
    if ((int64_t)B * Sq == 0) { *noop = true; return ATTN_OK; }
    if (Skv < 1) return ATTN_ERR_SHAPE;
    if (causal == 2 && Sq > Skv) return ATTN_ERR_CAUSAL;
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
                            int causal, bool mfma, int rows_per_wave, int waves, bool wide_heads = false) {
    attn::FwdParams p;
    // Bottom-right alignment shifts every query to position Skv - Sq + i.
    p.causal_off = causal == 2 ? Skv - Sq : 0;
    p.n_split = 1;
    p.part_o = nullptr;
    p.part_ml = nullptr;
    p.lse = nullptr;
    p.dsc_q = p.dsc_k = p.dsc_v = nullptr;
    p.q = q; p.k = k; p.v = v; p.out = out;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Skv = Skv;
    p.G = Hq / Hkv;
    attn::set_slot_map(p, mfma, rows_per_wave, waves, wide_heads);
    p.scale_log2 = scale_log2;
    p.out_mul = out_mul;
    return p;
}

// Dense (B, S, H, D) element strides of the batch, sequence and head axes.
void dense_strides(int64_t* st, int S, int H, int D) {
    st[0] = (int64_t)S * H * D;
    st[1] = (int64_t)H * D;
    st[2] = D;
}

void set_dense_strides(attn::FwdParams& p, int D) {
    dense_strides(p.sq, p.Sq, p.Hq, D);
    dense_strides(p.sk, p.Skv, p.Hkv, D);
    dense_strides(p.sv, p.Skv, p.Hkv, D);
    dense_strides(p.so, p.Sq, p.Hq, D);
}

const float kLog2e = 1.4426950408889634f;

// The kernels never see a zero score multiplier: scale 0 (every visible key
// weighted equally) is run with multiplier 2^-100 instead. For any score
// |s| < 2^35, exp2(s * 2^-100) rounds to exactly 1.0f, so the weights, and
// the result, are those of scale 0; and masked scores (+-inf) still map to
// -inf, which lets the kernels mask with a single select.
float nonzero_multiplier(float c) { return c == 0.0f ? 0x1p-100f : c; }

// strides: NULL (dense) or q, k, v, out element strides (batch, seq, head).
hipError_t launch_mfma(const void* q, const void* k, const void* v, void* out,
                       int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale_log2,
                       float out_mul, int dtype, int causal, const int64_t* strides, hipStream_t stream,
                       float* lse = nullptr, const float* const* dsc = nullptr) {
    attn::FwdParams p = make_params(q, k, v, out, B, Hq, Hkv, Sq, Skv, scale_log2, out_mul,
                                    causal, true, 32, 4, true);
    if (strides) {
        for (int i = 0; i < 3; ++i) {
            p.sq[i] = strides[i]; p.sk[i] = strides[3 + i]; p.sv[i] = strides[6 + i]; p.so[i] = strides[9 + i];
        }
    } else {
        set_dense_strides(p, D);
    }
    p.lse = lse;
    if (dsc) {
        p.dsc_q = dsc[0];
        p.dsc_k = dsc[1];
        p.dsc_v = dsc[2];
    }
    const bool masked = causal != 0;
    return dtype == ATTN_FP8_E4M3 ? attn::launch_fwd_fp8(p, D, masked, stream)
                                  : attn::launch_fwd_mfma(p, D, dtype == ATTN_BF16, masked, stream);
}

// Workgroups of the four-wave kernel for a shape (the unit of the split
// heuristic), and the key tiles a row block sees at most.
int64_t base_grid(int B, int Hq, int Hkv, int Sq) {
    const attn::FwdParams p = make_params(nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Sq, 1, 1.0f, 1.0f,
                                          0, true, 32, 4, true);
    return (int64_t)p.n_units * p.n_row_blocks;
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
    const int st = validate(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, eb, eb, &noop);
    if (st != ATTN_OK || noop) return st;
    hipError_t e;
    if (dtype == ATTN_F32) {
        attn::FwdParams p = make_params(q, k, v, out, B, Hq, Hkv, Sq, Skv,
                                        nonzero_multiplier(scale * kLog2e), 1.0f, causal, false, 32, 4);
        set_dense_strides(p, D);
        e = attn::launch_fwd_f32(p, D, causal != 0, stream);
    } else {
        e = launch_mfma(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, nonzero_multiplier(scale * kLog2e), 1.0f,
                        dtype, causal, nullptr, stream);
    }
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                            int B, int Hq, int Hkv, int Sq, int Skv, int D,
                            float scale, int causal, int dtype, hipStream_t stream) {
    int eb;
    switch (dtype) {
        case ATTN_F32: eb = 4; break;
        case ATTN_BF16: case ATTN_F16: eb = 2; break;
        default: return ATTN_ERR_DTYPE;
    }
    if (!lse) return ATTN_ERR_NULL;
    bool noop;
    const int st = validate(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, eb, eb, &noop);
    if (st != ATTN_OK || noop) return st;
    if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
    const int64_t nl = (int64_t)B * Hq * Sq * 4;
    const int64_t nq = (int64_t)B * Sq * Hq * D * eb, nk = (int64_t)B * Skv * Hkv * D * eb;
    if (ranges_overlap(lse, nl, q, nq) || ranges_overlap(lse, nl, k, nk) || ranges_overlap(lse, nl, v, nk) ||
        ranges_overlap(lse, nl, out, nq))
        return ATTN_ERR_ALIAS;
    hipError_t e;
    if (dtype == ATTN_F32) {
        attn::FwdParams p = make_params(q, k, v, out, B, Hq, Hkv, Sq, Skv,
                                        nonzero_multiplier(scale * kLog2e), 1.0f, causal, false, 32, 4);
        set_dense_strides(p, D);
        p.lse = lse;
        e = attn::launch_fwd_f32(p, D, causal != 0, stream);
    } else {
        e = launch_mfma(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, nonzero_multiplier(scale * kLog2e), 1.0f,
                        dtype, causal, nullptr, stream, lse);
    }
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fwd_fp8(const void* q, const void* k, const void* v, void* out,
                            int B, int Hq, int Hkv, int Sq, int Skv, int D,
                            float scale, int causal,
                            float q_descale, float k_descale, float v_descale,
                            hipStream_t stream) {
    bool noop;
    const int st = validate(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, 1, 2, &noop);
    if (st != ATTN_OK) return st;
    if (!isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale)) return ATTN_ERR_SCALE;
    if (noop) return ATTN_OK;
    const float sl2 = scale * q_descale * k_descale * kLog2e;
    if (!isfinite(sl2)) return ATTN_ERR_SCALE;
    const hipError_t e = launch_mfma(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, nonzero_multiplier(sl2), v_descale,
                                     ATTN_FP8_E4M3, causal, nullptr, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fwd_fp8_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                                int B, int Hq, int Hkv, int Sq, int Skv, int D,
                                float scale, int causal,
                                float q_descale, float k_descale, float v_descale,
                                hipStream_t stream) {
    if (!lse) return ATTN_ERR_NULL;
    bool noop;
    const int st = validate(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, 1, 2, &noop);
    if (st != ATTN_OK) return st;
    if (!isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale)) return ATTN_ERR_SCALE;
    if (noop) return ATTN_OK;
    if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
    const int64_t nl = (int64_t)B * Hq * Sq * 4;
    const int64_t nq = (int64_t)B * Sq * Hq * D, nk = (int64_t)B * Skv * Hkv * D;
    if (ranges_overlap(lse, nl, q, nq) || ranges_overlap(lse, nl, k, nk) || ranges_overlap(lse, nl, v, nk) ||
        ranges_overlap(lse, nl, out, nq * 2))
        return ATTN_ERR_ALIAS;
    const float sl2 = scale * q_descale * k_descale * kLog2e;
    if (!isfinite(sl2)) return ATTN_ERR_SCALE;
    const hipError_t e = launch_mfma(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, nonzero_multiplier(sl2), v_descale,
                                     ATTN_FP8_E4M3, causal, nullptr, stream, lse);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" size_t attn_split_workspace(int B, int Hq, int Sq, int D, int n_split) {
    if (n_split <= 1 || B <= 0 || Hq <= 0 || Sq <= 0 || D <= 0) return 0;
    return (size_t)n_split * B * Sq * Hq * (size_t)(D + 2) * sizeof(float);
}

extern "C" int attn_split_suggest(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0 || Hq % Hkv != 0 || (D != 32 && D != 64 && D != 128))
        return 1;
    // Aim at 256 workgroups (one per CU), with at least four 64-key tiles per
    // range. Measured on decode shapes (one to four queries, 4K to 64K keys,
    // GQA and MQA): more ranges than that cost more in partial results and
    // short ranges than they gain in parallelism.
    const int64_t base = base_grid(B, Hq, Hkv, Sq);
    const int64_t tiles = (Skv + 63) / 64;
    int64_t n = (256 + base - 1) / base;
    n = n < tiles / 4 ? n : tiles / 4;
    if (causal == 1) n = n < (Sq + 63) / 64 / 4 ? n : (Sq + 63) / 64 / 4;   // keys beyond the rows are never read
    if (n < 1) n = 1;
    return (int)(n > ATTN_MAX_SPLIT ? ATTN_MAX_SPLIT : n);
}

extern "C" int attn_fwd_split(const void* q, const void* k, const void* v, void* out,
                              int B, int Hq, int Hkv, int Sq, int Skv, int D,
                              float scale, int causal, int dtype, int n_split,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_DTYPE;
    bool noop;
    const int st = validate(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, 2, 2, &noop);
    if (st != ATTN_OK) return st;
    if (n_split < 1 || n_split > ATTN_MAX_SPLIT) return ATTN_ERR_SPLIT;
    if (noop) return ATTN_OK;
    if (n_split == 1) return attn_fwd(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, stream);
    const size_t need = attn_split_workspace(B, Hq, Sq, D, n_split);
    if (!workspace || ((uintptr_t)workspace & 15) || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    const int64_t nq = (int64_t)B * Sq * Hq * D, nk = (int64_t)B * Skv * Hkv * D;
    if (ranges_overlap(workspace, (int64_t)need, q, nq * 2) || ranges_overlap(workspace, (int64_t)need, k, nk * 2) ||
        ranges_overlap(workspace, (int64_t)need, v, nk * 2) || ranges_overlap(workspace, (int64_t)need, out, nq * 2))
        return ATTN_ERR_WORKSPACE;
    attn::FwdParams p = make_params(q, k, v, out, B, Hq, Hkv, Sq, Skv, nonzero_multiplier(scale * kLog2e), 1.0f,
                                    causal, true, 32, 4, true);
    set_dense_strides(p, D);
    p.n_split = n_split;
    p.part_o = (float*)workspace;
    p.part_ml = (float*)workspace + (size_t)n_split * B * Sq * Hq * D;
    hipError_t e = attn::launch_fwd_mfma(p, D, dtype == ATTN_BF16, causal != 0, stream);
    if (e == hipSuccess) e = attn::launch_combine(p, D, dtype == ATTN_BF16, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

namespace {

// (n - 1) * stride for n >= 1 and a non-negative stride, or -1 when the
// product does not fit in int64.
int64_t span(int64_t stride, int n) {
    int64_t r;
    return __builtin_mul_overflow((int64_t)(n - 1), stride, &r) ? -1 : r;
}

// Largest element offset a (B, S, H, D) view with non-negative strides
// reaches, plus 1; -1 when it does not fit in int64.
int64_t extent(const int64_t* st, int B, int S, int H, int D) {
    const int64_t a = span(st[0], B), b = span(st[1], S), c = span(st[2], H);
    if (a < 0 || b < 0 || c < 0) return -1;
    int64_t r;
    if (__builtin_add_overflow(a, b, &r) || __builtin_add_overflow(r, c, &r) || __builtin_add_overflow(r, (int64_t)D, &r))
        return -1;
    return r;
}

// No two (b, i, h, d) of a view share an element: sorted by stride, every
// axis of size > 1 steps over the whole extent of the faster ones.
bool injective(const int64_t* st, int B, int S, int H, int D) {
    int64_t s[4] = {1, st[0], st[1], st[2]};
    int64_t n[4] = {D, B, S, H};
    for (int a = 1; a < 4; ++a)
        for (int b = a; b > 0 && s[b] < s[b - 1]; --b) {
            int64_t t = s[b]; s[b] = s[b - 1]; s[b - 1] = t;
            t = n[b]; n[b] = n[b - 1]; n[b - 1] = t;
        }
    int64_t covered = 1;   // elements covered by the faster axes, as a stride unit
    for (int a = 0; a < 4; ++a) {
        if (n[a] == 1) continue;
        if (s[a] < covered) return false;
        if (__builtin_mul_overflow(s[a], n[a], &covered)) return false;
    }
    return true;
}

}  // namespace

extern "C" int attn_fwd_strided(const void* q, const void* k, const void* v, void* out,
                                int B, int Hq, int Hkv, int Sq, int Skv, int D,
                                const int64_t* q_strides, const int64_t* k_strides,
                                const int64_t* v_strides, const int64_t* out_strides,
                                float scale, int causal, int dtype, hipStream_t stream) {
    int eb;
    switch (dtype) {
        case ATTN_F32: eb = 4; break;
        case ATTN_BF16: case ATTN_F16: eb = 2; break;
        default: return ATTN_ERR_DTYPE;
    }
    if (!q || !k || !v || !out || !q_strides || !k_strides || !v_strides || !out_strides) return ATTN_ERR_NULL;
    if (B < 0 || Sq < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Skv < 0) return ATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATTN_ERR_GROUP;
    if (D != 32 && D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (causal < 0 || causal > 2) return ATTN_ERR_CAUSAL;
    if ((int64_t)B * Sq == 0) return ATTN_OK;
    if (Skv < 1) return ATTN_ERR_SHAPE;
    if (causal == 2 && Sq > Skv) return ATTN_ERR_CAUSAL;
    const int64_t* all[4] = {q_strides, k_strides, v_strides, out_strides};
    for (const int64_t* st : all)
        for (int i = 0; i < 3; ++i) {
            if (st[i] < 0 || st[i] > ((int64_t)1 << 40)) return ATTN_ERR_STRIDE;
            if ((st[i] * eb) % 16 != 0) return ATTN_ERR_ALIGN;
        }
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return ATTN_ERR_ALIGN;
    // Every product of a stride and an axis length must fit in int64 (a
    // stride is at most 2^40, an axis below 2^31: the product can reach
    // 2^71), and so must each view's extent in bytes.
    const int64_t xq = extent(q_strides, B, Sq, Hq, D), xk = extent(k_strides, B, Skv, Hkv, D);
    const int64_t xv = extent(v_strides, B, Skv, Hkv, D), xo = extent(out_strides, B, Sq, Hq, D);
    const int64_t kmax = ((int64_t)1 << 62) / eb;
    if (xq < 0 || xk < 0 || xv < 0 || xo < 0 || xq > kmax || xk > kmax || xv > kmax || xo > kmax)
        return ATTN_ERR_STRIDE;
    if (!injective(out_strides, B, Sq, Hq, D)) return ATTN_ERR_STRIDE;
    // A key tile's byte offsets inside one head must fit in 32 bits.
    const int64_t kspan = span(k_strides[1], Skv), vspan = span(v_strides[1], Skv);
    if ((kspan + D) * eb >= ((int64_t)1 << 32) || (vspan + D) * eb >= ((int64_t)1 << 32))
        return ATTN_ERR_SHAPE;
    const int64_t eq = xq * eb, ek = xk * eb, ev = xv * eb, eo = xo * eb;
    if (ranges_overlap(out, eo, q, eq) || ranges_overlap(out, eo, k, ek) || ranges_overlap(out, eo, v, ev))
        return ATTN_ERR_ALIAS;
    int64_t strides[12];
    for (int i = 0; i < 3; ++i) {
        strides[i] = q_strides[i]; strides[3 + i] = k_strides[i];
        strides[6 + i] = v_strides[i]; strides[9 + i] = out_strides[i];
    }
    hipError_t e;
    if (dtype == ATTN_F32) {
        attn::FwdParams p = make_params(q, k, v, out, B, Hq, Hkv, Sq, Skv,
                                        nonzero_multiplier(scale * kLog2e), 1.0f, causal, false, 32, 4);
        for (int i = 0; i < 3; ++i) {
            p.sq[i] = strides[i]; p.sk[i] = strides[3 + i]; p.sv[i] = strides[6 + i]; p.so[i] = strides[9 + i];
        }
        e = attn::launch_fwd_f32(p, D, causal != 0, stream);
    } else {
        e = launch_mfma(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, nonzero_multiplier(scale * kLog2e), 1.0f,
                        dtype, causal, strides, stream);
    }
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" size_t attn_bwd_workspace(int B, int Hq, int Sq) {
    if (B <= 0 || Hq <= 0 || Sq <= 0) return 0;
    return (size_t)2 * B * Hq * Sq * sizeof(float);
}

namespace {

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Byte offsets of the FP8 backward's workspace: bf16 copies of q, k, v and
// dout, then the per-row values of attn_bwd.
struct Fp8BwdLayout {
    size_t q, k, v, dout, rows, total;
};

Fp8BwdLayout fp8_bwd_layout(int B, int Hq, int Hkv, int Sq, int Skv, int D) {
    Fp8BwdLayout L;
    const size_t nq = (size_t)B * Sq * Hq * D, nk = (size_t)B * Skv * Hkv * D;
    L.q = 0;
    L.k = L.q + round_up(nq * 2);
    L.v = L.k + round_up(nk * 2);
    L.dout = L.v + round_up(nk * 2);
    L.rows = L.dout + round_up(nq * 2);
    L.total = L.rows + attn_bwd_workspace(B, Hq, Sq);
    return L;
}

struct BwdScalars {
    float scale_log2, dp_mul, delta_mul, dq_mul, dk_mul, dv_mul;
};

// Shared checks of both backward entry points. in_bytes: element size of q,
// k, v and dout; out and the gradients are 16-bit. ws_need: workspace bytes.
int bwd_validate(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                 int causal, int in_bytes, const void* workspace, size_t workspace_bytes, size_t ws_need,
                 bool* noop) {
    *noop = false;
    if (B < 0 || Sq < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Skv < 0) return ATTN_ERR_SHAPE;
    // Pointers of empty tensors may be NULL (the query side when B * Sq == 0,
    // the key side when B * Skv == 0).
    if ((int64_t)B * Sq > 0 && (!q || !out || !dout || !lse || !dq)) return ATTN_ERR_NULL;
    if ((int64_t)B * Skv > 0 && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL;
    if (Hq % Hkv != 0) return ATTN_ERR_GROUP;
    if (D != 32 && D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (causal < 0 || causal > 2) return ATTN_ERR_CAUSAL;
    if ((int64_t)B * Sq > 0 && Skv < 1) return ATTN_ERR_SHAPE;
    if (causal == 2 && Sq > Skv) return ATTN_ERR_CAUSAL;
    const int64_t nq = (int64_t)B * Sq * Hq * D, nk = (int64_t)B * Skv * Hkv * D;
    if (nq >= kMaxElems || nk >= kMaxElems) return ATTN_ERR_SHAPE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dq |
         (uintptr_t)dk | (uintptr_t)dv) & 15)
        return ATTN_ERR_ALIGN;
    if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
    if ((int64_t)B * (Sq + Skv) == 0) { *noop = true; return ATTN_OK; }   // nothing to write
    if (ws_need > 0 && (!workspace || ((uintptr_t)workspace & 15) || workspace_bytes < ws_need))
        return ATTN_ERR_WORKSPACE;
    // Outputs (dq, dk, dv, workspace) must not overlap inputs or each other.
    const int64_t nl = (int64_t)B * Hq * Sq * 4;
    const void* in_p[6] = {q, k, v, out, dout, lse};
    const int64_t in_n[6] = {nq * in_bytes, nk * in_bytes, nk * in_bytes, nq * 2, nq * in_bytes, nl};
    void* out_p[3] = {dq, dk, dv};
    const int64_t out_n[3] = {nq * 2, nk * 2, nk * 2};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 6; ++i)
            if (ranges_overlap(out_p[o], out_n[o], in_p[i], in_n[i])) return ATTN_ERR_ALIAS;
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (ranges_overlap(out_p[o], out_n[o], out_p[o2], out_n[o2])) return ATTN_ERR_ALIAS;
        if (ranges_overlap(out_p[o], out_n[o], workspace, (int64_t)ws_need)) return ATTN_ERR_WORKSPACE;
    }
    for (int i = 0; i < 6; ++i)
        if (ranges_overlap(workspace, (int64_t)ws_need, in_p[i], in_n[i])) return ATTN_ERR_WORKSPACE;
    return ATTN_OK;
}

// Enqueues the two backward kernels on 16-bit q, k, v, out, dout.
int bwd_launch(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
               void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
               bool is_bf16, const BwdScalars& sc, float* rows, hipStream_t stream,
               const float* const* dsc = nullptr, float raw_scale = 0.0f) {
    attn::BwdParams bp;
    bp.f = make_params(q, k, v, (void*)out, B, Hq, Hkv, Sq > 0 ? Sq : 1, Skv, sc.scale_log2, 1.0f,
                       causal, true, 32, 4, true);
    set_dense_strides(bp.f, D);
    if (Sq == 0) {   // no query rows: dK = dV = 0, the dQ kernel has nothing to do
        bp.f.Sq = 0;
        bp.f.n_row_blocks = 0;
    }
    bp.dout = dout;
    bp.lse = lse;
    bp.delta = rows;
    bp.lse2 = rows + (size_t)B * Hq * Sq;
    bp.dq = dq;
    bp.dk = dk;
    bp.dv = dv;
    bp.dp_mul = sc.dp_mul;
    bp.delta_mul = sc.delta_mul;
    bp.dq_mul = sc.dq_mul;
    bp.dk_mul = sc.dk_mul;
    bp.dv_mul = sc.dv_mul;
    bp.n_kblocks = (Skv + 127) / 128;
    for (int i = 0; i < 4; ++i) bp.dsc[i] = dsc ? dsc[i] : nullptr;
    bp.scale = raw_scale;
    const hipError_t e = attn::launch_bwd(bp, D, is_bf16, causal != 0, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv,
                        int B, int Hq, int Hkv, int Sq, int Skv, int D,
                        float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    if (dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_DTYPE;
    bool noop;
    const size_t need = (B > 0 && Hq > 0 && Sq > 0) ? attn_bwd_workspace(B, Hq, Sq) : 0;
    const int st = bwd_validate(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, scale, causal, 2,
                                workspace, workspace_bytes, need, &noop);
    if (st != ATTN_OK || noop) return st;
    const BwdScalars sc = {scale * kLog2e, 1.0f, 1.0f, scale, scale, 1.0f};
    return bwd_launch(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, causal, dtype == ATTN_BF16, sc,
                      (float*)workspace, stream);
}

extern "C" size_t attn_bwd_fp8_workspace(int B, int Hq, int Hkv, int Sq, int Skv, int D) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || D <= 0 || (int64_t)Sq + Skv == 0) return 0;
    return fp8_bwd_layout(B, Hq, Hkv, Sq, Skv, D).total;
}

extern "C" int attn_bwd_fp8(const void* q, const void* k, const void* v, const void* out, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv,
                            int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal,
                            float q_descale, float k_descale, float v_descale, float do_descale,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    bool noop;
    const bool shape_ok = B >= 0 && Sq >= 0 && Skv >= 0 && Hq > 0 && Hkv > 0 && D > 0;
    const size_t need = shape_ok ? attn_bwd_fp8_workspace(B, Hq, Hkv, Sq, Skv, D) : 0;
    const int st = bwd_validate(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, scale, causal, 1,
                                workspace, workspace_bytes, need, &noop);
    if (st != ATTN_OK) return st;
    if (D == 32) return ATTN_ERR_HEAD_DIM;   // as attn_fwd_fp8, whose out and lse it takes
    if (!isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale) || !isfinite(do_descale))
        return ATTN_ERR_SCALE;
    if (noop) return ATTN_OK;
    // On the codes: S = (scale qd kd) q.k, dP = (dd vd) dout.v, Delta = dd
    // rowsum(dout * out), dq = (scale kd) dS k, dk = (scale qd) dS^T q,
    // dv = dd P^T dout.
    const BwdScalars sc = {scale * q_descale * k_descale * kLog2e, do_descale * v_descale, do_descale,
                           scale * k_descale, scale * q_descale, do_descale};
    if (!isfinite(sc.scale_log2) || !isfinite(sc.dp_mul) || !isfinite(sc.dq_mul) || !isfinite(sc.dk_mul))
        return ATTN_ERR_SCALE;
    const Fp8BwdLayout L = fp8_bwd_layout(B, Hq, Hkv, Sq, Skv, D);
    uint8_t* ws = (uint8_t*)workspace;
    const int64_t nq = (int64_t)B * Sq * Hq * D, nk = (int64_t)B * Skv * Hkv * D;
    hipError_t e = hipSuccess;
    if (nq > 0) e = attn::launch_widen_fp8(q, ws + L.q, nq, false, stream);
    if (e == hipSuccess && nk > 0) e = attn::launch_widen_fp8(k, ws + L.k, nk, false, stream);
    if (e == hipSuccess && nk > 0) e = attn::launch_widen_fp8(v, ws + L.v, nk, false, stream);
    if (e == hipSuccess && nq > 0) e = attn::launch_widen_fp8(dout, ws + L.dout, nq, true, stream);
    if (e != hipSuccess) return ATTN_ERR_HIP;
    return bwd_launch(ws + L.q, ws + L.k, ws + L.v, out, ws + L.dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D,
                      causal, true, sc, (float*)(ws + L.rows), stream);
}

extern "C" int attn_bwd_fp8_dev(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv,
                                int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal,
                                const float* q_descale, const float* k_descale, const float* v_descale,
                                const float* do_descale, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    bool noop;
    const bool shape_ok = B >= 0 && Sq >= 0 && Skv >= 0 && Hq > 0 && Hkv > 0 && D > 0;
    const size_t need = shape_ok ? attn_bwd_fp8_workspace(B, Hq, Hkv, Sq, Skv, D) : 0;
    const int st = bwd_validate(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, scale, causal, 1,
                                workspace, workspace_bytes, need, &noop);
    if (st != ATTN_OK) return st;
    if (D == 32) return ATTN_ERR_HEAD_DIM;
    if (!q_descale || !k_descale || !v_descale || !do_descale) return ATTN_ERR_NULL;
    if (((uintptr_t)q_descale | (uintptr_t)k_descale | (uintptr_t)v_descale | (uintptr_t)do_descale) & 3)
        return ATTN_ERR_ALIGN;
    if (noop) return ATTN_OK;
    const Fp8BwdLayout L = fp8_bwd_layout(B, Hq, Hkv, Sq, Skv, D);
    uint8_t* ws = (uint8_t*)workspace;
    const int64_t nq = (int64_t)B * Sq * Hq * D, nk = (int64_t)B * Skv * Hkv * D;
    hipError_t e = hipSuccess;
    if (nq > 0) e = attn::launch_widen_fp8(q, ws + L.q, nq, false, stream);
    if (e == hipSuccess && nk > 0) e = attn::launch_widen_fp8(k, ws + L.k, nk, false, stream);
    if (e == hipSuccess && nk > 0) e = attn::launch_widen_fp8(v, ws + L.v, nk, false, stream);
    if (e == hipSuccess && nq > 0) e = attn::launch_widen_fp8(dout, ws + L.dout, nq, true, stream);
    if (e != hipSuccess) return ATTN_ERR_HIP;
    const float* dsc[4] = {q_descale, k_descale, v_descale, do_descale};
    const BwdScalars sc = {0.f, 1.f, 1.f, 1.f, 1.f, 1.f};   // formed on the device
    return bwd_launch(ws + L.q, ws + L.k, ws + L.v, out, ws + L.dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D,
                      causal, true, sc, (float*)(ws + L.rows), stream, dsc, scale);
}

// ---- FP8 delayed scaling --------------------------------------------------------------------

extern "C" size_t attn_fp8_state_bytes(void) { return ATTN_FP8_STATE_BYTES; }

extern "C" int attn_fp8_state_init(void* states, int n_states, int format, hipStream_t stream) {
    if (!states) return ATTN_ERR_NULL;
    if (n_states < 0) return ATTN_ERR_SHAPE;
    if (format != ATTN_FP8_E4M3 && format != ATTN_FP8_E5M2) return ATTN_ERR_DTYPE;
    if ((uintptr_t)states & 15) return ATTN_ERR_ALIGN;
    if (n_states == 0) return ATTN_OK;
    const hipError_t e = attn::launch_fp8_state_init(states, n_states, format == ATTN_FP8_E5M2 ? 1 : 0, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fp8_quantize(const void* x, int x_dtype, void* codes, int64_t n, void* state,
                                 hipStream_t stream) {
    if (!state) return ATTN_ERR_NULL;
    if (n < 0 || n >= ((int64_t)1 << 40)) return ATTN_ERR_SHAPE;
    if (n > 0 && (!x || !codes)) return ATTN_ERR_NULL;
    int eb;
    switch (x_dtype) {
        case ATTN_F32: eb = 4; break;
        case ATTN_BF16: case ATTN_F16: eb = 2; break;
        default: return ATTN_ERR_DTYPE;
    }
    if (((uintptr_t)x | (uintptr_t)codes | (uintptr_t)state) & 15) return ATTN_ERR_ALIGN;
    if (n == 0) return ATTN_OK;   // the amax of nothing (0) changes no history slot
    if (ranges_overlap(codes, n, x, n * eb) || ranges_overlap(codes, n, state, ATTN_FP8_STATE_BYTES) ||
        ranges_overlap(state, ATTN_FP8_STATE_BYTES, x, n * eb))
        return ATTN_ERR_ALIAS;
    const hipError_t e = attn::launch_fp8_quantize(x, x_dtype, codes, n, state, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fp8_update(void* states, int n_states, hipStream_t stream) {
    if (!states) return ATTN_ERR_NULL;
    if (n_states < 0) return ATTN_ERR_SHAPE;
    if ((uintptr_t)states & 15) return ATTN_ERR_ALIGN;
    if (n_states == 0) return ATTN_OK;
    const hipError_t e = attn::launch_fp8_update(states, n_states, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fwd_fp8_dev(const void* q, const void* k, const void* v, void* out, float* lse,
                                int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal,
                                const float* q_descale, const float* k_descale, const float* v_descale,
                                hipStream_t stream) {
    bool noop;
    const int st = validate(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, 1, 2, &noop);
    if (st != ATTN_OK) return st;
    if (!q_descale || !k_descale || !v_descale) return ATTN_ERR_NULL;
    if (((uintptr_t)q_descale | (uintptr_t)k_descale | (uintptr_t)v_descale) & 3) return ATTN_ERR_ALIGN;
    if (noop) return ATTN_OK;
    if (lse) {
        if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
        const int64_t nl = (int64_t)B * Hq * Sq * 4;
        const int64_t nq = (int64_t)B * Sq * Hq * D, nk = (int64_t)B * Skv * Hkv * D;
        if (ranges_overlap(lse, nl, q, nq) || ranges_overlap(lse, nl, k, nk) || ranges_overlap(lse, nl, v, nk) ||
            ranges_overlap(lse, nl, out, nq * 2))
            return ATTN_ERR_ALIAS;
    }
    const float* dsc[3] = {q_descale, k_descale, v_descale};
    const hipError_t e = launch_mfma(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, 1.0f, ATTN_FP8_E4M3, causal,
                                     nullptr, stream, lse, dsc);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" const char* attn_strerror(int status) {
    switch (status) {
        case ATTN_OK: return "success";
        case ATTN_ERR_NULL: return "a pointer argument is NULL";
        case ATTN_ERR_SHAPE: return "invalid shape (B, Sq >= 0; Hq, Hkv, D > 0; Skv >= 1 unless B*Sq == 0; < 2^31 elements per tensor)";
        case ATTN_ERR_GROUP: return "Hq is not a multiple of Hkv";
        case ATTN_ERR_HEAD_DIM: return "head dimension D must be 32, 64 or 128 (64 or 128 for E4M3 inputs)";
        case ATTN_ERR_DTYPE: return "unsupported dtype (attn_fwd takes F32, BF16, F16; E4M3 goes through attn_fwd_fp8; the split and backward entry points take BF16, F16)";
        case ATTN_ERR_ALIGN: return "q, k, v and out must be 16-byte aligned";
        case ATTN_ERR_ALIAS: return "an output (out, lse or a gradient) overlaps an input or another output";
        case ATTN_ERR_SCALE: return "scale or a descale is not finite";
        case ATTN_ERR_HIP: return "HIP kernel launch failed";
        case ATTN_ERR_CAUSAL: return "causal must be 0, 1 or 2 (2, bottom-right alignment, needs Sq <= Skv)";
        case ATTN_ERR_SPLIT: return "n_split must be between 1 and ATTN_MAX_SPLIT";
        case ATTN_ERR_STRIDE: return "a stride is negative or too large, or out's strides make two elements share memory";
        case ATTN_ERR_SCRATCH: return "the call needs more scratch than attn_fwd_split_noalloc holds (ATTN_NOALLOC_SCRATCH_BYTES); use attn_fwd_split with a workspace";
        case ATTN_ERR_WORKSPACE: return "workspace is NULL, not 16-byte aligned, smaller than the size function returns (attn_split_workspace / attn_bwd_workspace), or overlaps an input or an output";
        default: return "unknown status";
    }
}

// attn_fwd_mfma.hip — fused attention forward on gfx950 matrix cores.
//
// Computes out = softmax(scale * Q K^T [+ causal mask]) V, the formula and
// four steps of the codelab "Accelerate attention on GPU with cuDNN and
// TransformerEngine" (§1 "How attention works"), fused into one launch in the
// flash style the codelab describes for fused kernels (§8: the work is tiled
// so the (T x S) weight matrix is never materialised and memory stays O(T)).
// Causal mask: §7 (lower triangle, key j visible to query i iff j <= i).
// GQA / MQA: §9 (contiguous groups of query heads share one KV head).
// FP8: §10 (E4M3 inputs for the forward pass, per-tensor scaling).
//
// Input types: bf16, f16 (both products on v_mfma_f32_32x32x16_{bf16,f16}),
// and E4M3 (Q K^T on v_mfma_f32_32x32x64_f8f6f4; V widened exactly to bf16
// and P V on the bf16 instruction, because E4M3 weights would cost up to
// 2^-4 relative error per weight on rows that see only a few keys).
//
// Design (one workgroup = 4 wavefronts of 64 lanes):
//   * Each wave owns 32 query rows of one query head. A workgroup holds
//     `gpack` query heads that read the same KV head, 4 / gpack row blocks of
//     32 rows each, so every K/V tile staged in LDS serves 128 query rows.
//   * Scores are computed transposed, S^T = K Q^T: lane (h = lane / 32,
//     n = lane % 32) then holds 16 scores of query n per 32-key block, so a
//     row's max needs only one exchange between lanes n and n + 32, and its
//     sum is kept per lane until the end.
//   * O^T = V^T P^T. The score accumulator is used directly as the P operand:
//     the MFMA sums over k in any order as long as both operands agree, so
//     V is read from LDS with the same key permutation (V sits in LDS as
//     [key/4][d][key%4], which makes that read one 8-byte access per 4 keys).
//   * Online softmax in the exp2 domain with the scale folded into one
//     multiply; the running max is only raised when it grows by more than 8
//     (a factor 2^8): numerator and denominator share the stale max, so the
//     result is the same, and weights up to 256 are harmless in bf16 / f16.
//   * K/V tiles are double-buffered: the next tile's global loads are issued
//     before the current tile's math and written to LDS after it, with one
//     barrier per tile.
//   * Causal: tiles wholly above the workgroup's diagonal are never loaded;
//     32-key blocks wholly above a wave's diagonal skip their MFMAs.

#include "kernel_common.h"

namespace attn {

typedef uint8_t fp8_t;   // one OCP E4M3 code

__device__ inline uint32_t pack2_bf16(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ inline uint32_t pack2_f16(float lo, float hi) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}

// Per input type: the score product (QK), the weight product (PV) and the
// conversions around them.
template <typename T> struct Traits;

template <> struct Traits<__bf16> {
    static constexpr int IN_BYTES = 2;
    static constexpr int QK_LANE_BYTES = 16;    // bytes of one operand per lane per k-step
    static constexpr int QK_K = 16;             // contraction length of one QK MFMA
    using qk_frag = bf16x8;
    using pv_frag = bf16x8;
    using out_t = __bf16;
    __device__ static inline f32x16 qk(qk_frag a, qk_frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline f32x16 pv(pv_frag a, pv_frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline uint32_t pack_p(float lo, float hi) { return pack2_bf16(lo, hi); }
    __device__ static inline uint32_t pack_out(float lo, float hi) { return pack2_bf16(lo, hi); }
};

template <> struct Traits<_Float16> {
    static constexpr int IN_BYTES = 2;
    static constexpr int QK_LANE_BYTES = 16;
    static constexpr int QK_K = 16;
    using qk_frag = f16x8;
    using pv_frag = f16x8;
    using out_t = _Float16;
    __device__ static inline f32x16 qk(qk_frag a, qk_frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static inline f32x16 pv(pv_frag a, pv_frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static inline uint32_t pack_p(float lo, float hi) { return pack2_f16(lo, hi); }
    __device__ static inline uint32_t pack_out(float lo, float hi) { return pack2_f16(lo, hi); }
};

template <> struct Traits<fp8_t> {
    static constexpr int IN_BYTES = 1;
    static constexpr int QK_LANE_BYTES = 32;
    static constexpr int QK_K = 64;
    using qk_frag = i32x8;
    using pv_frag = bf16x8;
    using out_t = __bf16;
    __device__ static inline f32x16 qk(qk_frag a, qk_frag b, f32x16 c) {
        // Both operands E4M3 (format code 0), no block scales.
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
    __device__ static inline f32x16 pv(pv_frag a, pv_frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline uint32_t pack_p(float lo, float hi) { return pack2_bf16(lo, hi); }
    __device__ static inline uint32_t pack_out(float lo, float hi) { return pack2_bf16(lo, hi); }
};

// Swizzle of 16-byte chunks inside a K row in LDS: chunk c of row r is stored
// at chunk position c ^ kswz(r). Sixteen consecutive rows read at the same c
// then land in sixteen different 16-byte bank groups (64 banks x 4 bytes).
template <int NCK>
__device__ inline int kswz(int r) {
    return (r / (16 / NCK)) % NCK;
}

// Eight consecutive V elements of one key row, as four 32-bit words each
// holding two 16-bit values of the PV operand type.
template <typename T>
__device__ inline u32x4 load_v8(const T* src, bool ok);

template <> __device__ inline u32x4 load_v8<__bf16>(const __bf16* src, bool ok) {
    return ok ? *(const u32x4*)src : (u32x4){0, 0, 0, 0};
}
template <> __device__ inline u32x4 load_v8<_Float16>(const _Float16* src, bool ok) {
    return ok ? *(const u32x4*)src : (u32x4){0, 0, 0, 0};
}
// E4M3 -> bf16 is exact (3 mantissa bits and exponents 2^-9 .. 2^8 all fit).
template <> __device__ inline u32x4 load_v8<fp8_t>(const fp8_t* src, bool ok) {
    const u32x2 x = ok ? *(const u32x2*)src : (u32x2){0, 0};
    u32x4 r;
    for (int w = 0; w < 2; ++w) {
        const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[w], false);
        const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[w], true);
        r[2 * w] = pack2_bf16(a[0], a[1]);
        r[2 * w + 1] = pack2_bf16(b[0], b[1]);
    }
    return r;
}

template <typename T, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_mfma_kernel(FwdParams p) {
    using Tr = Traits<T>;
    using qk_frag = typename Tr::qk_frag;
    using pv_frag = typename Tr::pv_frag;
    using out_t = typename Tr::out_t;
    constexpr int ROW_BYTES = D * Tr::IN_BYTES;       // one K / Q row
    constexpr int NCK = ROW_BYTES / 16;               // 16-byte chunks per K row
    constexpr int CH = Tr::QK_LANE_BYTES / 16;        // chunks per lane per k-step
    constexpr int KSTEPS = D / Tr::QK_K;              // k-steps of the score product
    constexpr int NKB = BN / 32;                      // 32-key blocks per tile
    constexpr int NDB = D / 32;                       // 32-wide column blocks of O
    constexpr int K_LD = (BN * NCK) / 256;            // K chunks staged per thread
    static_assert(K_LD * 256 == BN * NCK, "K tile must split evenly over 256 threads");
    static_assert((BN / 4) * (D / 8) == 256, "V tile must be one 4 x 8 unit per thread");

    __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][BN * ROW_BYTES];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][BN * D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;              // which half of the wave
    const int n = lane & 31;              // query column inside the wave's 32 rows

    const WorkItem wi = map_workgroup(p, CAUSAL);
    const int hq = wi.hq0 + (wave % p.gpack);
    const int q0 = wi.row_base + (wave / p.gpack) * 32;
    const int Sq = p.Sq, Skv = p.Skv;
    const size_t qstride = (size_t)p.Hq * D;          // elements between query rows
    const size_t kstride = (size_t)p.Hkv * D;

    const T* qbase = (const T*)p.q + ((size_t)wi.b * Sq * p.Hq + hq) * D;
    const T* kbase = (const T*)p.k + ((size_t)wi.b * Skv * p.Hkv + wi.hkv) * D;
    const T* vbase = (const T*)p.v + ((size_t)wi.b * Skv * p.Hkv + wi.hkv) * D;

    // Q^T operand, kept in registers for the whole key loop: lane (h, n) holds
    // bytes [(2 ks + h) * QK_LANE_BYTES, +QK_LANE_BYTES) of row q0 + n.
    qk_frag qf[KSTEPS];
    {
        const int row = q0 + n;
        const uint8_t* src = (const uint8_t*)(qbase + row * qstride);
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 x[CH];
            for (int t = 0; t < CH; ++t) {
                x[t] = (u32x4){0, 0, 0, 0};
                if (row < Sq) x[t] = *(const u32x4*)(src + ((2 * ks + h) * CH + t) * 16);
            }
            if constexpr (CH == 1) {
                qf[ks] = __builtin_bit_cast(qk_frag, x[0]);
            } else {
                qf[ks] = __builtin_bit_cast(qk_frag, (i32x8){(int)x[0][0], (int)x[0][1], (int)x[0][2], (int)x[0][3],
                                                             (int)x[1][0], (int)x[1][1], (int)x[1][2], (int)x[1][3]});
            }
        }
    }

    int n_tiles = (Skv + BN - 1) / BN;
    if (CAUSAL) {
        const int last_row = min(wi.row_base + p.rows_per_wg, Sq) - 1;
        n_tiles = min(n_tiles, last_row / BN + 1);
    }

    // ---- tile staging: global -> registers -> LDS ------------------------
    u32x4 kreg[K_LD];
    u32x4 vreg[4];
    auto load_tile = [&](int j) {
        const int key0 = j * BN;
        for (int i = 0; i < K_LD; ++i) {
            const int id = i * 256 + tid;
            const int r = id / NCK, c = id % NCK;
            const int key = key0 + r;
            kreg[i] = (u32x4){0, 0, 0, 0};
            if (key < Skv) kreg[i] = *(const u32x4*)((const uint8_t*)(kbase + key * kstride) + c * 16);
        }
        const int g = tid / (D / 8), c = tid % (D / 8);
        for (int r = 0; r < 4; ++r) {
            const int key = key0 + 4 * g + r;
            vreg[r] = load_v8<T>(vbase + key * kstride + c * 8, key < Skv);
        }
    };
    auto store_tile = [&](int buf) {
        for (int i = 0; i < K_LD; ++i) {
            const int id = i * 256 + tid;
            const int r = id / NCK, c = id % NCK;
            *(u32x4*)(&lds_k[buf][r * ROW_BYTES + ((c ^ kswz<NCK>(r)) * 16)]) = kreg[i];
        }
        // V: this thread holds keys 4g..4g+3 at columns 8c..8c+7 (16-bit
        // values). Write them as [g][d][4 keys]: one column's four keys become
        // two 32-bit words.
        const int g = tid / (D / 8), c = tid % (D / 8);
        u32x4 outw[4];
        for (int e = 0; e < 4; ++e) {          // column pair (8c + 2e, 8c + 2e + 1)
            const uint32_t a0 = vreg[0][e], a1 = vreg[1][e], a2 = vreg[2][e], a3 = vreg[3][e];
            const uint32_t lo01 = __builtin_amdgcn_perm(a1, a0, 0x05040100u);   // column 8c+2e
            const uint32_t lo23 = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
            const uint32_t hi01 = __builtin_amdgcn_perm(a1, a0, 0x07060302u);   // column 8c+2e+1
            const uint32_t hi23 = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
            outw[e] = (u32x4){lo01, lo23, hi01, hi23};
        }
        uint16_t* dst = &lds_v[buf][(g * D + 8 * c) * 4];
        for (int e = 0; e < 4; ++e) *(u32x4*)(dst + e * 8) = outw[e];
    };

    // ---- running softmax state (per lane: query n, partial over its keys) --
    f32x16 oacc[NDB];
    for (int db = 0; db < NDB; ++db)
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = -INFINITY;   // running max in the log2 domain (same on both halves)
    float l_part = 0.f;        // this lane's share of the running denominator

    const float c_log2 = p.scale_log2;
    const int qrow = q0 + n;
    const int wave_last_row = q0 + 31;

    load_tile(0);
    store_tile(0);

    for (int j = 0; j < n_tiles; ++j) {
        const int buf = j & 1;
        __syncthreads();
        if (j + 1 < n_tiles) load_tile(j + 1);

        // ---- S^T = K Q^T for each 32-key block -------------------------
        f32x16 s[NKB];
        bool active[NKB];
        for (int kb = 0; kb < NKB; ++kb) {
            const int kstart = j * BN + kb * 32;
            active[kb] = kstart < Skv && (!CAUSAL || kstart <= wave_last_row);
            for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
            if (!active[kb]) continue;
            const int row = kb * 32 + n;                      // lane's key row (A operand)
            const uint8_t* krow = &lds_k[buf][row * ROW_BYTES];
            const int sw = kswz<NCK>(row);
            for (int ks = 0; ks < KSTEPS; ++ks) {
                qk_frag a;
                if constexpr (CH == 1) {
                    a = __builtin_bit_cast(qk_frag, *(const u32x4*)(krow + (((2 * ks + h) ^ sw) * 16)));
                } else {
                    const u32x4 x0 = *(const u32x4*)(krow + ((((2 * ks + h) * 2) ^ sw) * 16));
                    const u32x4 x1 = *(const u32x4*)(krow + ((((2 * ks + h) * 2 + 1) ^ sw) * 16));
                    a = __builtin_bit_cast(qk_frag, (i32x8){(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                                            (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]});
                }
                s[kb] = Tr::qk(a, qf[ks], s[kb]);
            }
        }

        // ---- scale, mask, online softmax ---------------------------------
        float mloc = -INFINITY;
        for (int kb = 0; kb < NKB; ++kb) {
            if (!active[kb]) continue;
            const int kstart = j * BN + kb * 32;
            const bool need_mask = (CAUSAL && kstart + 31 > q0) || (kstart + 32 > Skv);
            for (int i = 0; i < 16; ++i) {
                float x = s[kb][i] * c_log2;
                if (need_mask) {
                    const int key = kstart + 8 * (i >> 2) + 4 * h + (i & 3);
                    if (key >= Skv || (CAUSAL && key > qrow)) x = -INFINITY;
                }
                s[kb][i] = x;
                mloc = fmaxf(mloc, x);
            }
        }
        const float mt = xor32_max(mloc);
        const float mnew = fmaxf(m_run, mt);
        const bool grow = mnew > m_run + 8.0f;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float alpha = exp2f(m_run - mnew);          // 0 on the first tile
            for (int db = 0; db < NDB; ++db)
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
            l_part *= alpha;
            m_run = mnew;
        }
        const float muse = (m_run == -INFINITY) ? 0.f : m_run;

        // ---- O^T += V^T P^T ---------------------------------------------
        for (int kb = 0; kb < NKB; ++kb) {
            if (!active[kb]) continue;
            uint32_t pw[8];
            for (int i = 0; i < 8; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(s[kb][2 * i] - muse);
                const float p1 = __builtin_amdgcn_exp2f(s[kb][2 * i + 1] - muse);
                l_part += p0 + p1;
                pw[i] = Tr::pack_p(p0, p1);
            }
            for (int s2 = 0; s2 < 2; ++s2) {
                const pv_frag pf = __builtin_bit_cast(pv_frag, (u32x4){pw[4 * s2], pw[4 * s2 + 1], pw[4 * s2 + 2], pw[4 * s2 + 3]});
                const int g1 = (kb * 32 + 16 * s2) / 4 + h;   // keys 4*g1 .. 4*g1+3
                for (int db = 0; db < NDB; ++db) {
                    const int d = db * 32 + n;
                    const u32x2 lo = *(const u32x2*)(&lds_v[buf][(g1 * D + d) * 4]);
                    const u32x2 hi = *(const u32x2*)(&lds_v[buf][((g1 + 2) * D + d) * 4]);
                    const pv_frag vf = __builtin_bit_cast(pv_frag, (u32x4){lo[0], lo[1], hi[0], hi[1]});
                    oacc[db] = Tr::pv(vf, pf, oacc[db]);
                }
            }
        }

        if (j + 1 < n_tiles) store_tile(buf ^ 1);
    }

    // ---- epilogue: O = O^T / l, round once, store [b][row][hq][d] ----------
    const float l = xor32_sum(l_part);
    const float inv = p.out_mul / l;
    if (qrow < Sq) {
        out_t* orow = (out_t*)p.out + ((size_t)wi.b * Sq + qrow) * qstride + (size_t)hq * D;
        for (int db = 0; db < NDB; ++db) {
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = db * 32 + 8 * jj + 4 * h;
                const uint32_t w0 = Tr::pack_out(oacc[db][4 * jj + 0] * inv, oacc[db][4 * jj + 1] * inv);
                const uint32_t w1 = Tr::pack_out(oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv);
                *(u32x2*)(orow + d0) = (u32x2){w0, w1};
            }
        }
    }
}

template <typename T, int D, int BN>
static hipError_t launch_typed(const FwdParams& p, bool causal, hipStream_t stream) {
    const dim3 grid(p.n_units * p.n_row_blocks), block(256);
    if (causal)
        hipLaunchKernelGGL((fwd_mfma_kernel<T, D, BN, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_mfma_kernel<T, D, BN, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// bf16 (is_bf16 = true) or f16 inputs, D = 64 or 128.
hipError_t launch_fwd_mfma(const FwdParams& p, int D, bool is_bf16, bool causal, hipStream_t stream) {
    if (is_bf16) {
        return D == 64 ? launch_typed<__bf16, 64, 128>(p, causal, stream)
                       : launch_typed<__bf16, 128, 64>(p, causal, stream);
    }
    return D == 64 ? launch_typed<_Float16, 64, 128>(p, causal, stream)
                   : launch_typed<_Float16, 128, 64>(p, causal, stream);
}

// E4M3 inputs, bf16 output, D = 64 or 128.
hipError_t launch_fwd_fp8(const FwdParams& p, int D, bool causal, hipStream_t stream) {
    return D == 64 ? launch_typed<fp8_t, 64, 128>(p, causal, stream)
                   : launch_typed<fp8_t, 128, 64>(p, causal, stream);
}

}  // namespace attn

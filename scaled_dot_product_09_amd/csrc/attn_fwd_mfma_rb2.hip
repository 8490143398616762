// attn_fwd_mfma_rb2.hip — fused attention forward, 64 query rows per wavefront.
//
// The same computation as attn_fwd_mfma.hip, out = softmax(scale * Q K^T
// [+ causal mask]) V (codelab "Accelerate attention on GPU with cuDNN and
// TransformerEngine": §1 formula and four steps, §7 causal mask, §9 MHA / GQA
// / MQA head sharing, §10 E4M3 inputs), laid out for long sequences:
//
//   * One wavefront per SIMD (one 4-wave workgroup per CU). Each wave owns 64
//     query rows of one query head, held as two 32-row halves ("row blocks"
//     rb0, rb1). Every K / V operand read from LDS then feeds two MFMAs (one
//     per half), halving LDS traffic per flop against 32 rows per wave; the
//     64 x D fp32 output accumulator lives in the accumulation registers.
//   * The two halves ping-pong inside the wave: while the matrix cores run
//     the score product of one half, the vector ALUs form the softmax
//     weights of the other. Per K/V tile j the wave runs
//       max(rb0) | QK(rb1, j) + exp(rb0) | max(rb1) | PV(rb0, j) + exp(rb1)
//       | QK(rb0, j+1) + PV(rb1, j)
//     with the interleave pinned by scheduling barriers.
//   * LDS holds three K tiles and two V tiles (K is needed one tile ahead of
//     V). Tiles go HBM -> LDS directly (global_load_lds_dwordx4); each
//     iteration starts with one barrier and then issues K(j+2) and V(j+1).
//   * Online softmax, lazy rescale, masking, the V transpose read and the
//     E4M3 handling are those of the 32-row kernel (see mfma_common.h).

#include "mfma_common.h"

namespace attn {

template <typename T, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_rb2_kernel(FwdParams p) {
    using Tr = Traits<T>;
    using qk_frag = typename Tr::qk_frag;
    using pv_frag = typename Tr::pv_frag;
    using out_t = typename Tr::out_t;
    constexpr int KROWB = D * Tr::IN_BYTES;           // bytes of one K / Q row
    constexpr int VROWB = D * 2;                      // bytes of one V row in LDS (16-bit)
    constexpr int NCK = KROWB / 16;                   // 16-byte chunks per K row
    constexpr int NCV = VROWB / 16;
    constexpr int CH = Tr::QK_LANE_BYTES / 16;        // chunks per lane per k-step
    constexpr int KSTEPS = D / Tr::QK_K;              // k-steps of the score product
    constexpr int NKB = BN / 32;                      // 32-key blocks per tile
    constexpr int NDB = D / 32;                       // 32-wide column blocks of O
    constexpr int KTILE = BN * KROWB, VTILE = BN * VROWB;
    constexpr int NKBUF = 3, NVBUF = 2;
    static_assert(NKB == 2, "the interleave below assumes 64-key tiles");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[NKBUF * KTILE + NVBUF * VTILE];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;              // which half of the wave
    const int n = lane & 31;              // query column inside a 32-row block

    const WorkItem wi = map_workgroup(p, CAUSAL);
    const int hq = wi.hq0 + (wave % p.gpack);
    const int q0 = wi.row_base + (wave / p.gpack) * 64;
    const int Sq = p.Sq, Skv = p.Skv;
    const size_t qstride = (size_t)p.Hq * D;          // elements between query rows
    const size_t kstride = (size_t)p.Hkv * D;
    const size_t kstride_b = kstride * Tr::IN_BYTES;

    const T* qbase = (const T*)p.q + ((size_t)wi.b * Sq * p.Hq + hq) * D;
    const uint8_t* kbase = (const uint8_t*)((const T*)p.k + ((size_t)wi.b * Skv * p.Hkv + wi.hkv) * D);
    const uint8_t* vbase = (const uint8_t*)((const T*)p.v + ((size_t)wi.b * Skv * p.Hkv + wi.hkv) * D);

    // Q^T operands of both halves, in registers for the whole key loop.
    qk_frag qf[2][KSTEPS];
    for (int r = 0; r < 2; ++r) {
        const int row = q0 + 32 * r + n;
        const uint8_t* src = (const uint8_t*)(qbase + row * qstride);
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 x[CH];
            for (int t = 0; t < CH; ++t) {
                x[t] = (u32x4){0, 0, 0, 0};
                if (row < Sq) x[t] = *(const u32x4*)(src + ((2 * ks + h) * CH + t) * 16);
            }
            if constexpr (CH == 1) {
                qf[r][ks] = __builtin_bit_cast(qk_frag, x[0]);
            } else {
                qf[r][ks] = __builtin_bit_cast(qk_frag, (i32x8){(int)x[0][0], (int)x[0][1], (int)x[0][2], (int)x[0][3],
                                                                (int)x[1][0], (int)x[1][1], (int)x[1][2], (int)x[1][3]});
            }
        }
    }

    int n_tiles = (Skv + BN - 1) / BN;
    if (CAUSAL) {
        const int last_row = min(wi.row_base + p.rows_per_wg, Sq) - 1 + p.causal_off;
        n_tiles = min(n_tiles, last_row / BN + 1);
    }
    n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);

    // ---- tile staging --------------------------------------------------------
    uint8_t* const kbufs = lds;
    uint8_t* const vbufs = lds + NKBUF * KTILE;
    auto kbuf = [&](int j) { return kbufs + (j % NKBUF) * KTILE; };
    auto vbuf = [&](int j) { return vbufs + (j % NVBUF) * VTILE; };
    constexpr int V_ST = Tr::V_DMA ? 1 : (BN * D / 8) / 256;
    u32x2 vstage[V_ST];
    TileDma<KROWB, BN> kdma;
    TileDma<VROWB, BN> vdma;
    kdma.init(kbase, (uint32_t)kstride_b, wave, lane, kSwzK);
    if constexpr (Tr::V_DMA) vdma.init(vbase, (uint32_t)kstride_b, wave, lane, kSwzV);
    auto issue_k = [&](int j) { kdma.issue(j * BN, Skv, kbuf(j), wave); };
    auto issue_v = [&](int j) {
        if constexpr (Tr::V_DMA) {
            vdma.issue(j * BN, Skv, vbuf(j), wave);
        } else {
            for (int u = 0; u < V_ST; ++u) {
                const int id = u * 256 + tid;
                const int r = id / (D / 8), c = id % (D / 8);
                const int key = min(j * BN + r, Skv - 1);
                vstage[u] = *(const u32x2*)(vbase + key * kstride_b + c * 8);
            }
        }
    };
    auto finish_v = [&](int j) {   // FP8 only: widen the staged V(j) and write it
        if constexpr (!Tr::V_DMA) {
            uint8_t* vt = vbuf(j);
            for (int u = 0; u < V_ST; ++u) {
                const int id = u * 256 + tid;
                const int r = id / (D / 8), c = id % (D / 8);
                u32x4 w;
                for (int e = 0; e < 2; ++e) {
                    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)vstage[u][e], false);
                    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)vstage[u][e], true);
                    w[2 * e] = pack2_bf16(a[0], a[1]);
                    w[2 * e + 1] = pack2_bf16(b[0], b[1]);
                }
                *(u32x4*)(vt + r * VROWB + ((c ^ v_swz<NCV>(r)) * 16)) = w;
            }
        }
    };

    // ---- running softmax state, per half ----------------------------------
    f32x16 oacc[2][NDB];
    for (int r = 0; r < 2; ++r)
        for (int db = 0; db < NDB; ++db)
            for (int i = 0; i < 16; ++i) oacc[r][db][i] = 0.f;
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_part[2] = {0.f, 0.f};

    const float c_log2 = p.scale_log2;
    const bool c_nonneg = c_log2 >= 0.f;

    // Lane constants of the operand reads (see the 32-row kernel).
    const int L16 = lane & 15;
    const int G16 = (lane >> 4) & 1;
    const int v_row_in = 4 * h + (L16 >> 2);
    const int v_col_b = 32 * G16 + 8 * (L16 & 3);
    const int k_sw = k_swz<NCK>(n);
    const uint32_t k_lane_base0 = n * KROWB + ((((h * CH) ^ k_sw)) << 4);
    const uint32_t k_lane_base1 = n * KROWB + ((((h * CH + (CH - 1)) ^ k_sw)) << 4);
    int v_lane_off[NDB];
    for (int db = 0; db < NDB; ++db) {
        const int cb = db * 64 + v_col_b;
        v_lane_off[db] = v_row_in * VROWB + ((((cb >> 4) ^ v_swz<NCV>(v_row_in)) << 4) | (cb & 15));
    }
    auto load_k = [&](const uint8_t* kt, int kb, int ks) -> qk_frag {
        const uint8_t* kr = kt + kb * 32 * KROWB;
        if constexpr (CH == 1) {
            return __builtin_bit_cast(qk_frag, *(const u32x4*)(kr + (k_lane_base0 ^ (ks * 32 * CH))));
        } else {
            const u32x4 x0 = *(const u32x4*)(kr + (k_lane_base0 ^ (ks * 32 * CH)));
            const u32x4 x1 = *(const u32x4*)(kr + (k_lane_base1 ^ (ks * 32 * CH)));
            return __builtin_bit_cast(qk_frag, (i32x8){(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                                       (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]});
        }
    };
    auto load_v = [&](const uint8_t* vt, int kb, int s2, int db) -> pv_frag {
        const uint8_t* a_lo = vt + (kb * 32 + 16 * s2) * VROWB + v_lane_off[db];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a_lo));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a_lo + 8 * VROWB));
        return __builtin_bit_cast(pv_frag, (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };

    // Row max of half r's scores of tile j, lazy rescale of its O and l;
    // returns -m. Masked scores become -inf (scale >= 0) or +inf (scale < 0)
    // so that c * s = -inf; the test is skipped (wave-uniformly) for 32-key
    // blocks that hide no key from any row of the half.
    auto tile_max = [&](int r, f32x16 (&s)[NKB], int j) -> float {
        const float masked = c_nonneg ? -INFINITY : INFINITY;
        const int qrow = q0 + 32 * r + n;
        for (int kb = 0; kb < NKB; ++kb) {
            const int kbase_h = j * BN + kb * 32 + 4 * h;
            int lim = Skv - 1 - kbase_h;
            if (CAUSAL) lim = min(lim, qrow + p.causal_off - kbase_h);
            if (__builtin_amdgcn_ballot_w64(lim < 27) != 0) {
                for (int i = 0; i < 16; ++i)
                    s[kb][i] = (8 * (i >> 2) + (i & 3) > lim) ? masked : s[kb][i];
            }
        }
        float mk[NKB];
        if (c_nonneg) {
            for (int kb = 0; kb < NKB; ++kb) {
                float a = fmaxf(s[kb][0], fmaxf(s[kb][1], s[kb][2]));
                float b = fmaxf(s[kb][3], fmaxf(s[kb][4], s[kb][5]));
                a = fmaxf(a, fmaxf(s[kb][6], s[kb][7]));
                b = fmaxf(b, fmaxf(s[kb][8], s[kb][9]));
                a = fmaxf(a, fmaxf(s[kb][10], s[kb][11]));
                b = fmaxf(b, fmaxf(s[kb][12], s[kb][13]));
                a = fmaxf(a, fmaxf(s[kb][14], s[kb][15]));
                mk[kb] = fmaxf(a, b);
            }
        } else {
            for (int kb = 0; kb < NKB; ++kb) {
                float a = s[kb][0];
                for (int i = 1; i < 16; ++i) a = fminf(a, s[kb][i]);
                mk[kb] = a;
            }
        }
        float mraw = mk[0];
        for (int kb = 1; kb < NKB; ++kb) mraw = c_nonneg ? fmaxf(mraw, mk[kb]) : fminf(mraw, mk[kb]);
        const float mt = xor32_max(mraw * c_log2);
        const float mnew = fmaxf(m_run[r], mt);
        if (__builtin_amdgcn_ballot_w64(mnew > m_run[r] + 8.0f) != 0) {
            const float alpha = __builtin_amdgcn_exp2f(m_run[r] - mnew);
            for (int db = 0; db < NDB; ++db)
                for (int i = 0; i < 16; ++i) oacc[r][db][i] *= alpha;
            l_part[r] *= alpha;
            m_run[r] = mnew;
        }
        return (m_run[r] == -INFINITY) ? 0.f : -m_run[r];
    };

    // Weight pair pp (scores 2i, 2i+1 of block kb = pp / 8) of half r.
    auto weight_pair = [&](int r, const f32x16 (&s)[NKB], float neg_m, uint32_t (&pw)[NKB][8], int pp) {
        const int kb = pp / 8, i = pp % 8;
        const float x0 = fmaf(s[kb][2 * i], c_log2, neg_m);
        const float x1 = fmaf(s[kb][2 * i + 1], c_log2, neg_m);
        pw[kb][i] = Tr::pack(__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1));
        l_part[r] = Tr::sum2(pw[kb][i], l_part[r]);
    };

    // Scores of half r for the tile in kt, with weight pairs of the other
    // half (r ^ 1, scores s_o, offset neg_m_o) spread over the k-steps when
    // WITH_W.
    auto qk_half = [&](auto with_w, int r, const uint8_t* kt, f32x16 (&s)[NKB],
                       const f32x16 (&s_o)[NKB], float neg_m_o, uint32_t (&pw_o)[NKB][8]) {
        constexpr bool WITH_W = decltype(with_w)::value;
        constexpr int PER_STEP = (NKB * 8) / KSTEPS;
        for (int kb = 0; kb < NKB; ++kb)
            for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
        qk_frag cur[NKB], nxt[NKB];
        for (int kb = 0; kb < NKB; ++kb) cur[kb] = load_k(kt, kb, 0);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            if (ks + 1 < KSTEPS)
                for (int kb = 0; kb < NKB; ++kb) nxt[kb] = load_k(kt, kb, ks + 1);
            for (int kb = 0; kb < NKB; ++kb) s[kb] = Tr::qk(cur[kb], qf[r][ks], s[kb]);
            if constexpr (WITH_W)
                for (int t = 0; t < PER_STEP; ++t) weight_pair(r ^ 1, s_o, neg_m_o, pw_o, ks * PER_STEP + t);
            if (ks + 1 < KSTEPS)
                for (int kb = 0; kb < NKB; ++kb) cur[kb] = nxt[kb];
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // O^T += V^T P^T for half r, with weight pairs of the other half spread
    // over the (kb, s2) groups when WITH_W.
    auto pv_half = [&](auto with_w, int r, const uint8_t* vt, const uint32_t (&pw)[NKB][8],
                       const f32x16 (&s_o)[NKB], float neg_m_o, uint32_t (&pw_o)[NKB][8]) {
        constexpr bool WITH_W = decltype(with_w)::value;
#pragma unroll
        for (int g = 0; g < NKB * 2; ++g) {
            const int kb = g / 2, s2 = g % 2;
            const pv_frag pf = __builtin_bit_cast(pv_frag, (u32x4){pw[kb][4 * s2], pw[kb][4 * s2 + 1],
                                                                   pw[kb][4 * s2 + 2], pw[kb][4 * s2 + 3]});
            pv_frag vf[NDB];
            for (int db = 0; db < NDB; ++db) vf[db] = load_v(vt, kb, s2, db);
            for (int db = 0; db < NDB; ++db) {
                oacc[r][db] = Tr::pv(vf[db], pf, oacc[r][db]);
                if constexpr (WITH_W) {
                    constexpr int PER_G = (NKB * 8) / (NKB * 2 * NDB);
                    for (int t = 0; t < PER_G; ++t)
                        weight_pair(r ^ 1, s_o, neg_m_o, pw_o, (g * NDB + db) * PER_G + t);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    f32x16 s0[NKB], s1[NKB];
    uint32_t pw0[NKB][8], pw1[NKB][8];
    issue_k(0);
    issue_v(0);
    if (n_tiles > 1) issue_k(1);
    finish_v(0);
    dma_barrier();
    qk_half(std::false_type{}, 0, kbuf(0), s0, s1, 0.f, pw1);

    for (int j = 0; j < n_tiles; ++j) {
        dma_barrier();
        if (j + 2 < n_tiles) issue_k(j + 2);
        if (j + 1 < n_tiles) issue_v(j + 1);
        const uint8_t* kt = kbuf(j);
        const uint8_t* vt = vbuf(j);
        const float neg_m0 = tile_max(0, s0, j);
        qk_half(std::true_type{}, 1, kt, s1, s0, neg_m0, pw0);         // QK(rb1) + exp(rb0)
        const float neg_m1 = tile_max(1, s1, j);
        pv_half(std::true_type{}, 0, vt, pw0, s1, neg_m1, pw1);        // PV(rb0) + exp(rb1)
        if (j + 1 < n_tiles) qk_half(std::false_type{}, 0, kbuf(j + 1), s0, s1, 0.f, pw1);   // QK(rb0, j+1)
        pv_half(std::false_type{}, 1, vt, pw1, s0, 0.f, pw0);          // PV(rb1)
        if (j + 1 < n_tiles) finish_v(j + 1);
    }

    // ---- epilogue: O = O^T / l, round once, store [b][row][hq][d] ----------
    for (int r = 0; r < 2; ++r) {
        const float l = xor32_sum(l_part[r]);
        const float inv = p.out_mul / l;
        const int qrow = q0 + 32 * r + n;
        if (qrow < Sq) {
            out_t* orow = (out_t*)p.out + ((size_t)wi.b * Sq + qrow) * qstride + (size_t)hq * D;
            for (int db = 0; db < NDB; ++db) {
                for (int jj = 0; jj < 4; ++jj) {
                    const int d0 = db * 32 + 8 * jj + 4 * h;
                    const uint32_t w0 = Tr::pack(oacc[r][db][4 * jj + 0] * inv, oacc[r][db][4 * jj + 1] * inv);
                    const uint32_t w1 = Tr::pack(oacc[r][db][4 * jj + 2] * inv, oacc[r][db][4 * jj + 3] * inv);
                    *(u32x2*)(orow + d0) = (u32x2){w0, w1};
                }
            }
        }
    }
}

template <typename T, int D>
static hipError_t launch_rb2_typed(const FwdParams& p, bool causal, hipStream_t stream) {
    const dim3 grid(p.n_units * p.n_row_blocks), block(256);
    if (causal)
        hipLaunchKernelGGL((fwd_rb2_kernel<T, D, 64, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_rb2_kernel<T, D, 64, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// dtype: 1 = bf16, 2 = f16, 3 = E4M3 (bf16 output); D = 64 or 128.
hipError_t launch_fwd_rb2(const FwdParams& p, int D, int dtype, bool causal, hipStream_t stream) {
    switch (dtype) {
        case 1: return D == 64 ? launch_rb2_typed<__bf16, 64>(p, causal, stream)
                               : launch_rb2_typed<__bf16, 128>(p, causal, stream);
        case 2: return D == 64 ? launch_rb2_typed<_Float16, 64>(p, causal, stream)
                               : launch_rb2_typed<_Float16, 128>(p, causal, stream);
        default: return D == 64 ? launch_rb2_typed<uint8_t, 64>(p, causal, stream)
                                : launch_rb2_typed<uint8_t, 128>(p, causal, stream);
    }
}

}  // namespace attn

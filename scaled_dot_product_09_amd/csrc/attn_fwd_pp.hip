// attn_fwd_pp.hip — fused attention forward on gfx950 matrix cores, two wave
// groups in ping-pong.
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
// Design (one workgroup = 8 wavefronts of 64 lanes, one workgroup per CU):
//   * Each wave owns 32 query rows of one query head. A workgroup holds
//     `gpack` query heads that read the same KV head and 8 / gpack row
//     blocks of 32 rows, so every K/V tile staged in LDS serves 256 query
//     rows.
//   * Per 64-key tile a wave has two phases: X (matrix cores: the scores of
//     the next tile, S^T = K Q^T, and the output update of this tile,
//     O^T += V^T P^T) and Y (vector ALU: mask, row max, lazy rescale, and the
//     weights P = exp2(c s - m) of the next tile). The waves of a SIMD are
//     w and w + 4, so group 0 (waves 0-3) runs its phases one slot ahead of
//     group 1 (waves 4-7) and workgroup barriers separate the slots: in every
//     slot each SIMD has one wave in X and one in Y, so the softmax runs in
//     the shadow of the other wave's matrix products.
//   * K and V go from HBM straight into LDS (buffer loads to LDS, no register
//     staging), double-buffered; group 1 issues the copies for tile j+2 (K)
//     and j+1 (V) in its Y slot and drains them at the end of its next X
//     slot, two slots before they are read. 16-byte chunks are XOR-swizzled
//     per row so the operand reads are bank-conflict free.
//   * Scores are computed transposed: lane (h = lane / 32, n = lane % 32)
//     holds 16 scores of query n per 32-key block, so a row's max needs one
//     exchange between lanes n and n + 32 and its sum stays per lane until
//     the end. The score accumulator, rounded, is the P operand directly; V
//     is gathered in the matching key order by the gfx950 LDS transpose read
//     (ds_read_b64_tr_b16) from row-major V.
//   * Online softmax in the exp2 domain: one FMA (scale folded in) and one
//     v_exp per score; row sums by v_dot2 over the rounded weights, so the
//     normalisation uses exactly the weights that multiplied V. The running
//     max is only raised when it grows by more than 8 (a factor 2^8):
//     numerator and denominator share the stale max, so the result is
//     unchanged, and weights up to 256 are harmless in bf16 / f16.
//   * Causal: tiles wholly above the workgroup's diagonal are never loaded;
//     a wave's scores above its own diagonal are masked to -inf (weight 0).

#include "mfma_common.h"

// Lambdas in the kernel capture register arrays by reference: any call left
// out of line would move those arrays to scratch memory.
#define INLINE __attribute__((always_inline))

namespace attn {

template <typename T, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd_pp_kernel(FwdParams p) {
    using Tr = Traits<T>;
    using qk_frag = typename Tr::qk_frag;
    using pv_frag = typename Tr::pv_frag;
    using out_t = typename Tr::out_t;
    constexpr int KROWB = D * Tr::IN_BYTES;           // bytes of one K / Q row
    constexpr int VROWB = D * 2;                      // bytes of one V row in LDS (16-bit)
    constexpr int NCK = KROWB / 16;                   // 16-byte chunks per K row
    constexpr int NCV = VROWB / 16;
    constexpr int CH = Tr::QK_LANE_BYTES / 16;        // chunks per lane per k-step
    constexpr int KSTEPS = D / Tr::QK_K;              // MFMA k-steps of one score block
    constexpr int NKB = BN / 32;                      // 32-key blocks per tile
    constexpr int NDB = D / 32;                       // 32-wide column blocks of O
    constexpr int NPV = NKB * 2;                      // 16-key groups of one tile (PV k-steps)
    constexpr int KTILE = BN * KROWB, VTILE = BN * VROWB;
    static_assert(NKB == 2, "the phase-X interleave assumes 64-key tiles");

    // Separate LDS objects, so the compiler can prove that a copy landing in
    // one buffer never aliases reads of another.
    __shared__ __attribute__((aligned(1024))) uint8_t lds_k0[KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_k1[KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_v0[VTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_v1[VTILE];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;            // 0: waves 0-3, 1: waves 4-7 (w and w+4 share a SIMD)
    const int wq = wave & 3;              // wave inside its group
    const int h = lane >> 5;              // which half of the wave
    const int n = lane & 31;              // query column inside the wave's 32 rows

    const WorkItem wi = map_workgroup(p, CAUSAL);
    const int hq = wi.hq0 + (wave % p.gpack);
    const int q0 = wi.row_base + (wave / p.gpack) * 32;
    const int Sq = p.Sq, Skv = p.Skv;
    const size_t qstride = (size_t)p.Hq * D;          // elements between query rows
    const size_t kstride = (size_t)p.Hkv * D;

    const T* qbase = (const T*)p.q + ((size_t)wi.b * Sq * p.Hq + hq) * D;
    const uint8_t* kbase = (const uint8_t*)((const T*)p.k + ((size_t)wi.b * Skv * p.Hkv + wi.hkv) * D);
    const uint8_t* vbase = (const uint8_t*)((const T*)p.v + ((size_t)wi.b * Skv * p.Hkv + wi.hkv) * D);
    const size_t kstride_b = kstride * Tr::IN_BYTES;

    // Q^T operand, kept in registers for the whole key loop: lane (h, n) holds
    // bytes [(2 ks + h) * QK_LANE_BYTES, +QK_LANE_BYTES) of row q0 + n. A
    // negative scale is folded into Q: (-q).k is exactly -(q.k) (negation is
    // exact and the products are summed in the same order), with the
    // multiplier |c|, so the softmax only ever sees c > 0 and masks with -inf.
    qk_frag qf[KSTEPS];
    {
        const int row = q0 + n;
        const uint8_t* src = (const uint8_t*)(qbase + row * qstride);
        const uint32_t flip = p.scale_log2 < 0.f ? Tr::SIGN_BITS : 0u;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 x[CH];
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                x[t] = (u32x4){0, 0, 0, 0};
                if (row < Sq) x[t] = *(const u32x4*)(src + ((2 * ks + h) * CH + t) * 16);
                x[t] ^= flip;
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
        const int last_row = min(wi.row_base + p.rows_per_wg, Sq) - 1 + p.causal_off;
        n_tiles = min(n_tiles, last_row / BN + 1);
    }
    n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);

    // ---- tile staging (group 1 only) -----------------------------------------
    // K(j) lives in lds_k[j % 2], V(j) in lds_v[j % 2]; the schedule below is
    // unrolled by two tiles so every buffer is a distinct, static LDS object.
    // FP8: V is widened to bf16 in registers (exact) and written to LDS by
    // group 1's threads; 8 values (one 16-byte chunk) per thread and step.
    constexpr int V_ST = Tr::V_DMA ? 1 : (BN * D / 8) / 256;
    const int gtid = tid & 255;           // thread inside its group
    u32x2 vstage[V_ST];
    TileDma<KROWB, BN> kdma;
    TileDma<VROWB, BN> vdma;
    kdma.init(kbase, (uint32_t)kstride_b, wq, lane, kSwzK);
    if constexpr (Tr::V_DMA) vdma.init(vbase, (uint32_t)kstride_b, wq, lane, kSwzV);
    auto issue_k = [&](int j, uint8_t* kt) INLINE { kdma.issue(j * BN, Skv, kt, wq); };
    auto issue_v = [&](int j, uint8_t* vt) INLINE {
        if constexpr (Tr::V_DMA) {
            vdma.issue(j * BN, Skv, vt, wq);
        } else {
#pragma unroll
            for (int u = 0; u < V_ST; ++u) {
                const int id = u * 256 + gtid;
                const int r = id / (D / 8), c = id % (D / 8);
                const int key = min(j * BN + r, Skv - 1);
                vstage[u] = *(const u32x2*)(vbase + key * kstride_b + c * 8);
            }
        }
    };
    auto finish_v = [&](uint8_t* vt) INLINE {   // FP8 only: widen the staged V and write it
        if constexpr (!Tr::V_DMA) {
#pragma unroll
            for (int u = 0; u < V_ST; ++u) {
                const int id = u * 256 + gtid;
                const int r = id / (D / 8), c = id % (D / 8);
                u32x4 w;
#pragma unroll
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

    // ---- running softmax state (per lane: query n, partial over its keys) --
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = -INFINITY;   // running max of c * score in the log2 domain (same on both halves)
    float l_part = 0.f;        // this lane's share of the running denominator
    const float c_log2 = fabsf(p.scale_log2);   // > 0: the host never passes 0
    const int qrow = q0 + n;

    // Per-lane constants of the operand reads (see load_k / load_v).
    const int L16 = lane & 15;                 // lane inside its 16-lane group
    const int G16 = (lane >> 4) & 1;           // which 16 columns of a 32-column block
    const int v_row_in = 4 * h + (L16 >> 2);   // key row offset this lane addresses
    const int v_col_b = 32 * G16 + 8 * (L16 & 3);   // byte offset inside a 64-byte column block
    // K row kb*32 + n, 16-byte chunk (2 ks + h) * CH + t sits at byte
    // n * KROWB + ((((2 ks + h) * CH + t) ^ k_swz(n)) << 4): the k-step only
    // flips bits of the chunk index above those of (h, t), so the offset is
    // k_lane_base ^ (ks * 32 * CH) plus t * 16 (t ^ mask bit, folded below).
    const int k_sw = k_swz<NCK>(n);
    const uint32_t k_lane_base0 = n * KROWB + ((((h * CH) ^ k_sw)) << 4);
    const uint32_t k_lane_base1 = n * KROWB + ((((h * CH + (CH - 1)) ^ k_sw)) << 4);
    int v_lane_off[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int cb = db * 64 + v_col_b;
        v_lane_off[db] = v_row_in * VROWB + ((((cb >> 4) ^ v_swz<NCV>(v_row_in)) << 4) | (cb & 15));
    }

    auto load_k = [&](const uint8_t* kt, int kb, int ks) INLINE -> qk_frag {
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
    // V operand of the PV step for keys 16 g + {0..15} of the tile and output
    // columns 32 db + {0..31}. Lane (h, n) needs V[key][32 db + n] for keys
    // 16 g + 4h + {0..3} (frag elements 0..3) and 16 g + 8 + 4h + {0..3}
    // (elements 4..7), the key order of the score accumulator. The transpose
    // read hands lane i of a 16-lane group element i % 4 of the 8 bytes
    // addressed by lanes 4 s + i / 4 (s = 0..3), so lane L addresses key row
    // 16 g + 4h + L / 4 at columns 32 db + 16 G16 + 4 (L % 4) .. +3.
    auto load_v = [&](const uint8_t* vt, int g, int db) INLINE -> pv_frag {
        const uint8_t* a_lo = vt + (16 * g) * VROWB + v_lane_off[db];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a_lo));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a_lo + 8 * VROWB));
        return __builtin_bit_cast(pv_frag, (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };

    f32x16 s[NKB];             // scores of the tile being prepared
    uint32_t pw[NKB][8];       // rounded weights of the tile being accumulated

    // ---- phase X: scores of tile j+1 (if any) and O += V(j)^T P(j) ----------
    // The score and output MFMAs are independent; they are issued as one
    // stream, PV op p (key group p / NDB, column block p % NDB) followed by
    // the score ops [qlo(p), qlo(p+1)), so that neither accumulator chain
    // issues back to back. Each operand is fetched from LDS two ops of its
    // kind ahead, through a ring of three registers.
    // kt holds K(j+1), vt holds V(j); __restrict__ (once inlined) tells the
    // compiler these reads never alias the copies in flight to the others.
    auto phase_x = [&](auto has_next_tag, const uint8_t* __restrict__ kt, const uint8_t* __restrict__ vt) INLINE {
        constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
        constexpr int NQK = HAS_NEXT ? KSTEPS * NKB : 0;   // score ops: (ks, kb) = (q / NKB, q % NKB)
        constexpr int NPO = NPV * NDB;                      // output ops
        auto qlo = [](int pidx) INLINE { return (pidx * NQK + NPO - 1) / NPO; };
        auto fetch_k = [&](int q) INLINE { return load_k(kt, q % NKB, q / NKB); };
        auto fetch_v = [&](int pidx) INLINE { return load_v(vt, pidx / NDB, pidx % NDB); };
        qk_frag kr[3];
        pv_frag vr[3];
        if constexpr (HAS_NEXT) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[kb] = (f32x16){};
            kr[0] = fetch_k(0);
            if (NQK > 1) kr[1] = fetch_k(1);
        }
        vr[0] = fetch_v(0);
        vr[1] = fetch_v(1);
#pragma unroll
        for (int pidx = 0; pidx < NPO; ++pidx) {
            if (pidx + 2 < NPO) vr[(pidx + 2) % 3] = fetch_v(pidx + 2);
            const int g = pidx / NDB, db = pidx % NDB;
            const int kb = g / 2, s2 = g % 2;
            const pv_frag pf = __builtin_bit_cast(pv_frag, (u32x4){pw[kb][4 * s2], pw[kb][4 * s2 + 1],
                                                                   pw[kb][4 * s2 + 2], pw[kb][4 * s2 + 3]});
            oacc[db] = Tr::pv(vr[pidx % 3], pf, oacc[db]);
#pragma unroll
            for (int q = qlo(pidx); q < qlo(pidx + 1); ++q) {
                if (q + 2 < NQK) kr[(q + 2) % 3] = fetch_k(q + 2);
                s[q % NKB] = Tr::qk(kr[q % 3], qf[q / NKB], s[q % NKB]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- phase Y: softmax of tile t (scores in s) -> weights pw --------------
    auto phase_y = [&](int t) INLINE {
        // Mask keys past the end or above the causal diagonal to -inf. The
        // test is skipped (wave-uniformly) wherever no key of a 32-key block
        // is hidden from any row of the wave.
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const int kbase_h = t * BN + kb * 32 + 4 * h;       // key of element i: kbase_h + koff(i)
            int lim = Skv - 1 - kbase_h;                         // last existing key offset
            if (CAUSAL) lim = min(lim, qrow + p.causal_off - kbase_h);          // last visible key offset
            if (__builtin_amdgcn_ballot_w64(lim < 27) != 0) {   // 27 = largest koff(i)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    s[kb][i] = (8 * (i >> 2) + (i & 3) > lim) ? -INFINITY : s[kb][i];
            }
        }
        // Row max in the log2 domain (lanes n and n + 32 hold the two halves
        // of a row), then the lazy rescale of O and l.
        float mraw = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; i += 2) mraw = fmaxf(mraw, fmaxf(s[kb][i], s[kb][i + 1]));
        // c_log2 > 0, so a fully masked row gives -inf * c = -inf here.
        const float mt = xor32_max(mraw * c_log2);
        const float mnew = fmaxf(m_run, mt);
        if (__builtin_amdgcn_ballot_w64(mnew > m_run + 8.0f) != 0) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);   // 0 on the first tile
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
            l_part *= alpha;
            m_run = mnew;
        }
        const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
        // Weights exp2(c s - m), rounded to the input type; the row sum adds
        // exactly the rounded values.
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * i], c_log2, neg_m));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * i + 1], c_log2, neg_m));
                pw[kb][i] = Tr::pack(e0, e1);
                l_part = Tr::sum2(pw[kb][i], l_part);
            }
    };

    // Scores of tile 0 (both groups, before the ping-pong starts).
    auto scores_first = [&]() INLINE {
        const uint8_t* kt = lds_k0;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = (f32x16){};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[kb] = Tr::qk(load_k(kt, kb, ks), qf[ks], s[kb]);
    };

    // ---- schedule ----------------------------------------------------------
    // Phases in order: Y(0), X(0), Y(1), X(1), ..., Y(n-1), X(n-1) where Y(t)
    // prepares the weights of tile t and X(j) computes the scores of tile j+1
    // and accumulates tile j. Both groups run the same code; group 1 starts
    // one slot later (an extra barrier before its first phase) and group 0
    // ends with one extra barrier, so every wave executes the same number of
    // barriers and, in between, group 0 runs phase k in slot k while group 1
    // runs phase k-1: one wave of each SIMD is always in X and one in Y.
    // X(j) reads K(j+1) and V(j) in slots 2j+1 and 2j+2. Group 1 copies
    // K(j+2) and V(j+1) at the start of slot 2j+1 (into the buffers of K(j)
    // and V(j-1), last read in slot 2j) and drains them before the barrier
    // that ends slot 2j+2.
    const bool copier = grp == 1;
    if (copier) {
        issue_k(0, lds_k0);
        issue_v(0, lds_v0);
        if (n_tiles > 1) issue_k(1, lds_k1);
        finish_v(lds_v0);
    }
    dma_barrier();
    scores_first();
    if (copier) {
        __syncthreads();                               // group 1 lags one slot
        if (n_tiles > 2) issue_k(2, lds_k0);
        if (n_tiles > 1) issue_v(1, lds_v1);
    }
    phase_y(0);
    __syncthreads();
    // One pipelined step: X(j), the copies of K(j+3) and V(j+2), Y(j+1).
    auto step = [&](int j, uint8_t* __restrict__ kt, uint8_t* __restrict__ vt,
                    uint8_t* __restrict__ vt_next) INLINE {
        __builtin_amdgcn_s_setprio(1);
        phase_x(std::true_type{}, kt, vt);
        __builtin_amdgcn_s_setprio(0);
        if (copier) finish_v(vt_next);                 // FP8: V(j+1)
        dma_barrier();                                 // group 1: K(j+2), V(j+1) landed
        if (copier) {
            if (j + 3 < n_tiles) issue_k(j + 3, kt);
            if (j + 2 < n_tiles) issue_v(j + 2, vt);
        }
        phase_y(j + 1);
        __syncthreads();
    };
    int j = 0;
    for (; j + 2 < n_tiles; j += 2) {
        step(j, lds_k1, lds_v0, lds_v1);
        step(j + 1, lds_k0, lds_v1, lds_v0);
    }
    if (j + 1 < n_tiles) {
        step(j, lds_k1, lds_v0, lds_v1);
        ++j;
    }
    __builtin_amdgcn_s_setprio(1);
    if (j & 1) phase_x(std::false_type{}, lds_k0, lds_v1);
    else phase_x(std::false_type{}, lds_k1, lds_v0);
    __builtin_amdgcn_s_setprio(0);
    if (!copier) __syncthreads();                      // group 0 matches group 1's count

    // ---- epilogue: O = O^T / l, round once, store [b][row][hq][d] ----------
    const float l = xor32_sum(l_part);
    const float inv = p.out_mul / l;
    if (qrow < Sq) {
        out_t* orow = (out_t*)p.out + ((size_t)wi.b * Sq + qrow) * qstride + (size_t)hq * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = db * 32 + 8 * jj + 4 * h;
                const uint32_t w0 = Tr::pack(oacc[db][4 * jj + 0] * inv, oacc[db][4 * jj + 1] * inv);
                const uint32_t w1 = Tr::pack(oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv);
                *(u32x2*)(orow + d0) = (u32x2){w0, w1};
            }
        }
    }
}

template <typename T, int D>
static hipError_t launch_pp_typed(const FwdParams& p, bool causal, hipStream_t stream) {
    const dim3 grid(p.n_units * p.n_row_blocks), block(512);
    if (causal)
        hipLaunchKernelGGL((fwd_pp_kernel<T, D, 64, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_pp_kernel<T, D, 64, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// dtype: ATTN_BF16 (1), ATTN_F16 (2) or ATTN_FP8_E4M3 (3); D = 64 or 128.
hipError_t launch_fwd_pp(const FwdParams& p, int D, int dtype, bool causal, hipStream_t stream) {
    switch (dtype) {
        case 1: return D == 64 ? launch_pp_typed<__bf16, 64>(p, causal, stream)
                               : launch_pp_typed<__bf16, 128>(p, causal, stream);
        case 2: return D == 64 ? launch_pp_typed<_Float16, 64>(p, causal, stream)
                               : launch_pp_typed<_Float16, 128>(p, causal, stream);
        default: return D == 64 ? launch_pp_typed<fp8_t, 64>(p, causal, stream)
                                : launch_pp_typed<fp8_t, 128>(p, causal, stream);
    }
}

}  // namespace attn

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
// Design (one workgroup = 4 wavefronts of 64 lanes, two workgroups per CU;
// the launcher's shape rule picks the key-half form for very small grids and
// the sequential 32-key form, three workgroups per CU, for short rows of keys
// at head dim 128 — see the kernel template and launch_typed):
//   * Each wave owns 32 query rows of one query head. A workgroup holds
//     `gpack` query heads that read the same KV head, 4 / gpack row blocks of
//     32 rows each, so every K/V tile staged in LDS serves 128 query rows.
//   * K and V tiles go from HBM straight into LDS (buffer loads to LDS,
//     no register staging; FP8 V through registers, widened to bf16),
//     double-buffered: the next tile is in flight while one is computed,
//     with one barrier per tile. 16-byte chunks are
//     XOR-swizzled per row so the operand reads below are bank-conflict free.
//   * Scores are computed transposed, S^T = K Q^T: lane (h = lane / 32,
//     n = lane % 32) then holds 16 scores of query n per 32-key block, so a
//     row's max needs one exchange between lanes n and n + 32, and its sum
//     stays per lane until the end.
//   * O^T = V^T P^T. The score accumulator is used directly as the P operand:
//     the MFMA sums over k in any order as long as both operands agree, so
//     the V operand is gathered with the same key order by the gfx950 LDS
//     transpose read (ds_read_b64_tr_b16) from row-major V.
//   * Online softmax in the exp2 domain: one FMA (scale folded in) and one
//     v_exp per score; row max by v_max3; row sums by v_dot2 over the
//     rounded weights, so the normalisation uses exactly the weights that
//     multiplied V. The running max is only raised when it grows by more
//     than 8 (a factor 2^8): numerator and denominator share the stale max,
//     so the result is unchanged, and weights up to 256 are harmless in
//     bf16 / f16.
//   * Causal: tiles wholly above the workgroup's diagonal are never loaded;
//     from the first tile wholly above a wave's own rows on, that wave only
//     copies tiles and keeps the barriers; only 32-key blocks crossing the
//     diagonal (or the end of the keys) are masked.

#include "mfma_common.h"

namespace attn {

// RB = 32-row blocks per wave (1 or 2). With RB = 2 every K / V operand read
// from LDS feeds the MFMAs of both blocks, which halves LDS reads per flop;
// the doubled accumulators need the whole register file (one wave per SIMD).
// KS = key halves per workgroup (1 or 2). With KS = 2 the workgroup has
// twice the waves: waves 2 w and 2 w + 1 own the same query slots and take
// alternate key tiles (even and odd); the SIMD that runs one of them (waves
// go round the four SIMDs in order) also runs a half of query wave w + 2,
// which in a folded workgroup holds the mirror row block, so the causal
// work of the two blocks shares every SIMD. Each LDS stage then holds KS
// tiles side by side (a step of KS * BN keys, copied by all waves); half h
// computes on the tile at rows h * BN of it. At the end the two partial
// softmax states (running max, weight sum, unnormalised output) of a slot
// are merged through LDS. For grids too small to give every SIMD two waves.
template <typename T, int D, int BN, bool CAUSAL, int NWAVES, int RB, int KS = 1>
__global__ __launch_bounds__(64 * NWAVES, RB == 1 ? (BN == 32 ? 3 : 8 / NWAVES) : 1) void fwd_mfma_kernel(FwdParams p) {
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
    constexpr int KTILE = KS * BN * KROWB, VTILE = KS * BN * VROWB;   // one stage: KS tiles
    constexpr int NWQ = NWAVES / KS;                  // waves holding distinct query slots
    static_assert(KS == 1 || RB == 1, "the key halves merge one row block per wave");

    // Four separate LDS objects (not one array cut in four), so the compiler
    // can prove that a copy landing in one buffer never aliases reads of
    // another and does not make those reads wait for the copy.
    __shared__ __attribute__((aligned(1024))) uint8_t lds_k0[KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_k1[KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_v0[VTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_v1[VTILE];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = KS == 1 ? wave_all : wave_all / KS;    // which query slots
    const int half = KS == 1 ? 0 : wave_all % KS;           // which key half
    const int h = lane >> 5;              // which half of the wave
    const int n = lane & 31;              // query column inside the wave's 32 rows

    const WorkItem wi = map_workgroup(p, CAUSAL);
    float sl2, out_mul;
    fwd_scalars(p, sl2, out_mul);
    // The workgroup's 32 * NWAVES query slots cover gpack query heads (of one
    // KV head) times rows_per_wg rows, in runs of HS = head_stride rows of
    // one head: slot s is head hq0 + (s / HS) % gpack and row
    // row_base + (s / (HS gpack)) HS + s % HS. Lane n of a wave owns slot
    // 32 wave + n. With HS = 32 a wave holds 32 rows of one head; with
    // fewer rows than that per head (decode with GQA / MQA) a wave's 32 MFMA
    // columns hold rows of several heads instead of empty rows.
    // With RB = 2, row block r of the wave owns slots 32 (2 wave + r) + n.
    const int HS = p.head_stride;
    int hq[RB], qrow[RB];
    for (int r = 0; r < RB; ++r) {
        const int slot = (wave * RB + r) * 32 + n;
        hq[r] = wi.hq0 + slot_head(p, slot);
        qrow[r] = item_row(p, wi, slot);
    }
    // No slot of this wave holds a query row (its first slot has its
    // smallest row): it only copies tiles and keeps the workgroup's barriers.
    const bool wave_idle = __builtin_amdgcn_readfirstlane(item_row(p, wi, wave * RB * 32)) >= p.Sq;
    const int Sq = p.Sq;
    int Skv = p.Skv;                                   // keys of this workgroup's range, from its start

    const uint8_t* kbase = (const uint8_t*)((const T*)p.k + wi.b * p.sk[0] + wi.hkv * p.sk[2]);
    const uint8_t* vbase = (const uint8_t*)((const T*)p.v + wi.b * p.sv[0] + wi.hkv * p.sv[2]);
    const size_t krow_b = (size_t)p.sk[1] * Tr::IN_BYTES;   // bytes between keys
    const size_t vrow_b = (size_t)p.sv[1] * Tr::IN_BYTES;

    // Q^T operand, kept in registers for the whole key loop: lane (h, n) holds
    // bytes [(2 ks + h) * QK_LANE_BYTES, +QK_LANE_BYTES) of its slot's row.
    // A negative scale is folded into Q: the kernel computes (-q).k, which
    // is exactly -(q.k) (negation is exact and the products are summed in
    // the same order), with the multiplier |c|, so the softmax below only
    // ever sees c >= 0 and masks with -inf.
    qk_frag qf[RB][KSTEPS];
    for (int r = 0; r < RB; ++r) {
        const int row = qrow[r];
        const T* qbase = (const T*)p.q + wi.b * p.sq[0] + hq[r] * p.sq[2];
        const uint8_t* src = (const uint8_t*)(qbase + row * p.sq[1]);
        const uint32_t flip = sl2 < 0.f ? Tr::SIGN_BITS : 0u;
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 x[CH];
            for (int t = 0; t < CH; ++t) {
                x[t] = (u32x4){0, 0, 0, 0};
                if (row < Sq) x[t] = *(const u32x4*)(src + ((2 * ks + h) * CH + t) * 16);
                x[t] ^= flip;
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
        const int last_row = min(wi.row_end, Sq) - 1 + p.causal_off;
        n_tiles = min(n_tiles, last_row / BN + 1);
    }
    n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);
    // With KS = 2, half h takes the tiles h, h + 2, h + 4, ...: its local tile
    // j is tile gt(j) = 2 j + h of the workgroup's range; n_tiles becomes the
    // half's own count, nt_max the larger of the two halves' counts (both
    // halves run nt_max barrier steps).
    auto gt = [&](int j) { return KS == 1 ? j : KS * j + half; };
    auto local_count = [&](int n_glob) { return KS == 1 ? n_glob : max(0, (n_glob - half + KS - 1) / KS); };

    // Split keys (n_split > 1): this workgroup takes tiles [tb, te) of the
    // n_tiles it would otherwise loop over, and writes an unnormalised partial
    // result for a separate combine step. The key range is made to start at
    // 0: the K/V bases move to key tb * BN, and the key count and the causal
    // offset move with them.
    int coff = p.causal_off;
    const size_t qrow_idx = ((size_t)wi.split * p.B + wi.b) * Sq;   // partial-buffer row base
    if (p.n_split > 1) {
        const int tb = wi.split * n_tiles / p.n_split;
        const int te = (wi.split + 1) * n_tiles / p.n_split;
        n_tiles = te - tb;
        kbase += (size_t)tb * BN * krow_b;
        vbase += (size_t)tb * BN * vrow_b;
        Skv -= tb * BN;
        coff -= tb * BN;
        if (n_tiles == 0) {   // no keys in range: weight sum 0, max -inf, output 0
            for (int rb = 0; rb < RB; ++rb) {
                const int row = qrow[rb];
                if (row < Sq) {
                    const size_t r = (qrow_idx + row) * p.Hq + hq[rb];
                    for (int db = 0; db < NDB; ++db)
                        for (int jj = 0; jj < 4; ++jj)
                            *(f32x4*)(p.part_o + r * D + db * 32 + 8 * jj + 4 * h) = (f32x4){0.f, 0.f, 0.f, 0.f};
                    if (h == 0) *(f32x2*)(p.part_ml + r * 2) = (f32x2){-INFINITY, 0.f};
                }
            }
            return;
        }
    }
    const int nt_glob = n_tiles;
    const int nt_max = KS == 1 ? nt_glob : (nt_glob + KS - 1) / KS;
    n_tiles = local_count(nt_glob);

    // ---- tile staging ------------------------------------------------------
    // LDS: two K tiles and two V tiles. The loop below is software-pipelined
    // one tile deep (the scores of tile j+1 are computed while the weights of
    // tile j are formed), so K runs one tile ahead of V: iteration j reads
    // K(j+1) and V(j) and, meanwhile, loads K(j+2) into the K buffer K(j)
    // used and V(j+1) into the V buffer V(j-1) used.
    uint8_t* const kbuf0 = lds_k0;
    uint8_t* const kbuf1 = lds_k1;
    uint8_t* const vbuf0 = lds_v0;
    uint8_t* const vbuf1 = lds_v1;
    // FP8: V is widened to bf16 in registers (exact) and written to LDS by
    // the threads; 8 values (one 16-byte chunk) per thread and step. Thread
    // tid stages chunk c0 = tid % (D / 8) of rows r0 + u RSTEP of the stage
    // (u < V_ST); the row step keeps the chunk and the swizzle mask, so the
    // global and LDS offsets of every u are the thread's offsets for u = 0
    // plus a constant, and a stage only adds a scalar offset.
    constexpr int NTHR = 64 * NWAVES;
    constexpr int V_ST = Tr::V_DMA ? 1 : (KS * BN * D / 8) / NTHR;
    constexpr int RSTEP = NTHR / (D / 8);
    static_assert(Tr::V_DMA || (NTHR % (D / 8) == 0 && RSTEP % 16 == 0), "the V swizzle must repeat over RSTEP rows");
    u32x2 vstage[V_ST];
    const int v_r0 = tid / (D / 8), v_c0 = tid % (D / 8);
    const uint32_t v_goff = (uint32_t)v_r0 * (uint32_t)vrow_b + (uint32_t)v_c0 * 8;   // tile byte offset, u = 0
    const uint32_t v_loff = (uint32_t)(v_r0 * VROWB + ((v_c0 ^ v_swz<NCV>(v_r0)) << 4));
    const __amdgpu_buffer_rsrc_t v_rs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, -1, kBufferWord3);
    // The copies are split over all waves, or over the first four when a
    // tile has fewer 1 KiB pieces than there are waves.
    // j is a stage (a step of KS tiles); every wave of the workgroup copies.
    constexpr int NWK = (KS * BN * KROWB / 1024) % NWAVES == 0 ? NWAVES : 4;
    constexpr int NWV = (KS * BN * VROWB / 1024) % NWAVES == 0 ? NWAVES : 4;
    TileDma<KROWB, KS * BN, NWK> kdma;
    TileDma<VROWB, KS * BN, NWV> vdma;
    kdma.init(kbase, (uint32_t)krow_b, wave_all % NWK, lane, kSwzK);
    if constexpr (Tr::V_DMA) vdma.init(vbase, (uint32_t)vrow_b, wave_all % NWV, lane, kSwzV);
    auto issue_k = [&](int j, uint8_t* kt) {
        if (NWK == NWAVES || wave_all < NWK) kdma.issue(j * KS * BN, Skv, kt, wave_all);
    };
    auto issue_v = [&](int j, uint8_t* vt) {
        if constexpr (Tr::V_DMA) {
            if (NWV == NWAVES || wave_all < NWV) vdma.issue(j * KS * BN, Skv, vt, wave_all);
        } else {
            // Rows past the end of the keys (last stage only) repeat the last
            // key, as in the tile copies. Byte offsets stay below
            // Skv * row stride < 2^32.
            const int key0 = j * KS * BN;
            const uint32_t t0 = (uint32_t)key0 * (uint32_t)vrow_b;
            if (key0 + KS * BN <= Skv) {
                for (int u = 0; u < V_ST; ++u)
                    vstage[u] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                        v_rs, v_goff, t0 + (uint32_t)(u * RSTEP) * (uint32_t)vrow_b, 0));
            } else {
                for (int u = 0; u < V_ST; ++u) {
                    const int key = min(key0 + v_r0 + u * RSTEP, Skv - 1);
                    vstage[u] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                        v_rs, (uint32_t)key * (uint32_t)vrow_b + (uint32_t)v_c0 * 8, 0, 0));
                }
            }
        }
    };
    auto finish_v = [&](uint8_t* vt) {   // FP8 only: widen the staged V and write it
        if constexpr (!Tr::V_DMA) {
            for (int u = 0; u < V_ST; ++u) {
                u32x4 w;
                // Two E4M3 codes -> two bf16 per instruction (scale 1: exact,
                // every E4M3 value is a bf16 value; same bits as widening to
                // fp32 and rounding to bf16, checked on all 256 codes).
                for (int e = 0; e < 2; ++e) {
                    w[2 * e] = __builtin_bit_cast(
                        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vstage[u][e], 1.0f, false));
                    w[2 * e + 1] = __builtin_bit_cast(
                        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vstage[u][e], 1.0f, true));
                }
                *(u32x4*)(vt + v_loff + u * RSTEP * VROWB) = w;
            }
        }
    };

    // ---- running softmax state (per lane: query n, partial over its keys) --
    f32x16 oacc[RB][NDB];
    for (int r = 0; r < RB; ++r)
        for (int db = 0; db < NDB; ++db)
            for (int i = 0; i < 16; ++i) oacc[r][db][i] = 0.f;
    float m_run[RB];    // running max of scale*log2(e)*score (same on both halves)
    // This lane's share of the running denominator, as NLSUM partial sums
    // (the row-sum dot products of a tile form NLSUM independent chains
    // instead of one).
    constexpr int NLSUM = 2;
    float l_part[RB][NLSUM];
    float neg_m[RB];    // exponent offset -m_run of the tile being weighted
    for (int r = 0; r < RB; ++r) {
        m_run[r] = -INFINITY;
        for (int t = 0; t < NLSUM; ++t) l_part[r][t] = 0.f;
        neg_m[r] = 0.f;
    }

    const float c_log2 = fabsf(sl2);   // > 0: never 0 (see fwd_scalars)

    // Per-lane constants of the V transpose read (see load_v).
    const int L16 = lane & 15;                 // lane inside its 16-lane group
    const int G16 = (lane >> 4) & 1;           // which 16 columns of a 32-column block
    const int v_row_in = 4 * h + (L16 >> 2);   // key row offset this lane addresses
    const int v_col_b = 32 * G16 + 8 * (L16 & 3);   // byte offset inside a 64-byte column block
    // Byte offsets of this lane's operand reads inside a K / V tile. The
    // swizzle masks depend only on lane bits: K row kb*32 + n has mask
    // k_swz(n), and the V rows base + 4h + L16/4 (base a multiple of 16) have
    // mask v_swz(4h + L16/4); so every read below is a lane base plus a
    // compile-time offset.
    // K row kb*32 + n, 16-byte chunk (2 ks + h) * CH + t sits at byte
    // n * KROWB + ((((2 ks + h) * CH + t) ^ k_swz(n)) << 4): the k-step only
    // flips bits of the chunk index above those of (h, t), so the offset is
    // k_lane_base ^ (ks * 32 * CH) plus t * 16 (t ^ mask bit, folded below).
    const int k_sw = k_swz<NCK>(n);
    // With KS = 2 half h reads the tile at rows h * BN of each stage: a
    // multiple of the swizzle periods, and a power of two above every bit the
    // k-step XOR below touches.
    const uint32_t k_half = (uint32_t)(half * BN * KROWB), v_half = (uint32_t)(half * BN * VROWB);
    const uint32_t k_lane_base0 = k_half + n * KROWB + ((((h * CH) ^ k_sw)) << 4);
    const uint32_t k_lane_base1 = k_half + n * KROWB + ((((h * CH + (CH - 1)) ^ k_sw)) << 4);
    int v_lane_off[NDB];
    for (int db = 0; db < NDB; ++db) {
        const int cb = db * 64 + v_col_b;
        v_lane_off[db] = v_half + v_row_in * VROWB + ((((cb >> 4) ^ v_swz<NCV>(v_row_in)) << 4) | (cb & 15));
    }

    // Operand fetches from the LDS tiles (lane-base + compile-time offsets).
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
    // V operand of the PV step for keys kb*32 + 16 s2 + {0..15} and output
    // columns 32 db + {0..31}. Lane (h, n) needs V[key][32 db + n] for keys
    // base + 4h + {0..3} (frag elements 0..3) and base + 8 + 4h + {0..3}
    // (elements 4..7). The transpose read hands lane i of a 16-lane group
    // element i % 4 of the 8 bytes addressed by lanes 4 s + i / 4 (s = 0..3),
    // so lane L addresses key row base + 4h + L / 4 at columns
    // 32 db + 16 G16 + 4 (L % 4) .. +3 (v_lane_off holds that offset).
    auto load_v = [&](const uint8_t* vt, int kb, int s2, int db) -> pv_frag {
        const uint8_t* a_lo = vt + (kb * 32 + 16 * s2) * VROWB + v_lane_off[db];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a_lo));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a_lo + 8 * VROWB));
        return __builtin_bit_cast(pv_frag, (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };

    // S^T = K Q^T for one tile (all 32-key blocks), K operands fetched one
    // k-step ahead.
    auto qk_tile = [&](const uint8_t* kt, f32x16 (&s)[RB][NKB]) {
        for (int r = 0; r < RB; ++r)
            for (int kb = 0; kb < NKB; ++kb)
                for (int i = 0; i < 16; ++i) s[r][kb][i] = 0.f;
        qk_frag cur[NKB], nxt[NKB];
        for (int kb = 0; kb < NKB; ++kb) cur[kb] = load_k(kt, kb, 0);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            if (ks + 1 < KSTEPS)
                for (int kb = 0; kb < NKB; ++kb) nxt[kb] = load_k(kt, kb, ks + 1);
            for (int kb = 0; kb < NKB; ++kb)
                for (int r = 0; r < RB; ++r) s[r][kb] = Tr::qk(cur[kb], qf[r][ks], s[r][kb]);
            if (ks + 1 < KSTEPS)
                for (int kb = 0; kb < NKB; ++kb) cur[kb] = nxt[kb];
        }
    };

    // Masking of one tile's scores: keys past the end or above the causal
    // diagonal become -inf, so that c * s = -inf for them. The test costs a
    // few instructions per 32-key block and is skipped (wave-uniformly)
    // wherever no key of the block is hidden from any row of the wave.
    const float masked = -INFINITY;
    auto mask_tile = [&](f32x16 (&s)[NKB], int j, int r) {
        for (int kb = 0; kb < NKB; ++kb) {
            const int kbase_h = gt(j) * BN + kb * 32 + 4 * h;      // key of element i: kbase_h + koff(i)
            int lim = Skv - 1 - kbase_h;                            // last existing key offset
            if (CAUSAL) lim = min(lim, qrow[r] + coff - kbase_h);   // last visible key offset
            if (__builtin_amdgcn_ballot_w64(lim < 27) != 0) {   // 27 = largest koff(i)
                for (int i = 0; i < 16; ++i)
                    s[kb][i] = (8 * (i >> 2) + (i & 3) > lim) ? masked : s[kb][i];
            }
        }
    };
    // Partial row max of one of NP equal pieces of a tile's scores, so it can
    // ride along the PV MFMA groups (NP = 2 NKB of them) or be formed in
    // four steps after the first tile's scores.
    auto max_piece = [&](const f32x16 (&s)[NKB], int piece, float m, auto np_tag) -> float {
        constexpr int PER = NKB * 16 / decltype(np_tag)::value;   // scores per piece
        const int base = piece * PER;
        for (int e = 0; e < PER; e += 2) {
            const int x = base + e;
            m = fmaxf(fmaxf(m, s[x / 16][x % 16]), s[x / 16][(x + 1) % 16]);
        }
        return m;
    };
    // From this lane's raw max of a tile: the row max in the log2 domain, the
    // lazy rescale of O and l (only when the max grew by more than 8, i.e. a
    // factor 2^8), and the new exponent offset -m.
    auto finish_max = [&](float mraw, int r) -> float {
        // c_log2 > 0, so a fully masked row gives -inf * c = -inf here.
        const float mt = xor32_max(mraw * c_log2);
        const float mnew = fmaxf(m_run[r], mt);
        if (__builtin_amdgcn_ballot_w64(mnew > m_run[r] + 8.0f) != 0) {
            const float alpha = __builtin_amdgcn_exp2f(m_run[r] - mnew);   // 0 on the first tile
            for (int db = 0; db < NDB; ++db)
                for (int i = 0; i < 16; ++i) oacc[r][db][i] *= alpha;
            for (int t = 0; t < NLSUM; ++t) l_part[r][t] *= alpha;
            m_run[r] = mnew;
        }
        return (m_run[r] == -INFINITY) ? 0.f : -m_run[r];
    };

    // Causal bf16 / f16: a wave stops computing after the last tile its own
    // rows can see (see wave_tiles below). Not for E4M3, whose V copies go
    // through registers: keeping them in the last-tile iteration would
    // spill.
    constexpr bool WAVE_SKIP = CAUSAL && Tr::V_DMA;
    // One pipelined iteration over tile j. With HAS_NEXT (tile j+1 exists):
    //   A: scores of tile j+1 (MFMA) interleaved with the weights of tile j
    //      (exp2(c s - m), packed, summed) — the offset -m of tile j is known;
    //   A': masking of tile j+1's scores, only on boundary tiles;
    //   B: PV of tile j (MFMA) interleaved with the row max of tile j+1;
    //   C: cross-half max, lazy rescale of O (after PV of tile j), new -m.
    // Buffers: K(j+1) in kb_next, V(j) in vb_cur; meanwhile K(j+2) goes to
    // kb_cur and V(j+1) to vb_next. Every wave runs exactly one barrier per
    // iteration. Tiles above a wave's own diagonal (in workgroups holding
    // several row blocks of one head) are computed like masked tiles: all
    // their weights are 0.
    // The buffer pointers are __restrict__: once inlined, that marks every LDS
    // access of the iteration with its buffer's scope, which is what lets
    // the compiler see that copies into kb_cur / vb_next never alias reads of
    // kb_next / vb_cur (otherwise it makes the reads wait for the copies).
    auto iteration = [&](auto has_next_tag, int j, f32x16 (&s_cur)[RB][NKB], f32x16 (&s_nxt)[RB][NKB],
                         uint8_t* __restrict__ kb_cur, uint8_t* __restrict__ kb_next,
                         uint8_t* __restrict__ vb_cur, uint8_t* __restrict__ vb_next) {
        constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
        dma_barrier();
        // The copies follow the workgroup's stages, which (with WAVE_SKIP, or
        // for the key half with one tile fewer) may run past this wave's last
        // computed tile. With HAS_NEXT, stage j + 1 exists by construction
        // (j + 1 < wave_tiles <= n_tiles <= nt_max).
        if constexpr (HAS_NEXT || WAVE_SKIP || KS == 2) {
            if (HAS_NEXT || j + 1 < nt_max) {
                if (j + 2 < nt_max) issue_k(j + 2, kb_cur);
                issue_v(j + 1, vb_next);
            }
        }
        uint32_t pw[RB][NKB][8];
        pv_frag vf[2][NDB];     // V operands of two consecutive PV groups
        // Weights of tile j in two stages, so that no dependency chain sits
        // inside one k-step: stage 1 (scale, offset, exp2) of group g runs in
        // k-step g, stage 2 (round to the input type) in k-step g + 1, when
        // the exp2 results have long been ready. The rounded weights are
        // added to the row sum in phase B, beside the PV products that use
        // them, where the vector unit has more room than in phase A
        // (measured: 1.7 % faster at head dim 64, 3.8 % at 32, same at 128).
        float ex[RB][NKB * 8][2];
        auto weight_exp = [&](int r, int pp) {
            const int kb = pp / 8, i = pp % 8;
            const float x0 = fmaf(s_cur[r][kb][2 * i], c_log2, neg_m[r]);
            const float x1 = fmaf(s_cur[r][kb][2 * i + 1], c_log2, neg_m[r]);
            ex[r][pp][0] = __builtin_amdgcn_exp2f(x0);
            ex[r][pp][1] = __builtin_amdgcn_exp2f(x1);
            // Keep the weights where they are computed (between the score
            // MFMAs) instead of letting the compiler sink them to their use.
            asm volatile("" : "+v"(ex[r][pp][0]), "+v"(ex[r][pp][1]));
        };
        auto weight_pack = [&](int r, int pp) {
            const int kb = pp / 8, i = pp % 8;
            pw[r][kb][i] = Tr::pack(ex[r][pp][0], ex[r][pp][1]);
            asm volatile("" : "+v"(pw[r][kb][i]));
        };
        // ---- A ---------------------------------------------------------------
        // Phase A mixes the score MFMAs with the softmax VALU work, phase B
        // is mostly P V MFMAs. One of them runs at raised wave priority, so
        // that it wins the issue arbitration over the SIMD's other wave: at
        // D = 128 (matrix-bound) phase A, which keeps both the matrix core and
        // the VALU fed (+2 % over equal priority); at D = 64 and 32 (vector-
        // bound) phase B, which keeps the matrix products from queuing behind
        // the other wave's softmax (+1.6 % causal, +8 % non-causal against
        // phase A at D = 64; +1.6 % at D = 32).
        constexpr int PRIO_A = D == 128 ? 1 : 0;
        __builtin_amdgcn_s_setprio(PRIO_A);
        // With BAL, the exponentials of the last PV group's four weight pairs
        // move from phase A into the first two PV groups of phase B (the last
        // group is the first to need them), which evens out the vector work
        // per matrix product between the two phases (measured: E4M3 S=4096
        // +2 %, head dim 32 +5 %, MQA S=1024 +1.4 %, GQA S=4096 and head dim
        // 64 within 1 %).
        constexpr int PAIRS = NKB * 8;
        constexpr bool BAL = NKB >= 2 && RB == 1;
        constexpr int PA = BAL ? PAIRS - 4 : PAIRS;   // pairs weighted in phase A
        if constexpr (HAS_NEXT) {
            for (int r = 0; r < RB; ++r)
                for (int kb = 0; kb < NKB; ++kb)
                    for (int i = 0; i < 16; ++i) s_nxt[r][kb][i] = 0.f;
            // K operands are fetched two k-steps ahead; the V operands of the
            // first PV group are fetched during the last k-step.
            qk_frag kf[3][NKB];
            for (int kb = 0; kb < NKB; ++kb) kf[0][kb] = load_k(kb_next, kb, 0);
            if (KSTEPS > 1)
                for (int kb = 0; kb < NKB; ++kb) kf[1][kb] = load_k(kb_next, kb, 1);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                if (ks + 2 < KSTEPS)
                    for (int kb = 0; kb < NKB; ++kb) kf[(ks + 2) % 3][kb] = load_k(kb_next, kb, ks + 2);
                if (ks + 1 == KSTEPS)
                    for (int db = 0; db < NDB; ++db) vf[0][db] = load_v(vb_cur, 0, 0, db);
                for (int kb = 0; kb < NKB; ++kb)
                    for (int r = 0; r < RB; ++r) s_nxt[r][kb] = Tr::qk(kf[ks % 3][kb], qf[r][ks], s_nxt[r][kb]);
#pragma unroll
                for (int r = 0; r < RB; ++r)
                    for (int pp = ks * PA / KSTEPS; pp < (ks + 1) * PA / KSTEPS; ++pp) weight_exp(r, pp);
                if (ks > 0) {
#pragma unroll
                    for (int r = 0; r < RB; ++r)
                        for (int pp = (ks - 1) * PA / KSTEPS; pp < ks * PA / KSTEPS; ++pp) weight_pack(r, pp);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int r = 0; r < RB; ++r)
                for (int pp = (KSTEPS - 1) * PA / KSTEPS; pp < PA; ++pp) weight_pack(r, pp);
            // ---- A' ------------------------------------------------------------
            for (int r = 0; r < RB; ++r) mask_tile(s_nxt[r], j + 1, r);
        } else {
#pragma unroll
            for (int r = 0; r < RB; ++r)
                for (int pp = 0; pp < NKB * 8; ++pp) weight_exp(r, pp);
#pragma unroll
            for (int r = 0; r < RB; ++r)
                for (int pp = 0; pp < NKB * 8; ++pp) weight_pack(r, pp);
            for (int db = 0; db < NDB; ++db) vf[0][db] = load_v(vb_cur, 0, 0, db);
        }
        // ---- B -----------------------------------------------------------------
        __builtin_amdgcn_s_setprio(1 - PRIO_A);
        float mraw[RB];
        for (int r = 0; r < RB; ++r) mraw[r] = masked;
#pragma unroll
        for (int g = 0; g < NKB * 2; ++g) {
            const int kb = g / 2, s2 = g % 2;
            // V operands of the next group are fetched while this group's MFMAs run.
            if (g + 1 < NKB * 2)
                for (int db = 0; db < NDB; ++db) vf[(g + 1) & 1][db] = load_v(vb_cur, (g + 1) / 2, (g + 1) % 2, db);
            for (int r = 0; r < RB; ++r) {
                const pv_frag pf = __builtin_bit_cast(pv_frag, (u32x4){pw[r][kb][4 * s2], pw[r][kb][4 * s2 + 1],
                                                                       pw[r][kb][4 * s2 + 2], pw[r][kb][4 * s2 + 3]});
                for (int db = 0; db < NDB; ++db) oacc[r][db] = Tr::pv(vf[g & 1][db], pf, oacc[r][db]);
            }
            if constexpr (BAL && HAS_NEXT) {
                if (g < 2)
                    for (int r = 0; r < RB; ++r)
                        for (int pp = PA + 2 * g; pp < PA + 2 * g + 2; ++pp) weight_exp(r, pp);
                if (g == 1 || g == 2)
                    for (int r = 0; r < RB; ++r)
                        for (int pp = PA + 2 * (g - 1); pp < PA + 2 * g; ++pp) weight_pack(r, pp);
            }
            // Row sum over this group's rounded weights (left unpinned, so the
            // compiler places the dot products in the gaps between the MFMAs).
            for (int r = 0; r < RB; ++r)
                for (int t = 0; t < 4; ++t)
                    l_part[r][t % NLSUM] = Tr::sum2(pw[r][kb][4 * s2 + t], l_part[r][t % NLSUM]);
            if constexpr (HAS_NEXT) {
                constexpr auto np = std::integral_constant<int, NKB * 2>{};
                for (int r = 0; r < RB; ++r) {
                    if (BAL) {
                        // The row max of tile j + 1 goes to the last two
                        // groups (the first two carry the moved exponentials).
                        if (g >= NKB * 2 - 2) {
                            const int p0 = (g - (NKB * 2 - 2)) * NKB;
                            for (int pc = p0; pc < p0 + NKB; ++pc)
                                mraw[r] = max_piece(s_nxt[r], pc, mraw[r], np);
                        }
                    } else {
                        mraw[r] = max_piece(s_nxt[r], g, mraw[r], np);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- C -----------------------------------------------------------------
        if constexpr (HAS_NEXT)
            for (int r = 0; r < RB; ++r) neg_m[r] = finish_max(mraw[r], r);
        if constexpr (HAS_NEXT || KS == 2)
            if (HAS_NEXT || j + 1 < nt_max) finish_v(vb_next);
    };

    // BN = 32: the sequential form for workgroups with few tiles. One score
    // tile is live per wave (tile j's K and V in the buffers of parity
    // j & 1, the copies of tile j + 1 issued after the barrier; scores, row
    // max, weights and P V of tile j in order), so a wave needs 160
    // registers and a workgroup 32 KiB of LDS: three workgroups per CU, whose
    // start-up and end hide behind each other where a workgroup's life is
    // short. With many tiles the pipelined form below (64-key tiles, the
    // scores of tile j + 1 beside the weights of tile j, two workgroups per
    // CU) is faster.
    constexpr bool SEQ = BN == 32;
    static_assert(!SEQ || (Tr::V_DMA && KS == 1 && RB == 1), "the sequential form is for 16-bit inputs, KS = RB = 1");
    if constexpr (SEQ) {
        int wave_tiles = n_tiles;
        if constexpr (WAVE_SKIP) {
            const int s_last = 32 * RB * (wave + 1) - 1;
            const int last_row = min(item_row(p, wi, s_last), Sq - 1);
            const int last_key = last_row + coff;
            wave_tiles = __builtin_amdgcn_readfirstlane(local_count(last_key < 0 ? 0 : min(nt_glob, last_key / BN + 1)));
        }
        issue_k(0, kbuf0);
        issue_v(0, vbuf0);
        for (int j = 0; j < nt_max; ++j) {
            uint8_t* const kt = (j & 1) ? kbuf1 : kbuf0;
            uint8_t* const vt = (j & 1) ? vbuf1 : vbuf0;
            dma_barrier();
            if (j + 1 < nt_max) {
                issue_k(j + 1, (j & 1) ? kbuf0 : kbuf1);
                issue_v(j + 1, (j & 1) ? vbuf0 : vbuf1);
            }
            if (wave_idle || j >= wave_tiles) continue;
            f32x16 s[RB][NKB];
            qk_tile(kt, s);
            for (int r = 0; r < RB; ++r) {
                mask_tile(s[r], j, r);
                float mraw = masked;
#pragma unroll
                for (int g = 0; g < 4; ++g) mraw = max_piece(s[r], g, mraw, std::integral_constant<int, 4>{});
                neg_m[r] = finish_max(mraw, r);
            }
            uint32_t pw[RB][NKB][8];
#pragma unroll
            for (int r = 0; r < RB; ++r)
                for (int kb = 0; kb < NKB; ++kb)
                    for (int i = 0; i < 8; ++i)
                        pw[r][kb][i] = Tr::pack(__builtin_amdgcn_exp2f(fmaf(s[r][kb][2 * i], c_log2, neg_m[r])),
                                                __builtin_amdgcn_exp2f(fmaf(s[r][kb][2 * i + 1], c_log2, neg_m[r])));
            pv_frag vf[2][NDB];
            for (int db = 0; db < NDB; ++db) vf[0][db] = load_v(vt, 0, 0, db);
#pragma unroll
            for (int g = 0; g < NKB * 2; ++g) {
                const int kb = g / 2, s2 = g % 2;
                if (g + 1 < NKB * 2)
                    for (int db = 0; db < NDB; ++db) vf[(g + 1) & 1][db] = load_v(vt, (g + 1) / 2, (g + 1) % 2, db);
                for (int r = 0; r < RB; ++r) {
                    const pv_frag pf = __builtin_bit_cast(pv_frag, (u32x4){pw[r][kb][4 * s2], pw[r][kb][4 * s2 + 1],
                                                                           pw[r][kb][4 * s2 + 2], pw[r][kb][4 * s2 + 3]});
                    for (int db = 0; db < NDB; ++db) oacc[r][db] = Tr::pv(vf[g & 1][db], pf, oacc[r][db]);
                    for (int t = 0; t < 4; ++t)
                        l_part[r][t % NLSUM] = Tr::sum2(pw[r][kb][4 * s2 + t], l_part[r][t % NLSUM]);
                }
            }
        }
    } else {
        f32x16 s0[RB][NKB], s1[RB][NKB];
        // Every wave copies its share of each stage, also a key half without
        // tiles of its own (KS = 2 with a single tile).
        issue_k(0, kbuf0);
        issue_v(0, vbuf0);
        if (nt_max > 1) issue_k(1, kbuf1);
        finish_v(vbuf0);
        dma_barrier();
        if (!wave_idle && n_tiles > 0) {
            qk_tile(kbuf0, s0);
            for (int r = 0; r < RB; ++r) {
                mask_tile(s0[r], 0, r);
                float mraw = masked;
    #pragma unroll
                for (int g = 0; g < 4; ++g) mraw = max_piece(s0[r], g, mraw, std::integral_constant<int, 4>{});
                neg_m[r] = finish_max(mraw, r);
            }
        }
        if constexpr (!WAVE_SKIP) {
            if (wave_idle || n_tiles == 0) {
                // Same copies and barriers as an iteration, no compute.
                for (int j = 0; j < nt_max; ++j) {
                    dma_barrier();
                    if (j + 1 < nt_max) {
                        if (j + 2 < nt_max) issue_k(j + 2, (j & 1) ? kbuf1 : kbuf0);
                        issue_v(j + 1, (j & 1) ? vbuf0 : vbuf1);
                        finish_v((j & 1) ? vbuf0 : vbuf1);
                    }
                }
            } else {
                int j = 0;
                for (; j + 2 < n_tiles; j += 2) {
                    iteration(std::true_type{}, j, s0, s1, kbuf0, kbuf1, vbuf0, vbuf1);
                    iteration(std::true_type{}, j + 1, s1, s0, kbuf1, kbuf0, vbuf1, vbuf0);
                }
                if (j + 1 < n_tiles) {
                    iteration(std::true_type{}, j, s0, s1, kbuf0, kbuf1, vbuf0, vbuf1);
                    iteration(std::false_type{}, j + 1, s1, s0, kbuf1, kbuf0, vbuf1, vbuf0);
                } else {
                    iteration(std::false_type{}, j, s0, s1, kbuf0, kbuf1, vbuf0, vbuf1);
                }
                // The other key half's last stage, if it has one tile more (no
                // copies left). The branch above already ran nt_max steps.
                for (j = n_tiles; j < nt_max; ++j) dma_barrier();
            }
        } else {
            // The wave's own rows need tiles 0 .. wave_tiles - 1 only. Its
            // highest row is that of its last slot (rows grow with the slot's run
            // index, and the last slot ends a run); rows past Sq count as row
            // Sq - 1 (their results are never stored). From tile wave_tiles on,
            // every score of the wave is masked and every weight 0, so the wave
            // only copies and keeps the barriers, leaving its SIMD to the other
            // workgroup's wave. This happens where the waves of a workgroup hold
            // different rows (several row blocks of one head).
            const int s_last = 32 * RB * (wave + 1) - 1;
            const int last_row = min(item_row(p, wi, s_last), Sq - 1);
            const int last_key = last_row + coff;   // from the start of this workgroup's key range
            const int wave_tiles =
                __builtin_amdgcn_readfirstlane(local_count(last_key < 0 ? 0 : min(nt_glob, last_key / BN + 1)));
            int j = 0;
            if (!wave_idle) {
                for (; j + 2 < wave_tiles; j += 2) {
                    iteration(std::true_type{}, j, s0, s1, kbuf0, kbuf1, vbuf0, vbuf1);
                    iteration(std::true_type{}, j + 1, s1, s0, kbuf1, kbuf0, vbuf1, vbuf0);
                }
                if (j + 1 < wave_tiles) {
                    iteration(std::true_type{}, j, s0, s1, kbuf0, kbuf1, vbuf0, vbuf1);
                    iteration(std::false_type{}, j + 1, s1, s0, kbuf1, kbuf0, vbuf1, vbuf0);
                    j += 2;
                } else if (j < wave_tiles) {
                    iteration(std::false_type{}, j, s0, s1, kbuf0, kbuf1, vbuf0, vbuf1);
                    j += 1;
                }
            }
            // Tiles j .. n_tiles - 1: the same copies and barriers, no compute
            // (and, with KS = 2, the other key half's last step).
            for (; j < nt_max; ++j) {
                dma_barrier();
                if (j + 1 < nt_max) {
                    if (j + 2 < nt_max) issue_k(j + 2, (j & 1) ? kbuf1 : kbuf0);
                    issue_v(j + 1, (j & 1) ? vbuf0 : vbuf1);
                    finish_v((j & 1) ? vbuf0 : vbuf1);
                }
            }
        }
    }

    uint8_t* ost_half = nullptr;   // KS = 2: this wave's region of the merge exchange (consumed below)
    if constexpr (KS == 2) {
        // Merge the key halves: half 1 publishes each lane's running max,
        // weight sum and unnormalised output in LDS (the tile buffers are free
        // once every wave has passed this barrier); half 0 rescales both to
        // the larger maximum and adds. Slot wave w's outputs (64 lanes x D/2
        // floats = 128 D bytes) go to the V buffers (each holds two), the
        // (max, sum) pairs to the first K buffer.
        __syncthreads();
        float lsum = l_part[0][0];
        for (int t = 1; t < NLSUM; ++t) lsum += l_part[0][t];
        float* xo = (float*)((wave < 2 ? lds_v0 : lds_v1) + (wave & 1) * 128 * D);
        float* xml = (float*)lds_k0 + wave * 128;
        if (half == 1) {
            for (int db = 0; db < NDB; ++db)
                for (int q4 = 0; q4 < 4; ++q4)
                    *(f32x4*)(xo + ((db * 4 + q4) * 64 + lane) * 4) =
                        (f32x4){oacc[0][db][4 * q4], oacc[0][db][4 * q4 + 1], oacc[0][db][4 * q4 + 2],
                                oacc[0][db][4 * q4 + 3]};
            *(f32x2*)(xml + lane * 2) = (f32x2){m_run[0], lsum};
        }
        __syncthreads();
        if (half == 1) return;
        const f32x2 ml1 = *(const f32x2*)(xml + lane * 2);
        const float m = fmaxf(m_run[0], ml1[0]);
        const float a0 = m_run[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[0] - m);
        const float a1 = ml1[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml1[0] - m);
        for (int db = 0; db < NDB; ++db)
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 o1 = *(const f32x4*)(xo + ((db * 4 + q4) * 64 + lane) * 4);
                for (int e = 0; e < 4; ++e) oacc[0][db][4 * q4 + e] = a0 * oacc[0][db][4 * q4 + e] + a1 * o1[e];
            }
        l_part[0][0] = a0 * lsum + a1 * ml1[1];
        for (int t = 1; t < NLSUM; ++t) l_part[0][t] = 0.f;
        m_run[0] = m;
        ost_half = (uint8_t*)xo;
    }

    // ---- epilogue: O = O^T / l, round once, store [b][row][hq][d] ----------
    // With D = 128 and a wave holding 32 consecutive rows of one head (HS =
    // 32), the rounded tile goes through LDS first: each lane holds 4 consecutive
    // values of one row per store, so storing from the accumulator layout
    // takes 4 D / 32 instructions that each touch 32 rows at 16 bytes; read
    // back row by row, the same bytes leave in 16-byte pieces of whole rows
    // (D / 32 instructions, each 1 KiB of complete rows), a quarter of the
    // instructions and an eighth of the memory requests. The wave's slice of
    // the V buffers (32 rows of D 16-bit values) is free once every wave has
    // passed the barrier below; chunks are XOR-swizzled by row as in K tiles.
    // With the key halves (KS = 2) only half 0 is left, and each of its waves
    // stages the tile in its own region of the merge exchange, which it has
    // just read.
    if constexpr (RB == 1 && D == 128) {
        if (p.n_split == 1 && HS == 32) {
            float lsum = l_part[0][0];
            for (int t = 1; t < NLSUM; ++t) lsum += l_part[0][t];
            const float l = xor32_sum(lsum);
            const float inv = out_mul / l;
            const int row = qrow[0];
            if (p.lse && row < Sq && h == 0)
                p.lse[((size_t)wi.b * p.Hq + hq[0]) * Sq + row] = (m_run[0] + __builtin_amdgcn_logf(l)) * kLn2;
            if constexpr (KS == 1) __syncthreads();
            // Each wave needs 32 rows of VROWB bytes: two per V buffer when a V
            // buffer holds 64 rows, else one buffer of the four per wave.
            static_assert(KS == 2 || VTILE >= 2 * 32 * VROWB || (VTILE >= 32 * VROWB && KTILE >= 32 * VROWB), "");
            uint8_t* const ost = KS == 2 ? ost_half
                               : VTILE >= 2 * 32 * VROWB ? (wave < 2 ? lds_v0 : lds_v1) + (wave & 1) * 32 * VROWB
                               : (wave == 0 ? lds_k0 : wave == 1 ? lds_k1 : wave == 2 ? lds_v0 : lds_v1);
            const int osw_n = k_swz<NCV>(n);
            for (int db = 0; db < NDB; ++db)
                for (int jj = 0; jj < 4; ++jj) {
                    const uint32_t w0 = Tr::pack(oacc[0][db][4 * jj + 0] * inv, oacc[0][db][4 * jj + 1] * inv);
                    const uint32_t w1 = Tr::pack(oacc[0][db][4 * jj + 2] * inv, oacc[0][db][4 * jj + 3] * inv);
                    *(u32x2*)(ost + n * VROWB + (((db * 4 + jj) ^ osw_n) << 4) + h * 8) = (u32x2){w0, w1};
                }
            constexpr int RPI = 1024 / VROWB;   // rows per 1 KiB read / store
            const int row0 = __builtin_amdgcn_readfirstlane(qrow[0] - n);   // the wave's first row
            const int hw = __builtin_amdgcn_readfirstlane(hq[0]);
            const int cc = lane % NCV;
            out_t* const obase = (out_t*)p.out + wi.b * p.so[0] + hw * p.so[2] + cc * 8;
            for (int it = 0; it < 32 / RPI; ++it) {
                const int r = it * RPI + lane / NCV;
                const u32x4 v = *(const u32x4*)(ost + r * VROWB + ((cc ^ k_swz<NCV>(r)) << 4));
                if (row0 + r < Sq) *(u32x4*)(obase + (size_t)(row0 + r) * p.so[1]) = v;
            }
            return;
        }
    }
    for (int rb = 0; rb < RB; ++rb) {
        float lsum = l_part[rb][0];
        for (int t = 1; t < NLSUM; ++t) lsum += l_part[rb][t];
        const float l = xor32_sum(lsum);
        const int row = qrow[rb];
        if (p.n_split > 1) {
            // Partial result of this key range: O and l relative to 2^m_run.
            if (row < Sq) {
                const size_t r = (qrow_idx + row) * p.Hq + hq[rb];
                for (int db = 0; db < NDB; ++db)
                    for (int jj = 0; jj < 4; ++jj)
                        *(f32x4*)(p.part_o + r * D + db * 32 + 8 * jj + 4 * h) =
                            (f32x4){oacc[rb][db][4 * jj], oacc[rb][db][4 * jj + 1], oacc[rb][db][4 * jj + 2],
                                    oacc[rb][db][4 * jj + 3]};
                if (h == 0) *(f32x2*)(p.part_ml + r * 2) = (f32x2){m_run[rb], l};
            }
            continue;
        }
        const float inv = out_mul / l;
        // Row log-sum-exp: the weights are 2^(c s - m_run) with c = scale log2(e),
        // so sum_j e^(scale s_j) = 2^m_run l and its logarithm is (m_run + log2 l) ln 2.
        if (p.lse && row < Sq && h == 0)
            p.lse[((size_t)wi.b * p.Hq + hq[rb]) * Sq + row] = (m_run[rb] + __builtin_amdgcn_logf(l)) * kLn2;
        if (row < Sq) {
            out_t* orow = (out_t*)p.out + wi.b * p.so[0] + row * p.so[1] + hq[rb] * p.so[2];
            for (int db = 0; db < NDB; ++db) {
                for (int jj = 0; jj < 4; ++jj) {
                    const int d0 = db * 32 + 8 * jj + 4 * h;
                    const uint32_t w0 = Tr::pack(oacc[rb][db][4 * jj + 0] * inv, oacc[rb][db][4 * jj + 1] * inv);
                    const uint32_t w1 = Tr::pack(oacc[rb][db][4 * jj + 2] * inv, oacc[rb][db][4 * jj + 3] * inv);
                    *(u32x2*)(orow + d0) = (u32x2){w0, w1};
                }
            }
        }
    }
}

// MI355X has 256 compute units; the four-wave kernel runs two workgroups
// per CU. A launch with fewer than 1.5 workgroups per CU leaves SIMDs with a
// single wave (nothing hides its stalls) or none; then, if a row block (or,
// with split keys, a key range) has enough key tiles, the key halves (KS = 2:
// eight waves per workgroup, one workgroup per CU, two waves per SIMD) halve
// each wave's chain of tiles.
constexpr int kComputeUnits = 256;

template <typename T, int D, int BN>
static hipError_t launch_typed(const FwdParams& p0, bool causal, hipStream_t stream) {
    FwdParams p = p0;
    int wgs = p.n_units * p.n_row_blocks * p.n_split;
    // Key tiles of one key range (all of them without a split). Split-key
    // launches take the key halves only with long ranges (at least 32
    // tiles): measured on decode shapes (GQA one query against 16K to 64K
    // keys -4 to -37 %), while 16-tile ranges whose four waves all hold
    // rows lose up to 9 % to the merge.
    const int range_tiles = ((p.Skv + BN - 1) / BN + p.n_split - 1) / p.n_split;
    const bool halves = wgs * 2 < kComputeUnits * 3 && range_tiles >= (p.n_split == 1 ? 8 : 32);
    // Causal key halves fold the row blocks (see fold_row_blocks): two mirror
    // blocks per workgroup, the same number of workgroups.
    if (halves && causal && Traits<T>::V_DMA && p.n_split == 1 && fold_row_blocks(p))
        wgs = p.n_units * p.n_row_blocks;
    set_divisors(p);
    // Head dim 128 with few 64-key tiles per workgroup on average (a masked
    // row sees causal_off + its index + 1 keys, on average causal_off + Sq / 2):
    // the sequential form at three workgroups per CU (measured: causal
    // S = 512 and 1024 +7 to +15 %; causal S = 2048 and non-causal S = 1024
    // 3-7 % slower).
    const int64_t vis = causal ? std::min<int64_t>(p.Skv, (int64_t)p.causal_off + (p.Sq + 1) / 2) : p.Skv;
    const int64_t avg_tiles = (vis + 63) / 64;
    const bool seq = D == 128 && Traits<T>::V_DMA && p.n_split == 1 && !halves && avg_tiles <= 9;
    const dim3 grid(wgs), block(64 * (halves ? 8 : 4));
    if (halves) {
        if (causal)
            hipLaunchKernelGGL((fwd_mfma_kernel<T, D, BN, true, 8, 1, 2>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((fwd_mfma_kernel<T, D, BN, false, 8, 1, 2>), grid, block, 0, stream, p);
    } else if (seq) {
        if constexpr (D == 128 && Traits<T>::V_DMA) {
            if (causal)
                hipLaunchKernelGGL((fwd_mfma_kernel<T, D, 32, true, 4, 1>), grid, block, 0, stream, p);
            else
                hipLaunchKernelGGL((fwd_mfma_kernel<T, D, 32, false, 4, 1>), grid, block, 0, stream, p);
        }
    } else if (causal) {
        hipLaunchKernelGGL((fwd_mfma_kernel<T, D, BN, true, 4, 1>), grid, block, 0, stream, p);
    } else {
        hipLaunchKernelGGL((fwd_mfma_kernel<T, D, BN, false, 4, 1>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

// bf16 (is_bf16 = true) or f16 inputs, D = 32, 64 or 128.
hipError_t launch_fwd_mfma(const FwdParams& p, int D, bool is_bf16, bool causal, hipStream_t stream) {
    if (is_bf16) {
        return D == 32 ? launch_typed<__bf16, 32, 64>(p, causal, stream)
             : D == 64 ? launch_typed<__bf16, 64, 64>(p, causal, stream)
                       : launch_typed<__bf16, 128, 64>(p, causal, stream);
    }
    return D == 32 ? launch_typed<_Float16, 32, 64>(p, causal, stream)
         : D == 64 ? launch_typed<_Float16, 64, 64>(p, causal, stream)
                   : launch_typed<_Float16, 128, 64>(p, causal, stream);
}

// E4M3 inputs, bf16 output, D = 64 or 128 (one FP8 score MFMA spans 64 of D).
hipError_t launch_fwd_fp8(const FwdParams& p, int D, bool causal, hipStream_t stream) {
    return D == 64 ? launch_typed<fp8_t, 64, 64>(p, causal, stream)
                   : launch_typed<fp8_t, 128, 64>(p, causal, stream);
}

}  // namespace attn


// attn_bwd.hip — backward pass of the fused attention on gfx950 matrix cores.
//
// Gradients of out = softmax(scale * Q K^T [+ causal mask]) V (codelab
// "Accelerate attention on GPU with cuDNN and TransformerEngine", §1: the
// formula, and the scale that keeps the softmax's gradients from vanishing;
// §7 mask; §9 head grouping). With the weights rebuilt from the forward's
// row log-sum-exp, P = exp(S - lse), and Delta_i = rowsum(dO_i * O_i), which
// equals rowsum(P_i * dP_i):
//
//     dP = dO V^T,  dS = P * (dP - Delta),  dV = P^T dO,
//     dK = scale dS^T Q,  dQ = scale dS K
//
// (dK and dV of a KV head summed over the query heads of its group).
//
// Two kernels, no atomics, deterministic:
//   * bwd_dq_kernel: the forward's workgroup map (32 query rows per wave),
//     looping over 64-key tiles staged in LDS: S^T = K Q^T, dP^T = V dO^T,
//     dS^T, and dQ^T += K^T dS^T, with the dS^T accumulator used directly as
//     the second operand (the K^T operand is gathered in the same key order
//     by the LDS transpose read). It also forms Delta for its rows and
//     stores it for the second kernel.
//   * bwd_dkdv_kernel: one workgroup per 128 keys of one KV head (32 keys
//     per wave, K and V operands held in registers), looping over the query
//     heads of the group and 64-row query steps staged in LDS (three stages,
//     copies two steps ahead): S = Q K^T,
//     dP = dO V^T, dS, then dV += P^T dO and dK += dS^T Q with P^T and dS^T
//     taken straight from the accumulators.
// S and dP are thus computed twice, 7 matrix products instead of 5. The
// alternative, one kernel adding dQ into an fp32 buffer with atomics, moves
// Sq * D * 4 bytes per 128 keys through the atomic units; measured on
// MI355X they sustain about 1.4 TB/s in that pattern, which at S = 4096
// would take about three times as long as all the products.

#include "mfma_common.h"

namespace attn {

namespace {

template <typename T>
__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (std::is_same_v<T, __bf16>)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

template <typename T>
__device__ inline T round_to(float x) { return (T)x; }

// Transpose read of 16 keys (rows base + 4h + {0..3} and base + 8 + 4h +
// {0..3}) of one 32-column block: the operand layout that pairs with an
// accumulator used as the other operand (see the forward kernel).
template <typename frag>
__device__ inline frag tr_read(const uint8_t* base, uint32_t off_lo, uint32_t off_hi) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + off_lo));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + off_hi));
    return __builtin_bit_cast(frag, (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// acc += a b on the matrix cores with acc pinned to the accumulation
// registers (AGPRs): for accumulators that only matrix instructions touch
// until the end, so that everything the vector ALU reads can stay in
// ordinary VGPRs. The leading s_nop covers the wait states between a vector
// write of a or b (or of acc, at its initialisation) and the MFMA reading
// it; consecutive uses of one accumulator are always several MFMAs apart.
template <typename T, typename frag>
__device__ inline void mfma_agpr(f32x16& acc, frag a, frag b) {
    if constexpr (std::is_same_v<T, __bf16>)
        asm("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm("s_nop 4\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

struct BwdScalars {
    float c2, dp_mul, delta_mul, dq_mul, dk_mul, dv_mul;
};

// The backward's scalar factors: from the parameters, or (FP8 with
// device-side factors) formed from the bare scale and the q, k, v, dout
// factors in device memory by the expressions the host uses.
__device__ inline BwdScalars bwd_scalars(const BwdParams& bp) {
    BwdScalars s = {bp.f.scale_log2, bp.dp_mul, bp.delta_mul, bp.dq_mul, bp.dk_mul, bp.dv_mul};
    if (bp.dsc[0]) {
        const float qd = *bp.dsc[0], kd = *bp.dsc[1], vd = *bp.dsc[2], dd = *bp.dsc[3];
        s.c2 = ((bp.scale * qd) * kd) * kLog2eF32;
        s.dp_mul = dd * vd;
        s.delta_mul = dd;
        s.dq_mul = bp.scale * kd;
        s.dk_mul = bp.scale * qd;
        s.dv_mul = dd;
    }
    return s;
}

}  // namespace

// ---------------------------------------------------------------------------
// dQ (and Delta): one workgroup = 4 waves x 32 query slots, the forward's map.
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdParams bp) {
    using Tr = Traits<T>;
    using frag = typename Tr::qk_frag;
    const FwdParams& p = bp.f;
    constexpr int ROWB = D * 2;             // bytes of one row of K, V, Q, dO
    constexpr int NC = ROWB / 16;           // 16-byte chunks per row
    constexpr int KSTEPS = D / 16;          // k-steps of S^T and dP^T
    constexpr int BN = 64;                  // keys per tile
    constexpr int NKB = BN / 32, NDB = D / 32;
    constexpr int TILE = BN * ROWB;
    __shared__ __attribute__((aligned(1024))) uint8_t lds_k0[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_k1[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_v0[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_v1[TILE];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, n = lane & 31;

    const WorkItem wi = map_workgroup(p, CAUSAL);
    const BwdScalars sc = bwd_scalars(bp);
    const int slot = wave * 32 + n;
    const int hq = wi.hq0 + slot_head(p, slot);
    const int qrow = wi.row_base + slot_row(p, slot);
    const bool wave_idle = __builtin_amdgcn_readfirstlane(wi.row_base + slot_row(p, wave * 32)) >= p.Sq;
    const int Sq = p.Sq, Skv = p.Skv;
    const bool row_ok = qrow < Sq;

    // This lane's query row: Q^T and dO^T operands (16 bytes per k-step,
    // chunk 2 ks + h) and its part of Delta = dO . O.
    const size_t roff = (size_t)wi.b * p.sq[0] + (size_t)qrow * p.sq[1] + (size_t)hq * p.sq[2];
    frag qf[KSTEPS], gf[KSTEPS];
    float dsum = 0.f;
    {
        const uint8_t* qsrc = (const uint8_t*)((const T*)p.q + roff);
        const uint8_t* gsrc = (const uint8_t*)((const T*)bp.dout + roff);
        const uint8_t* osrc = (const uint8_t*)((const T*)p.out + roff);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 xq = {0, 0, 0, 0}, xg = {0, 0, 0, 0}, xo = {0, 0, 0, 0};
            if (row_ok) {
                const int off = (2 * ks + h) * 16;
                xq = *(const u32x4*)(qsrc + off);
                xg = *(const u32x4*)(gsrc + off);
                xo = *(const u32x4*)(osrc + off);
            }
            qf[ks] = __builtin_bit_cast(frag, xq);
            gf[ks] = __builtin_bit_cast(frag, xg);
#pragma unroll
            for (int e = 0; e < 4; ++e) dsum = dot2<T>(xg[e], xo[e], dsum);
        }
    }
    const float delta = sc.delta_mul * xor32_sum(dsum);
    const float dp_mul = sc.dp_mul;
    const size_t srow = ((size_t)wi.b * p.Hq + hq) * Sq + qrow;
    const float lse2 = row_ok ? bp.lse[srow] * kLog2eF32 : 0.f;
    if (row_ok && h == 0) {   // for the dK / dV kernel
        bp.delta[srow] = delta;
        bp.lse2[srow] = lse2;
    }
    const float c2 = sc.c2;                   // scale * log2(e), any sign
    const int coff = p.causal_off;

    int n_tiles = (Skv + BN - 1) / BN;
    if (CAUSAL) {
        const int last_row = min(wi.row_base + p.rows_per_wg, Sq) - 1 + coff;
        n_tiles = min(n_tiles, last_row / BN + 1);
    }
    n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);

    const uint8_t* kbase = (const uint8_t*)((const T*)p.k + wi.b * p.sk[0] + wi.hkv * p.sk[2]);
    const uint8_t* vbase = (const uint8_t*)((const T*)p.v + wi.b * p.sv[0] + wi.hkv * p.sv[2]);
    TileDma<ROWB, BN, 4> kdma, vdma;
    kdma.init(kbase, (uint32_t)(p.sk[1] * 2), wave, lane, kSwzKV);   // read as rows and transposed
    vdma.init(vbase, (uint32_t)(p.sv[1] * 2), wave, lane, kSwzK);    // read as rows

    // Row reads (first operand of S^T = K Q^T and dP^T = V dO^T): lane (h, n)
    // reads row 32 kb + n, chunk 2 ks + h; the k-step only flips chunk bits
    // above h, so the offset is a lane base XOR (ks << 5).
    const uint32_t krd = n * ROWB + ((h ^ kv_swz<NC>(n)) << 4);
    const uint32_t vrd = n * ROWB + ((h ^ k_swz<NC>(n)) << 4);
    // Transpose reads of K (first operand of dQ^T = K^T dS^T): lane L of a
    // 16-lane group addresses row 4h + L / 4 (and that + 8) at byte
    // 64 db + 32 G16 + 8 (L % 4) of the row.
    const int L16 = lane & 15, G16 = (lane >> 4) & 1;
    const int rlo = 4 * h + (L16 >> 2), rhi = rlo + 8;
    uint32_t tlo[NDB], thi[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int cb = db * 64 + 32 * G16 + 8 * (L16 & 3);
        tlo[db] = rlo * ROWB + ((((cb >> 4) ^ kv_swz<NC>(rlo)) << 4) | (cb & 15));
        thi[db] = rhi * ROWB + ((((cb >> 4) ^ kv_swz<NC>(rhi)) << 4) | (cb & 15));
    }

    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;

    // One tile: kt / vt hold tile j, kn / vn receive tile j + 1. The buffers
    // are distinct LDS objects passed as __restrict__ pointers into an
    // inlined body, which lets the compiler see that the copies into kn / vn
    // never alias the reads of kt / vt; otherwise it makes those reads wait
    // for the copies, and no copy overlaps the tile's products.
    auto tile = [&](int j, const uint8_t* __restrict__ kt, const uint8_t* __restrict__ vt,
                    uint8_t* __restrict__ kn, uint8_t* __restrict__ vn) __attribute__((always_inline)) {
        dma_barrier();   // tile j has landed; every wave is done with tile j - 1
        if (j + 1 < n_tiles) {
            kdma.issue((j + 1) * BN, Skv, kn, wave);
            vdma.issue((j + 1) * BN, Skv, vn, wave);
        }
        if (wave_idle) return;
        // Four phases with operands fetched from LDS two MFMA pairs ahead,
        // and the weights of one 32-key block computed alongside the other
        // block's MFMAs:
        //   1: S^T, dP^T of block 0     2: S^T, dP^T of block 1 + weights of block 0
        //   3: dQ^T from block 0 + weights of block 1     4: dQ^T from block 1
        f32x16 s[NKB], dp[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) { s[kb][i] = 0.f; dp[kb][i] = 0.f; }
        // dS^T = P^T (dp_mul dP^T - Delta), P^T = 2^(c2 s - lse2) on visible
        // keys, rounded to the input type in pairs of consecutive keys;
        // elements i0 .. i0 + cnt - 1 of block kb.
        uint32_t pw[NKB][8];
        // Key of element i of block kb: key0 + 8 (i / 4) + i % 4, visible iff
        // its offset 8 (i / 4) + i % 4 <= lim. Blocks where every element of
        // every lane is visible (offsets reach 27) skip the test.
        int lim[NKB];
        bool masked[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const int key0 = j * BN + kb * 32 + 4 * h;
            lim[kb] = Skv - 1 - key0;
            if (CAUSAL) lim[kb] = min(lim[kb], qrow + coff - key0);
            masked[kb] = __builtin_amdgcn_ballot_w64(lim[kb] < 27) != 0;
        }
        auto weights = [&](int kb, int i0, int cnt) __attribute__((always_inline)) {
            if (masked[kb]) {
#pragma unroll
                for (int i = i0; i < i0 + cnt; i += 2) {
                    const int ko = 8 * (i >> 2) + (i & 3);
                    const float p0 = ko <= lim[kb] ? __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, -lse2)) : 0.f;
                    const float p1 = ko + 1 <= lim[kb] ? __builtin_amdgcn_exp2f(fmaf(s[kb][i + 1], c2, -lse2)) : 0.f;
                    pw[kb][i / 2] = Tr::pack(p0 * fmaf(dp[kb][i], dp_mul, -delta),
                                             p1 * fmaf(dp[kb][i + 1], dp_mul, -delta));
                }
            } else {
#pragma unroll
                for (int i = i0; i < i0 + cnt; i += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, -lse2));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][i + 1], c2, -lse2));
                    pw[kb][i / 2] = Tr::pack(p0 * fmaf(dp[kb][i], dp_mul, -delta),
                                             p1 * fmaf(dp[kb][i + 1], dp_mul, -delta));
                }
            }
        };
        // A wave in phases 3-4 (the dQ products, with the second block's
        // weights between them) runs at raised priority, so its products
        // issue ahead of the score products and weights of the other wave on
        // the SIMD (1 to 4 % faster than equal priority at D = 32, 64 and
        // 128, causal or not).
        __builtin_amdgcn_s_setprio(0);
        // Phases 1-2: u = kb KSTEPS + ks.
        constexpr int U = NKB * KSTEPS;
        constexpr int PER_U = 16 / KSTEPS;
        auto ldk = [&](int u) __attribute__((always_inline)) {
            return __builtin_bit_cast(frag, *(const u32x4*)(kt + (u / KSTEPS) * 32 * ROWB + (krd ^ ((u % KSTEPS) << 5))));
        };
        auto ldv = [&](int u) __attribute__((always_inline)) {
            return __builtin_bit_cast(frag, *(const u32x4*)(vt + (u / KSTEPS) * 32 * ROWB + (vrd ^ ((u % KSTEPS) << 5))));
        };
        frag ka[3], va[3];
        ka[0] = ldk(0); va[0] = ldv(0);
        ka[1] = ldk(1); va[1] = ldv(1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u + 2 < U) { ka[(u + 2) % 3] = ldk(u + 2); va[(u + 2) % 3] = ldv(u + 2); }
            const int kb = u / KSTEPS, ks = u % KSTEPS;
            s[kb] = Tr::qk(ka[u % 3], qf[ks], s[kb]);
            dp[kb] = Tr::qk(va[u % 3], gf[ks], dp[kb]);
            if (kb == 1) weights(0, ks * PER_U, PER_U);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(1);
        // Phases 3-4: v = (kb 2 + s2) NDB + db.
        constexpr int V = NKB * 2 * NDB;
        constexpr int PER_V = 16 / (2 * NDB);
        auto ldt = [&](int v) __attribute__((always_inline)) {
            const int kb = v / (2 * NDB), s2 = (v / NDB) % 2, db = v % NDB;
            return tr_read<frag>(kt + (kb * 32 + 16 * s2) * ROWB, tlo[db], thi[db]);
        };
        frag ta[3];
        ta[0] = ldt(0);
        ta[1] = ldt(1);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            if (v + 2 < V) ta[(v + 2) % 3] = ldt(v + 2);
            const int kb = v / (2 * NDB), s2 = (v / NDB) % 2, db = v % NDB;
            const frag sf = __builtin_bit_cast(frag, (u32x4){pw[kb][4 * s2], pw[kb][4 * s2 + 1],
                                                             pw[kb][4 * s2 + 2], pw[kb][4 * s2 + 3]});
            dq[db] = Tr::qk(ta[v % 3], sf, dq[db]);
            if (kb == 0) weights(1, v * PER_V, PER_V);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    kdma.issue(0, Skv, lds_k0, wave);
    vdma.issue(0, Skv, lds_v0, wave);
    int j = 0;
    for (; j + 2 <= n_tiles; j += 2) {
        tile(j, lds_k0, lds_v0, lds_k1, lds_v1);
        tile(j + 1, lds_k1, lds_v1, lds_k0, lds_v0);
    }
    if (j < n_tiles) tile(j, lds_k0, lds_v0, lds_k1, lds_v1);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // no copy may still be in flight when the workgroup ends

    if (row_ok) {
        const float dqm = sc.dq_mul;
        T* dst = (T*)bp.dq + roff;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = db * 32 + 8 * jj + 4 * h;
                const uint32_t w0 = Tr::pack(dq[db][4 * jj] * dqm, dq[db][4 * jj + 1] * dqm);
                const uint32_t w1 = Tr::pack(dq[db][4 * jj + 2] * dqm, dq[db][4 * jj + 3] * dqm);
                *(u32x2*)(dst + d0) = (u32x2){w0, w1};
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup = 128 keys of one KV head, 32 per wave.
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams bp) {
    using Tr = Traits<T>;
    using frag = typename Tr::qk_frag;
    const FwdParams& p = bp.f;
    constexpr int ROWB = D * 2, NC = ROWB / 16, KSTEPS = D / 16, NDB = D / 32;
    constexpr int BM = 64;                             // query rows per step (two 32-row blocks)
    // With D = 128 the kernel needs more than the 256 VGPRs: dK and dV, which
    // only MFMAs touch in the loop, live in AGPRs.
    constexpr bool ACC_AGPR = D == 128;
    // LDS operands are fetched PF MFMA pairs ahead of their use.
    constexpr int PF = 3, RING = PF + 1;
    constexpr int NMB = BM / 32;
    constexpr int TILE = BM * ROWB;
    // One LDS object per stage and tensor (see the step body below).
    __shared__ __attribute__((aligned(1024))) uint8_t lds_q0[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_q1[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_q2[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_g0[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_g1[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_g2[TILE];
    __shared__ __attribute__((aligned(16))) float lds_s0[2 * BM];   // [lse, Delta][row]
    __shared__ __attribute__((aligned(16))) float lds_s1[2 * BM];
    __shared__ __attribute__((aligned(16))) float lds_s2[2 * BM];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, n = lane & 31;

    // Key blocks are the slowest index, so with a causal mask the blocks
    // that see the most query rows (the first ones) go out first, for every
    // (batch, KV head) alike; the workgroups of one (batch, KV head) then
    // sit on the same XCD (workgroup i runs on XCD i % 8).
    const int id = (int)__builtin_amdgcn_workgroup_id_x();
    const int nbh = p.B * p.Hkv;
    const int kblk = id / nbh;
    const int hkv = (id % nbh) % p.Hkv, b = (id % nbh) / p.Hkv;
    const int Sq = p.Sq, Skv = p.Skv, G = p.G;
    const int kw0 = kblk * 128 + 32 * wave;            // this wave's first key
    const int key = kw0 + n;                           // the key of lane column n

    // K and V as second operands of S = Q K^T and dP = dO V^T: lane (h, n)
    // holds 16 bytes (chunk 2 ks + h) of key n, for the whole kernel.
    frag kf[KSTEPS], vf[KSTEPS];
    {
        const int kr = min(key, Skv - 1);
        const uint8_t* ksrc = (const uint8_t*)((const T*)p.k + b * p.sk[0] + (size_t)kr * p.sk[1] + hkv * p.sk[2]);
        const uint8_t* vsrc = (const uint8_t*)((const T*)p.v + b * p.sv[0] + (size_t)kr * p.sv[1] + hkv * p.sv[2]);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            kf[ks] = __builtin_bit_cast(frag, *(const u32x4*)(ksrc + (2 * ks + h) * 16));
            vf[ks] = __builtin_bit_cast(frag, *(const u32x4*)(vsrc + (2 * ks + h) * 16));
        }
    }

    const int coff = p.causal_off;
    const BwdScalars sc = bwd_scalars(bp);
    const float c2 = sc.c2;
    const float dp_mul = sc.dp_mul;
    const int n_qs = (Sq + BM - 1) / BM;
    // First query step holding a row that sees a key of this block.
    const int qs0 = CAUSAL ? min(n_qs, max(0, kblk * 128 - coff) / BM) : 0;
    const int per_head = n_qs - qs0;
    const int n_steps = G * per_head;

    // Copies of one step: the Q and dO tiles (all four waves), the rows'
    // lse log2(e) (wave 0) and Delta (wave 1), each lane of those one row
    // (rows past the end repeat the last row; they are masked).
    // Step t covers rows [step_row(t), + BM) of query head t % G: the query
    // steps run from the last one down to the block's first, and the G heads
    // of the group take turns within each, so that all key blocks of a KV
    // head, which run side by side on one XCD, read the same (head, rows)
    // tile of Q and dO at about the same time and share it through its L2,
    // whatever the number of steps each block sees (the causal diagonal step
    // comes last).
    auto step_row = [&](int t) { return (n_qs - 1 - t / G) * BM; };
    TileDma<ROWB, BM, 4> qdma, gdma;
    constexpr int NV = 2 * TileDma<ROWB, BM, 4>::PER_WAVE;   // tile copy instructions per wave and step
    static_assert(NV + 1 < 16, "the wait below encodes the count in four bits");
    const uint32_t qrow_b = (uint32_t)(p.sq[1] * 2);
    auto issue_step = [&](int t, uint8_t* qd, uint8_t* gd, float* sd) __attribute__((always_inline)) {
        const int g = t % G, r0 = step_row(t);
        const int hq = hkv * G + g;
        const size_t hoff = (size_t)b * p.sq[0] + (size_t)hq * p.sq[2];
        qdma.init((const uint8_t*)((const T*)p.q + hoff), qrow_b, wave, lane, kSwzKV);
        gdma.init((const uint8_t*)((const T*)bp.dout + hoff), qrow_b, wave, lane, kSwzKV);
        qdma.issue(r0, Sq, qd, wave);
        gdma.issue(r0, Sq, gd, wave);
        if (wave < 2) {
            const float* src = (wave == 0 ? bp.lse2 : bp.delta) + ((size_t)b * p.Hq + hq) * Sq;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, -1, kBufferWord3);
            const uint32_t off = (uint32_t)min(r0 + lane, Sq - 1) * 4;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(sd + wave * BM), 4, off, 0, 0, 0);
        }
    };

    // Row reads of the Q and dO tiles (first operand of S and dP): row
    // 32 mb + n, chunk 2 ks + h. Transpose reads (second operand of dV and
    // dK): rows 4h + L / 4 and + 8 at byte 64 db + 32 G16 + 8 (L % 4).
    const uint32_t qrd = n * ROWB + ((h ^ kv_swz<NC>(n)) << 4);
    const int L16 = lane & 15, G16 = (lane >> 4) & 1;
    const int rlo = 4 * h + (L16 >> 2), rhi = rlo + 8;
    uint32_t tlo[NDB], thi[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int cb = db * 64 + 32 * G16 + 8 * (L16 & 3);
        tlo[db] = rlo * ROWB + ((((cb >> 4) ^ kv_swz<NC>(rlo)) << 4) | (cb & 15));
        thi[db] = rhi * ROWB + ((((cb >> 4) ^ kv_swz<NC>(rhi)) << 4) | (cb & 15));
    }

    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) { dk[db][i] = 0.f; dv[db][i] = 0.f; }

    // Step t reads stage t % 3 (qt, gt, stt) and, after the barrier, starts
    // the copies of step t + 2 into stage (t + 2) % 3 (qn, gn, sn), the one
    // step t - 1 used. Distinct LDS objects passed as __restrict__ pointers
    // into an inlined body let the compiler see that those copies never
    // alias this step's reads (otherwise the reads would wait for them).
    auto step = [&](int t, const uint8_t* __restrict__ qt, const uint8_t* __restrict__ gt,
                    const float* __restrict__ stt, uint8_t* __restrict__ qn, uint8_t* __restrict__ gn,
                    float* __restrict__ sn) __attribute__((always_inline)) {
        // Step t's copies have landed (each wave waits for its own, the
        // barrier for everyone's), and every wave is done with step t - 1,
        // whose stage the copies of step t + 2 reuse.
        // Copies complete in issue order, so waiting until no more than step
        // t + 1's own copies are outstanding (NV per wave, plus one for the
        // statistics in waves 0 and 1) means step t's have landed.
        if (t + 1 < n_steps) {
            if (wave < 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (NV + 1));
            else __builtin_amdgcn_s_waitcnt(0x0F70 | NV);
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        __syncthreads();
        if (t + 2 < n_steps) issue_step(t + 2, qn, gn, sn);
        const int r0 = step_row(t);

        // Four phases, each a run of MFMAs with operands fetched from LDS PF
        // MFMA pairs ahead (one wave per SIMD: nothing else hides the LDS
        // latency), and the vector work of one 32-row block riding along the
        // MFMAs of the other:
        //   1: S, dP of block 0        2: S, dP of block 1 + weights of block 0
        //   3: dV, dK of block 0 + weights of block 1        4: dV, dK of block 1
        f32x16 s[NMB], dp[NMB];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) { s[mb][i] = 0.f; dp[mb][i] = 0.f; }

        // Element i of block mb, lane (h, n): query r0 + 32 mb + 8 (i / 4) + 4h + i % 4, key kw0 + n.
        // It is visible iff the key exists, the row exists and (causal) key <= row + coff.
        const bool key_ok = key < Skv;
        uint32_t pw[NMB][8], sw[NMB][8];
        // Weights P = 2^(c2 s - lse log2 e) and dS = P (dP - Delta) of
        // elements i0 .. i0 + cnt - 1 of block mb, rounded in pairs.
        // Row offsets (8 (i / 4) + i % 4, up to 27) at or above qlim see the
        // key; at or above qend the row does not exist. Blocks where no lane
        // has a hidden element skip the test.
        int qlim[NMB], qend[NMB];
        bool masked[NMB];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            const int qb = r0 + 32 * mb + 4 * h;
            qlim[mb] = CAUSAL ? key - coff - qb : -(1 << 30);
            qend[mb] = key_ok ? Sq - qb : -(1 << 30);
            masked[mb] = __builtin_amdgcn_ballot_w64(qlim[mb] > 0 || qend[mb] <= 27) != 0;
        }
        // The rows' lse log2(e) and Delta: four 16-byte LDS reads per block,
        // issued ahead of the weights that use them.
        f32x4 lst[NMB][4], dst[NMB][4];
        auto load_stats = [&](int mb) __attribute__((always_inline)) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                lst[mb][jj] = *(const f32x4*)&stt[32 * mb + 8 * jj + 4 * h];
                dst[mb][jj] = *(const f32x4*)&stt[BM + 32 * mb + 8 * jj + 4 * h];
            }
        };
        // Weights P = 2^(c2 s - lse log2 e) and dS = P (dP - Delta) of
        // elements i0 .. i0 + cnt - 1 of block mb, rounded in pairs.
        auto weights = [&](int mb, int i0, int cnt) __attribute__((always_inline)) {
#pragma unroll
            for (int i = i0; i < i0 + cnt; i += 2) {
                const int jj = i >> 2, e = i & 3;
                float p0 = __builtin_amdgcn_exp2f(fmaf(s[mb][i], c2, -lst[mb][jj][e]));
                float p1 = __builtin_amdgcn_exp2f(fmaf(s[mb][i + 1], c2, -lst[mb][jj][e + 1]));
                if (masked[mb]) {
                    const int qo = 8 * jj + e;
                    p0 = (qo >= qlim[mb] && qo < qend[mb]) ? p0 : 0.f;
                    p1 = (qo + 1 >= qlim[mb] && qo + 1 < qend[mb]) ? p1 : 0.f;
                }
                pw[mb][i / 2] = Tr::pack(p0, p1);
                sw[mb][i / 2] = Tr::pack(p0 * fmaf(dp[mb][i], dp_mul, -dst[mb][jj][e]),
                                         p1 * fmaf(dp[mb][i + 1], dp_mul, -dst[mb][jj][e + 1]));
            }
        };

        // Phases 1-2: u = mb KSTEPS + ks.
        constexpr int U = NMB * KSTEPS;
        constexpr int PER_U = 16 / KSTEPS;                 // elements of block 0 weighted per k-step of block 1
        auto ldq = [&](int u) __attribute__((always_inline)) {
            return __builtin_bit_cast(frag, *(const u32x4*)(qt + (u / KSTEPS) * 32 * ROWB + (qrd ^ ((u % KSTEPS) << 5))));
        };
        auto ldg = [&](int u) __attribute__((always_inline)) {
            return __builtin_bit_cast(frag, *(const u32x4*)(gt + (u / KSTEPS) * 32 * ROWB + (qrd ^ ((u % KSTEPS) << 5))));
        };
        frag qa[RING], ga[RING];
#pragma unroll
        for (int u = 0; u < PF; ++u) { qa[u] = ldq(u); ga[u] = ldg(u); }
        load_stats(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u + PF < U) { qa[(u + PF) % RING] = ldq(u + PF); ga[(u + PF) % RING] = ldg(u + PF); }
            const int mb = u / KSTEPS, ks = u % KSTEPS;
            s[mb] = Tr::qk(qa[u % RING], kf[ks], s[mb]);
            dp[mb] = Tr::qk(ga[u % RING], vf[ks], dp[mb]);
            if (mb == 1) {
                weights(0, ks * PER_U, PER_U);
                if (ks == KSTEPS - 1) load_stats(1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // Phases 3-4: v = (mb 2 + s2) NDB + db.
        constexpr int V = NMB * 2 * NDB;
        constexpr int PER_V = 16 / (2 * NDB);              // elements of block 1 weighted per MFMA pair of block 0
        auto ldt = [&](const uint8_t* tile, int v) __attribute__((always_inline)) {
            const int mb = v / (2 * NDB), s2 = (v / NDB) % 2, db = v % NDB;
            return tr_read<frag>(tile + (32 * mb + 16 * s2) * ROWB, tlo[db], thi[db]);
        };
        frag tg[RING], tq[RING];
#pragma unroll
        for (int v = 0; v < PF; ++v) { tg[v] = ldt(gt, v); tq[v] = ldt(qt, v); }
#pragma unroll
        for (int v = 0; v < V; ++v) {
            if (v + PF < V) { tg[(v + PF) % RING] = ldt(gt, v + PF); tq[(v + PF) % RING] = ldt(qt, v + PF); }
            const int mb = v / (2 * NDB), s2 = (v / NDB) % 2, db = v % NDB;
            const frag pa = __builtin_bit_cast(frag, (u32x4){pw[mb][4 * s2], pw[mb][4 * s2 + 1],
                                                             pw[mb][4 * s2 + 2], pw[mb][4 * s2 + 3]});
            const frag sa = __builtin_bit_cast(frag, (u32x4){sw[mb][4 * s2], sw[mb][4 * s2 + 1],
                                                             sw[mb][4 * s2 + 2], sw[mb][4 * s2 + 3]});
            if constexpr (ACC_AGPR) {
                mfma_agpr<T>(dv[db], pa, tg[v % RING]);
                mfma_agpr<T>(dk[db], sa, tq[v % RING]);
            } else {
                dv[db] = Tr::qk(pa, tg[v % RING], dv[db]);
                dk[db] = Tr::qk(sa, tq[v % RING], dk[db]);
            }
            if (mb == 0) weights(1, v * PER_V, PER_V);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (n_steps > 0) issue_step(0, lds_q0, lds_g0, lds_s0);
    if (n_steps > 1) issue_step(1, lds_q1, lds_g1, lds_s1);
    int t = 0;
    for (; t + 3 <= n_steps; t += 3) {
        step(t, lds_q0, lds_g0, lds_s0, lds_q2, lds_g2, lds_s2);
        step(t + 1, lds_q1, lds_g1, lds_s1, lds_q0, lds_g0, lds_s0);
        step(t + 2, lds_q2, lds_g2, lds_s2, lds_q1, lds_g1, lds_s1);
    }
    if (t < n_steps) step(t, lds_q0, lds_g0, lds_s0, lds_q2, lds_g2, lds_s2);
    if (t + 1 < n_steps) step(t + 1, lds_q1, lds_g1, lds_s1, lds_q0, lds_g0, lds_s0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if constexpr (ACC_AGPR) {
        // Wait states between the last MFMA writing the accumulators and the
        // vector reads below (more than the 32x32 MFMA's write latency).
        static_assert(NDB == 4, "");
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(dk[0]), "+a"(dk[1]), "+a"(dk[2]), "+a"(dk[3]),
                       "+a"(dv[0]), "+a"(dv[1]), "+a"(dv[2]), "+a"(dv[3]));
    }

    // Element i of the accumulators: key kw0 + 8 (i / 4) + 4h + i % 4, column 32 db + n.
    const float sk_mul = sc.dk_mul, sv_mul = sc.dv_mul;
    T* dkb = (T*)bp.dk + b * p.sk[0] + hkv * p.sk[2];
    T* dvb = (T*)bp.dv + b * p.sv[0] + hkv * p.sv[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int kr = kw0 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (kr < Skv) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                dkb[(size_t)kr * p.sk[1] + 32 * db + n] = round_to<T>(dk[db][i] * sk_mul);
                dvb[(size_t)kr * p.sv[1] + 32 * db + n] = round_to<T>(dv[db][i] * sv_mul);
            }
        }
    }
}

// FP8 codes (E4M3, or E5M2 with E5M2 = true) widened to bfloat16, exactly:
// both formats' values are bfloat16 values (fewer exponent and mantissa
// bits). 16 codes per thread; n is a multiple of 16.
template <bool E5M2>
__global__ __launch_bounds__(256) void widen_fp8_kernel(const uint8_t* __restrict__ in, __bf16* __restrict__ out,
                                                        int64_t n16) {
    const int64_t t = (int64_t)__builtin_amdgcn_workgroup_id_x() * 256 + __builtin_amdgcn_workitem_id_x();
    if (t >= n16) return;
    const u32x4 c = *(const u32x4*)(in + t * 16);
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f32x2 lo, hi;
        if constexpr (E5M2) {
            lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)c[e], false);
            hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)c[e], true);
        } else {
            lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[e], false);
            hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[e], true);
        }
        w[2 * e] = pack2_bf16(lo[0], lo[1]);
        w[2 * e + 1] = pack2_bf16(hi[0], hi[1]);
    }
    *(u32x4*)(out + t * 16) = (u32x4){w[0], w[1], w[2], w[3]};
    *(u32x4*)(out + t * 16 + 8) = (u32x4){w[4], w[5], w[6], w[7]};
}

hipError_t launch_widen_fp8(const void* in, void* out, int64_t n, bool e5m2, hipStream_t stream) {
    const int64_t n16 = n / 16;
    if (n16 == 0) return hipSuccess;
    const dim3 grid((unsigned)((n16 + 255) / 256)), block(256);
    if (e5m2) hipLaunchKernelGGL((widen_fp8_kernel<true>), grid, block, 0, stream, (const uint8_t*)in, (__bf16*)out, n16);
    else hipLaunchKernelGGL((widen_fp8_kernel<false>), grid, block, 0, stream, (const uint8_t*)in, (__bf16*)out, n16);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_bwd_typed(const BwdParams& bp0, bool causal, hipStream_t stream) {
    BwdParams bp = bp0;
    set_divisors(bp.f);
    const FwdParams& p = bp.f;
    const unsigned gq = (unsigned)(p.n_units * p.n_row_blocks);
    const unsigned gk = (unsigned)(p.B * p.Hkv * bp.n_kblocks);
    if (gq > 0) {
        if (causal) hipLaunchKernelGGL((bwd_dq_kernel<T, D, true>), dim3(gq), dim3(256), 0, stream, bp);
        else hipLaunchKernelGGL((bwd_dq_kernel<T, D, false>), dim3(gq), dim3(256), 0, stream, bp);
    }
    if (gk > 0) {
        if (causal) hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true>), dim3(gk), dim3(256), 0, stream, bp);
        else hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false>), dim3(gk), dim3(256), 0, stream, bp);
    }
    return hipGetLastError();
}

// bf16 (is_bf16) or f16, D = 32, 64 or 128. The dQ kernel runs first: it
// writes Delta, which the dK / dV kernel reads.
hipError_t launch_bwd(const BwdParams& bp, int D, bool is_bf16, bool causal, hipStream_t stream) {
    if (is_bf16) {
        return D == 32 ? launch_bwd_typed<__bf16, 32>(bp, causal, stream)
             : D == 64 ? launch_bwd_typed<__bf16, 64>(bp, causal, stream)
                       : launch_bwd_typed<__bf16, 128>(bp, causal, stream);
    }
    return D == 32 ? launch_bwd_typed<_Float16, 32>(bp, causal, stream)
         : D == 64 ? launch_bwd_typed<_Float16, 64>(bp, causal, stream)
                   : launch_bwd_typed<_Float16, 128>(bp, causal, stream);
}

}  // namespace attn

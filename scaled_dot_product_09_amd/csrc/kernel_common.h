// kernel_common.h — shared device-side definitions of the attention kernels.
//
// Parameter block, vector types and the workgroup -> work-item mapping used by
// every kernel in libattn.so. Only the library's own .hip files include it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// Division by a divisor fixed at launch, for dividends in [0, 2^31): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1 (< 2^32),
// n / d = (umulhi(n, m) + n) >> l (the round-up multiplier method of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994; exact for 31-bit dividends because m d - 2^(32+l)
// is at most d <= 2^l). The sum stays below 2^32 for n < 2^31. Replaces a
// ~40-instruction integer division by a multiply, an add and a shift.
struct FastDiv {
    uint32_t m;
    int l;
};

inline FastDiv make_fastdiv(int d) {   // host side, d >= 1
    FastDiv f;
    f.l = 0;
    while ((1ll << f.l) < (long long)d) ++f.l;
    f.m = (uint32_t)(((((uint64_t)1 << f.l) - (uint64_t)d) << 32) / (uint64_t)d + 1);
    return f;
}

__host__ __device__ inline int fdiv(int n, FastDiv f) {
    const uint32_t hi = (uint32_t)(((uint64_t)(uint32_t)n * f.m) >> 32);
    return (int)((hi + (uint32_t)n) >> f.l);
}

// Everything a forward kernel needs, passed by value as one kernel argument.
struct FwdParams {
    const void* q;      // (B, Sq, Hq, D), element strides sq
    const void* k;      // (B, Skv, Hkv, D), element strides sk
    const void* v;      // (B, Skv, Hkv, D), element strides sv
    void* out;          // (B, Sq, Hq, D), element strides so
    // Element strides of the batch, sequence and head axes (D is contiguous);
    // dense (B, S, H, D) tensors have {S H D, H D, D}.
    int64_t sq[3], sk[3], sv[3], so[3];
    int B, Hq, Hkv, Sq, Skv;
    int G;              // query heads per KV head, Hq / Hkv
    int gpack;          // query heads of one KV head handled by one workgroup
    int head_stride;    // consecutive query slots of one head (see the slot map of the kernels)
    int rows_per_wg;    // query rows per head handled by one workgroup
    int n_row_blocks;   // ceil(Sq / rows_per_wg)
    int n_units;        // B * Hkv * (G / gpack): (batch, KV head, head group) units
    int xcd_remap;      // 1 when n_units % 8 == 0 (see map_workgroup)
    float scale_log2;   // softmax scale * log2(e) (FP8: times q and k descales)
    float out_mul;      // factor applied to the normalised output (FP8: v descale)
    int causal_off;     // causal: key j is visible to query row i iff j <= i + causal_off
    int n_split;        // key ranges per (unit, row block); 1 = no split
    float* part_o;      // n_split > 1: unnormalised partial outputs [n_split][B][Sq][Hq][D]
    float* part_ml;     // n_split > 1: (running max, weight sum) pairs [n_split][B][Sq][Hq][2]
    float* lse;         // null, or the natural-log row log-sum-exp of the scaled scores, [B][Hq][Sq]
    // FP8 with device-side dequantisation factors: when dsc_q is not null,
    // scale_log2 holds the bare softmax scale and the kernel reads q, k, v
    // factors from device memory: multiplier ((scale qd) kd) log2(e),
    // out_mul = vd (the same expressions, in the same order, as the host
    // computes for host-side factors).
    const float* dsc_q;
    const float* dsc_k;
    const float* dsc_v;
    // Divisors of the workgroup map (set by set_divisors before a launch):
    // n_row_blocks * n_split, n_units, n_split, G / gpack, Hkv; and log2 of
    // head_stride and gpack (both powers of two).
    FastDiv div_ranks, div_per, div_units, div_split, div_groups, div_hkv;
    int hs_log2, gpack_log2;
    int unit_major;     // with xcd_remap: an XCD runs its units one after another (see map_workgroup)
    // 0, or R >= 2: folded row blocks. The workgroup's slots with a row
    // offset below rows_per_wg hold row block rb of R blocks of rows_per_wg
    // rows, the others block R - 1 - rb (none when that is rb itself), and
    // n_row_blocks = ceil(R / 2). Under a causal mask the two blocks' key
    // counts add up to about the same for every workgroup.
    int fold;
};

// Slot map of a launch (host side; from B, Hkv, G and Sq): a workgroup of
// `waves` waves of rows_per_wave query slots shares one KV head between
// gpack query heads and covers rows_per_wave * waves / gpack rows of each.
// gpack is the largest of 4, 2, 1 dividing G (1 without the matrix cores).
// The matrix-core kernel (wide_heads), whose MFMA columns may mix heads,
// doubles it while G allows and the heads' Sq rows still fit the
// workgroup's slots (gpack * Sq <= rows_per_wave * waves): with few query
// rows (decode with GQA / MQA) the slots then hold rows of many heads
// instead of empty rows of one. Slots come in runs of head_stride
// consecutive rows of one head, heads interleaved between runs: 32 (one
// head per wave, 32 rows) when there are that many rows; with fewer rows,
// the smallest power of two >= Sq, so the rows of all gpack heads sit in
// the first waves and the rest have no work. No folding.
inline void set_slot_map(FwdParams& p, bool mfma, int rows_per_wave, int waves, bool wide_heads) {
    p.gpack = mfma ? ((p.G % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1) : 1;
    if (mfma && wide_heads) {
        const int slots = rows_per_wave * waves;
        while (p.G % (2 * p.gpack) == 0 && 2 * p.gpack <= slots && (int64_t)2 * p.gpack * p.Sq <= slots)
            p.gpack *= 2;
    }
    p.rows_per_wg = rows_per_wave * waves / p.gpack;
    int hs = 1;
    while (hs < p.Sq && hs < 32) hs *= 2;
    p.head_stride = hs < p.rows_per_wg ? hs : p.rows_per_wg;
    p.n_row_blocks = (p.Sq + p.rows_per_wg - 1) / p.rows_per_wg;
    p.n_units = p.B * p.Hkv * (p.G / p.gpack);
    p.xcd_remap = (p.n_units % 8 == 0) ? 1 : 0;
    p.fold = 0;
}

// Folded row blocks for the four-query-wave (128-slot) map of set_slot_map
// (host side): blocks of 64 / gpack rows with gpack at most 2, so that a
// wave still holds 32 rows of one head, two mirror blocks per workgroup,
// the same number of workgroups. Needs runs of 32 rows (head_stride 32) and
// at least two blocks; returns whether it folded.
inline bool fold_row_blocks(FwdParams& p) {
    if (p.head_stride != 32 || p.rows_per_wg * p.gpack != 128) return false;
    const int gp = p.gpack < 2 ? p.gpack : 2;
    const int rpw = 64 / gp;
    const int R = (p.Sq + rpw - 1) / rpw;
    if (R < 2) return false;
    p.gpack = gp;
    p.rows_per_wg = rpw;
    p.fold = R;
    p.n_row_blocks = (R + 1) / 2;
    p.n_units = p.B * p.Hkv * (p.G / gp);
    p.xcd_remap = p.n_units % 8 == 0 ? 1 : 0;
    return true;
}

// Fills the divisor fields from the shape fields (host side; call after the
// last change to n_units, n_split, G, gpack, Hkv or head_stride).
inline void set_divisors(FwdParams& p) {
    const int ranks = p.n_row_blocks * p.n_split;
    p.div_ranks = make_fastdiv(ranks > 0 ? ranks : 1);
    const int per = p.n_units >> 3;
    p.div_per = make_fastdiv(per > 0 ? per : 1);
    // A unit's row blocks fill an XCD's 64 workgroup slots (32 CUs, two
    // each) on their own: its longest ones then start while at least a
    // unit's worth of work remains, and the causal tail stays short.
    p.unit_major = ranks >= 64;
    p.div_units = make_fastdiv(p.n_units > 0 ? p.n_units : 1);
    p.div_split = make_fastdiv(p.n_split > 0 ? p.n_split : 1);
    const int groups = p.gpack > 0 ? p.G / p.gpack : 1;
    p.div_groups = make_fastdiv(groups > 0 ? groups : 1);
    p.div_hkv = make_fastdiv(p.Hkv > 0 ? p.Hkv : 1);
    p.hs_log2 = 0;
    while ((1 << p.hs_log2) < p.head_stride) ++p.hs_log2;
    p.gpack_log2 = 0;
    while ((1 << p.gpack_log2) < p.gpack) ++p.gpack_log2;
}

// Query slot s of a matrix-core workgroup: head offset (s / HS) % gpack and
// row offset (s / (HS gpack)) HS + s % HS from the workgroup's first head and
// row (see the slot map of the kernels; HS = head_stride).
__host__ __device__ inline int slot_head(const FwdParams& p, int s) {
    return (s >> p.hs_log2) & ((1 << p.gpack_log2) - 1);
}
__host__ __device__ inline int slot_row(const FwdParams& p, int s) {
    return ((s >> (p.hs_log2 + p.gpack_log2)) << p.hs_log2) + (s & ((1 << p.hs_log2) - 1));
}

constexpr float kLog2eF32 = 1.4426950408889634f;

// The forward's score multiplier and output factor, from the parameters or
// from device memory. A zero multiplier becomes 2^-100, as on the host (see
// the C API): every weight is then exp2(0) = 1, the weights of scale 0.
__device__ inline void fwd_scalars(const FwdParams& p, float& sl2, float& out_mul) {
    sl2 = p.scale_log2;
    out_mul = p.out_mul;
    if (p.dsc_q) {
        sl2 = ((p.scale_log2 * *p.dsc_q) * *p.dsc_k) * kLog2eF32;
        out_mul = *p.dsc_v;
        if (sl2 == 0.0f) sl2 = 0x1p-100f;
    }
}

constexpr float kLn2 = 0.6931471805599453f;

// Backward pass: the forward's block (q, k, v, out = the forward's output,
// shapes, slot map, scale_log2 = scale log2(e), causal_off) plus the
// gradient tensors. dout and dq have q's layout, dk and dv k's.
struct BwdParams {
    FwdParams f;
    const void* dout;   // (B, Sq, Hq, D) gradient of the loss with respect to out
    const float* lse;   // [B][Hq][Sq] natural-log row log-sum-exp from the forward
    float* delta;       // [B][Hq][Sq] workspace: rowsum(dout * out), written by the dQ kernel
    float* lse2;        // [B][Hq][Sq] workspace: lse * log2(e), written by the dQ kernel
    void* dq;           // (B, Sq, Hq, D)
    void* dk;           // (B, Skv, Hkv, D)
    void* dv;           // (B, Skv, Hkv, D)
    // Scalar factors (all 1 but dq_mul = dk_mul = scale for 16-bit inputs;
    // for FP8 codes they fold in the per-tensor dequantisation factors):
    //   dP = dp_mul (dout v^T), Delta = delta_mul rowsum(dout * out),
    //   dq = dq_mul (dS k), dk = dk_mul (dS^T q), dv = dv_mul (P^T dout).
    float dp_mul, delta_mul, dq_mul, dk_mul, dv_mul;
    int n_kblocks;      // key blocks of the dK / dV kernel, ceil(Skv / 128)
    // FP8 with device-side factors (q, k, v, dout), or null: then the
    // factors above are formed on the device from scale (the bare softmax
    // scale) by the expressions the host uses.
    const float* dsc[4];
    float scale;
};

struct WorkItem {
    int b, hkv, hq0;    // batch, KV head, first query head of the workgroup
    int row_base;       // first query row of the workgroup (of its first row block)
    int row_hi;         // folded: first row of the second row block minus rows_per_wg; else row_base
    int row_end;        // one past the workgroup's last query row (not clamped to Sq)
    int split;          // which of the n_split key ranges
};

// Workgroup -> (unit, row block, key range). The hardware hands workgroup i
// to XCD i % 8 (MI355X has 8 XCDs, each with its own L2). When the units
// split evenly over the XCDs, XCD x gets a contiguous range of units, so
// every workgroup that reads a given KV head runs on the same XCD and shares
// its L2. Row blocks go out in order of decreasing causal work (the last row
// block first) so the short ones fill the tail of the launch; the key ranges
// of one row block are neighbours. With many row blocks per unit
// (unit_major) the XCD runs its units one after another, all row blocks of
// one before the next, so that about one unit's K and V are live in its L2
// at a time; otherwise it interleaves them (every unit's longest row block
// first).
__host__ __device__ inline WorkItem map_item(const FwdParams& p, bool causal, int pid) {
    int rank, unit;
    if (p.xcd_remap) {
        const int per = p.n_units >> 3;
        const int xcd = pid & 7;
        const int slot = pid >> 3;
        int ul;
        if (p.unit_major) {
            ul = fdiv(slot, p.div_ranks);
            rank = slot - ul * (p.n_row_blocks * p.n_split);
        } else {
            rank = fdiv(slot, p.div_per);
            ul = slot - rank * per;
        }
        unit = xcd * per + ul;
    } else {
        rank = fdiv(pid, p.div_units);
        unit = pid - rank * p.n_units;
    }
    const int rb_rank = fdiv(rank, p.div_split);
    const int split = rank - rb_rank * p.n_split;
    const int rb = causal ? (p.n_row_blocks - 1 - rb_rank) : rb_rank;
    const int groups = p.G / p.gpack;
    const int t = fdiv(unit, p.div_groups);
    const int hgrp = unit - t * groups;
    WorkItem w;
    w.b = fdiv(t, p.div_hkv);
    w.hkv = t - w.b * p.Hkv;
    w.hq0 = w.hkv * p.G + hgrp * p.gpack;
    w.row_base = rb * p.rows_per_wg;
    w.row_hi = w.row_base;
    w.row_end = w.row_base + p.rows_per_wg;
    if (p.fold) {
        // The mirror block; for the middle block of an odd R the second
        // half's rows start at Sq (no work).
        const int rb2 = p.fold - 1 - rb;
        w.row_hi = (rb2 > rb ? rb2 * p.rows_per_wg : p.Sq) - p.rows_per_wg;
        if (rb2 > rb) w.row_end = (rb2 + 1) * p.rows_per_wg;
    }
    w.split = split;
    return w;
}

// The calling workgroup's item.
__device__ inline WorkItem map_workgroup(const FwdParams& p, bool causal) {
    return map_item(p, causal, (int)__builtin_amdgcn_workgroup_id_x());
}

// Query row of slot s of a workgroup (see slot_row; slots of the second
// half of a folded workgroup belong to its second row block).
__host__ __device__ inline int item_row(const FwdParams& p, const WorkItem& w, int s) {
    const int r = slot_row(p, s);
    return (r < p.rows_per_wg ? w.row_base : w.row_hi) + r;
}

// The values of lanes l and l ^ 32 of a 64-wide wavefront, as (a, b) in some
// order: v_permlane32_swap exchanges the upper half of one operand with the
// lower half of the other, so each lane ends up holding both.
__device__ inline void xor32_pair(float x, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
    a = __builtin_bit_cast(float, (unsigned)r[0]);
    b = __builtin_bit_cast(float, (unsigned)r[1]);
}

// Maximum of a value over lanes l and l ^ 32 of a 64-wide wavefront.
__device__ inline float xor32_max(float x) {
    float a, b;
    xor32_pair(x, a, b);
    return fmaxf(a, b);
}

__device__ inline float xor32_sum(float x) {
    float a, b;
    xor32_pair(x, a, b);
    return a + b;
}

}  // namespace attn

// attn_fwd_f32.hip — fused attention forward in float32 on the vector ALUs.
//
// The float32 path of out = softmax(scale * Q K^T [+ causal mask]) V (codelab
// "Accelerate attention on GPU with cuDNN and TransformerEngine", §1 formula,
// §4 float32 from-scratch computation, §7 mask, §9 head grouping). It keeps
// every product and sum in float32 so the result stays within 1e-5 of the
// exact value on N(0, 1) inputs; it is not the throughput path (bf16 / f16 /
// FP8 run on the matrix cores).
//
// Layout of the work: one workgroup (256 threads) takes a block of query rows
// of one query head. Each row is split over TPR = D / 32 neighbouring lanes
// that each keep 32 columns of Q and of the output accumulator in registers.
// K and V tiles of 32 keys are staged in LDS; every lane reads them with
// broadcast 16-byte loads. Scores of one tile are finished with a reduction
// over the TPR lanes of the row, then one online-softmax update per tile.

#include "kernel_common.h"

namespace attn {

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdParams p) {
    constexpr int TPR = D / 32;           // lanes per query row
    constexpr int RPW = 256 / TPR;        // query rows per workgroup
    constexpr int BK = 32;                // keys per tile
    __shared__ __attribute__((aligned(16))) float lk[BK][D];
    __shared__ __attribute__((aligned(16))) float lv[BK][D];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int part = tid % TPR;
    const int rows_blocks = (p.Sq + RPW - 1) / RPW;
    int bid = (int)__builtin_amdgcn_workgroup_id_x();
    const int rb = bid % rows_blocks;  bid /= rows_blocks;
    const int hq = bid % p.Hq;
    const int b = bid / p.Hq;
    const int hkv = hq / p.G;
    const int row = rb * RPW + tid / TPR;
    const int Sq = p.Sq, Skv = p.Skv;
    const int64_t kstride = p.sk[1], vstride = p.sv[1];

    const float* qrow = (const float*)p.q + b * p.sq[0] + row * p.sq[1] + hq * p.sq[2] + part * 32;
    const float* kb = (const float*)p.k + b * p.sk[0] + hkv * p.sk[2];
    const float* vb = (const float*)p.v + b * p.sv[0] + hkv * p.sv[2];

    float qv[32], o[32];
    for (int d = 0; d < 32; ++d) { qv[d] = row < Sq ? qrow[d] : 0.f; o[d] = 0.f; }
    float m_run = -INFINITY, l_run = 0.f;

    int kend = Skv;
    if (CAUSAL) kend = min(Skv, min(rb * RPW + RPW, Sq) + p.causal_off);   // keys 0 .. last visible
    for (int k0 = 0; k0 < kend; k0 += BK) {
        __syncthreads();
        for (int e = tid; e < BK * D / 4; e += 256) {
            const int r = e / (D / 4), c = (e % (D / 4)) * 4;
            f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
            if (k0 + r < Skv) {
                kx = *(const f32x4*)(kb + (k0 + r) * kstride + c);
                vx = *(const f32x4*)(vb + (k0 + r) * vstride + c);
            }
            *(f32x4*)&lk[r][c] = kx;
            *(f32x4*)&lv[r][c] = vx;
        }
        __syncthreads();

        float s[BK];
        float mt = -INFINITY;
        for (int j = 0; j < BK; ++j) {
            float acc = 0.f;
            for (int d = 0; d < 32; d += 4) {
                const f32x4 kx = *(const f32x4*)&lk[j][part * 32 + d];
                acc = fmaf(qv[d], kx[0], acc);
                acc = fmaf(qv[d + 1], kx[1], acc);
                acc = fmaf(qv[d + 2], kx[2], acc);
                acc = fmaf(qv[d + 3], kx[3], acc);
            }
            for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
            float x = acc * p.scale_log2;
            const int key = k0 + j;
            if (key >= Skv || (CAUSAL && key > row + p.causal_off)) x = -INFINITY;
            s[j] = x;
            mt = fmaxf(mt, x);
        }
        const float mnew = fmaxf(m_run, mt);
        if (mnew == -INFINITY) continue;                   // nothing visible yet
        const float alpha = exp2f(m_run - mnew);
        l_run *= alpha;
        for (int d = 0; d < 32; ++d) o[d] *= alpha;
        m_run = mnew;
        for (int j = 0; j < BK; ++j) {
            const float pj = exp2f(s[j] - mnew);
            l_run += pj;
            for (int d = 0; d < 32; d += 4) {
                const f32x4 vx = *(const f32x4*)&lv[j][part * 32 + d];
                o[d] = fmaf(pj, vx[0], o[d]);
                o[d + 1] = fmaf(pj, vx[1], o[d + 1]);
                o[d + 2] = fmaf(pj, vx[2], o[d + 2]);
                o[d + 3] = fmaf(pj, vx[3], o[d + 3]);
            }
        }
    }

    if (row < Sq) {
        // Row log-sum-exp: sum_j e^(scale s_j) = 2^m_run l_run.
        if (p.lse && part == 0) p.lse[((size_t)b * p.Hq + hq) * Sq + row] = (m_run + log2f(l_run)) * kLn2;
        const float inv = p.out_mul / l_run;
        float* orow = (float*)p.out + b * p.so[0] + row * p.so[1] + hq * p.so[2] + part * 32;
        for (int d = 0; d < 32; d += 4)
            *(f32x4*)(orow + d) = (f32x4){o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv};
    }
}

hipError_t launch_fwd_f32(const FwdParams& p, int D, bool causal, hipStream_t stream) {
    const int rpw = 256 / (D / 32);
    const dim3 grid((unsigned)p.B * p.Hq * ((p.Sq + rpw - 1) / rpw)), block(256);
    if (D == 32) {
        if (causal) hipLaunchKernelGGL((fwd_f32_kernel<32, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((fwd_f32_kernel<32, false>), grid, block, 0, stream, p);
    } else if (D == 64) {
        if (causal) hipLaunchKernelGGL((fwd_f32_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((fwd_f32_kernel<64, false>), grid, block, 0, stream, p);
    } else {
        if (causal) hipLaunchKernelGGL((fwd_f32_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((fwd_f32_kernel<128, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace attn

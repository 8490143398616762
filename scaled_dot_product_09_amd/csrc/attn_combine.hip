// attn_combine.hip — merge of the partial results of a split-key launch.
//
// With the keys of every query row cut into n_split ranges (the split-key,
// "flash decoding" form of the fused kernel, for grids too small to fill the
// GPU, e.g. the few query rows of key-value-cache inference that the
// codelab's §9 motivates GQA / MQA with), range s leaves, per (row, head):
//   m_s  the running max of c * score (log2 domain) it weighted against,
//   l_s  the sum of its weights exp2(c s - m_s),
//   O_s  the sum of its weights times V rows.
// The softmax over all keys ([Attention codelab §1], step 2) is then
//   out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s,
// which is exactly the single-pass result: every range's weights are
// rescaled to the common offset M before the division.

#include "mfma_common.h"

namespace attn {

// One thread per 4 output elements of one (row, head).
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const FwdParams p, int rows) {
    const int n_split = p.n_split;
    using Tr = Traits<T>;
    constexpr int TPR = D / 4;
    const int t = (int)__builtin_amdgcn_workgroup_id_x() * 256 + (int)__builtin_amdgcn_workitem_id_x();
    const int r = t / TPR;
    if (r >= rows) return;
    const int d0 = (t % TPR) * 4;
    float M = -INFINITY;
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, part_ml[((size_t)s * rows + r) * 2]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    for (int s = 0; s < n_split; ++s) {
        const f32x2 ml = *(const f32x2*)(part_ml + ((size_t)s * rows + r) * 2);
        const float w = ml[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[0] - M);
        L = fmaf(w, ml[1], L);
        const f32x4 o = *(const f32x4*)(part_o + ((size_t)s * rows + r) * D + d0);
        acc[0] = fmaf(w, o[0], acc[0]);
        acc[1] = fmaf(w, o[1], acc[1]);
        acc[2] = fmaf(w, o[2], acc[2]);
        acc[3] = fmaf(w, o[3], acc[3]);
    }
    const float inv = p.out_mul / L;
    const uint32_t w0 = Tr::pack(acc[0] * inv, acc[1] * inv);
    const uint32_t w1 = Tr::pack(acc[2] * inv, acc[3] * inv);
    // r = (b Sq + row) Hq + hq, the partials' (row, head) order.
    const int hq = r % p.Hq, t2 = r / p.Hq, row = t2 % p.Sq, b = t2 / p.Sq;
    typename Tr::out_t* o = (typename Tr::out_t*)p.out + b * p.so[0] + row * p.so[1] + hq * p.so[2] + d0;
    *(u32x2*)o = (u32x2){w0, w1};
}

template <typename T, int D>
static hipError_t launch_combine_typed(const FwdParams& p, hipStream_t stream) {
    const int rows = p.B * p.Sq * p.Hq;
    const int threads = rows * (D / 4);
    hipLaunchKernelGGL((combine_kernel<T, D>), dim3((threads + 255) / 256), dim3(256), 0, stream,
                       (const float*)p.part_o, (const float*)p.part_ml, p, rows);
    return hipGetLastError();
}

// is_bf16: bfloat16 output, else float16; D = 32, 64 or 128.
hipError_t launch_combine(const FwdParams& p, int D, bool is_bf16, hipStream_t stream) {
    if (is_bf16) {
        return D == 32 ? launch_combine_typed<__bf16, 32>(p, stream)
             : D == 64 ? launch_combine_typed<__bf16, 64>(p, stream) : launch_combine_typed<__bf16, 128>(p, stream);
    }
    return D == 32 ? launch_combine_typed<_Float16, 32>(p, stream)
         : D == 64 ? launch_combine_typed<_Float16, 64>(p, stream) : launch_combine_typed<_Float16, 128>(p, stream);
}

}  // namespace attn

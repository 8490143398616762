// attn_fp8_scaling.hip — FP8 delayed scaling on the device.
//
// The codelab "Accelerate attention on GPU with cuDNN and TransformerEngine"
// (§10) runs attention in FP8 under a delayed-scaling recipe: an
// absolute-maximum history per tensor (1024 entries, reduced with max,
// margin 0), E4M3 for the forward pass and E5M2 for the backward pass. This
// file keeps that state in device memory and updates it with kernels, so a
// whole FP8 step (casts, attention, scale updates) runs without the host
// reading any value back:
//
//   * fp8_state_init_kernel: scale = scale_inv = 1, step 0, empty history.
//   * fp8_quantize_kernel: codes = nearest-even, saturating FP8 of
//     float32(x * scale) with the state's current scale (the one derived
//     from earlier steps), and amax(|x|) of this call folded into history
//     slot (step mod 1024) with one atomic max per workgroup (on the bit
//     patterns of non-negative floats, whose unsigned order is their order;
//     NaN patterns sort above infinity, so a NaN propagates).
//   * fp8_update_kernel: amax = max(history); if finite and positive,
//     scale = fmax / amax and scale_inv = 1 / scale (binary32, correctly
//     rounded divisions); step + 1; the next step's slot is cleared.

#include "kernel_common.h"

namespace attn {

// Word layout of one state (the C header documents the same).
struct Fp8State {
    float scale;
    float scale_inv;
    uint32_t step;
    uint32_t fmt;        // 0: E4M3, 1: E5M2
    float history[1024];
};
static_assert(sizeof(Fp8State) == 16 + 4096, "state layout");

namespace {

constexpr int kHistory = 1024;

__device__ inline float fmt_max(uint32_t fmt) { return fmt == 0 ? 448.0f : 57344.0f; }

// Nearest-even, saturating FP8 code of y from the fields of binary32 y.
// E4M3 (bias 7, 3 mantissa bits, largest finite 448, NaN S.1111.111) or
// E5M2 (bias 15, 2 mantissa bits, largest finite 57344, NaN S.11111.10).
__device__ inline uint32_t encode_fp8(float y, uint32_t fmt) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, y);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const uint32_t mag = bits & 0x7FFFFFFFu;
    const bool e4m3 = fmt == 0;
    if (mag > 0x7F800000u) return sign | (e4m3 ? 0x7Fu : 0x7Eu);          // NaN
    const uint32_t max_code = e4m3 ? 0x7Eu : 0x7Bu;
    const int mbits = e4m3 ? 3 : 2;
    const int bias = e4m3 ? 7 : 15;
    const int emin = 1 - bias;                                             // exponent of the smallest normal
    const float a = __builtin_bit_cast(float, mag);
    uint32_t code;
    if (a < __builtin_ldexpf(1.0f, emin)) {
        // Subnormal (or zero): a / 2^(emin - mbits) rounded to an integer,
        // nearest-even; 2^mbits (a carry into the smallest normal) is that code.
        code = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, mbits - emin));
    } else if (mag >= 0x7F800000u) {
        code = max_code;                                                   // infinity saturates
    } else {
        const int e = (int)(mag >> 23) - 127;                              // a = 1.f * 2^e, a normal binary32
        const uint32_t frac = mag & 0x7FFFFFu;
        const int drop = 23 - mbits;
        uint32_t m = frac >> drop;
        const uint32_t rem = frac & ((1u << drop) - 1u), half = 1u << (drop - 1);
        if (rem > half || (rem == half && (m & 1u))) ++m;                  // nearest, ties to even
        code = ((uint32_t)(e + bias) << mbits) + m;                        // a carry moves into the exponent
        if (code > max_code) code = max_code;
    }
    return sign | code;
}

__global__ __launch_bounds__(256) void fp8_state_init_kernel(Fp8State* states, uint32_t fmt) {
    Fp8State* st = states + __builtin_amdgcn_workgroup_id_x();
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    for (int i = tid; i < kHistory; i += 256) st->history[i] = 0.f;
    if (tid == 0) {
        st->scale = 1.0f;
        st->scale_inv = 1.0f;
        st->step = 0;
        st->fmt = fmt;
    }
}

template <typename T>
__device__ inline float load_f32(const T* p) { return (float)*p; }

// Each thread handles 8 consecutive elements per round, grid-stride over n8
// rounds; the tail (n % 8) is done element by element by the last threads.
template <typename T>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const T* __restrict__ x, uint8_t* __restrict__ codes,
                                                           int64_t n, Fp8State* st) {
    __shared__ float red[4];
    const float scale = st->scale;
    const uint32_t fmt = st->fmt;
    const uint32_t slot = st->step % kHistory;
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int64_t gid = (int64_t)__builtin_amdgcn_workgroup_id_x() * 256 + tid;
    const int64_t nthreads = (int64_t)__builtin_amdgcn_grid_size_x();
    // |v| as bit patterns: their unsigned maximum is the maximum of |v|,
    // with a NaN (pattern above infinity) taking precedence.
    uint32_t ab = 0;
    const int64_t n8 = n / 8;
    for (int64_t i = gid; i < n8; i += nthreads) {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = load_f32(x + i * 8 + e);
            const uint32_t vb = __builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu;
            ab = vb > ab ? vb : ab;
            w[e / 4] |= encode_fp8(v * scale, fmt) << (8 * (e % 4));
        }
        *(u32x2*)(codes + i * 8) = (u32x2){w[0], w[1]};
    }
    for (int64_t i = n8 * 8 + gid; i < n; i += nthreads) {
        const float v = load_f32(x + i);
        const uint32_t vb = __builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu;
        ab = vb > ab ? vb : ab;
        codes[i] = (uint8_t)encode_fp8(v * scale, fmt);
    }
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)ab, off, 64);
        ab = o > ab ? o : ab;
    }
    if ((tid & 63) == 0) red[tid >> 6] = __builtin_bit_cast(float, ab);
    __syncthreads();
    if (tid == 0) {
        uint32_t m = 0;
        for (int w = 0; w < 4; ++w) {
            const uint32_t b = __builtin_bit_cast(uint32_t, red[w]);
            m = b > m ? b : m;
        }
        atomicMax((unsigned int*)&st->history[slot], m);
    }
}

__global__ __launch_bounds__(256) void fp8_update_kernel(Fp8State* states) {
    __shared__ uint32_t red[4];
    Fp8State* st = states + __builtin_amdgcn_workgroup_id_x();
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    uint32_t m = 0;
    for (int i = tid; i < kHistory; i += 256) {
        const uint32_t b = __builtin_bit_cast(uint32_t, st->history[i]);
        m = b > m ? b : m;
    }
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
        m = o > m ? o : m;
    }
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) {
        uint32_t mm = 0;
        for (int w = 0; w < 4; ++w) mm = red[w] > mm ? red[w] : mm;
        // Finite and positive: 0 < bits < the infinity pattern.
        if (mm > 0u && mm < 0x7F800000u) {
            const float amax = __builtin_bit_cast(float, mm);
            const float s = fmt_max(st->fmt) / amax;
            st->scale = s;
            st->scale_inv = 1.0f / s;
        }
        const uint32_t next = st->step + 1;
        st->step = next;
        st->history[next % kHistory] = 0.f;
    }
}

}  // namespace

hipError_t launch_fp8_state_init(void* states, int n_states, int fmt, hipStream_t stream) {
    hipLaunchKernelGGL(fp8_state_init_kernel, dim3(n_states), dim3(256), 0, stream, (Fp8State*)states,
                       (uint32_t)fmt);
    return hipGetLastError();
}

// dtype: 0 float32, 1 bfloat16, 2 float16.
hipError_t launch_fp8_quantize(const void* x, int dtype, void* codes, int64_t n, void* state, hipStream_t stream) {
    // Enough workgroups to fill the GPU, each thread at least 8 elements a round.
    int64_t groups = (n / 8 + 255) / 256;
    if (groups < 1) groups = 1;
    if (groups > 2048) groups = 2048;
    const dim3 grid((unsigned)groups), block(256);
    if (dtype == 0)
        hipLaunchKernelGGL(fp8_quantize_kernel<float>, grid, block, 0, stream, (const float*)x, (uint8_t*)codes, n,
                           (Fp8State*)state);
    else if (dtype == 1)
        hipLaunchKernelGGL(fp8_quantize_kernel<__bf16>, grid, block, 0, stream, (const __bf16*)x, (uint8_t*)codes, n,
                           (Fp8State*)state);
    else
        hipLaunchKernelGGL(fp8_quantize_kernel<_Float16>, grid, block, 0, stream, (const _Float16*)x,
                           (uint8_t*)codes, n, (Fp8State*)state);
    return hipGetLastError();
}

hipError_t launch_fp8_update(void* states, int n_states, hipStream_t stream) {
    hipLaunchKernelGGL(fp8_update_kernel, dim3(n_states), dim3(256), 0, stream, (Fp8State*)states);
    return hipGetLastError();
}

}  // namespace attn

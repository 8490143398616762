// mfma_common.h — device building blocks shared by the matrix-core kernels.
//
// Number formats and their MFMA instructions (Traits), the LDS swizzles and
// the HBM -> LDS tile copy. Only the library's own .hip files include it.
#pragma once

#include <type_traits>

#include "kernel_common.h"

namespace attn {

typedef uint8_t fp8_t;   // one OCP E4M3 code
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Word 3 of a CDNA buffer descriptor for raw (unformatted, unswizzled) byte
// access: data format 32, every other field zero.
constexpr int kBufferWord3 = 0x00020000;

__device__ inline uint32_t pack2_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ inline uint32_t pack2_f16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}

// Workgroup barrier after which every wave's HBM -> LDS buffer copies have
// landed. Those copies complete on the vector memory counter, and the
// workgroup fence of __syncthreads() does not wait for them, so each wave
// first drains its own outstanding copies.
__device__ inline void dma_barrier() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt and lgkmcnt left alone
    __syncthreads();
}

// Per input type: the score product (QK), the weight product (PV) and the
// conversions around them.
template <typename T> struct Traits;

template <> struct Traits<__bf16> {
    static constexpr int IN_BYTES = 2;
    static constexpr int QK_LANE_BYTES = 16;    // bytes of one operand per lane per k-step
    static constexpr int QK_K = 16;             // contraction length of one QK MFMA
    static constexpr bool V_DMA = true;         // V goes to LDS unchanged
    static constexpr uint32_t SIGN_BITS = 0x80008000u;   // sign bits of the inputs in one dword
    using qk_frag = bf16x8;
    using pv_frag = bf16x8;
    using out_t = __bf16;
    __device__ static inline f32x16 qk(qk_frag a, qk_frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline f32x16 pv(pv_frag a, pv_frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline uint32_t pack(float lo, float hi) { return pack2_bf16(lo, hi); }
    // l += lo + hi of a packed pair, summed in fp32.
    __device__ static inline float sum2(uint32_t w, float l) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                              (bf16x2){(__bf16)1.0f, (__bf16)1.0f}, l, false);
    }
};

template <> struct Traits<_Float16> {
    static constexpr int IN_BYTES = 2;
    static constexpr int QK_LANE_BYTES = 16;
    static constexpr int QK_K = 16;
    static constexpr bool V_DMA = true;
    static constexpr uint32_t SIGN_BITS = 0x80008000u;
    using qk_frag = f16x8;
    using pv_frag = f16x8;
    using out_t = _Float16;
    __device__ static inline f32x16 qk(qk_frag a, qk_frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static inline f32x16 pv(pv_frag a, pv_frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static inline uint32_t pack(float lo, float hi) { return pack2_f16(lo, hi); }
    __device__ static inline float sum2(uint32_t w, float l) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w),
                                      (f16x2){(_Float16)1.0f, (_Float16)1.0f}, l, false);
    }
};

template <> struct Traits<fp8_t> {
    static constexpr int IN_BYTES = 1;
    static constexpr int QK_LANE_BYTES = 32;
    static constexpr int QK_K = 64;
    static constexpr bool V_DMA = false;        // V is widened to bf16 on its way to LDS
    static constexpr uint32_t SIGN_BITS = 0x80808080u;
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
    __device__ static inline uint32_t pack(float lo, float hi) { return pack2_bf16(lo, hi); }
    __device__ static inline float sum2(uint32_t w, float l) { return Traits<__bf16>::sum2(w, l); }
};

// XOR swizzles of 16-byte chunks inside LDS rows (chunk c of row r lives at
// chunk position c ^ swz(r)). The hardware serves 256 bytes (64 banks x 4
// bytes) per pass.
//  * K rows are read by 32 lanes at one chunk index and 32 different rows
//    (the A operand of S^T = K Q^T): consecutive rows get different masks.
//  * V rows are read by the transpose read: per half-wave 4 rows x 4 chunks.
//  * Tiles read both ways (row reads by 16 lanes per pass, transpose reads
//    of 4 rows x 64 bytes per half-wave) use kv_swz: it maps 16 consecutive
//    rows at one chunk index to 16 different chunk positions (bank groups)
//    and 4 consecutive rows starting at a multiple of 4 to 4 different
//    64-byte column groups. With u = r / (16 / NCH) (the row's 256-byte
//    bank window) and G = NCH / 4 column groups per row, the mask is
//    ((u mod G) << 2) | ((u / G) mod 4); it repeats every 16 rows.
template <int NCH>   // chunks per row
__device__ inline int k_swz(int r) { return (r / (16 / NCH)) % NCH; }
template <int NCH>
__device__ inline int v_swz(int r) { return 4 * ((r / (16 / NCH)) % (NCH / 4)); }
template <int NCH>
__device__ inline int kv_swz(int r) {
    const int u = r / (16 / NCH);
    return ((u % (NCH / 4)) << 2) | ((u / (NCH / 4)) % 4);
}

enum SwzKind { kSwzK, kSwzV, kSwzKV };

template <int NCH>
__device__ inline int swz(SwzKind kind, int r) {
    return kind == kSwzK ? k_swz<NCH>(r) : kind == kSwzV ? v_swz<NCH>(r) : kv_swz<NCH>(r);
}

// Copying one K or V tile (NROWS rows of ROWB bytes) from HBM straight into
// LDS, by NW waves. Each buffer_load_dwordx4 ... lds moves 1 KiB: lane l lands
// at byte 16 l of it, i.e. at row i * RPI + l / NCH, chunk position l % NCH,
// and fetches the global chunk (l % NCH) ^ swz(row) of that row. The per-lane
// byte offset of that chunk inside a tile (row * row stride + chunk * 16)
// does not depend on the tile, so it is computed once; each tile only adds a
// scalar offset.
template <int ROWB, int NROWS, int NW = 4>
struct TileDma {
    static constexpr int NCH = ROWB / 16;
    static constexpr int RPI = 1024 / ROWB;             // rows per instruction
    static constexpr int NINSTR = NROWS * ROWB / 1024;
    static constexpr int PER_WAVE = NINSTR / NW;
    static constexpr int ROW_STEP = NW * RPI;           // rows between a wave's instructions
    static_assert(NINSTR % NW == 0, "tile must split evenly over the copying waves");
    // Instruction t of this wave covers rows r0 + ROW_STEP t. ROW_STEP is a
    // multiple of 256 / NCH, so every swizzle gives the same mask for every t
    // (they depend on r / (16 / NCH) modulo at most 16, and ROW_STEP /
    // (16 / NCH) is a multiple of 16): one lane offset serves all of the
    // wave's instructions.
    __amdgpu_buffer_rsrc_t rs;  // the whole head: base of its row 0, no range limit
    uint32_t gstride;           // bytes between consecutive rows (keys)
    uint32_t off;               // lane's byte offset inside the tile, instruction 0
    uint32_t cb;                // lane's byte offset inside its row
    int r0;                     // lane's tile row, instruction 0

    __device__ void init(const uint8_t* head, uint32_t row_bytes_stride, int wave, int lane, SwzKind kind) {
        gstride = row_bytes_stride;
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)head, 0, -1, kBufferWord3);
        r0 = wave * RPI + lane / NCH;
        const int c = (lane % NCH) ^ swz<NCH>(kind, r0);
        cb = (uint32_t)c * 16;
        off = (uint32_t)r0 * gstride + cb;
    }
    // Rows [key0, key0 + NROWS) of the head. Rows past the end of the keys
    // (only in the last tile) repeat the last key: finite values whose
    // weights are 0 after masking.
    //
    // The copy is a buffer load into LDS (MUBUF, not a FLAT global load):
    // the head's base address lives in a scalar buffer descriptor built
    // once, the tile's and each instruction's row offset in a scalar offset
    // register, so a tile costs a handful of scalar adds and the lanes only
    // hold their fixed offset `off`. Unlike the FLAT form, the compiler's LDS
    // wait bookkeeping does not treat the copy as an LDS access of unknown
    // order (which would force every later LDS operand read to wait for all
    // outstanding reads). Every byte offset stays below Skv * gstride < 2^32
    // (a tensor has fewer than 2^31 elements of at most 2 bytes).
    __device__ void issue(int key0, int Skv, uint8_t* tile, int wave) const {
        const uint32_t t0 = (uint32_t)key0 * gstride;
        const uint32_t step = (uint32_t)ROW_STEP * gstride;
        if (key0 + NROWS <= Skv) {
            for (int t = 0; t < PER_WAVE; ++t)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(tile + (wave + NW * t) * 1024), 16,
                                                         off, t0 + t * step, 0, 0);
        } else {
            const int last = Skv - 1 - key0;        // last row of the tile that exists
            for (int t = 0; t < PER_WAVE; ++t) {
                const uint32_t o = (uint32_t)min(r0 + t * ROW_STEP, last) * gstride + cb;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(tile + (wave + NW * t) * 1024), 16,
                                                         o, t0, 0, 0);
            }
        }
    }
};


}  // namespace attn

// device_common.h -- element-type traits, MFMA wrappers and conversions for
// the gfx950 (CDNA4) kernels.  Device-side only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace cnv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- conversions (round to nearest even; the hardware default mode) -------
__device__ inline float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ inline float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
__device__ inline uint16_t f32_to_f16(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
__device__ inline uint16_t f32_to_bf16(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

// ---- element traits --------------------------------------------------------
// EPC: elements per 16-byte chunk.  One MFMA consumes 64 bytes of each
// operand row: 16x16x32 for 16-bit types, 16x16x64 for int8.
struct EF16 {
    using elem = uint16_t;
    using acc = f32x4;
    static constexpr int EPC = 8;
    static constexpr int kDtype = CONV2D_DTYPE_F16;
    __device__ static inline acc mfma(u32x4 a, u32x4 b, acc c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static inline float to_f32(elem e) { return f16_to_f32(e); }
    __device__ static inline elem from_f32(float v) { return f32_to_f16(v); }
};

struct EBF16 {
    using elem = uint16_t;
    using acc = f32x4;
    static constexpr int EPC = 8;
    static constexpr int kDtype = CONV2D_DTYPE_BF16;
    __device__ static inline acc mfma(u32x4 a, u32x4 b, acc c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static inline float to_f32(elem e) { return bf16_to_f32(e); }
    __device__ static inline elem from_f32(float v) { return f32_to_bf16(v); }
};

struct EI8 {
    using elem = int8_t;
    using acc = i32x4;
    static constexpr int EPC = 16;
    static constexpr int kDtype = CONV2D_DTYPE_I8;
    __device__ static inline acc mfma(u32x4 a, u32x4 b, acc c)
    {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                                      __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
    }
};

// ---- direct-to-LDS loads (buffer_load_dwordx4 ... lds) -------------------
// Lane i of the wave writes its 16 bytes at LDS address lds + 16*i; the
// global offset voff is checked against the buffer's byte range and reads
// past it return zeros (padding without branches).  The instruction is
// issued from inline asm so that the compiler does not track it: it would
// otherwise wait for every such load before any later LDS access, which
// serialises the prefetch with the compute.  Callers make the data visible
// themselves: s_waitcnt vmcnt(0) on every wave, then a barrier.
constexpr uint32_t kBufOOB = 0x7ffffff0u;  // past every range under 2 GB: reads as zero
// Past every buffer of at most kBufMaxBytes (internal.h), the largest
// tensor the implicit-GEMM kernels take:
constexpr uint32_t kBufOOBFar = 0xfffffff0u;

// Raw buffer descriptor (base, stride 0, num_records = bytes, 32-bit data
// format for CDNA), wave-uniform.
__device__ inline u32x4 make_buf_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    u32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    r.z = __builtin_amdgcn_readfirstlane(bytes);
    r.w = 0x00020000u;
    return r;
}
// Wave-uniform 32-bit LDS address of a __shared__ location.
__device__ inline uint32_t lds_addr(const void *p)
{
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char *)p);
}
// M0 (the LDS base of the transfer) is saved and restored around the load,
// so the compiler's own use of M0 is untouched.
// rsrc and lds must be wave-uniform; they are read from the first lane so
// that they sit in scalar registers whatever the compiler inferred.
__device__ inline void dma16(const u32x4 &rsrc_in, uint32_t lds_in, uint32_t voff)
{
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_in);
    u32x4 rsrc;
    rsrc.x = __builtin_amdgcn_readfirstlane(rsrc_in.x);
    rsrc.y = __builtin_amdgcn_readfirstlane(rsrc_in.y);
    rsrc.z = __builtin_amdgcn_readfirstlane(rsrc_in.z);
    rsrc.w = __builtin_amdgcn_readfirstlane(rsrc_in.w);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(rsrc)
        : "memory");
}
__device__ inline void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)
// s_waitcnt with vmcnt = N (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ inline void wait_vm_n()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// int8 requantisation of one accumulator: + bias, ReLU, * m in fp64,
// round half to even (v_rndne_f64), saturate.
__device__ inline int8_t requant_i8(int v, double m)
{
    double t = rint((double)v * m);
    t = t > 127.0 ? 127.0 : t;
    t = t < -128.0 ? -128.0 : t;
    return (int8_t)(int)t;
}

typedef float f2v __attribute__((ext_vector_type(2)));
typedef short s2v __attribute__((ext_vector_type(2)));
template <class E>
struct Pack2;
template <>
struct Pack2<EF16> {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    __device__ static inline uint32_t cvt(f2v v) { return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2)); }
};
template <>
struct Pack2<EBF16> {
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    __device__ static inline uint32_t cvt(f2v v) { return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2)); }
};
// Two epilogue values to a packed pair, rounded to nearest even by one packed
// conversion.  ReLU (v <= 0, -0 and NaN included, -> +0), which commutes with
// the rounding: a max against 0 that maps NaN to 0 (packed fp16 after the
// conversion; fp32 before it for bf16, which has no packed max), then an
// int16 max of the packed halves, which turns a -0 into +0.
template <class E, bool RELU>
__device__ inline uint32_t out_pair(float a, float b)
{
    constexpr bool F16 = E::kDtype == CONV2D_DTYPE_F16;
    if (RELU && !F16) {
        a = __builtin_fmaxf(a, 0.0f);
        b = __builtin_fmaxf(b, 0.0f);
    }
    uint32_t p = Pack2<E>::cvt(f2v{a, b});
    if (RELU && F16) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        p = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(h2, p), h2{0, 0}));
    }
    if (RELU) p = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s2v, p), s2v{0, 0}));
    return p;
}

// acc + (both 16-bit values of the packed pair w), in fp32: a two-element
// dot product with (1, 1) (exact products, one fp32 accumulation)
template <class E>
struct DotOne {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    __device__ static inline float add(uint32_t w, float acc)
    {
        if constexpr (E::kDtype == CONV2D_DTYPE_F16)
            return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), h2{(_Float16)1.0f, (_Float16)1.0f}, acc, false);
        else
            return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w), b2{(__bf16)1.0f, (__bf16)1.0f}, acc,
                                                   false);
    }
};
// Float epilogue value: acc + bias, then ReLU (v <= 0, including -0, -> +0).
__device__ inline float bias_relu_f32(float v, float b, int relu)
{
    v += b;
    return (relu && !(v > 0.0f)) ? 0.0f : v;
}

}  // namespace cnv

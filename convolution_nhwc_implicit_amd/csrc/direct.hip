// direct.hip -- direct convolution for grouped problems (groups > 1).
//
// The burn CubeCL dispatch (conv_forward_nhwc, conv_weight_backward,
// conv_data_backward) routes groups != 1 to a direct kernel rather than the
// implicit GEMM; this file is that path for gfx950.  Each thread owns one
// output element and sums its products in a fixed (r, s, channel) order in
// fp32 (int32 for int8), so results are deterministic.  Consecutive threads
// own consecutive channels, so the NHWC / KRSC reads and the writes coalesce.
// wgrad cuts its long pixel sum into slices whose fp32 partials are reduced in
// slice order by the same split-K reduction as the implicit-GEMM wgrad.
#include <type_traits>

#include "device_common.h"

namespace cnv {

template <class E>
__device__ inline float ld_f(const typename E::elem *p)
{
    return E::to_f32(*p);
}

// ---------------------------------------------------------------- fprop ----
// alpha * acc + beta * cmat[idx] when the linear-combination epilogue is on
template <class E>
__device__ inline float axpby_at(const DirectArgs &a, float acc, size_t idx)
{
    if (!a.axpby) return acc;
    const float c = a.cmat ? ld_f<E>((const typename E::elem *)a.cmat + idx) : 0.0f;
    return a.alpha * acc + a.beta * c;
}

template <class E>
__global__ __launch_bounds__(256) void direct_fprop_kernel(const DirectArgs a)
{
    using elem = typename E::elem;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.total) return;
    const int k = (int)(idx % a.K);
    const long long pix = idx / a.K;
    const int q = (int)(pix % a.Q);
    const int p = (int)((pix / a.Q) % a.P);
    const int n = (int)(pix / ((long long)a.P * a.Q));
    const int g = k / a.Kg;
    const elem *x = (const elem *)a.a + g * a.Cg;
    const elem *w = (const elem *)a.b + (size_t)k * a.R * a.S * a.Cg;

    if constexpr (E::kDtype == CONV2D_DTYPE_I8) {
        int acc = 0;
        for (int r = 0; r < a.R; ++r) {
            const int h = p * a.sh - a.pad_h + r * a.dh;
            if ((unsigned)h >= (unsigned)a.H) continue;
            for (int s = 0; s < a.S; ++s) {
                const int wc = q * a.sw - a.pad_w + s * a.dw;
                if ((unsigned)wc >= (unsigned)a.W) continue;
                const elem *xp = x + (((size_t)n * a.H + h) * a.W + wc) * a.C;
                const elem *wp = w + ((size_t)r * a.S + s) * a.Cg;
                for (int c = 0; c < a.Cg; ++c) acc += (int)xp[c] * (int)wp[c];
            }
        }
        int v = acc + (a.bias ? ((const int32_t *)a.bias)[k] : 0);
        if (a.relu && v < 0) v = 0;
        ((int8_t *)a.out)[idx] = requant_i8(v, a.requant_m);
    } else {
        float acc = 0.0f;
        for (int r = 0; r < a.R; ++r) {
            const int h = p * a.sh - a.pad_h + r * a.dh;
            if ((unsigned)h >= (unsigned)a.H) continue;
            for (int s = 0; s < a.S; ++s) {
                const int wc = q * a.sw - a.pad_w + s * a.dw;
                if ((unsigned)wc >= (unsigned)a.W) continue;
                const elem *xp = x + (((size_t)n * a.H + h) * a.W + wc) * a.C;
                const elem *wp = w + ((size_t)r * a.S + s) * a.Cg;
                for (int c = 0; c < a.Cg; ++c) acc += ld_f<E>(xp + c) * ld_f<E>(wp + c);
            }
        }
        const float b = a.bias ? ld_f<E>((const elem *)a.bias + k) : 0.0f;
        ((elem *)a.out)[idx] = E::from_f32(bias_relu_f32(axpby_at<E>(a, acc, idx), b, a.relu));
    }
}

// ---------------------------------------------------------------- dgrad ----
// dx[n,h,w,c] = sum over taps (r,s) that reach (h,w) from a valid output
// pixel, and over the output channels k of c's group, of dy[n,p,q,k]*w[k,r,s,c'].
template <class E>
__global__ __launch_bounds__(256) void direct_dgrad_kernel(const DirectArgs a)
{
    using elem = typename E::elem;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.total) return;
    const int c = (int)(idx % a.C);
    const long long pix = idx / a.C;
    const int wc = (int)(pix % a.W);
    const int h = (int)((pix / a.W) % a.H);
    const int n = (int)(pix / ((long long)a.H * a.W));
    const int g = c / a.Cg, cl = c - g * a.Cg;
    const elem *dy = (const elem *)a.a;
    const elem *w = (const elem *)a.b;
    float acc = 0.0f;
    for (int r = 0; r < a.R; ++r) {
        const int th = h + a.pad_h - r * a.dh;
        if (th < 0 || th % a.sh) continue;
        const int p = th / a.sh;
        if (p >= a.P) continue;
        for (int s = 0; s < a.S; ++s) {
            const int tw = wc + a.pad_w - s * a.dw;
            if (tw < 0 || tw % a.sw) continue;
            const int q = tw / a.sw;
            if (q >= a.Q) continue;
            const elem *dyp = dy + (((size_t)n * a.P + p) * a.Q + q) * a.K + (size_t)g * a.Kg;
            const elem *wp = w + (((size_t)g * a.Kg * a.R + r) * a.S + s) * a.Cg + cl;
            const size_t kstride = (size_t)a.R * a.S * a.Cg;
            for (int kl = 0; kl < a.Kg; ++kl) acc += ld_f<E>(dyp + kl) * ld_f<E>(wp + kl * kstride);
        }
    }
    ((elem *)a.out)[idx] = E::from_f32(axpby_at<E>(a, acc, idx));
}

// ---------------------------------------------------------------- wgrad ----
// One thread per (slice z, k, r, s, c'); sums its slice of output pixels.
template <class E>
__global__ __launch_bounds__(256) void direct_wgrad_kernel(const DirectArgs a)
{
    using elem = typename E::elem;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.total) return;
    const int z = blockIdx.y;
    const int cl = (int)(idx % a.Cg);
    long long t = idx / a.Cg;
    const int s = (int)(t % a.S);
    t /= a.S;
    const int r = (int)(t % a.R);
    const int k = (int)(t / a.R);
    const int g = k / a.Kg;
    const elem *x = (const elem *)a.a + g * a.Cg + cl;
    const elem *dy = (const elem *)a.b + k;
    const uint32_t pbeg = (uint32_t)z * a.pix_per_split;
    uint32_t pend = pbeg + a.pix_per_split;
    if (pend > a.npix || pend < pbeg) pend = a.npix;
    float acc = 0.0f;
    if (pbeg < pend) {
        uint32_t q = pbeg % a.Q, rest = pbeg / a.Q;
        uint32_t p = rest % a.P, n = rest / a.P;
        for (uint32_t pix = pbeg; pix < pend; ++pix) {
            const int h = (int)p * a.sh - a.pad_h + r * a.dh;
            const int w = (int)q * a.sw - a.pad_w + s * a.dw;
            if ((unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W)
                acc += ld_f<E>(dy + (size_t)pix * a.K) *
                       ld_f<E>(x + (((size_t)n * a.H + h) * a.W + w) * a.C);
            if (++q == (uint32_t)a.Q) {
                q = 0;
                if (++p == (uint32_t)a.P) {
                    p = 0;
                    ++n;
                }
            }
        }
    }
    if (a.splits == 1 && !a.to_parts)
        ((elem *)a.out)[idx] = E::from_f32(acc);
    else
        ((float *)a.out)[(size_t)z * a.part_stride + idx] = acc;
}

// ------------------------------------------------------- tiled kernels ----
// For 16-bit types with channel counts that allow 16-byte vectors, a
// workgroup stages what it reads in LDS (the group's filter slice and the
// input rows of a few output rows) and each thread computes four outputs at
// once with two-element dot products (v_dot2_f32_f16 / _bf16: exact
// products, fp32 sums) in a fixed (tap, channel) order.
template <class E>
struct Dot2;
template <>
struct Dot2<EF16> {
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    __device__ static inline float run(uint32_t a, uint32_t b, float c)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2, a), __builtin_bit_cast(v2, b), c, false);
    }
};
template <>
struct Dot2<EBF16> {
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    __device__ static inline float run(uint32_t a, uint32_t b, float c)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2, a), __builtin_bit_cast(v2, b), c, false);
    }
};
template <class E>
__device__ inline float dot8(u32x4 a, u32x4 b, float c)
{
    c = Dot2<E>::run(a.x, b.x, c);
    c = Dot2<E>::run(a.y, b.y, c);
    c = Dot2<E>::run(a.z, b.z, c);
    return Dot2<E>::run(a.w, b.w, c);
}

constexpr int kDirectLds = 64 * 1024;

// fprop: workgroup = (image, `rows` output rows, group).  LDS: the group's
// filters [Kg][R][S][Cg] as stored, and input rows [rows][R][W][Cg] (zeros
// outside the image).  Thread item = (row, output column, 4 output channels).
template <class E>
__global__ __launch_bounds__(256) void direct_fprop_tiled(const DirectArgs a)
{
    using elem = typename E::elem;
    extern __shared__ __attribute__((aligned(16))) unsigned char dsm[];
    const int tid = threadIdx.x, g = blockIdx.y, rows = a.rows;
    const int ptiles = (a.P + rows - 1) / rows;
    const int n = blockIdx.x / ptiles, p0 = (blockIdx.x - n * ptiles) * rows;
    const int RSC = a.R * a.S * a.Cg, CG8 = a.Cg / 8;
    elem *wsm = (elem *)dsm;
    elem *xsm = wsm + (size_t)a.Kg * RSC;
    {
        const u32x4 *wg = (const u32x4 *)((const elem *)a.b + (size_t)g * a.Kg * RSC);
        for (int i = tid; i < a.Kg * RSC / 8; i += 256) ((u32x4 *)wsm)[i] = wg[i];
        const elem *x = (const elem *)a.a;
        const int nx = rows * a.R * a.W * CG8;
        for (int i = tid; i < nx; i += 256) {
            int t = i / CG8;
            const int c8 = i - t * CG8;
            const int wc = t % a.W;
            t /= a.W;
            const int r = t % a.R, ri = t / a.R;
            const int p = p0 + ri, h = p * a.sh - a.pad_h + r * a.dh;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (p < a.P && (unsigned)h < (unsigned)a.H)
                v = *(const u32x4 *)(x + (((size_t)n * a.H + h) * a.W + wc) * a.C + g * a.Cg + c8 * 8);
            ((u32x4 *)xsm)[i] = v;
        }
    }
    __syncthreads();
    const int KBN = a.Kg / 4, items = rows * a.Q * KBN;
    for (int it = tid; it < items; it += 256) {
        const int kb = it % KBN, t = it / KBN;
        const int q = t % a.Q, ri = t / a.Q;
        const int p = p0 + ri;
        if (p >= a.P) continue;
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int r = 0; r < a.R; ++r) {
            const int h = p * a.sh - a.pad_h + r * a.dh;
            if ((unsigned)h >= (unsigned)a.H) continue;
            for (int s = 0; s < a.S; ++s) {
                const int wc = q * a.sw - a.pad_w + s * a.dw;
                if ((unsigned)wc >= (unsigned)a.W) continue;
                const u32x4 *xr = (const u32x4 *)(xsm + ((size_t)(ri * a.R + r) * a.W + wc) * a.Cg);
                const u32x4 *wr = (const u32x4 *)(wsm + (size_t)kb * 4 * RSC + (r * a.S + s) * a.Cg);
                for (int c8 = 0; c8 < CG8; ++c8) {
                    const u32x4 xv = xr[c8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = dot8<E>(xv, wr[e * (RSC / 8) + c8], acc[e]);
                }
            }
        }
        const int k0 = g * a.Kg + kb * 4;
        const size_t o = (((size_t)n * a.P + p) * a.Q + q) * a.K + k0;
        uint32_t v[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
            uint32_t lohi[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int k = k0 + 2 * e2 + e;
                const float b = a.bias ? ld_f<E>((const elem *)a.bias + k) : 0.0f;
                lohi[e] = E::from_f32(bias_relu_f32(axpby_at<E>(a, acc[2 * e2 + e], o + 2 * e2 + e), b, a.relu));
            }
            v[e2] = lohi[0] | (lohi[1] << 16);
        }
        *(uint2 *)((elem *)a.out + o) = uint2{v[0], v[1]};
    }
}

// dgrad: workgroup = (image, `rows` dx rows, group).  LDS: the group's
// filters transposed to [R][S][Cg][Kg], and for each (row, r) the dy row
// p = (h + pad - r*d)/stride that reaches it ([rows][R][Q][Kg], zeros when no
// row does).  Thread item = (row, dx column, 4 channels).
template <class E>
__global__ __launch_bounds__(256) void direct_dgrad_tiled(const DirectArgs a)
{
    using elem = typename E::elem;
    extern __shared__ __attribute__((aligned(16))) unsigned char dsm[];
    const int tid = threadIdx.x, g = blockIdx.y, rows = a.rows;
    const int htiles = (a.H + rows - 1) / rows;
    const int n = blockIdx.x / htiles, h0 = (blockIdx.x - n * htiles) * rows;
    const int RSC = a.R * a.S * a.Cg, KG8 = a.Kg / 8;
    elem *wt = (elem *)dsm;                      // [R][S][Cg][Kg]
    elem *dys = wt + (size_t)RSC * a.Kg;         // [rows][R][Q][Kg]
    {
        const elem *w = (const elem *)a.b + (size_t)g * a.Kg * RSC;
        for (int i = tid; i < RSC * a.Kg; i += 256) {
            const int kl = i % a.Kg, rsc = i / a.Kg;
            wt[i] = w[(size_t)kl * RSC + rsc];
        }
        const elem *dy = (const elem *)a.a;
        const int nd = rows * a.R * a.Q * KG8;
        for (int i = tid; i < nd; i += 256) {
            int t = i / KG8;
            const int k8 = i - t * KG8;
            const int q = t % a.Q;
            t /= a.Q;
            const int r = t % a.R, hi = t / a.R;
            const int h = h0 + hi, th = h + a.pad_h - r * a.dh;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (h < a.H && th >= 0 && th % a.sh == 0 && th / a.sh < a.P)
                v = *(const u32x4 *)(dy + (((size_t)n * a.P + th / a.sh) * a.Q + q) * a.K + g * a.Kg + k8 * 8);
            ((u32x4 *)dys)[i] = v;
        }
    }
    __syncthreads();
    const int CBN = a.Cg / 4, items = rows * a.W * CBN;
    for (int it = tid; it < items; it += 256) {
        const int cb = it % CBN, t = it / CBN;
        const int wc = t % a.W, hi = t / a.W;
        const int h = h0 + hi;
        if (h >= a.H) continue;
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int r = 0; r < a.R; ++r) {
            const int th = h + a.pad_h - r * a.dh;
            if (th < 0 || th % a.sh || th / a.sh >= a.P) continue;
            for (int s = 0; s < a.S; ++s) {
                const int tw = wc + a.pad_w - s * a.dw;
                if (tw < 0 || tw % a.sw) continue;
                const int q = tw / a.sw;
                if (q >= a.Q) continue;
                const u32x4 *dr = (const u32x4 *)(dys + ((size_t)(hi * a.R + r) * a.Q + q) * a.Kg);
                const u32x4 *wr = (const u32x4 *)(wt + ((size_t)(r * a.S + s) * a.Cg + cb * 4) * a.Kg);
                for (int k8 = 0; k8 < KG8; ++k8) {
                    const u32x4 dv = dr[k8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = dot8<E>(dv, wr[e * KG8 + k8], acc[e]);
                }
            }
        }
        const size_t o = (((size_t)n * a.H + h) * a.W + wc) * a.C + g * a.Cg + cb * 4;
        uint32_t v[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2)
            v[e2] = (uint32_t)E::from_f32(axpby_at<E>(a, acc[2 * e2], o + 2 * e2)) |
                    ((uint32_t)E::from_f32(axpby_at<E>(a, acc[2 * e2 + 1], o + 2 * e2 + 1)) << 16);
        *(uint2 *)((elem *)a.out + o) = uint2{v[0], v[1]};
    }
}

// wgrad: thread = (group, 4 output channels kl, tap (r, s), 8 channels cl) of
// the filter, summing its pixel slice in order (fp32).  The dy and x vectors
// it reads per pixel are shared with its neighbours through the caches.
template <class E>
__global__ __launch_bounds__(256) void direct_wgrad_tiled(const DirectArgs a)
{
    using elem = typename E::elem;
    const int KBN = a.Kg / 4, CG8 = a.Cg / 8;
    const int per_g = KBN * a.R * a.S * CG8;
    const int id = blockIdx.x * 256 + threadIdx.x;
    if (id >= per_g) return;
    const int g = blockIdx.y, z = blockIdx.z;
    int t = id;
    const int c8 = t % CG8;
    t /= CG8;
    const int s = t % a.S;
    t /= a.S;
    const int r = t % a.R, kb = t / a.R;
    const elem *x = (const elem *)a.a + g * a.Cg + c8 * 8;
    const elem *dy = (const elem *)a.b + g * a.Kg + kb * 4;
    const uint32_t pbeg = (uint32_t)z * a.pix_per_split;
    uint32_t pend = pbeg + a.pix_per_split;
    if (pend > a.npix || pend < pbeg) pend = a.npix;
    float acc[4][8];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[e][j] = 0.0f;
    if (pbeg < pend) {
        uint32_t q = pbeg % a.Q, rest = pbeg / a.Q;
        uint32_t p = rest % a.P, n = rest / a.P;
        for (uint32_t pix = pbeg; pix < pend; ++pix) {
            const int h = (int)p * a.sh - a.pad_h + r * a.dh;
            const int w = (int)q * a.sw - a.pad_w + s * a.dw;
            if ((unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W) {
                const uint2 dv = *(const uint2 *)(dy + (size_t)pix * a.K);
                const u32x4 xv = *(const u32x4 *)(x + (((size_t)n * a.H + h) * a.W + w) * a.C);
                float df[4], xf[8];
                const uint32_t dw4[2] = {dv.x, dv.y}, xw8[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) df[e] = E::to_f32((elem)(dw4[e >> 1] >> (16 * (e & 1))));
#pragma unroll
                for (int j = 0; j < 8; ++j) xf[j] = E::to_f32((elem)(xw8[j >> 1] >> (16 * (j & 1))));
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[e][j] += df[e] * xf[j];
            }
            if (++q == (uint32_t)a.Q) {
                q = 0;
                if (++p == (uint32_t)a.P) {
                    p = 0;
                    ++n;
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int k = g * a.Kg + kb * 4 + e;
        const size_t o = (((size_t)k * a.R + r) * a.S + s) * a.Cg + c8 * 8;
        if (a.splits == 1 && !a.to_parts) {
            uint32_t v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = (uint32_t)E::from_f32(acc[e][2 * j]) | ((uint32_t)E::from_f32(acc[e][2 * j + 1]) << 16);
            *(u32x4 *)((elem *)a.out + o) = u32x4{v[0], v[1], v[2], v[3]};
        } else {
            float *dst = (float *)a.out + (size_t)z * a.part_stride + o;
#pragma unroll
            for (int j = 0; j < 8; j += 4) *(f32x4 *)(dst + j) = f32x4{acc[e][j], acc[e][j + 1], acc[e][j + 2], acc[e][j + 3]};
        }
    }
}

// ---------------------------------------------------------- depthwise ----
// groups = C = K (one channel per group): per-channel 2-D filters, no
// reduction over channels.  A thread owns 8 channels (one 16-byte vector of
// the NHWC pixel) of DWT consecutive output columns and accumulates their
// taps in fp32, (r, s) in order.  Neighbouring threads take neighbouring
// channel vectors, so every load of a wave is whole 16-byte pieces of
// consecutive pixels; the re-reads of the 3x3 neighbourhood hit the caches.
constexpr int DWT = 4;
constexpr int DW_MAX_TAPS = 9;  // wgrad keeps one fp32 sum per tap and channel
constexpr int DWW = 4;          // output columns per work unit of the wgrad row kernel

// The row kernels: unit column stride and dilation, R and S up to 3, and
// the tensors they read through buffer offsets under 1 GB.
static bool rows_ok(int R, int S, int sw, int dw, long long in_bytes, long long in2_bytes)
{
    return R <= 3 && S <= 3 && sw == 1 && dw == 1 && in_bytes < (1LL << 30) && in2_bytes < (1LL << 30);
}

template <class E>
__device__ inline void unpack8(u32x4 v, float *f)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = E::to_f32((typename E::elem)(w[j >> 1] >> (16 * (j & 1))));
}

// acc + (fp16 in the low / high half of x2, widened exactly) * w, one rounding.
__device__ inline float fma_mix_lo(uint32_t x2, float w, float acc)
{
    asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(x2), "v"(w));
    return acc;
}
__device__ inline float fma_mix_hi(uint32_t x2, float w, float acc)
{
    asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(x2), "v"(w));
    return acc;
}

// acc + a * b for the fp16 pair in the low / high halves of a2 and b2.
__device__ inline float fma_mix2_lo(uint32_t a2, uint32_t b2, float acc)
{
    asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[1,1,0]" : "+v"(acc) : "v"(a2), "v"(b2));
    return acc;
}
__device__ inline float fma_mix2_hi(uint32_t a2, uint32_t b2, float acc)
{
    asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[1,1,0] op_sel_hi:[1,1,0]" : "+v"(acc) : "v"(a2), "v"(b2));
    return acc;
}

// Bias of the thread's 8 channels (zeros without bias), loaded once.
template <class E>
__device__ inline void load_bias8(const DirectArgs &a, int c0, float *b8)
{
#pragma unroll
    for (int j = 0; j < 8; ++j) b8[j] = a.bias ? ld_f<E>((const typename E::elem *)a.bias + c0 + j) : 0.0f;
}

// out[o .. o+7] = epilogue(v): alpha/beta with C, then bias and ReLU when b8
// is given (fprop).
template <class E>
__device__ inline void store8(const DirectArgs &a, typename E::elem *dst, size_t o, const float *v,
                              const float *b8)
{
    uint32_t w[4];
#pragma unroll
    for (int j2 = 0; j2 < 4; ++j2) {
        uint32_t h[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int j = 2 * j2 + e;
            float t = axpby_at<E>(a, v[j], o + j);
            if (b8) t = bias_relu_f32(t, b8[j], a.relu);
            h[e] = E::from_f32(t);
        }
        w[j2] = h[0] | (h[1] << 16);
    }
    __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, (u32x4 *)(dst + o));  // streamed out
}

// The filter [C][R][S] is C*R*S contiguous elements, a whole number of
// 16-byte chunks.  It is staged per workgroup in LDS as [R*S][C] fp32 (taps
// reversed when flip), so a thread reads its 8 channels' weight of a tap as
// two 16-byte LDS reads.  The caller loads chunk threadIdx.x (filter_chunk)
// before its own input loads, so the two share one trip to memory.
template <class E>
__device__ inline u32x4 filter_chunk(const DirectArgs &a, int i)
{
    return i < a.C * a.R * a.S / 8 ? *(const u32x4 *)((const typename E::elem *)a.b + (size_t)i * 8)
                                   : u32x4{0, 0, 0, 0};
}

template <class E>
__device__ inline void stage_filter(const DirectArgs &a, float *wsh, bool flip, u32x4 first)
{
    const int RS = a.R * a.S, nch = a.C * RS / 8;
    for (int i = threadIdx.x; i < nch; i += 256) {
        float f[8];
        unpack8<E>(i == (int)threadIdx.x ? first : filter_chunk<E>(a, i), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int fl = i * 8 + e, c = fl / RS, k = fl - c * RS;
            wsh[(flip ? RS - 1 - k : k) * a.C + c] = f[e];
        }
    }
}

__device__ inline void filter8(const float *wsh, int k, int C, int c0, float *wv)
{
    const f32x4 lo = *(const f32x4 *)(wsh + k * C + c0), hi = *(const f32x4 *)(wsh + k * C + c0 + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        wv[j] = lo[j];
        wv[4 + j] = hi[j];
    }
}

// Geometry of the row kernel: an input of ih x iw pixels, an output of oh x ow
// pixels; output row p reads input rows p*sh - ph + r*dh, output column q reads
// input columns q - pw + s (unit column stride and dilation).  The thread
// index t < nthr is (row n*oh + p, column strip qt, channel vector c8),
// c8 fastest; in_bytes is the input's size (under 2 GB).
struct DwGeom {
    int ih, iw, oh, ow, sh, dh, ph, pw;
    uint32_t nthr, in_bytes;
    FastDiv div_c8, div_qt, div_oh;
};

// Row kernel, R <= 3 and S <= 3 with unit column stride and dilation.  (R and
// S stay run-time values: fixing them at compile time lets the compiler widen
// every row's pixels to fp32 at once, which costs occupancy and time.)  A
// thread's DWT outputs read
// DWT + S - 1 input pixels of each of R input rows; they are all loaded, as
// buffer loads whose out-of-range offsets read zeros (the padding), before
// the filter and bias are staged, so the kernel makes one trip to memory;
// every tap then reuses them from registers.  fprop: in = x, filter as
// stored, bias and ReLU.  dgrad at stride 1 (FLIP): in = dy, the filter
// reversed in r and s, pads (R-1)*dh - pad_h and (S-1) - pad_w, no bias.
template <class E, bool FLIP>
__global__ __launch_bounds__(256) void depthwise_rows(const DirectArgs a, const DwGeom g)
{
    using elem = typename E::elem;
    extern __shared__ __attribute__((aligned(16))) float wsh[];  // [R*S][C] filter, then [C] bias
    const int R = a.R, S = a.S;
    const uint32_t C8 = (uint32_t)a.C / 8, QT = (uint32_t)(g.ow + DWT - 1) / DWT;
    uint32_t t = blockIdx.x * 256u + threadIdx.x;
    const bool live = t < g.nthr;
    if (!live) t = 0;
    const uint32_t rest = fdiv(t, g.div_c8), c8 = t - rest * C8;
    const uint32_t prow = fdiv(rest, g.div_qt), qt = rest - prow * QT;
    const uint32_t n = fdiv(prow, g.div_oh), p = prow - n * (uint32_t)g.oh;
    const int c0 = (int)c8 * 8, w0 = (int)qt * DWT - g.pw;
    const uint32_t pixb = (uint32_t)a.C * 2;
    // filter chunk and bias first: staging them waits for these loads only
    const u32x4 fch = filter_chunk<E>(a, threadIdx.x);
    const bool has_bias = !FLIP && a.bias;
    const float bias0 = has_bias && (int)threadIdx.x < a.C ? ld_f<E>((const elem *)a.bias + threadIdx.x) : 0.0f;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)a.a, (short)0, (int)g.in_bytes, 0x00020000);
    u32x4 raw[3][DWT + 2];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const int h = (int)p * g.sh - g.ph + r * g.dh;
        const bool rok = live && r < R && (unsigned)h < (unsigned)g.ih;
        const uint32_t base = rok ? ((n * (uint32_t)g.ih + (uint32_t)h) * (uint32_t)g.iw) * pixb + (uint32_t)c0 * 2 : kBufOOB;
#pragma unroll
        for (int u = 0; u < DWT + 2; ++u) {
            const int wc = w0 + u;
            const uint32_t off = (unsigned)wc < (unsigned)g.iw && u < DWT + S - 1 ? base + (uint32_t)wc * pixb : kBufOOB;
            raw[r][u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
        }
    }
    stage_filter<E>(a, wsh, FLIP, fch);
    float *bsh = wsh + R * S * a.C;
    if (has_bias) {
        for (int i = threadIdx.x; i < a.C; i += 256)
            bsh[i] = i == (int)threadIdx.x ? bias0 : ld_f<E>((const elem *)a.bias + i);
    }
    __syncthreads();
    if (!live) return;
    float acc[DWT][8];
#pragma unroll
    for (int i = 0; i < DWT; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        if (r >= R) break;
        if constexpr (std::is_same<E, EF16>::value) {
            // fp16 pixels feed v_fma_mix_f32 straight from their packed
            // words (exact widening, one rounding: the same result as
            // converting first), which saves a conversion per element
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                if (s >= S) break;
                float wv[8];
                filter8(wsh, r * S + s, a.C, c0, wv);
#pragma unroll
                for (int i = 0; i < DWT; ++i) {
                    const u32x4 v = raw[r][i + s];
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int j = 0; j < 8; j += 2) {
                        acc[i][j] = fma_mix_lo(w4[j >> 1], wv[j], acc[i][j]);
                        acc[i][j + 1] = fma_mix_hi(w4[j >> 1], wv[j + 1], acc[i][j + 1]);
                    }
                }
            }
        } else {
            float xf[DWT + 2][8];
#pragma unroll
            for (int u = 0; u < DWT + 2; ++u) unpack8<E>(raw[r][u], xf[u]);
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                if (s >= S) break;
                float wv[8];
                filter8(wsh, r * S + s, a.C, c0, wv);
#pragma unroll
                for (int i = 0; i < DWT; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[i][j] += xf[i + s][j] * wv[j];
            }
        }
    }
    float b8[8];
    if (has_bias) {
        const f32x4 lo = *(const f32x4 *)(bsh + c0), hi = *(const f32x4 *)(bsh + c0 + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b8[j] = lo[j];
            b8[4 + j] = hi[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) b8[j] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < DWT; ++i) {
        const int q = (int)qt * DWT + i;
        if (q < g.ow)
            store8<E>(a, (elem *)a.out, (((size_t)n * g.oh + p) * g.ow + q) * a.C + c0, acc[i],
                      FLIP ? nullptr : b8);
    }
}

// General fprop (any column stride or dilation, up to 9 taps): per tap, the
// thread's DWT output columns each load their input pixel.
template <class E>
__global__ __launch_bounds__(256) void depthwise_fprop(const DirectArgs a)
{
    using elem = typename E::elem;
    extern __shared__ __attribute__((aligned(16))) float wsh[];  // [R*S][C]
    const int C8 = a.C / 8, QT = (a.Q + DWT - 1) / DWT;
    stage_filter<E>(a, wsh, false, filter_chunk<E>(a, threadIdx.x));
    __syncthreads();
    long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    if (t >= (long long)a.N * a.P * QT * C8) return;
    const int c8 = (int)(t % C8);
    t /= C8;
    const int qt = (int)(t % QT);
    t /= QT;
    const int p = (int)(t % a.P), n = (int)(t / a.P);
    const int c0 = c8 * 8;
    const elem *x = (const elem *)a.a;
    float acc[DWT][8];
#pragma unroll
    for (int i = 0; i < DWT; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    for (int r = 0; r < a.R; ++r) {
        const int h = p * a.sh - a.pad_h + r * a.dh;
        if ((unsigned)h >= (unsigned)a.H) continue;
        const elem *xrow = x + ((size_t)n * a.H + h) * a.W * a.C + c0;
        for (int s = 0; s < a.S; ++s) {
            float wv[8];
            filter8(wsh, r * a.S + s, a.C, c0, wv);
#pragma unroll
            for (int i = 0; i < DWT; ++i) {
                const int q = qt * DWT + i;
                const int wc = q * a.sw - a.pad_w + s * a.dw;
                if (q >= a.Q || (unsigned)wc >= (unsigned)a.W) continue;
                float xf[8];
                unpack8<E>(*(const u32x4 *)(xrow + (size_t)wc * a.C), xf);
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] += xf[j] * wv[j];
            }
        }
    }
    float b8[8];
    load_bias8<E>(a, c0, b8);
#pragma unroll
    for (int i = 0; i < DWT; ++i) {
        const int q = qt * DWT + i;
        if (q < a.Q) store8<E>(a, (elem *)a.out, (((size_t)n * a.P + p) * a.Q + q) * a.C + c0, acc[i], b8);
    }
}

template <class E>
__global__ __launch_bounds__(256) void depthwise_dgrad(const DirectArgs a)
{
    using elem = typename E::elem;
    extern __shared__ __attribute__((aligned(16))) float wsh[];  // [R*S][C]
    const int C8 = a.C / 8, WT = (a.W + DWT - 1) / DWT;
    stage_filter<E>(a, wsh, false, filter_chunk<E>(a, threadIdx.x));
    __syncthreads();
    long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    if (t >= (long long)a.N * a.H * WT * C8) return;
    const int c8 = (int)(t % C8);
    t /= C8;
    const int wt = (int)(t % WT);
    t /= WT;
    const int h = (int)(t % a.H), n = (int)(t / a.H);
    const int c0 = c8 * 8;
    const elem *dy = (const elem *)a.a;
    float acc[DWT][8];
#pragma unroll
    for (int i = 0; i < DWT; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    for (int r = 0; r < a.R; ++r) {
        const int th = h + a.pad_h - r * a.dh;
        if (th < 0 || th % a.sh) continue;
        const int p = th / a.sh;
        if (p >= a.P) continue;
        const elem *drow = dy + ((size_t)n * a.P + p) * a.Q * a.C + c0;
        for (int s = 0; s < a.S; ++s) {
            float wv[8];
            filter8(wsh, r * a.S + s, a.C, c0, wv);
#pragma unroll
            for (int i = 0; i < DWT; ++i) {
                const int wc = wt * DWT + i;
                const int tw = wc + a.pad_w - s * a.dw;
                if (wc >= a.W || tw < 0 || tw % a.sw) continue;
                const int q = tw / a.sw;
                if (q >= a.Q) continue;
                float df[8];
                unpack8<E>(*(const u32x4 *)(drow + (size_t)q * a.C), df);
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] += df[j] * wv[j];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < DWT; ++i) {
        const int wc = wt * DWT + i;
        if (wc < a.W)
            store8<E>(a, (elem *)a.out, (((size_t)n * a.H + h) * a.W + wc) * a.C + c0, acc[i], nullptr);
    }
}

// wgrad: dw[c,r,s] = sum over output pixels of dy[pix,c] * x[tap pixel,c].
// Workgroup z takes pixels [z*pix_per_split, ...); its threads are (channel
// vector c8, pixel lane pl): lane pl sums pixels pl, pl + npl, ... of the
// slice, then the lanes' sums are added in lane order through LDS and the
// workgroup writes one fp32 partial per (c, r, s).
template <class E>
__global__ __launch_bounds__(256) void depthwise_wgrad(const DirectArgs a)
{
    using elem = typename E::elem;
    __shared__ float red[256][8];
    const int C8 = a.C / 8, npl = 256 / C8, RS = a.R * a.S;
    const int tid = threadIdx.x, c8 = tid % C8, pl = tid / C8;
    const bool live = pl < npl;
    const int c0 = c8 * 8;
    const elem *x = (const elem *)a.a + c0;
    const elem *dy = (const elem *)a.b + c0;
    const uint32_t pbeg = (uint32_t)blockIdx.x * a.pix_per_split;
    uint32_t pend = pbeg + a.pix_per_split;
    if (pend > a.npix || pend < pbeg) pend = a.npix;
    float acc[DW_MAX_TAPS][8];
#pragma unroll
    for (int k = 0; k < DW_MAX_TAPS; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[k][j] = 0.0f;
    if (live) {
        for (uint32_t pix = pbeg + pl; pix < pend; pix += npl) {
            const uint32_t rest = fdiv(pix, a.div_q), q = pix - rest * (uint32_t)a.Q;
            const uint32_t n = fdiv(rest, a.div_p), p = rest - n * (uint32_t)a.P;
            float df[8];
            unpack8<E>(*(const u32x4 *)(dy + (size_t)pix * a.C), df);
#pragma unroll
            for (int k = 0; k < DW_MAX_TAPS; ++k) {
                const int r = k / a.S, s = k - r * a.S;
                const int h = (int)p * a.sh - a.pad_h + r * a.dh;
                const int wc = (int)q * a.sw - a.pad_w + s * a.dw;
                if (k < RS && (unsigned)h < (unsigned)a.H && (unsigned)wc < (unsigned)a.W) {
                    float xf[8];
                    unpack8<E>(*(const u32x4 *)(x + (((size_t)n * a.H + h) * a.W + wc) * a.C), xf);
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[k][j] += df[j] * xf[j];
                }
            }
        }
    }
    float *part = (float *)a.out + (size_t)blockIdx.x * a.part_stride;
#pragma unroll
    for (int k = 0; k < DW_MAX_TAPS; ++k) {
        if (k >= RS) continue;  // uniform
#pragma unroll
        for (int j = 0; j < 8; ++j) red[tid][j] = acc[k][j];
        __syncthreads();
        if (pl == 0) {
            float sum[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) sum[j] = 0.0f;
            for (int l = 0; l < npl; ++l)
#pragma unroll
                for (int j = 0; j < 8; ++j) sum[j] += red[l * C8 + c8][j];
            const int r = k / a.S, s = k - r * a.S;
#pragma unroll
            for (int j = 0; j < 8; ++j) part[((size_t)(c0 + j) * a.R + r) * a.S + s] = sum[j];
        }
        __syncthreads();
    }
}

// wgrad, R <= 3 and S <= 3 with unit column stride and dilation: a work unit
// is a strip of DWW output columns of one output row.  The thread loads the
// strip's dy pixels and the DWW + S - 1 input pixels of each of its R input
// rows, then adds dy[q] * x[q - pad_w + s] over the strip into its fp32 sum
// of every tap.  Workgroup z takes units [z*units_per_split, ...), thread
// lane sl the units sl, sl + nsl, ... of them; the lanes' sums are added in
// lane order through LDS and the workgroup writes one fp32 partial per
// (c, r, s).
template <class E, int T>
__global__ __launch_bounds__(256) void depthwise_wgrad_rows(const DirectArgs a)
{
    using elem = typename E::elem;
    __shared__ float red[256][8];
    const int C8 = a.C / 8, nsl = 256 / C8, RS = a.R * a.S;
    const int tid = threadIdx.x, c8 = tid % C8, sl = tid / C8;
    const int c0 = c8 * 8;
    const elem *x = (const elem *)a.a + c0;
    const elem *dy = (const elem *)a.b + c0;
    const uint32_t beg = (uint32_t)blockIdx.x * a.pix_per_split;
    uint32_t end = beg + a.pix_per_split;
    if (end > a.npix || end < beg) end = a.npix;
    const uint32_t QT = (uint32_t)(a.Q + T - 1) / T, pixb = (uint32_t)a.C * 2;
    // x and dy as buffers (each under 1 GB): out-of-range offsets read zeros
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x - c0), (short)0, (int)((uint32_t)a.N * a.H * a.W * pixb), 0x00020000);
    const __amdgpu_buffer_rsrc_t ds = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(dy - c0), (short)0, (int)((uint32_t)a.N * a.P * a.Q * pixb), 0x00020000);
    float acc[3][3][8];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int s = 0; s < 3; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[r][s][j] = 0.0f;
    if (sl < nsl) {
        for (uint32_t u = beg + sl; u < end; u += nsl) {
            const uint32_t rest = fdiv(u, a.div_q), qt = u - rest * QT;
            const uint32_t n = fdiv(rest, a.div_p), p = rest - n * (uint32_t)a.P;
            const int q0 = (int)qt * T, w0 = q0 - a.pad_w;
            const uint32_t dbase = ((n * (uint32_t)a.P + p) * (uint32_t)a.Q + (uint32_t)q0) * pixb + (uint32_t)c0 * 2;
            u32x4 draw[T];
#pragma unroll
            for (int i = 0; i < T; ++i)
                draw[i] = __builtin_amdgcn_raw_buffer_load_b128(ds, q0 + i < a.Q ? dbase + i * pixb : kBufOOB, 0, 0);
            u32x4 xraw[3][T + 2];
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const int h = (int)p * a.sh - a.pad_h + r * a.dh;
                const bool rok = r < a.R && (unsigned)h < (unsigned)a.H;
                const uint32_t base = rok ? (n * (uint32_t)a.H + (uint32_t)h) * (uint32_t)a.W * pixb + (uint32_t)c0 * 2
                                          : kBufOOB;
#pragma unroll
                for (int v = 0; v < T + 2; ++v) {
                    const int wc = w0 + v;
                    const uint32_t off =
                        v < T + a.S - 1 && (unsigned)wc < (unsigned)a.W ? base + (uint32_t)wc * pixb : kBufOOB;
                    xraw[r][v] = __builtin_amdgcn_raw_buffer_load_b128(xs, off, 0, 0);
                }
            }
            if constexpr (std::is_same<E, EF16>::value) {
                // both operands fp16: v_fma_mix_f32 takes them from their
                // packed words (exact products' widening, one rounding)
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    if (r >= a.R) break;
#pragma unroll
                    for (int s = 0; s < 3; ++s) {
                        if (s >= a.S) break;
#pragma unroll
                        for (int i = 0; i < T; ++i) {
                            const uint32_t d4[4] = {draw[i].x, draw[i].y, draw[i].z, draw[i].w};
                            const u32x4 xv = xraw[r][i + s];
                            const uint32_t x4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                            for (int j = 0; j < 8; j += 2) {
                                acc[r][s][j] = fma_mix2_lo(d4[j >> 1], x4[j >> 1], acc[r][s][j]);
                                acc[r][s][j + 1] = fma_mix2_hi(d4[j >> 1], x4[j >> 1], acc[r][s][j + 1]);
                            }
                        }
                    }
                }
            } else {
                float df[T][8];
#pragma unroll
                for (int i = 0; i < T; ++i) unpack8<E>(draw[i], df[i]);
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    if (r >= a.R) break;
                    float xf[T + 2][8];
#pragma unroll
                    for (int v = 0; v < T + 2; ++v) unpack8<E>(xraw[r][v], xf[v]);
#pragma unroll
                    for (int s = 0; s < 3; ++s) {
                        if (s >= a.S) break;
#pragma unroll
                        for (int i = 0; i < T; ++i)
#pragma unroll
                            for (int j = 0; j < 8; ++j) acc[r][s][j] += df[i][j] * xf[i + s][j];
                    }
                }
            }
        }
    }
    float *part = (float *)a.out + (size_t)blockIdx.x * a.part_stride;
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            if (r >= a.R || s >= a.S) continue;  // uniform
#pragma unroll
            for (int j = 0; j < 8; ++j) red[tid][j] = acc[r][s][j];
            __syncthreads();
            for (int o = tid; o < C8 * 8; o += 256) {
                const int oc8 = o >> 3, j = o & 7;
                float sum = 0.0f;
                for (int l = 0; l < nsl; ++l) sum += red[l * C8 + oc8][j];
                part[(size_t)o * RS + r * a.S + s] = sum;
            }
            __syncthreads();
        }
}

int direct_depthwise_wgrad_cols(int N, int H, int W, int C, int P, int Q, int R, int S, int sw, int dw)
{
    const long long xb = (long long)N * H * W * C * 2, dyb = (long long)N * P * Q * C * 2;
    return rows_ok(R, S, sw, dw, xb, dyb) ? DWW : 1;
}

bool direct_depthwise_ok(int dtype, int C, int Cg, int Kg, int R, int S)
{
    return (dtype == CONV2D_DTYPE_F16 || dtype == CONV2D_DTYPE_BF16) && Cg == 1 && Kg == 1 && C % 8 == 0 &&
           C / 8 <= 256 && R * S <= DW_MAX_TAPS && (size_t)R * S * C * sizeof(float) <= 64 * 1024;
}

int direct_tiled_rows(int op, int dtype, int R, int S, int W, int Q, int Cg, int Kg)
{
    if (dtype != CONV2D_DTYPE_F16 && dtype != CONV2D_DTYPE_BF16) return 0;
    long long fixed, per_row;
    if (op == 0) {
        if (Cg % 8 || Kg % 4) return 0;
        fixed = (long long)Kg * R * S * Cg;
        per_row = (long long)R * W * Cg;
    } else {
        if (Kg % 8 || Cg % 4) return 0;
        fixed = (long long)R * S * Cg * Kg;
        per_row = (long long)R * Q * Kg;
    }
    for (int rows = 4; rows >= 1; --rows)
        if ((fixed + rows * per_row) * 2 <= kDirectLds) return rows;
    return 0;
}

bool direct_wgrad_tiled_ok(int dtype, int Cg, int Kg)
{
    return (dtype == CONV2D_DTYPE_F16 || dtype == CONV2D_DTYPE_BF16) && Kg % 4 == 0 && Cg % 8 == 0;
}

long long direct_wgrad_tiled_wgs(int R, int S, int Cg, int Kg, int G)
{
    return ((long long)(Kg / 4) * R * S * (Cg / 8) + 255) / 256 * G;
}

static unsigned blocks_for(long long total) { return (unsigned)((total + 255) / 256); }

static DwGeom dw_geom(const DirectArgs &a, int ih, int iw, int oh, int ow, int sh, int dh, int ph, int pw,
                      long long thr, long long in_bytes)
{
    DwGeom g{ih, iw, oh, ow, sh, dh, ph, pw, (uint32_t)thr, (uint32_t)in_bytes, {}, {}, {}};
    g.div_c8 = make_fastdiv((uint32_t)(a.C / 8));
    g.div_qt = make_fastdiv((uint32_t)((ow + DWT - 1) / DWT));
    g.div_oh = make_fastdiv((uint32_t)oh);
    return g;
}

template <bool FLIP>
static hipError_t launch_rows(int dtype, const DirectArgs &a, const DwGeom &g, hipStream_t st)
{
    const size_t lds = ((size_t)a.R * a.S * a.C + a.C) * sizeof(float);
    const unsigned blocks = (unsigned)((g.nthr + 255) / 256);
    switch (dtype) {
    case CONV2D_DTYPE_F16: depthwise_rows<EF16, FLIP><<<blocks, 256, lds, st>>>(a, g); break;
    case CONV2D_DTYPE_BF16: depthwise_rows<EBF16, FLIP><<<blocks, 256, lds, st>>>(a, g); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_direct_fprop(int dtype, const DirectArgs &a, hipStream_t st)
{
    if (a.total == 0) return hipSuccess;
    if (a.depthwise) {
        const long long thr = (long long)a.N * a.P * ((a.Q + DWT - 1) / DWT) * (a.C / 8);
        const long long in_bytes = (long long)a.N * a.H * a.W * a.C * 2;
        if (rows_ok(a.R, a.S, a.sw, a.dw, in_bytes, 0) && thr < (1LL << 31)) {
            const DwGeom g = dw_geom(a, a.H, a.W, a.P, a.Q, a.sh, a.dh, a.pad_h, a.pad_w, thr, in_bytes);
            return launch_rows<false>(dtype, a, g, st);
        }
        const size_t lds = (size_t)a.R * a.S * a.C * sizeof(float);
        switch (dtype) {
        case CONV2D_DTYPE_F16: depthwise_fprop<EF16><<<blocks_for(thr), 256, lds, st>>>(a); break;
        case CONV2D_DTYPE_BF16: depthwise_fprop<EBF16><<<blocks_for(thr), 256, lds, st>>>(a); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (a.tiled) {
        const size_t lds = ((size_t)a.Kg * a.R * a.S * a.Cg + (size_t)a.rows * a.R * a.W * a.Cg) * 2;
        dim3 grid((unsigned)(a.N * ((a.P + a.rows - 1) / a.rows)), (unsigned)a.G);
        switch (dtype) {
        case CONV2D_DTYPE_F16: direct_fprop_tiled<EF16><<<grid, 256, lds, st>>>(a); break;
        case CONV2D_DTYPE_BF16: direct_fprop_tiled<EBF16><<<grid, 256, lds, st>>>(a); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (dtype) {
    case CONV2D_DTYPE_F16: direct_fprop_kernel<EF16><<<blocks_for(a.total), 256, 0, st>>>(a); break;
    case CONV2D_DTYPE_BF16: direct_fprop_kernel<EBF16><<<blocks_for(a.total), 256, 0, st>>>(a); break;
    case CONV2D_DTYPE_I8: direct_fprop_kernel<EI8><<<blocks_for(a.total), 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_direct_dgrad(int dtype, const DirectArgs &a, hipStream_t st)
{
    if (a.total == 0) return hipSuccess;
    if (a.depthwise) {
        const long long thr = (long long)a.N * a.H * ((a.W + DWT - 1) / DWT) * (a.C / 8);
        const long long in_bytes = (long long)a.N * a.P * a.Q * a.C * 2;
        if (a.sh == 1 && rows_ok(a.R, a.S, a.sw, a.dw, in_bytes, 0) && thr < (1LL << 31)) {
            // stride 1: the fprop row kernel over dy with the filter reversed
            const DwGeom g = dw_geom(a, a.P, a.Q, a.H, a.W, 1, a.dh, (a.R - 1) * a.dh - a.pad_h,
                                     (a.S - 1) - a.pad_w, thr, in_bytes);
            return launch_rows<true>(dtype, a, g, st);
        }
        const size_t lds = (size_t)a.R * a.S * a.C * sizeof(float);
        switch (dtype) {
        case CONV2D_DTYPE_F16: depthwise_dgrad<EF16><<<blocks_for(thr), 256, lds, st>>>(a); break;
        case CONV2D_DTYPE_BF16: depthwise_dgrad<EBF16><<<blocks_for(thr), 256, lds, st>>>(a); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (a.tiled) {
        const size_t lds = ((size_t)a.R * a.S * a.Cg * a.Kg + (size_t)a.rows * a.R * a.Q * a.Kg) * 2;
        dim3 grid((unsigned)(a.N * ((a.H + a.rows - 1) / a.rows)), (unsigned)a.G);
        switch (dtype) {
        case CONV2D_DTYPE_F16: direct_dgrad_tiled<EF16><<<grid, 256, lds, st>>>(a); break;
        case CONV2D_DTYPE_BF16: direct_dgrad_tiled<EBF16><<<grid, 256, lds, st>>>(a); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (dtype) {
    case CONV2D_DTYPE_F16: direct_dgrad_kernel<EF16><<<blocks_for(a.total), 256, 0, st>>>(a); break;
    case CONV2D_DTYPE_BF16: direct_dgrad_kernel<EBF16><<<blocks_for(a.total), 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_direct_wgrad(int dtype, const DirectArgs &a, hipStream_t st)
{
    if (a.total == 0) return hipSuccess;
    if (a.depthwise) {  // always fp32 partials, one per workgroup (grid = splits)
        const bool rows = direct_depthwise_wgrad_cols(a.N, a.H, a.W, a.C, a.P, a.Q, a.R, a.S, a.sw, a.dw) > 1;
        switch (dtype) {
        case CONV2D_DTYPE_F16:
            if (rows)
                depthwise_wgrad_rows<EF16, DWW><<<(unsigned)a.splits, 256, 0, st>>>(a);
            else
                depthwise_wgrad<EF16><<<(unsigned)a.splits, 256, 0, st>>>(a);
            break;
        case CONV2D_DTYPE_BF16:
            if (rows)
                depthwise_wgrad_rows<EBF16, DWW><<<(unsigned)a.splits, 256, 0, st>>>(a);
            else
                depthwise_wgrad<EBF16><<<(unsigned)a.splits, 256, 0, st>>>(a);
            break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (a.tiled) {
        const long long per_g = (long long)(a.Kg / 4) * a.R * a.S * (a.Cg / 8);
        dim3 grid(blocks_for(per_g), (unsigned)a.G, (unsigned)a.splits);
        switch (dtype) {
        case CONV2D_DTYPE_F16: direct_wgrad_tiled<EF16><<<grid, 256, 0, st>>>(a); break;
        case CONV2D_DTYPE_BF16: direct_wgrad_tiled<EBF16><<<grid, 256, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    dim3 grid(blocks_for(a.total), (unsigned)a.splits);
    switch (dtype) {
    case CONV2D_DTYPE_F16: direct_wgrad_kernel<EF16><<<grid, 256, 0, st>>>(a); break;
    case CONV2D_DTYPE_BF16: direct_wgrad_kernel<EBF16><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cnv

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

hipError_t launch_direct_fprop(int dtype, const DirectArgs &a, hipStream_t st)
{
    if (a.total == 0) return hipSuccess;
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

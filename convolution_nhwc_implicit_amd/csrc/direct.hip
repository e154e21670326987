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
        ((elem *)a.out)[idx] = E::from_f32(bias_relu_f32(acc, b, a.relu));
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
    ((elem *)a.out)[idx] = E::from_f32(acc);
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
    if (a.splits == 1)
        ((elem *)a.out)[idx] = E::from_f32(acc);
    else
        ((float *)a.out)[(size_t)z * a.part_stride + idx] = acc;
}

static unsigned blocks_for(long long total) { return (unsigned)((total + 255) / 256); }

hipError_t launch_direct_fprop(int dtype, const DirectArgs &a, hipStream_t st)
{
    if (a.total == 0) return hipSuccess;
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
    dim3 grid(blocks_for(a.total), (unsigned)a.splits);
    switch (dtype) {
    case CONV2D_DTYPE_F16: direct_wgrad_kernel<EF16><<<grid, 256, 0, st>>>(a); break;
    case CONV2D_DTYPE_BF16: direct_wgrad_kernel<EBF16><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cnv

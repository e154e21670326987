// pointwise_wgrad.hip -- weight gradient of a 1x1 stride-1 convolution as one
// streaming pass over dy and x (gfx950).
//
// With a 1x1 filter, stride 1 and no padding, dw[k][c] = sum over all pixels
// p of dy[p][k] * x[p][c]: a GEMM with rows k, columns c and a reduction over
// the N*H*W pixels (the tensorcore "Conv2D" page's note that a 1x1
// convolution is a plain GEMM).  When K and C are 64, 128 or 256 with K*C at
// most 16384, the whole K x C result fits in the MFMA accumulators of one
// workgroup.  So each workgroup takes one contiguous slice of pixels, reads
// its dy and x rows exactly once (contiguous bytes, direct-to-LDS), and writes
// one fp32 partial of dw; the split-K reduction adds the partials in slice
// order and applies the epilogue.  The pass is then as close to a plain copy
// of dy and x as the partials allow.
//
//   * 4 waves.  Wave w holds a 64 x 64 piece of the tile (2 x 2 blocks of
//     32x32x16 MFMA accumulators): rows 64*(w % WK), columns
//     64*((w / WK) % WC), and the 16-pixel steps t = w / (WK*WC) (mod PH),
//     where WK = K/64, WC = C/64 and PH = 4 / (WK*WC).  With PH > 1 the
//     phases' sums are added in phase order through LDS at the end.
//   * Groups of 64 pixels arrive in a ring of LDS buffers (3 for the 256 x 64
//     tile, up to 8 for smaller ones): all but one of them are in flight
//     while a group is computed, and only loads are ever waited for.  Pixels
//     past the slice read as zeros (buffer range check).
//   * MFMA operands need 8 consecutive pixels of one channel per lane;
//     ds_read_b64_tr_b16 gives them from the pixel-major rows (in each group
//     of 16 lanes, lane L points at 4 channels of pixel L/4 and lane i
//     receives channel i of the 4 pixels).  The 16-byte chunks of each pixel
//     are XOR-swizzled by the pixel so that the 4 pixels of one read fall on
//     different LDS banks.
//   * With the bias gradient, the waves of the first column set also add up
//     the dy values of their fragments (every dy value of the slice once) and
//     the slice carries K more floats.
#include "device_common.h"

namespace cnv {

namespace pwwk {
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
constexpr int NT = 256;
constexpr int GP = 64;    // pixels per group
constexpr int LDS_MAX = 163840;
// ring of group buffers: about 96 KB of them, at least 3 and at most 8 (a
// deeper ring measured no faster on the 256 x 64 tile)
constexpr int nbuf(int bufb) { return 98304 / bufb < 3 ? 3 : 98304 / bufb > 8 ? 8 : 98304 / bufb; }

// stored slot of 16-byte chunk j of pixel v in rows of ROWB bytes.  A
// transposing read covers 32 bytes of 4 consecutive pixels: 128-byte rows
// flip chunk bit 2 when bit 1 of v is set (the pixels then sit 32, 16 and 48
// banks apart); rows of 256 bytes or more (a multiple of the 64 banks) move
// the 32-byte pair by v mod 4.
template <int ROWB>
__device__ inline int swz(int j, int v)
{
    static_assert(ROWB == 128 || ROWB == 256 || ROWB == 512, "64, 128 or 256 channels");
    if constexpr (ROWB == 128) return j ^ (((v >> 1) & 1) << 2);
    return j ^ ((v & 3) << 1);
}

template <class E>
struct Mfma32;
template <>
struct Mfma32<EF16> {
    __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <>
struct Mfma32<EBF16> {
    __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
// s_waitcnt vmcnt(younger * PER) for younger in 0 .. M (a compile-time count)
template <int PER, int M>
__device__ __attribute__((always_inline)) inline void wait_younger(int younger)
{
    if constexpr (M == 0) {
        wait_vm_all();
    } else {
        if (younger == M)
            wait_vm_n<M * PER>();
        else
            wait_younger<PER, M - 1>(younger);
    }
}
}  // namespace pwwk

template <class E, int WK, int WC, bool DB>
__global__ __launch_bounds__(pwwk::NT) void pointwise_wgrad_kernel(const PwWgradArgs a)
{
    using namespace pwwk;
    constexpr int K = 64 * WK, C = 64 * WC, PH = 4 / (WK * WC);
    static_assert(WK * WC * PH == 4, "four waves");
    constexpr int DROWB = 2 * K, XROWB = 2 * C;          // bytes of a dy / x pixel
    constexpr int DBYTES = GP * DROWB, XBYTES = GP * XROWB;
    constexpr int BUFB = DBYTES + XBYTES;
    constexpr int NBUF = nbuf(BUFB);
    constexpr int DBLK = DBYTES / 1024, XBLK = XBYTES / 1024;  // 1 KB direct-to-LDS blocks
    constexpr int PER = (DBLK + XBLK) / 4;                // blocks per wave and group
    constexpr int TSTEPS = GP / 16 / PH;                  // steps per wave and group
    constexpr int ACCB = 4 * 64 * 64;                     // one wave's 4 blocks, bytes
    static_assert((DBLK + XBLK) % 4 == 0, "whole blocks per wave");
    static_assert(NBUF >= 3 && NBUF * BUFB <= LDS_MAX && (PH - 1) * 4 / PH * ACCB <= NBUF * BUFB, "LDS");
    static_assert((NBUF - 2) * PER < 64, "vmcnt range");
    __shared__ __attribute__((aligned(16))) unsigned char smem[NBUF * BUFB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = wave % WK, wc = (wave / WK) % WC, phase = wave / (WK * WC);

    const uint32_t p0 = (uint32_t)blockIdx.x * (uint32_t)a.pix_per_split;
    const uint32_t np = p0 < a.npix ? min((uint32_t)a.pix_per_split, a.npix - p0) : 0u;
    const int ngroups = (int)((np + GP - 1) / GP);
    const u32x4 d_rs = make_buf_rsrc((const unsigned char *)a.dy + (size_t)p0 * DROWB, np * DROWB);
    const u32x4 x_rs = make_buf_rsrc((const unsigned char *)a.x + (size_t)p0 * XROWB, np * XROWB);
    const uint32_t lds0 = lds_addr(smem);

    // block b of group g: lane i fills stored slot s of pixel v (the bytes
    // 1024*b + 16*i of the group's rows) with source chunk swz(s, v)
    auto dma_group = [&](int g) __attribute__((always_inline)) {
        if (g >= ngroups) return;
        const uint32_t buf = lds0 + (uint32_t)((g % NBUF) * BUFB);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int b = wave + 4 * j;
            if (b < DBLK) {
                const int off = 1024 * b + 16 * lane, v = off / DROWB, s = (off % DROWB) / 16;
                dma16(d_rs, buf + 1024 * b, (uint32_t)((g * GP + v) * DROWB + swz<DROWB>(s, v) * 16));
            } else {
                const int bx = b - DBLK;
                const int off = 1024 * bx + 16 * lane, v = off / XROWB, s = (off % XROWB) / 16;
                dma16(x_rs, buf + DBYTES + 1024 * bx, (uint32_t)((g * GP + v) * XROWB + swz<XROWB>(s, v) * 16));
            }
        }
    };

    // fragment reads: lane points at pixel 16*t + 8*(lane/32) + (L/4) (+4 for
    // the second read), channels base + 16*((lane/16)&1) + 4*(L%4), L = lane%16
    const int L = lane & 15, lhi = lane >> 5;
    const int pv = 8 * lhi + (L >> 2);
    const int cl = 16 * ((lane >> 4) & 1) + 4 * (L & 3);
    typedef __attribute__((address_space(3))) unsigned char lds_u8;
    int dofs[2], xofs[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int kc = 64 * wk + 32 * i + cl, xc = 64 * wc + 32 * i + cl;
        dofs[i] = pv * DROWB + swz<DROWB>(kc >> 3, pv) * 16 + (kc & 7) * 2;
        xofs[i] = DBYTES + pv * XROWB + swz<XROWB>(xc >> 3, pv) * 16 + (xc & 7) * 2;
    }
    auto tr = [](const unsigned char *p) -> uint2 {
        return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                             (__attribute__((address_space(3))) s16x4 *)(lds_u8 *)p));
    };
    auto frag = [&](const unsigned char *p, int rowb) -> u32x4 {
        const uint2 lo = tr(p), hi = tr(p + 4 * rowb);
        return u32x4{lo.x, lo.y, hi.x, hi.y};
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    float dbacc[2] = {0.0f, 0.0f};

    for (int g = 0; g < NBUF - 1; ++g) dma_group(g);
    for (int g = 0; g < ngroups; ++g) {
        // group g has landed when only this wave's loads of the younger
        // groups in flight remain
        const int younger = min(NBUF - 2, ngroups - 1 - g);
        wait_younger<PER, NBUF - 2>(younger);
        __syncthreads();  // every wave's loads of group g are visible; group g - 1 is consumed
        dma_group(g + NBUF - 1);
        const unsigned char *base = smem + (g % NBUF) * BUFB;
#pragma unroll
        for (int j = 0; j < TSTEPS; ++j) {
            const int t = phase + PH * j;
            u32x4 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                fa[i] = frag(base + dofs[i] + t * 16 * DROWB, DROWB);
                fb[i] = frag(base + xofs[i] + t * 16 * XROWB, XROWB);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) acc[i][jj] = Mfma32<E>::run(fa[i], fb[jj], acc[i][jj]);
            if constexpr (DB) {
                if (wc == 0) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int e = 0; e < 4; ++e) dbacc[i] = DotOne<E>::add(fa[i][e], dbacc[i]);
                }
            }
        }
    }

    // ---- phase sums in phase order (PH > 1): phases 1 .. PH-1 park their
    // blocks, phase 0 adds them.  A parked block is [4][64 lanes] of 16-byte
    // pieces; the wave's four blocks follow each other.
    __syncthreads();  // every wave is done with the ring
    f32x4 *const lds4 = (f32x4 *)smem + lane;
    if constexpr (PH > 1) {
        auto slot = [&](int ph) { return lds4 + ((ph - 1) * (WK * WC) + wk + WK * wc) * (ACCB / 16); };
        if (phase > 0) {
            f32x4 *p = slot(phase);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x16 &v = acc[i][jj];
                        p[((2 * i + jj) * 4 + q) * 64] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
                    }
        }
        __syncthreads();
        if (phase == 0) {
            for (int ph = 1; ph < PH; ++ph) {
                const f32x4 *p = slot(ph);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const f32x4 u = p[((2 * i + jj) * 4 + q) * 64];
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[i][jj][4 * q + e] += u[e];
                        }
            }
        }
    }
    float *const out = (float *)a.out + (size_t)blockIdx.x * a.part_stride;
    if (phase == 0) {
        // lane holds column 32*jj + lane%32 of a block, rows 8*(r/4) +
        // 4*(lane/32) + r%4
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int k = 64 * wk + 32 * i + 8 * (r >> 2) + 4 * lhi + (r & 3);
                    const int c = 64 * wc + 32 * jj + (lane & 31);
                    __builtin_nontemporal_store(acc[i][jj][r], &out[(size_t)k * C + c]);
                }
    }
    if constexpr (DB) {
        // lanes l and l + 32 hold the two pixel halves of channel l%32; the
        // phases' sums are added in phase order
        float *dbs = (float *)smem;  // [PH][K]
        __syncthreads();             // every wave is done with the parked blocks
        if (wc == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float v = dbacc[i] + __shfl_xor(dbacc[i], 32);
                if (lane < 32) dbs[phase * K + 64 * wk + 32 * i + lane] = v;
            }
        }
        __syncthreads();
        for (int k = tid; k < K; k += NT) {
            float s = dbs[k];
            for (int ph = 1; ph < PH; ++ph) s += dbs[ph * K + k];
            out[(size_t)K * C + k] = s;
        }
    }
}

bool pointwise_wgrad_supported(int dtype, int K, int C)
{
    if (dtype != CONV2D_DTYPE_F16 && dtype != CONV2D_DTYPE_BF16) return false;
    auto ok = [](int n) { return n == 64 || n == 128 || n == 256; };
    return ok(K) && ok(C) && K * C <= 16384;
}

template <class E, bool DB>
static hipError_t launch_pw_wgrad_e(const PwWgradArgs &a, hipStream_t st)
{
    const dim3 grid((unsigned)a.splits);
    const int wk = a.K / 64, wc = a.C / 64;
#define PWW_CASE(A, B)                                                                  \
    if (wk == A && wc == B) {                                                           \
        pointwise_wgrad_kernel<E, A, B, DB><<<grid, pwwk::NT, 0, st>>>(a);              \
        return hipGetLastError();                                                       \
    }
    PWW_CASE(1, 1)
    PWW_CASE(1, 2)
    PWW_CASE(2, 1)
    PWW_CASE(1, 4)
    PWW_CASE(2, 2)
    PWW_CASE(4, 1)
#undef PWW_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_pointwise_wgrad(int dtype, const PwWgradArgs &a, hipStream_t st)
{
    if (!pointwise_wgrad_supported(dtype, a.K, a.C) || a.splits < 1 || a.pix_per_split % pwwk::GP != 0)
        return hipErrorInvalidValue;
    switch (dtype) {
    case CONV2D_DTYPE_F16:
        return a.with_db ? launch_pw_wgrad_e<EF16, true>(a, st) : launch_pw_wgrad_e<EF16, false>(a, st);
    case CONV2D_DTYPE_BF16:
        return a.with_db ? launch_pw_wgrad_e<EBF16, true>(a, st) : launch_pw_wgrad_e<EBF16, false>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace cnv

// pointwise.hip -- 1x1 stride-1 convolution (fprop, and dgrad with the
// filter read transposed) as a streaming GEMM for gfx950.
//
// A 1x1 stride-1 convolution with no padding is one GEMM over the pixels:
// y[p][n] = sum over k of x[p][k] * w[n][k] (fprop), dx[p][c] = sum over k of
// dy[p][k] * w[k][c] (dgrad) -- the tensorcore "Conv2D" page's note that a
// 1x1 convolution degenerates to a plain GEMM.  With GEMM-K of 64 to 256 its
// arithmetic intensity is far below the ridge, so the work is moving pixels:
// the kernel reads each source pixel once and writes each output pixel once,
// as whole contiguous rows.
//
//   * A workgroup (4 waves) owns PWG consecutive pixels and NWG output
//     channels.  Its filter slice (NWG x GK, 32 KB at most) is read into
//     registers once: wave w holds channels [w*NWG/4, (w+1)*NWG/4) as the
//     A operand of 16x16x32 MFMAs (fprop: rows of w as they lie; dgrad: w
//     is [K][C], read with the transposing LDS read ds_read_b64_tr_b16).
//   * The workgroup's pixels arrive at the start by direct-to-LDS loads,
//     all of them, so no wait ever covers a store.  Then 64 pixels at a
//     time: MFMAs (the pixels are the B operand, 16-byte LDS reads), bias,
//     ReLU and rounding, the 64 x NWG outputs staged in LDS, and 16-byte
//     nontemporal stores of the contiguous output rows.
//   * 16-byte chunks of every LDS row are XOR-swizzled by the row so that
//     the fragment reads and the staging writes of 16 rows at one column
//     fall on different banks.
#include "device_common.h"

namespace cnv {

namespace pwk {
constexpr int NT = 256;
constexpr int TP = 64;  // pixels per sub-tile
// stored chunk of chunk j in row `row` of a tile with CHR 16-byte chunks per
// row: j ^ rswz(row)
template <int CHR>
__device__ inline int rswz(int row)
{
    static_assert(CHR == 8 || CHR == 16 || CHR == 32, "rows of 128, 256 or 512 bytes");
    if constexpr (CHR == 8) return (row >> 1) & 7;
    return row & 15;
}
// the transposed filter staging (dgrad, rows = k): rows r, r+1, r+2, r+3 and
// r+8 .. r+11 (one transposing read of 32 lanes) on different banks
template <int CHR>
__device__ inline int tswz(int row)
{
    const int b3 = ((row >> 3) & 1) << 1;
    if constexpr (CHR == 8) return (((row >> 1) & 1) << 2) | b3;
    return ((row & 3) << 2) | b3;
}
template <int GK>
struct Cfg {
    static constexpr int PWG = GK == 64 ? 256 : GK == 128 ? 128 : 64;  // pixels per workgroup
};
}  // namespace pwk

template <class E, int GK, int NWG, bool TRANS, bool RELU>
__global__ __launch_bounds__(pwk::NT) void pointwise_kernel(const PwArgs a)
{
    using namespace pwk;
    using elem = typename E::elem;
    using acc_t = typename E::acc;
    constexpr int NW = NWG / 4;    // output channels per wave
    constexpr int NB = NW / 16;    // 16-channel blocks per wave
    constexpr int KS = GK / 32;    // k32 steps
    constexpr int ROWB = GK * 2;   // bytes of a source pixel
    constexpr int XCH = GK / 8;    // chunks of a source pixel
    constexpr int OCH = NWG / 8;   // chunks of a staged output pixel
    constexpr int PWG = Cfg<GK>::PWG;
    constexpr int XB = PWG * ROWB;
    constexpr int FB = NWG * GK * 2;
    constexpr int OB = TP * NWG * 2;
    constexpr int SB = FB > OB ? FB : OB;
    static_assert(NB >= 1 && NW % 16 == 0 && FB <= 32768, "16-channel blocks; the filter slice fits 32 KB");
    static_assert(XB % 1024 == 0 && FB % 1024 == 0, "whole 1 KB direct-to-LDS blocks");
    __shared__ __attribute__((aligned(16))) unsigned char smem[XB + SB];
    unsigned char *xs = smem;       // the workgroup's source pixels
    unsigned char *fs = smem + XB;  // the filter slice, then the output staging

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p0 = blockIdx.x * PWG;
    const int np = min(PWG, a.npix - p0);  // >= 1
    const int n0 = blockIdx.y * NWG;

    // ---- loads: the source pixels, then the filter slice
    {
        const u32x4 x_rs = make_buf_rsrc(a.src, (uint32_t)a.src_bytes);
        for (int b = wave; b * 1024 < XB; b += 4) {
            const int o = b * 1024 + lane * 16;
            const int q = o / ROWB, j = ((o - q * ROWB) >> 4) ^ rswz<XCH>(q);
            dma16(x_rs, lds_addr(xs + b * 1024),
                  q < np ? (uint32_t)((size_t)(p0 + q) * ROWB + j * 16) : kBufOOBFar);
        }
        const u32x4 w_rs = make_buf_rsrc(a.w, (uint32_t)a.w_bytes);
        for (int b = wave; b * 1024 < FB; b += 4) {
            const int o = b * 1024 + lane * 16;
            uint32_t voff;
            if constexpr (!TRANS) {
                // row n (output channel n0 + n), GK elements as in w[n][k]
                const int n = o / ROWB, j = ((o - n * ROWB) >> 4) ^ rswz<XCH>(n);
                voff = (uint32_t)(((size_t)(n0 + n) * GK + j * 8) * 2);
            } else {
                // row k (dy channel), NWG dx channels of w[k][c]
                const int k = o / (NWG * 2), j = ((o - k * NWG * 2) >> 4) ^ tswz<OCH>(k);
                voff = (uint32_t)(((size_t)k * a.nout + n0 + j * 8) * 2);
            }
            dma16(w_rs, lds_addr(fs + b * 1024), voff);
        }
    }
    // the bias of the lane's output channels (fprop)
    float bias_v[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n0 + wave * NW + nb * 16 + 4 * (lane >> 4) + i;
            bias_v[nb][i] = a.bias ? E::to_f32(((const elem *)a.bias)[n]) : 0.0f;
        }
    wait_vm_all();
    __syncthreads();  // pixels and filter in LDS

    // ---- the wave's filter fragments: A = 16 channels x 32 k; lane holds
    // channel (lane & 15) of the block, k = 32*ks + 8*(lane >> 4) + 0..7
    u32x4 fa[NB][KS];
    if constexpr (!TRANS) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = wave * NW + nb * 16 + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                fa[nb][ks] = *(const u32x4 *)(fs + n * ROWB + (((4 * ks + (lane >> 4)) ^ rswz<XCH>(n)) << 4));
        }
    } else {
        // ds_read_b64_tr_b16: in each group of 16 lanes, lane L points at
        // row L/4, columns 4*(L%4)..+3 of a 4 x 16 tile (rows k, columns dx
        // channels) and receives column L of the 4 rows
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        const int L = lane & 15;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                uint2 h[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int k = 32 * ks + 8 * (lane >> 4) + 4 * t + (L >> 2);
                    const int chunk = (wave * NW + nb * 16) / 8 + ((L & 3) >> 1);
                    h[t] = __builtin_bit_cast(
                        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                   (__attribute__((address_space(3))) s16x4 *)(fs + k * NWG * 2 +
                                                                                ((chunk ^ tswz<OCH>(k)) << 4) +
                                                                                (L & 1) * 8)));
                }
                fa[nb][ks] = u32x4{h[0].x, h[0].y, h[1].x, h[1].y};
            }
    }
    __syncthreads();  // the filter slice becomes the output staging

    elem *dst = (elem *)a.dst;
    for (int s0 = 0; s0 < np; s0 += TP) {
        // MFMAs: pixels (B operand) of 16-pixel block pb: lane holds pixel
        // (lane & 15), k = 32*ks + 8*(lane >> 4) + 0..7
        acc_t acc[TP / 16][NB];
#pragma unroll
        for (int pb = 0; pb < TP / 16; ++pb) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[pb][nb] = acc_t{bias_v[nb][0], bias_v[nb][1], bias_v[nb][2], bias_v[nb][3]};
            const int q = s0 + pb * 16 + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 bx = *(const u32x4 *)(xs + q * ROWB + (((4 * ks + (lane >> 4)) ^ rswz<XCH>(q)) << 4));
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[pb][nb] = E::mfma(fa[nb][ks], bx, acc[pb][nb]);
            }
        }
        // epilogue: lane holds channels 4*(lane >> 4) + 0..3 of block nb for
        // pixel pb*16 + (lane & 15): 8 bytes, half (lane >> 4) & 1 of a chunk
#pragma unroll
        for (int pb = 0; pb < TP / 16; ++pb) {
            const int q = pb * 16 + (lane & 15);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int c = wave * NW + nb * 16 + 4 * (lane >> 4);
                const uint32_t lo = out_pair<E, RELU>(acc[pb][nb][0], acc[pb][nb][1]);
                const uint32_t hi = out_pair<E, RELU>(acc[pb][nb][2], acc[pb][nb][3]);
                *(uint2 *)(fs + q * NWG * 2 + (((c >> 3) ^ rswz<OCH>(q)) << 4) + (c & 4) * 2) = uint2{lo, hi};
            }
        }
        __syncthreads();  // the sub-tile is staged
        // the sub-tile's output rows: TP pixels x NWG channels, 16 bytes a thread
#pragma unroll
        for (int i = 0; i < TP * OCH / NT; ++i) {
            const int id = tid + i * NT;
            const int q = id / OCH, j = id - q * OCH;
            const u32x4 v = *(const u32x4 *)(fs + q * NWG * 2 + ((j ^ rswz<OCH>(q)) << 4));
            if (s0 + q < np)
                __builtin_nontemporal_store(v, (u32x4 *)(dst + (size_t)(p0 + s0 + q) * a.nout + n0 + j * 8));
        }
        __syncthreads();  // the staging is free for the next sub-tile
    }
}

bool pointwise_supported(int dtype, int gk, int nout)
{
    if (dtype != CONV2D_DTYPE_F16 && dtype != CONV2D_DTYPE_BF16) return false;
    if (gk != 64 && gk != 128 && gk != 256) return false;
    const int nwg = pointwise_nwg(gk, nout);
    return nwg > 0;
}

int pointwise_nwg(int gk, int nout)
{
    // output channels per workgroup: a multiple of 64 dividing nout, the
    // filter slice within 32 KB
    for (int nwg : {256, 128, 64})
        if (nout % nwg == 0 && nwg * gk <= 16384) return nwg;
    return 0;
}

int pointwise_pixels_per_wg(int gk) { return gk == 64 ? 256 : gk == 128 ? 128 : 64; }

template <class E, int GK, bool TRANS, bool RELU>
static hipError_t launch_gk(const PwArgs &a, int nwg, hipStream_t st)
{
    const dim3 grid((unsigned)((a.npix + pwk::Cfg<GK>::PWG - 1) / pwk::Cfg<GK>::PWG), (unsigned)(a.nout / nwg));
    switch (nwg) {
    case 64: pointwise_kernel<E, GK, 64, TRANS, RELU><<<grid, pwk::NT, 0, st>>>(a); break;
    case 128:
        if constexpr (GK <= 128) {
            pointwise_kernel<E, GK, 128, TRANS, RELU><<<grid, pwk::NT, 0, st>>>(a);
            break;
        }
        return hipErrorInvalidValue;
    case 256:
        if constexpr (GK == 64) {
            pointwise_kernel<E, GK, 256, TRANS, RELU><<<grid, pwk::NT, 0, st>>>(a);
            break;
        }
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class E, bool TRANS, bool RELU>
static hipError_t launch_e(const PwArgs &a, hipStream_t st)
{
    const int nwg = pointwise_nwg(a.gk, a.nout);
    switch (a.gk) {
    case 64: return launch_gk<E, 64, TRANS, RELU>(a, nwg, st);
    case 128: return launch_gk<E, 128, TRANS, RELU>(a, nwg, st);
    case 256: return launch_gk<E, 256, TRANS, RELU>(a, nwg, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_pointwise(int dtype, const PwArgs &a, hipStream_t st)
{
    if (!pointwise_supported(dtype, a.gk, a.nout) || a.npix <= 0) return hipErrorInvalidValue;
    if (dtype == CONV2D_DTYPE_F16) {
        if (a.trans) return launch_e<EF16, true, false>(a, st);
        return a.relu ? launch_e<EF16, false, true>(a, st) : launch_e<EF16, false, false>(a, st);
    }
    if (a.trans) return launch_e<EBF16, true, false>(a, st);
    return a.relu ? launch_e<EBF16, false, true>(a, st) : launch_e<EBF16, false, false>(a, st);
}

}  // namespace cnv

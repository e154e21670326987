// fewchan.hip -- forward convolution of inputs with few channels (C not a
// multiple of 8: the 3-channel RGB stem of the tensorcore "Conv2D" page's
// 224 -> 112 example), without padding the channels.
//
// The GEMM view (tensorcore page, "Conv2D vs GEMM tradeoffs"; CUTLASS
// notebook, "Iterator Algorithm", few/fixed channels) has rows = output
// channels, columns = output pixels and a reduction over (r, s, c).  With C
// this small an output pixel's patch is short and, within one filter row r,
// contiguous in the NHWC input row: taps s = 0..S-1 of pixel q cover the S*C
// elements from ((q*sw - pw)*C) on.  So the reduction is laid out per filter
// row as a window of Lw elements (a multiple of 8) that starts delta elements
// before that run, and a pixel's 8-element operand chunk is one 16-byte read
// of the input row as it sits in LDS: no im2col, no zero channels.  The filter
// is read in the same layout (zero where a window position is not one of the
// row's S*C taps), so window positions outside the run multiply zeros.
// delta (0 or 1) keeps every chunk 4-byte aligned in LDS, which needs
// stride_w*C even.
//
// A workgroup (4 waves) owns a band of output rows of one image:
//   * the input rows the band reads arrive by direct-to-LDS loads into one
//     contiguous buffer of padded rows, and the left/right padding and rows
//     outside the image come from the buffer range check as zeros;
//   * the filter is loaded into LDS as it is and read into VGPRs in the
//     window layout (the A operand, one or two blocks of 32 output channels);
//   * the band's pixels, numbered row by row, are cut into blocks of 32 (the
//     B operand columns of one 32x32x16 MFMA); wave w takes blocks w, w+4, ...
//     Each block adds bias, applies ReLU, rounds, and is staged in LDS so
//     that its 32 output pixels -- contiguous in y -- leave as 16-byte
//     stores.
#include "device_common.h"

namespace cnv {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace fc {
constexpr int NT = 256;
constexpr int WAVES = NT / 64;

template <class E>
__device__ inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ inline f32x16 mfma32<EF16>(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                   0, 0, 0);
}
template <>
__device__ inline f32x16 mfma32<EBF16>(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                    c, 0, 0, 0);
}
}  // namespace fc

// KB blocks of 32 output channels (K = 32*KB); NST 16-element reduction
// steps (2*NST chunks of 8 >= R*Lw/8; chunks past R*Lw have a zero filter).
template <class E, int KB, int NST>
__global__ __launch_bounds__(fc::NT) void fewchan_fprop_kernel(const FewArgs a)
{
    using elem = typename E::elem;
    constexpr int K = 32 * KB;
    constexpr int OPITCH = K * 2 + 16;    // staged output pixel (bytes)
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char *rows = smem;                             // a.buf_bytes
    unsigned char *stage = smem + a.buf_bytes;              // the filter, then output staging
    unsigned char *bias_raw = smem + a.buf_bytes + a.stage_bytes;  // 1 KB: the bias, then zeros

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int img = blockIdx.x / a.bands;
    const int band = blockIdx.x - img * a.bands;
    const int p0 = band * a.rows_per_wg;
    const int rows_out = min(a.rows_per_wg, a.P - p0);
    const int npix = rows_out * a.Q;
    const int h0 = p0 * a.sh - a.pad_h;  // input row of buffer row 0

    // ---- direct-to-LDS loads, in the order they are needed: the filter as it
    // is ([K][R][S*C], K*R*S*C a multiple of 8 elements) into the staging
    // area, the bias (raw elements; zeros without one), then the input rows.
    // Input row chunk u of the buffer is row u / cpr, element (u % cpr)*8 -
    // left of that row; everything outside the image reads zero.
    const int fchunks = K * a.R * a.SC / 8;
    int nrow_ops = 0;  // this wave's row loads, issued last
    {
        const u32x4 wr = make_buf_rsrc(a.w, (uint32_t)fchunks * 16u);
        const uint32_t st_lds = lds_addr(stage);
        for (int blk = wave; blk * 64 < fchunks; blk += fc::WAVES) {
            const int u = blk * 64 + lane;
            dma16(wr, st_lds + (uint32_t)(blk * 1024), u < fchunks ? (uint32_t)u * 16u : kBufOOB);
        }
        if (wave == 0) {
            // whole 16-byte chunks from the boundary at or below the bias (the
            // range check zeroes a chunk that is partly out of range; a chunk
            // never crosses a page)
            const uint32_t bshift = (uint32_t)((uintptr_t)a.bias & 15u);
            const u32x4 br = make_buf_rsrc((const unsigned char *)a.bias - bshift,
                                           a.bias ? (bshift + (uint32_t)(K * sizeof(elem)) + 15u) & ~15u : 0u);
            dma16(br, lds_addr(bias_raw), (uint32_t)lane * 16u);
        }
        const u32x4 xr = make_buf_rsrc(a.x, a.x_bytes);
        const uint32_t rows_lds = lds_addr(rows);
        const int nblk = a.buf_bytes >> 10;
        for (int blk = wave; blk < nblk; blk += fc::WAVES) {
            const uint32_t u = (uint32_t)(blk * 64 + lane);
            const uint32_t rr = fdiv(u, a.div_cpr);
            const int e0 = (int)(u - rr * (uint32_t)a.cpr) * 8 - a.left;
            const int h = h0 + (int)rr;
            const bool in = (int)rr < a.nrows && (unsigned)h < (unsigned)a.H && e0 >= 0 && e0 < a.WC;
            dma16(xr, rows_lds + (uint32_t)(blk * 1024),
                  in ? ((uint32_t)(img * a.H + h) * (uint32_t)a.WC + (uint32_t)e0) * 2u : kBufOOBFar);
            ++nrow_ops;
        }
    }
    // loads complete in issue order: with only the row loads outstanding,
    // this wave's share of the filter and the bias has landed
    switch (nrow_ops) {
    case 0: wait_vm_all(); break;
    case 1: wait_vm_n<1>(); break;
    case 2: wait_vm_n<2>(); break;
    case 3: wait_vm_n<3>(); break;
    case 4: wait_vm_n<4>(); break;
    case 5: wait_vm_n<5>(); break;
    case 6: wait_vm_n<6>(); break;
    case 7: wait_vm_n<7>(); break;
    case 8: wait_vm_n<8>(); break;
    case 9: wait_vm_n<9>(); break;
    case 10: wait_vm_n<10>(); break;
    case 11: wait_vm_n<11>(); break;
    case 12: wait_vm_n<12>(); break;
    case 13: wait_vm_n<13>(); break;
    case 14: wait_vm_n<14>(); break;
    case 15: wait_vm_n<15>(); break;
    default: wait_vm_all(); break;
    }
    __syncthreads();  // the filter and bias visible to every wave; the rows still on their way

    // ---- A operand: output channel m = 32*mb + l32, chunk 2*j + lhi of the
    // reduction (lane holds k = 8*lhi + 0..7 of step j): the 8 consecutive
    // filter elements of row m from a.step[j].fbase[lhi], with the halves
    // outside the filter row's S*C taps masked to zero (reads past the
    // filter stay inside the staging area, which has room past it).  B
    // operand chunks sit a.step[j].coff[lhi] bytes from a pixel's window.
    const int l32 = lane & 31, lhi = lane >> 5;
    u32x4 fa[KB][NST];
    uint32_t coff[NST];
    {
        const int RSC = a.R * a.SC;
#pragma unroll
        for (int j = 0; j < NST; ++j) {
            const FewStep &st = a.step[j];
            const int base = lhi ? st.fbase[1] : st.fbase[0];
            coff[j] = lhi ? st.coff[1] : st.coff[0];
            uint32_t mk[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) mk[p] = lhi ? st.mask[1][p] : st.mask[0][p];
#pragma unroll
            for (int mb = 0; mb < KB; ++mb) {
                // 16 bytes at a 2-byte aligned offset: five aligned dwords,
                // shifted into place
                const uint32_t off = (uint32_t)((32 * mb + l32) * RSC + base) * 2u;
                const uint32_t *d4 = (const uint32_t *)(stage + (off & ~3u));
                const uint32_t sh = (off & 2u) * 8u;
                uint32_t d[5];
#pragma unroll
                for (int i = 0; i < 5; ++i) d[i] = d4[i];
                uint32_t v[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) v[p] = __builtin_amdgcn_alignbit(d[p + 1], d[p], sh) & mk[p];
                fa[mb][j] = u32x4{v[0], v[1], v[2], v[3]};
            }
        }
    }
    // the bias in the accumulator layout: channels 32*mb + 8*g + 4*lhi + 0..3
    f32x4 bv[KB][4];
#pragma unroll
    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const elem *bp = (const elem *)(bias_raw + ((uintptr_t)a.bias & 15u)) + 32 * mb + 8 * g + 4 * lhi;
            bv[mb][g] = f32x4{E::to_f32(bp[0]), E::to_f32(bp[1]), E::to_f32(bp[2]), E::to_f32(bp[3])};
        }
    wait_vm_all();    // this wave's row loads
    __syncthreads();  // the rows visible to every wave; the filter staging is free for the outputs

    unsigned char *ost = stage + wave * 32 * OPITCH;
    const int nblocks = (npix + 31) >> 5;
    elem *ybase = (elem *)a.y + ((size_t)img * a.P + p0) * a.Q * K;
    for (int blk = wave; blk < nblocks; blk += fc::WAVES) {
        const int v = min(blk * 32 + l32, npix - 1);
        const int pl = (int)fdiv((uint32_t)v, a.div_q);
        const int q = v - pl * a.Q;
        // window start of pixel (pl, q) in buffer row pl*sh: element
        // left + (q*sw - pw)*C - delta, 4-byte aligned
        const unsigned char *pb = rows + pl * a.sh * a.pitch + (a.win0 + q * a.qstep) * 2;
        // all of the block's pixel chunks first (2-dword reads: the chunks
        // are 4-byte aligned), then the MFMAs
        u32x4 bf[NST];
#pragma unroll
        for (int j = 0; j < NST; ++j) {
            const uint32_t *p = (const uint32_t *)(pb + coff[j]);
            bf[j] = u32x4{p[0], p[1], p[2], p[3]};
        }
        __builtin_amdgcn_sched_barrier(0);  // every read in flight before the first MFMA
        f32x16 acc[KB];
#pragma unroll
        for (int mb = 0; mb < KB; ++mb) acc[mb] = f32x16{};
#pragma unroll
        for (int j = 0; j < NST; ++j)
#pragma unroll
            for (int mb = 0; mb < KB; ++mb) acc[mb] = fc::mfma32<E>(fa[mb][j], bf[j], acc[mb]);
        // epilogue: lane holds pixel l32, channels 32*mb + 8*g + 4*lhi + 0..3
        // in acc[mb][4*g + 0..3]
#pragma unroll
        for (int mb = 0; mb < KB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = bias_relu_f32(acc[mb][4 * g + i], bv[mb][g][i], a.relu);
                const uint2 pk = {out_pair<E, false>(o[0], o[1]), out_pair<E, false>(o[2], o[3])};
                *(uint2 *)(ost + l32 * OPITCH + (32 * mb + 8 * g + 4 * lhi) * 2) = pk;
            }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's staging writes are done
        __builtin_amdgcn_wave_barrier();
        // 32 pixels x K channels, contiguous in y from pixel blk*32
        const int npx = min(32, npix - blk * 32);
#pragma unroll
        for (int it = 0; it < 32 * K * 2 / 1024; ++it) {
            const int o = it * 1024 + lane * 16;
            const int px = o / (K * 2), off = o - px * (K * 2);
            const u32x4 val = *(const u32x4 *)(ost + px * OPITCH + off);
            if (px < npx)  // streaming stores: y is not read again here
                __builtin_nontemporal_store(val, (u32x4 *)((unsigned char *)(ybase + (size_t)(blk * 32 + px) * K) + off));
        }
        __builtin_amdgcn_wave_barrier();
    }
}

bool fewchan_supported(int dtype, int C, int K, int S, int sw, int dw, int W)
{
    if (dtype != CONV2D_DTYPE_F16 && dtype != CONV2D_DTYPE_BF16) return false;
    if (C % 8 == 0 || dw != 1 || (sw * C) % 2 || (W * C) % 8) return false;
    if (K != 32 && K != 64) return false;
    return true;
}

// Reduction steps (of 16) the kernels are built for.
static int fewchan_nst(int need)
{
    static const int kSteps[] = {4, 8, 11, 12, 16};
    for (int s : kSteps)
        if (s >= need) return s;
    return 0;
}
int fewchan_steps(int R, int lw) { return fewchan_nst((R * lw + 15) / 16); }

template <class E, int KB>
static hipError_t launch_kb(int nst, const FewArgs &a, hipStream_t st)
{
    const dim3 grid((unsigned)(a.N * a.bands)), block(fc::NT);
    const size_t lds = (size_t)a.buf_bytes + a.stage_bytes + 1024;
    switch (nst) {
    case 4: fewchan_fprop_kernel<E, KB, 4><<<grid, block, lds, st>>>(a); break;
    case 8: fewchan_fprop_kernel<E, KB, 8><<<grid, block, lds, st>>>(a); break;
    case 11: fewchan_fprop_kernel<E, KB, 11><<<grid, block, lds, st>>>(a); break;
    case 12: fewchan_fprop_kernel<E, KB, 12><<<grid, block, lds, st>>>(a); break;
    case 16: fewchan_fprop_kernel<E, KB, 16><<<grid, block, lds, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_fewchan_fprop(int dtype, const FewArgs &a, hipStream_t st)
{
    const int nst = fewchan_steps(a.R, a.lw);
    if (a.K == 64)
        return dtype == CONV2D_DTYPE_F16 ? launch_kb<EF16, 2>(nst, a, st) : launch_kb<EBF16, 2>(nst, a, st);
    if (a.K == 32)
        return dtype == CONV2D_DTYPE_F16 ? launch_kb<EF16, 1>(nst, a, st) : launch_kb<EBF16, 1>(nst, a, st);
    return hipErrorInvalidValue;
}

}  // namespace cnv

// fewchan_dgrad.hip -- data gradient of a stride-2 convolution whose input has
// few channels (C <= 4: the 3-channel stem of the tensorcore "Conv2D" page's
// 224 -> 112 example), without padding the channels.
//
// dx[h][w][c] = sum over (k, r, s) of dy[p][q][k] * w[k][r][s][c] with
// h = 2p - ph + r, w = 2q - pw + s.  Output pixel (2i + a, 2j + b) (a, b in
// {0, 1}: its stride phase) reads dy pixel (i + dp, j + dq) through filter tap
// r = a + ph - 2*dp, s = b + pw - 2*dq, and over both phases dp and dq take
// only a few values (four for a 7x7 filter).  So the 2x2 block of output
// pixels (i, j) -- a "super-pixel" -- with its 4*C <= 16 outputs (a, b, c) is
// one row of a GEMM:
//   rows    = super-pixels (16 consecutive j of one i),
//   columns = (a, b, c), 16 (12 used for C = 3),
//   K       = (dp, dq, k): the dy pixels around (i, j), 64 channels each,
// with B[(dp, dq, k)][(a, b, c)] = w[k][a + ph - 2dp][b + pw - 2dq][c] (zero
// where the tap does not exist).  A rows are 16 consecutive dy pixels of one
// dy row, 32 channels at a time: plain 128-bit LDS reads of the NHWC dy rows,
// no transposition; B (at most 32 steps of 16x16x32) is built once per
// workgroup in LDS from the filter and then lives in every wave's VGPRs.  The
// phase decomposition of the pages' col2im picture is folded into B, and
// every dx element is written once, with no atomics.
//
// A workgroup (8 waves) owns a band of super-rows of one image, two at a time:
// a ring of dy rows filled by direct-to-LDS loads (the rows of the next pair
// in flight while a pair is computed; zeros outside the image from the range
// check), blocks of 16 super-pixels dealt to the waves, each block's 2 x 32
// output pixels staged in LDS and written as 16-byte pieces of the two dx
// rows.
#include "device_common.h"

namespace cnv {

namespace fd {
constexpr int NT = 512;
constexpr int WAVES = NT / 64;
constexpr int K = 64;
constexpr int PIXB = K * 2;     // bytes of a dy pixel
constexpr int PF = 4;           // A reads in flight
constexpr int LDS_BYTES = 163840;
__device__ inline int swz(int ps) { return (ps >> 1) & 7; }  // chunk swizzle of pixel slot ps
}  // namespace fd

template <class E, int NDH, int NDW>
__global__ __launch_bounds__(fd::NT) void fewchan_dgrad_kernel(const FewDgradArgs a)
{
    using namespace fd;
    using elem = typename E::elem;
    constexpr int NSTEPS = 2 * NDH * NDW;  // k-steps of 32 (dp, dq, channel) values
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
    unsigned char *ring = smem;                                   // nslot dy rows of rowb bytes
    unsigned char *filt = smem + a.ring_bytes;                    // the filter as it is
    unsigned char *bmat = smem + a.ring_bytes + a.filt_bytes;     // the B fragments, 16 B each
    unsigned char *stage = bmat + NSTEPS * 64 * 16;               // per wave: 2 x 32 x C outputs

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int img = blockIdx.x / a.bands;
    const int band = blockIdx.x - img * a.bands;
    const int i0 = band * a.rows_per_wg;                // first super-row
    const int nsr = min(a.rows_per_wg, a.HS - i0);      // super-rows of the band (>= 1)
    const int niter = (nsr + 1) >> 1;
    const int prow0 = i0 + a.dp_min;                    // dy row of ring index 0
    const int nrel = nsr + NDH - 1;                     // dy rows the band reads

    // ---- loads.  Ring index rel (dy row prow0 + rel) sits in slot rel %
    // nslot; lane i of a 1 KB block fills stored chunk i % 8 of pixel slot
    // ps = 8*blk + i/8 (dy pixel q = ps + dq_min) with source chunk
    // (i % 8) ^ swz(ps).
    const u32x4 d_rs = make_buf_rsrc(a.dy, a.dy_bytes);
    const uint32_t lds0 = lds_addr(smem);
    const int rblk = a.rsl / 8;  // blocks per row
    auto dma_rows = [&](int rel0, int cnt) {
        for (int b = wave; b < cnt * rblk; b += WAVES) {
            const int rel = rel0 + b / rblk, blk = b - (b / rblk) * rblk;
            const int ps = 8 * blk + (lane >> 3);
            const int p = prow0 + rel, q = ps + a.dq_min;
            const int c = (lane & 7) ^ swz(ps);
            const bool in = rel < nrel && (unsigned)p < (unsigned)a.P && (unsigned)q < (unsigned)a.Q;
            dma16(d_rs, lds0 + (uint32_t)((rel % a.nslot) * a.rowb + blk * 1024),
                  in ? (uint32_t)(((img * a.P + p) * a.Q + q) * PIXB + c * 16) : kBufOOBFar);
        }
    };
    {
        const int fchunks = K * a.R * a.S * a.C / 8;
        const u32x4 wr = make_buf_rsrc(a.w, (uint32_t)fchunks * 16u);
        for (int blk = wave; blk * 64 < fchunks; blk += WAVES) {
            const int u = blk * 64 + lane;
            dma16(wr, lds_addr(filt) + (uint32_t)(blk * 1024), u < fchunks ? (uint32_t)u * 16u : kBufOOB);
        }
    }
    dma_rows(0, NDH + 1);  // the first pair's rows
    wait_vm_all();
    __syncthreads();
    if (niter > 1) dma_rows(NDH + 1, 2);

    // ---- B: lane holds column n = lane % 16 = (a, b, c) and K values
    // 8*(lane/16) + 0..7 of each step; step st covers K values [32*st,
    // 32*st + 32) = dy pixel (dp, dq) = pair st/2, channels 32*(st%2) +
    // 0..31.  Every wave holds the same B, so the workgroup builds it once in
    // LDS (fragment (st, lane) at 16*(64*st + lane)) and each wave reads its
    // copy into VGPRs.
    const int n = lane & 15, kq = lane >> 4;
    u32x4 fb[NSTEPS];
    {
        const elem *fs = (const elem *)filt;
        const int RSC = a.R * a.S * a.C;
        for (int f = tid; f < NSTEPS * 64; f += NT) {
            const int st = f >> 6, fl = f & 63;
            const int fn = fl & 15, fk = fl >> 4;
            const int ca = fn / (2 * a.C), cb = (fn / a.C) & 1, cc = fn % a.C;
            const int pair = st >> 1, k0 = 32 * (st & 1) + 8 * fk;
            const int dpi = pair / NDW, dqi = pair % NDW;
            const int r = ca + a.pad_h - 2 * (a.dp_min + dpi), s = cb + a.pad_w - 2 * (a.dq_min + dqi);
            const bool ok = fn < 4 * a.C && (unsigned)r < (unsigned)a.R && (unsigned)s < (unsigned)a.S;
            const int base = ok ? (k0 * a.R + r) * a.S * a.C + s * a.C + cc : 0;
            uint32_t v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = fs[base + (2 * e) * RSC], hi = fs[base + (2 * e + 1) * RSC];
                v[e] = ok ? (lo | hi << 16) : 0u;
            }
            *(u32x4 *)(bmat + 16 * f) = u32x4{v[0], v[1], v[2], v[3]};
        }
        __syncthreads();
#pragma unroll
        for (int st = 0; st < NSTEPS; ++st) fb[st] = *(const u32x4 *)(bmat + 16 * (64 * st + lane));
    }
    // the A read of step st: ring row rel0 + dp_index, pixel slot j0 + m +
    // dq_index, chunk 4*(st%2) + kq at its swizzled place (the swizzle of slot
    // j0 + m + dq_index is that of m + dq_index, j0 being a multiple of 16)
    const int m = lane & 15;
    int pixoff[NDW][2];
#pragma unroll
    for (int dqi = 0; dqi < NDW; ++dqi)
#pragma unroll
        for (int h = 0; h < 2; ++h) pixoff[dqi][h] = (m + dqi) * PIXB + ((4 * h + kq) ^ swz(m + dqi)) * 16;
    unsigned char *wst = stage + wave * a.stage_wave;  // this wave's output staging

    for (int it = 0; it < niter; ++it) {
        if (it > 0) {
            wait_vm_all();    // this pair's rows (and this wave's older stores)
            __syncthreads();  // the pair's rows are in LDS; the previous pair's slots are free
            if (it + 1 < niter) dma_rows(2 * it + NDH + 1, 2);
        }
        const int nbl = (2 * it + 1 < nsr ? 2 : 1) * a.nblk_r;  // blocks of this pair
        for (int bl = wave; bl < nbl; bl += WAVES) {
            const int ir = bl >= a.nblk_r ? 1 : 0, jb = bl - ir * a.nblk_r;
            const int j0 = 16 * jb;
            const int rel0 = 2 * it + ir;  // ring index of dp = dp_min for this super-row
            // A reads PF steps ahead of their MFMAs; two accumulators (even and
            // odd steps) so that consecutive MFMAs do not wait on each other
            f32x4 acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            u32x4 fa[NSTEPS];
            const unsigned char *rowp[NDH];
#pragma unroll
            for (int dpi = 0; dpi < NDH; ++dpi) rowp[dpi] = ring + ((rel0 + dpi) % a.nslot) * a.rowb + j0 * PIXB;
            auto ld = [&](int st) __attribute__((always_inline)) {
                const int pair = st >> 1, dpi = pair / NDW, dqi = pair % NDW;
                fa[st] = *(const u32x4 *)(rowp[dpi] + pixoff[dqi][st & 1]);
            };
#pragma unroll
            for (int st = 0; st < PF; ++st) ld(st);
#pragma unroll
            for (int st = 0; st < NSTEPS; ++st) {
                if (st + PF < NSTEPS) ld(st + PF);
                acc2[st & 1] = E::mfma(fa[st], fb[st], acc2[st & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = acc2[0][e] + acc2[1][e];
            // D: lane holds column n = (a, b, c) for super-pixels j0 + 4*kq + 0..3
            const int i = i0 + 2 * it + ir;
            if (n < 4 * a.C) {
                const int oa = n / (2 * a.C), ob = (n / a.C) & 1, oc = n % a.C;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int jl = 4 * kq + e;  // super-pixel within the block
                    ((elem *)wst)[oa * 32 * a.C + (2 * jl + ob) * a.C + oc] = E::from_f32(acc[e]);
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's staging writes are done
            __builtin_amdgcn_wave_barrier();
            // 2 rows x 32 pixels x C elements: 4*C 16-byte pieces per row
            const int pieces = 4 * a.C;
            if (lane < 2 * pieces) {
                const int oa = lane / pieces, pc = lane - oa * pieces;
                const int h = 2 * i + oa;
                const int valid = (a.W - 2 * j0) * a.C;  // elements of the row segment inside the image
                if (h < a.H && 8 * pc < valid) {
                    const u32x4 v = *(const u32x4 *)(wst + oa * 64 * a.C + 16 * pc);
                    elem *dst = (elem *)a.dx + (((size_t)img * a.H + h) * a.W + 2 * j0) * a.C + 8 * pc;
                    __builtin_nontemporal_store(v, (u32x4 *)dst);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

bool fewchan_dgrad_supported(int dtype, int C, int K, int sh, int sw, int dh, int dw, int W)
{
    if (dtype != CONV2D_DTYPE_F16 && dtype != CONV2D_DTYPE_BF16) return false;
    return C % 8 != 0 && C <= 4 && K == fd::K && sh == 2 && sw == 2 && dh == 1 && dw == 1 && (W * C) % 8 == 0;
}
int fewchan_dgrad_lds_bytes() { return fd::LDS_BYTES; }
int fewchan_dgrad_max_offsets() { return 4; }  // dp (and dq) values per axis: 2 to 4

template <class E, int NDH>
static hipError_t launch_ndh(const FewDgradArgs &a, dim3 grid, hipStream_t st)
{
    switch (a.ndw) {
    case 2: fewchan_dgrad_kernel<E, NDH, 2><<<grid, fd::NT, 0, st>>>(a); break;
    case 3: fewchan_dgrad_kernel<E, NDH, 3><<<grid, fd::NT, 0, st>>>(a); break;
    case 4: fewchan_dgrad_kernel<E, NDH, 4><<<grid, fd::NT, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
template <class E>
static hipError_t launch_e(const FewDgradArgs &a, dim3 grid, hipStream_t st)
{
    switch (a.ndh) {
    case 2: return launch_ndh<E, 2>(a, grid, st);
    case 3: return launch_ndh<E, 3>(a, grid, st);
    case 4: return launch_ndh<E, 4>(a, grid, st);
    default: return hipErrorInvalidValue;
    }
}
hipError_t launch_fewchan_dgrad(int dtype, const FewDgradArgs &a, hipStream_t st)
{
    const dim3 grid((unsigned)(a.N * a.bands));
    return dtype == CONV2D_DTYPE_F16 ? launch_e<EF16>(a, grid, st) : launch_e<EBF16>(a, grid, st);
}

}  // namespace cnv

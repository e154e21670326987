// fewchan_wgrad.hip -- weight gradient for inputs with few channels (C not a
// multiple of 8: the 3-channel stem of the tensorcore "Conv2D" page's
// 224 -> 112 example), without padding the channels.
//
// dw[k][r][s][c] = sum over output pixels (p, q) of dy[p, q, k] *
// x[p*sh - ph + r*dh, q*sw - pw + s, c] is a GEMM with rows k, a reduction
// over pixels and, as in the few-channel forward kernel, columns laid out per
// filter row as a window of Lw elements of the NHWC input row: window
// position kk of pixel q in filter row r is input-row element
// (q*sw - pw)*C - delta + kk, i.e. tap (s, c) with s*C + c = kk - delta when
// that is in [0, S*C); the other positions are computed and dropped.
//
// Both MFMA operands need eight consecutive pixels per lane, which gfx950's
// transposing LDS read ds_read_b64_tr_b16 gives from pixel-major data: in each
// group of 16 lanes, lane L points at 4 consecutive 16-bit values of "row"
// L/4 and lane i receives value i of the 4 rows.  For dy a row is a pixel (4
// channels per lane); for x it is a pixel's window (4 window positions per
// lane), which is 4 consecutive elements of the input row in LDS.  That read
// needs 8-byte alignment.  The window start moves by sw*C elements from pixel
// to pixel; delta (0..3) aligns the even pixels' windows, and when sw*C is 2
// mod 4 the odd pixels' windows sit 4 bytes off, so each group's input rows
// are also kept as a second copy shifted by 4 bytes, from which the odd
// pixels are read.  The pixels of an output row are taken as two classes
// (even q, odd q) of steps of 16 (the MFMA's reduction), so every step reads
// one copy; dy pixels past Q are zero and add nothing.
//
// A workgroup (8 waves, two per SIMD) owns a band of output rows of one image
// and all of dw: K = 64 rows (two k-blocks) by ceil(R*Lw / 32) column blocks,
// split in two column sets (waves 0-3 and 4-7).  Wave w takes the steps
// t = w (mod 4) of each group of two output rows.  Each group's dy rows and
// input rows arrive by direct-to-LDS loads (zeros outside the image from the
// range check) into one of two buffers while the previous group is computed.
// The four phases' sums are added in a fixed order and the band's fp32
// partial is written; the split-K reduce adds the bands in order.
#include "device_common.h"

namespace cnv {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

namespace fw {
constexpr int NT = 512;
constexpr int WAVES = NT / 64;
constexpr int PHASES = 4;
constexpr int K = 64, KB = 2;    // output channels, k-blocks
constexpr int PIXB = K * 2;      // bytes of a dy pixel
constexpr int LDS_BYTES = 163840;
constexpr int TILE_BYTES = 64 * 16 * 4;  // one 32x32 fp32 accumulator block, all lanes

template <class E>
__device__ inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ inline f32x16 mfma<EF16>(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                   0, 0, 0);
}
template <>
__device__ inline f32x16 mfma<EBF16>(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                    c, 0, 0, 0);
}
typedef __attribute__((address_space(3))) unsigned char lds_u8;
__device__ inline s16x4 tr(const lds_u8 *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
__device__ inline u32x4 join(s16x4 lo, s16x4 hi)
{
    const uint2 l = __builtin_bit_cast(uint2, lo), h = __builtin_bit_cast(uint2, hi);
    return u32x4{l.x, l.y, h.x, h.y};
}
// dy pixel q's 16-byte channel chunk c sits at chunk slot c ^ swz(q): the four
// pixels of a transposing read (q, q+2, q+4, q+6 of one class) then cover
// eight different chunk slots, i.e. all 32 banks of their 128 bytes
__device__ inline int swz(int q) { return ((q >> 1) & 3) << 1; }
}  // namespace fw

template <class E, int NCBW, int CB0>
__device__ __attribute__((always_inline)) inline void fewchan_wgrad_wave(const FewWgradArgs &a,
                                                                        unsigned char *smem, const int wave,
                                                                        const int lane)
{
    using namespace fw;
    const int phase = wave & (PHASES - 1);
    const int img = blockIdx.x / a.bands;
    const int band = blockIdx.x - img * a.bands;
    const int p0 = band * a.rows_per_wg;
    const int nrows = min(a.rows_per_wg, a.P - p0);  // >= 1 by construction of the grid
    const int ngroups = (nrows + a.grw - 1) / a.grw;
    const int DQ = a.dq;
    const int nsteps_row = 2 * a.spc;

    // ---- loads of group g into buffer g & 1: dy (grw rows of DQ pixel slots,
    // 8 pixels per 1 KB block), then the input rows (nxr rows of cpr 16-byte
    // chunks, 64 chunks per block).  Block b of the group goes to wave b % 8.
    const u32x4 d_rs = make_buf_rsrc(a.dy, a.dy_bytes);
    const u32x4 x_rs = make_buf_rsrc(a.x, a.x_bytes);
    const uint32_t lds0 = lds_addr(smem);
    auto dma_group = [&](int g) -> int {  // returns this wave's load count
        if (g >= ngroups) return 0;
        const uint32_t buf = lds0 + (uint32_t)((g & 1) * a.buf_bytes);
        const int prow = p0 + g * a.grw;                 // first output row of the group
        const int grows = min(a.grw, p0 + nrows - prow);  // its rows
        int n = 0;
        for (int b = wave; b < a.nblk_dy + a.nblk_x; b += WAVES) {
            if (b < a.nblk_dy) {
                const int v = 8 * b + (lane >> 3);
                const int gr = v / DQ, q = v - gr * DQ;
                const int c = (lane & 7) ^ swz(q);
                const bool in = gr < grows && q < a.Q;
                dma16(d_rs, buf + (uint32_t)(b * 1024),
                      in ? (uint32_t)(((img * a.P + prow + gr) * a.Q + q) * PIXB + c * 16) : kBufOOBFar);
            } else {
                const int bx = b - a.nblk_dy;
                const uint32_t u = (uint32_t)(bx * 64 + lane);
                const uint32_t rr = fdiv(u, a.div_cpr);
                const int e0 = (int)(u - rr * (uint32_t)a.cpr) * 8 - a.left;
                const int h = prow * a.sh - a.pad_h + (int)rr;
                const bool in = (int)rr < a.nxr && (unsigned)h < (unsigned)a.H && e0 >= 0 && e0 < a.WC;
                dma16(x_rs, buf + (uint32_t)(a.xa_off + bx * 1024),
                      in ? ((uint32_t)(img * a.H + h) * (uint32_t)a.WC + (uint32_t)e0) * 2u : kBufOOBFar);
            }
            ++n;
        }
        return n;
    };
    // wait until at most n of this wave's loads are outstanding
    auto wait_n = [](int n) {
        switch (n) {
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
        default: wait_vm_all(); break;
        }
    };

    // ---- per-lane read offsets.  In a 16-lane group (g16 = lane/16 within
    // the half-wave), lane L points at pixel L/4 of the read's four and at
    // values 4*(L%4)..+3 of the group's 16 channels (dy) or 16 window
    // positions (x).
    const int L = lane & 15, g16 = (lane >> 4) & 1, lhi = lane >> 5, l32 = lane & 31;
    const int psub = L >> 2;  // pixel of the read's four
    int dyc[KB];             // byte offset of the lane's 4 channels inside a dy pixel
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int ch = 32 * kb + 16 * g16 + 4 * (L & 3);
        dyc[kb] = ((ch >> 3) ^ (2 * psub)) * 16 + (ch & 7) * 2;  // swz(q) = 2 * psub for every q of the read
    }
    int xo[NCBW];  // byte offset of the lane's 4 window positions from its pixel's window start
#pragma unroll
    for (int i = 0; i < NCBW; ++i) {
        const int t = 32 * (CB0 + i) + 16 * g16 + 4 * (L & 3);
        const int r = t / a.lw, kk = t - r * a.lw;
        xo[i] = r < a.R ? r * a.dh * a.pitch + 2 * kk : 0;  // columns past the filter: any valid address
    }

    f32x16 acc[KB][NCBW];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < NCBW; ++i) acc[kb][i] = f32x16{};

    // one step: 16 pixels of one class of output row gr of the group; its
    // fragments are read one step ahead of their MFMAs
    struct Frags {
        s16x4 d[KB][2], x[NCBW][2];
    };
    auto read = [&](const unsigned char *buf, int t, Frags &f) __attribute__((always_inline)) {
        const int gr = t / nsteps_row, rem = t - gr * nsteps_row;
        const int cls = rem >= a.spc ? 1 : 0, j = rem - cls * a.spc;
        const lds_u8 *dyp = (const lds_u8 *)buf + gr * DQ * PIXB;
        const lds_u8 *xp = (const lds_u8 *)buf + (cls && a.odd_shift ? a.xb_off + 4 : a.xa_off) +
                           gr * a.sh * a.pitch + 2 * a.win0;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            const int q = 2 * (16 * j + 8 * lhi + 4 * rd + psub) + cls;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) f.d[kb][rd] = tr(dyp + q * PIXB + dyc[kb]);
#pragma unroll
            for (int i = 0; i < NCBW; ++i) f.x[i][rd] = tr(xp + 2 * q * a.qstep + xo[i]);
        }
    };
    auto mma = [&](const Frags &f) __attribute__((always_inline)) {
        u32x4 fa[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) fa[kb] = join(f.d[kb][0], f.d[kb][1]);
#pragma unroll
        for (int i = 0; i < NCBW; ++i) {
            const u32x4 fb = join(f.x[i][0], f.x[i][1]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) acc[kb][i] = mfma<E>(fa[kb], fb, acc[kb][i]);
        }
    };
    // this wave's steps t = phase, phase + 4, ... < nst of a group; the reads
    // past the last step (clamped to it) are discarded
    auto steps = [&](const unsigned char *buf, int nst) __attribute__((always_inline)) {
        if (phase >= nst) return;
        const int last = nst - 1;
        Frags f0, f1;
        int t = phase;
        read(buf, t, f0);
        while (true) {
            read(buf, min(t + PHASES, last), f1);
            mma(f0);
            t += PHASES;
            if (t >= nst) break;
            read(buf, min(t + PHASES, last), f0);
            mma(f1);
            t += PHASES;
            if (t >= nst) break;
        }
    };

    int nxt = dma_group(0);
    nxt = dma_group(1);
    for (int g = 0; g < ngroups; ++g) {
        wait_n(nxt);      // this wave's loads of group g (those of group g + 1 may still run)
        __syncthreads();  // group g is in LDS
        unsigned char *buf = smem + (g & 1) * a.buf_bytes;
        if (a.odd_shift) {
            // the shifted copy: byte j + 4 of copy B is byte j of copy A
            const unsigned char *xa = buf + a.xa_off;
            unsigned char *xb = buf + a.xb_off;
            for (int c = threadIdx.x; c < a.xcopy_chunks; c += NT) {
                const u32x4 v = *(const u32x4 *)(xa + 16 * c);
                uint32_t *d = (uint32_t *)(xb + 16 * c + 4);
                d[0] = v.x;
                d[1] = v.y;
                d[2] = v.z;
                d[3] = v.w;
            }
            if (threadIdx.x == 0) *(uint32_t *)xb = 0u;
            __syncthreads();
        }
        const int grows = min(a.grw, nrows - g * a.grw);
        steps(buf, grows * nsteps_row);
        __syncthreads();  // every wave is done with buffer g & 1
        nxt = dma_group(g + 2);
    }

    // ---- the four phases' sums of each column set, in the fixed order
    // (p0 + p2) + (p1 + p3), through LDS (free after the last barrier):
    // phases 2 and 3 park their blocks, phases 0 and 1 add them, phase 1
    // parks the result and phase 0 adds it and stores.  A parked block is
    // [4][64 lanes] of 16-byte pieces (4 consecutive accumulator rows).
    constexpr int NT_ = KB * NCBW;
    const int set_base = CB0 == 0 ? 0 : 2 * KB * a.ncba * TILE_BYTES;
    f32x4 *const lds4 = (f32x4 *)smem + lane;
    auto part = [&](int h) { return lds4 + (set_base + h * NT_ * TILE_BYTES) / 16; };
    auto park = [&](f32x4 *p, int t, const f32x16 &v) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) p[(t * 4 + q) * 64] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    };
    auto add = [&](const f32x4 *p, int t, f32x16 &v) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 u = p[(t * 4 + q) * 64];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] += u[e];
        }
    };
    if (phase >= 2) {
#pragma unroll
        for (int t = 0; t < NT_; ++t) park(part(phase - 2), t, acc[t / NCBW][t % NCBW]);
    }
    __syncthreads();
    if (phase < 2) {
#pragma unroll
        for (int t = 0; t < NT_; ++t) add(part(phase), t, acc[t / NCBW][t % NCBW]);
    }
    __syncthreads();
    if (phase == 1) {
#pragma unroll
        for (int t = 0; t < NT_; ++t) park(part(0), t, acc[t / NCBW][t % NCBW]);
    }
    __syncthreads();
    if (phase == 0) {
        // column t of the window layout -> (r, s*C + c); rows k = 32*kb +
        // 8*(e/4) + 4*lhi + e%4 of the lane's accumulator entry e
        float *const out = (float *)a.out + (size_t)blockIdx.x * a.part_stride;
        const int RSC = a.R * a.SC;
#pragma unroll
        for (int i = 0; i < NCBW; ++i) {
            const int t = 32 * (CB0 + i) + l32;
            const int r = t / a.lw, sc = t - r * a.lw - a.delta;
            const bool ok = r < a.R && sc >= 0 && sc < a.SC;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x16 &v = acc[kb][i];
                add(part(0), kb * NCBW + i, v);
                if (ok) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        __builtin_nontemporal_store(
                            v[e], &out[(size_t)(32 * kb + 8 * (e >> 2) + 4 * lhi + (e & 3)) * RSC + r * a.SC + sc]);
                }
            }
        }
    }
}

template <class E, int NCBA, int NCBB>
__global__ __launch_bounds__(512) void fewchan_wgrad_kernel(const FewWgradArgs a)
{
    __shared__ __attribute__((aligned(16))) unsigned char smem[fw::LDS_BYTES];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // waves 0-3 (one per SIMD) and 4-7 (the second of each SIMD) take the two column sets
    if (wave < fw::PHASES)
        fewchan_wgrad_wave<E, NCBA, 0>(a, smem, wave, lane);
    else
        fewchan_wgrad_wave<E, NCBB, NCBA>(a, smem, wave, lane);
}

bool fewchan_wgrad_supported(int dtype, int C, int K, int S, int sw, int dw, int W)
{
    if (dtype != CONV2D_DTYPE_F16 && dtype != CONV2D_DTYPE_BF16) return false;
    return C % 8 != 0 && K == fw::K && dw == 1 && (sw * C) % 2 == 0 && (W * C) % 8 == 0;
}
int fewchan_wgrad_lds_bytes() { return fw::LDS_BYTES; }

template <class E, int NCBA, int NCBB>
static void launch_sets(const FewWgradArgs &a, dim3 grid, hipStream_t st)
{
    fewchan_wgrad_kernel<E, NCBA, NCBB><<<grid, fw::NT, 0, st>>>(a);
}

template <class E>
static hipError_t launch_e(const FewWgradArgs &a, hipStream_t st)
{
    const dim3 grid((unsigned)(a.N * a.bands));
    switch (a.ncb) {
    case 2: launch_sets<E, 1, 1>(a, grid, st); break;
    case 3: launch_sets<E, 2, 1>(a, grid, st); break;
    case 4: launch_sets<E, 2, 2>(a, grid, st); break;
    case 5: launch_sets<E, 3, 2>(a, grid, st); break;
    case 6: launch_sets<E, 3, 3>(a, grid, st); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_fewchan_wgrad(int dtype, const FewWgradArgs &a, hipStream_t st)
{
    if (a.ncba != (a.ncb + 1) / 2) return hipErrorInvalidValue;
    return dtype == CONV2D_DTYPE_F16 ? launch_e<EF16>(a, st) : launch_e<EBF16>(a, st);
}

}  // namespace cnv

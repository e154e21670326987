// wgrad_band.hip -- stride-1 3x3 weight gradient with dy and x pixels resident
// in LDS and transposing LDS reads (gfx950).
//
// dw[k][r][s][c] = sum over output pixels (p,q) of dy[p,q,k] * x[p-ph+r*d, q-pw+s*d, c]
// is a GEMM with rows k, columns (r,s,c) and a reduction over pixels.  Both
// operands arrive pixel-major (NHWC), while an MFMA operand needs eight
// consecutive reduction elements (pixels) per lane.  gfx950's
// ds_read_b64_tr_b16 gives exactly that from a pixel-major tile: in each group
// of 16 lanes, lane L points at 4 channels of pixel L/4 and lane i receives
// channel i of the 4 pixels.  So dy and x pixels are copied into LDS as they
// are, and all R*S tap shifts of x are just different read addresses.
//
// Pixels are numbered with the padded pitch XW = Q + dil*(S-1): output pixel
// (p, q) of the band is v = p*XW + q, and its tap (r, s) of x is v + r*dil*XW
// + s*dil (with one filter row a workgroup, v + s*dil of that row's window).  dy is zero at the XW - Q padding columns, so the band is one
// linear stream of rows*XW pixels, cut into steps of 16 (one MFMA's
// reduction) and groups of 16 steps that ignore row boundaries.  Steps past
// the band's end read zero dy pixels (their loads fall outside the band's
// rows) and add exact zeros; the last group runs only the steps per wave
// that its band pixels need.
//
// A workgroup (8 waves, two per SIMD) owns a band of output rows and a set of
// column blocks of 32, all of K, and writes the band's fp32 partial for its
// columns; the split-K reduction adds the bands' partials in order.  Two
// splits of the 18 column blocks:
//   * column halves (9 blocks each), bands within one image, two workgroups
//     a band; the x window holds the group's pixels plus R-1 rows of halo;
//   * filter rows (6 blocks each: the S taps x two channel halves of one r),
//     three workgroups a band: 85 bands (255 workgroups) of the stacked rows
//     of all images (row n*P + p; a band may cross image boundaries).  The
//     host picks the split with the lower estimated time.  Window row i is x row
//     p + r - pad of dy row i's image, gathered row by row, so the x window
//     is the dy window plus S-1 pixels and the partials are two thirds of
//     the halves' (85 slices of the whole filter against 128 on 64x56x56).
// Waves 0-3 hold the first ceil(n/2) of the workgroup's n column blocks and
// waves 4-7 the rest, both k-blocks (32x32x16 MFMA accumulators); wave w
// takes the steps t = w (mod 4).  The two waves of a SIMD work on the same
// steps: with halves each SIMD does 18 MFMAs per step and per step a wave
// reads its 2 dy fragments and one x fragment per column block, 13 fragments
// for 18 MFMAs per SIMD (filter rows: 10 for 12).  Two waves per SIMD keep
// twice as many transposing reads in flight as one, and the LDS read rate
// grows with the reads in flight.  The four waves' sums of each column set
// are added at the end in a fixed order.
//
// Each group's dy pixels and x window (the group's pixels plus the tap
// shifts) arrive by direct-to-LDS loads (buffer_load ... lds; pixels outside
// the image and the padding come from the buffer range check as zeros) into
// one of two buffers while the previous group is computed from the other.
// The barrier between groups sits inside a wave's last step of a group: once
// that step's fragments are in registers, the wave waits for its share of the
// next group's loads, meets the others, reads the next group's first
// fragments during the last step's MFMAs and issues the loads of the group
// after next, a few blocks at a time, between them.
//
// 16-byte channel chunks of buffer pixel v are stored with chunk bit 2
// flipped when bit 1 of v is set: the transposing reads of 4 consecutive
// pixels x 32 channels then cover all 64 LDS banks.  Groups, steps and the
// second read of a fragment move by multiples of 4 pixels, which keep bit 1.
#include "device_common.h"

namespace cnv {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <class E>
struct Mfma32w;
template <>
struct Mfma32w<EF16> {
    __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <>
struct Mfma32w<EBF16> {
    __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

namespace wb {
constexpr int NT = 512;                   // 8 waves, two per SIMD
constexpr int WAVES = NT / 64;
constexpr int PHASES = 4;                 // wave w takes the steps t = w (mod 4)
constexpr int CH = 64;                    // C = K = 64 channels, 128 bytes per pixel
constexpr int PIXB = CH * 2;
constexpr int R = 3, S = 3, DIL = 1;
constexpr int NCOLS = R * S * CH;         // 576 columns (r, s, c)
constexpr int KB = CH / 32;               // k-blocks
constexpr int GSTEPS = 16;                // steps of 16 pixels per group
constexpr int GPIX = GSTEPS * 16;         // dy pixels per group
constexpr int SLOTS = GSTEPS / PHASES;    // steps per wave per group
constexpr int QMAX = 56;
constexpr int XWMAX = QMAX + DIL * (S - 1);
constexpr int DCAP = GPIX;
constexpr int D_BYTES = DCAP * PIXB;
constexpr int DBLK = DCAP / 8;             // 1 KB direct-to-LDS blocks of 8 pixels
constexpr int STEPB = PHASES * 16 * PIXB;  // a wave's next step in a group: 64 pixels on
constexpr int RDB = 4 * PIXB;              // the second read of a fragment: 4 pixels on
constexpr int TILE_BYTES = 64 * 16 * 4;    // one 32x32 fp32 accumulator block, all lanes
static_assert(DBLK % WAVES == 0, "every wave loads the same dy blocks");
static_assert(GSTEPS % PHASES == 0 && SLOTS == 4, "four steps per wave per group");

// The column split: NSPLIT workgroups share a band's pixels, each with
// NCOLS / NSPLIT columns.  NSPLIT = 2: column halves, the x window holds the
// R tap rows.  NSPLIT = 3: one filter row r per workgroup (its S taps, all
// channels); its x window is the band's rows shifted by r, so a window row
// lines up with its dy row and only the S - 1 column shifts reach past it.
template <int NSPLIT>
struct Cfg {
    static constexpr int CB_WG = NCOLS / 32 / NSPLIT;  // column blocks per workgroup: 9 or 6
    static constexpr int NCB_A = (CB_WG + 1) / 2;       // column blocks of waves 0-3
    static constexpr int NCB_B = CB_WG - NCB_A;         // and of waves 4-7
    static constexpr int HALO = (NSPLIT == 2 ? DIL * (R - 1) * XWMAX : 0) + DIL * (S - 1);  // x pixels past a group's dy pixels
    static constexpr int XCAP = (GPIX + HALO + 63) / 64 * 64;  // whole 1 KB blocks for each of the 8 waves
    static constexpr int X_BYTES = XCAP * PIXB;
    static constexpr int BUF_BYTES = D_BYTES + X_BYTES;
    static constexpr int LDS_BYTES = 2 * BUF_BYTES;
    static constexpr int XBLK = XCAP / 8;
    static constexpr int NB_WAVE = (DBLK + XBLK) / WAVES;  // blocks per wave per group
    static_assert(NSPLIT == 2 || NSPLIT == 3, "column halves or filter rows");
    static_assert(NSPLIT == 2 || R == 3, "one filter row per workgroup of three");
    static_assert(XBLK % WAVES == 0, "every wave loads the same x blocks");
    static_assert(LDS_BYTES <= 163840, "fits in the 160 KB LDS");
    static_assert(2 * KB * CB_WG * TILE_BYTES <= LDS_BYTES, "two phases' blocks of both sets fit in LDS");
    static_assert((SLOTS - 1) * STEPB + RDB + 32 < 65536, "read offsets fit the 16-bit immediate");
};

template <int V>
struct IntC {
    static constexpr int value = V;
};
// f(IntC<B>{}), f(IntC<B + 1>{}), ..., f(IntC<E - 1>{})
template <int B, int E, class F>
__device__ __attribute__((always_inline)) inline void static_for(F &&f)
{
    if constexpr (B < E) {
        f(IntC<B>{});
        static_for<B + 1, E>(f);
    }
}
__device__ inline int swz_chunk(int chunk, int v) { return chunk ^ (((v >> 1) & 1) << 2); }
}  // namespace wb

// The work of one wave: NCB column blocks from block CB0 of the workgroup's
// columns, the steps t = phase (mod 4); then the set's sums and the
// partial's stores.
template <class E, bool DB, int NSPLIT, int NCB, int CB0>
__device__ __attribute__((always_inline)) inline void wgrad_band_wave(const WgradBandArgs &a, unsigned char *smem,
                                                                     const int wave, const int lane)
{
    using namespace wb;
    using elem = typename E::elem;
    using Cf = Cfg<NSPLIT>;
    constexpr int CB_WG = Cf::CB_WG, NB_WAVE = Cf::NB_WAVE, BUF_BYTES = Cf::BUF_BYTES;
    const int phase = wave & (PHASES - 1);
    // Workgroup -> (band, column set colh).  A band is output rows [t0, t0 +
    // nrows) of the stack of all images' rows (row n*P + p is row p of image
    // n).  Workgroups are dealt to the 8 XCDs in turn; the column sets of a
    // band go 8 apart where the grid allows, so they share an XCD and the
    // later ones' loads hit that XCD's L2.
    int band, colh, t0, nrows, img;
    if constexpr (NSPLIT == 2) {
        // bands within one image: chunks_per_img bands of rows_per_wg rows
        if (a.xcd_pairs) {
            const int bid = blockIdx.x;
            colh = (bid >> 3) & 1;
            band = (bid & 7) + 8 * (bid >> 4);
        } else {
            colh = blockIdx.x & 1;
            band = blockIdx.x >> 1;
        }
        img = band / a.chunks_per_img;
        const int p_start = (band - img * a.chunks_per_img) * a.rows_per_wg;
        nrows = min(p_start + a.rows_per_wg, a.P) - p_start;  // >= 1 by construction of the grid
        t0 = img * a.P + p_start;
    } else {
        // nbands bands of about rows_total / nbands rows, across image
        // boundaries.  XCD x takes the three filter rows
        // of bands x*F .. x*F + F - 1 (F = band_f) in its first 3F
        // workgroups; the rest of the grid deals the last bands in order.
        const int bid = blockIdx.x, xcd = bid & 7, m = bid >> 3, F = a.band_f;
        if (m < 3 * F) {
            band = xcd * F + m / 3;
            colh = m - (m / 3) * 3;
        } else {
            const int idx = (m - 3 * F) * 8 + xcd;
            band = 8 * F + idx / 3;
            colh = idx - (idx / 3) * 3;
        }
        t0 = (int)(((long long)band * a.rows_total) / a.nbands);
        nrows = (int)(((long long)(band + 1) * a.rows_total) / a.nbands) - t0;
        img = t0 / a.P;
    }
    const int Q = a.Q, XW = a.xw;
    const int h_base = t0 - img * a.P - a.pad_h;  // column halves: input row of band row 0, tap row 0
    const int nsteps = (nrows * XW + 15) >> 4;
    const int ngroups = (nsteps + GSTEPS - 1) / GSTEPS;

    // ---- loads.  Group g covers the band's pixels [g*GPIX, g*GPIX + DCAP)
    // of dy and [g*GPIX, g*GPIX + XCAP) of x.  Lane i of a 1 KB block fills
    // stored chunk i%8 of buffer pixel 8*blk + i/8 with source chunk
    // swz_chunk(i%8, pixel); the lane's pixel within a block and its chunk
    // are the same in every block (bit 1 of the pixel index is bit 1 of
    // i/8).  The per-block arithmetic is redone in each call from an opaque
    // copy of them, so that the compiler does not keep every block's
    // addresses in registers across the loop.
    // x: the images the band's rows belong to; offsets past them read zeros
    // (window rows past the band's end meet zero dy)
    const int ximgs = NSPLIT == 2 ? 1 : (t0 + nrows - 1) / a.P - img + 1;
    const u32x4 x_rs =
        make_buf_rsrc((const elem *)a.x + (size_t)img * a.H * a.W * CH, (uint32_t)ximgs * (uint32_t)(a.H * a.W * CH * 2));
    const u32x4 d_rs = make_buf_rsrc((const elem *)a.dy + (size_t)t0 * Q * CH, (uint32_t)(nrows * Q * CH * 2));
    const uint32_t lds0 = lds_addr(smem);
    const int lane_px = lane >> 3;
    const int lane_chunk16 = swz_chunk(lane & 7, lane_px) * 16;
    // block jb (0 .. NB_WAVE-1) of this wave's share of group g: dy blocks
    // first, then x blocks; nothing for a group past the band
    auto dma_block = [&](int g, int px, int ch, auto jb_c) __attribute__((always_inline)) {
        constexpr int JB = decltype(jb_c)::value;
        if (g >= ngroups) return;
        const uint32_t buf = lds0 + (uint32_t)((g & 1) * BUF_BYTES);
        if constexpr (JB < DBLK / WAVES) {
            const int b = wave + WAVES * JB;
            const int v = px + b * 8;  // band pixel of this lane
            const int row = (int)fdiv((uint32_t)v, a.div_xw), col = v - row * XW;
            const bool in = row < nrows && col < Q;
            dma16(d_rs, buf + b * 1024, in ? (unsigned)((row * Q + col) * PIXB + ch) : kBufOOB);
        } else {
            const int b = wave + WAVES * (JB - DBLK / WAVES);
            const int v = px + b * 8;
            const int row = (int)fdiv((uint32_t)v, a.div_xw), col = v - row * XW;
            // window pixels past the last one a fragment reads are not fetched
            const int w = b * 8 + lane_px < GPIX + Cf::HALO ? col - a.pad_w : -1;
            if constexpr (NSPLIT == 2) {
                const int h = h_base + row;
                const bool in = (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W;
                dma16(x_rs, buf + D_BYTES + b * 1024, in ? (unsigned)((h * a.W + w) * PIXB + ch) : kBufOOB);
            } else {
                // window row `row` is dy row t0 + row of image n, shifted by the filter row
                const int t = t0 + row, n = (int)fdiv((uint32_t)t, a.div_p);
                const int h = t - n * a.P - a.pad_h + colh * DIL;
                const bool in = (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W && n - img < ximgs;
                dma16(x_rs, buf + D_BYTES + b * 1024,
                      in ? (unsigned)(((n - img) * a.H + h) * a.W + w) * (unsigned)PIXB + (unsigned)ch : kBufOOB);
            }
        }
    };
    auto dma_lane = [&](int g, int &px, int &ch) __attribute__((always_inline)) {
        px = g * GPIX + lane_px;
        ch = lane_chunk16;
        asm volatile("" : "+v"(px), "+v"(ch));
    };

    // ---- fragment reads.  Read rd of a fragment covers pixels v = 16*t +
    // 8*(lane/32) + 4*rd + 0..3 of step t; this lane points at pixel
    // v + L/4 (L = lane%16), channels 4*(L%4)..+3 of its 16-channel group.
    // Column block cb (of the 18) is tap cb/2 = (r, s), channel half cb%2.
    const int l32 = lane & 31, lhi = lane >> 5;
    auto dy_off = [&](int kb) {
        const int L_ = lane & 15, g_ = (lane >> 4) & 1;
        const int c_ = 16 * g_ + 4 * (L_ & 3);
        const int v = 16 * phase + 8 * lhi + (L_ >> 2);
        return v * PIXB + swz_chunk(kb * 4 + (c_ >> 3), v) * 16 + (c_ & 7) * 2;
    };
    auto x_off = [&](int cb) {
        const int L_ = lane & 15, g_ = (lane >> 4) & 1;
        const int c_ = 16 * g_ + 4 * (L_ & 3);
        const int v = 16 * phase + 8 * lhi + (L_ >> 2);
        const int tap = cb >> 1, tr_ = tap / S, ts_ = tap - tr_ * S;
        const int xv = v + (NSPLIT == 2 ? tr_ * DIL * XW : 0) + ts_ * DIL;  // filter rows: the row is in the window
        return D_BYTES + xv * PIXB + swz_chunk((cb & 1) * 4 + (c_ >> 3), xv) * 16 + (c_ & 7) * 2;
    };
    typedef __attribute__((address_space(3))) unsigned char lds_u8;  // 32-bit LDS addresses
    auto tr = [](const lds_u8 *p) -> s16x4 {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    };
    // Lane addresses of this wave's step of slot 0 in the current buffer; slot
    // J and the second read of a fragment are immediate offsets, and the
    // other buffer is BUF_BYTES away.  The empty asm keeps the compiler from
    // folding the offsets into one address register per slot.
    const lds_u8 *ad[KB], *ax[NCB];
    auto pin = [](const lds_u8 *&p) __attribute__((always_inline)) { asm volatile("" : "+v"(p)); };
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) ad[kb] = (const lds_u8 *)smem + dy_off(kb);
#pragma unroll
    for (int i = 0; i < NCB; ++i) ax[i] = (const lds_u8 *)smem + x_off(colh * CB_WG + CB0 + i);
    auto switch_buffer = [&](int delta) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            ad[kb] += delta;
            pin(ad[kb]);
        }
#pragma unroll
        for (int i = 0; i < NCB; ++i) {
            ax[i] += delta;
            pin(ax[i]);
        }
    };
    typedef s16x4 DyFrag[KB][2];
    s16x4 fx[NCB][2];  // x fragments, read in place
    auto read_dy = [&](DyFrag &d, auto j_c) __attribute__((always_inline)) {
        constexpr int J = decltype(j_c)::value;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int rd = 0; rd < 2; ++rd) d[kb][rd] = tr(ad[kb] + rd * RDB + J * STEPB);
    };
    auto read_x = [&](int i, auto j_c) __attribute__((always_inline)) {
        constexpr int J = decltype(j_c)::value;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) fx[i][rd] = tr(ax[i] + rd * RDB + J * STEPB);
    };
    auto join = [](s16x4 lo, s16x4 hi) -> u32x4 {
        const uint2 l = __builtin_bit_cast(uint2, lo), h = __builtin_bit_cast(uint2, hi);
        return u32x4{l.x, l.y, h.x, h.y};
    };

    f32x16 acc[KB][NCB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < NCB; ++i) acc[kb][i] = f32x16{};
    // bias gradient (DB): the first column half's waves 0-3 add up the dy
    // values of their fragments (every dy pixel of the band exactly once);
    // the lane holds channel 32*kb + l32, the pixels of half lhi
    constexpr bool DBW = DB && CB0 == 0;
    float dbacc[KB] = {};

    // One slot (one step): column block by column block, its two MFMAs (one
    // per k-block), then the next slot's read of that block's x fragment into
    // the same registers, and extra(i); the next dy fragments go to the other
    // set, read after the first block.  Every fragment is read NCB - 1 MFMA
    // pairs of this wave (and as many of its SIMD partner's) before its first
    // use.  No MFMA and no read is conditional: a branch around MFMAs makes
    // the compiler shuffle the accumulators between register files, one
    // around reads makes it drain every outstanding read before each slot.
    auto slot = [&](const DyFrag &od, DyFrag &nod, auto j_c, auto &&extra) __attribute__((always_inline)) {
        u32x4 a_[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) a_[kb] = join(od[kb][0], od[kb][1]);
#pragma unroll
        for (int i = 0; i < NCB; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            const u32x4 b = join(fx[i][0], fx[i][1]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) acc[kb][i] = Mfma32w<E>::run(a_[kb], b, acc[kb][i]);
            __builtin_amdgcn_sched_barrier(0);
            if (i == 0) read_dy(nod, j_c);
            read_x(i, j_c);
            extra(i);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DBW) {
            if (colh == 0) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const u32x4 u = a_[kb];
#pragma unroll
                    for (int e = 0; e < 4; ++e) dbacc[kb] = DotOne<E>::add(u[e], dbacc[kb]);
                }
            }
        }
    };
    using J0 = IntC<0>;
    using J1 = IntC<1>;
    using J2 = IntC<2>;
    using J3 = IntC<3>;
    auto none = [](int) __attribute__((always_inline)) {};

    DyFrag odA, odB;
    {
        int px, ch;
        dma_lane(0, px, ch);
        static_for<0, NB_WAVE>([&](auto jb) __attribute__((always_inline)) { dma_block(0, px, ch, jb); });
    }
    wait_vm_all();
    __syncthreads();
    {
        int px, ch;
        dma_lane(1, px, ch);
        static_for<0, NB_WAVE>([&](auto jb) __attribute__((always_inline)) { dma_block(1, px, ch, jb); });
    }
    read_dy(odA, J0{});
#pragma unroll
    for (int i = 0; i < NCB; ++i) read_x(i, J0{});
    // A last group of at most 12 steps computes only the slots its steps
    // need, two or three (the steps of a slot are its four phases).
    // (Column halves: two slots or the whole group; a third tail shape makes
    // the compiler spill their ten accumulator blocks.)
    int tail_slots = (nsteps - (ngroups - 1) * GSTEPS + PHASES - 1) / PHASES;  // 1 .. 4
    if (NSPLIT == 2 && tail_slots == 3) tail_slots = SLOTS;
    const int nfull = tail_slots == SLOTS ? ngroups : ngroups - 1;
    for (int g = 0; g < nfull; ++g) {
        slot(odA, odB, J1{}, none);
        slot(odB, odA, J2{}, none);
        slot(odA, odB, J3{}, none);
        // Last slot of the group.  The barrier (which waits for this wave's
        // LDS reads, this slot's fragments included, and for its loads of
        // group g + 1) frees this group's buffer for group g + 2 and makes
        // group g + 1 visible; the next group's first fragments are then read
        // during this slot (after the last group: slot 0 again, unused), and
        // the loads of group g + 2 are issued a few blocks at a time between
        // its MFMAs (dma_block does nothing past the band).
        int px = 0, ch = 0;
        if (g + 1 < ngroups) {  // workgroup-uniform
            wait_vm_all();
            __syncthreads();
            switch_buffer(g & 1 ? -BUF_BYTES : BUF_BYTES);
            dma_lane(g + 2, px, ch);
        }
        const int gd = g + 1 < ngroups ? g + 2 : ngroups;
        slot(odB, odA, J0{}, [&](int i) __attribute__((always_inline)) {  // i: 0 .. NCB - 1, unrolled
            static_for<0, NB_WAVE>([&](auto jb) __attribute__((always_inline)) {
                if (decltype(jb)::value * NCB / NB_WAVE == i) dma_block(gd, px, ch, jb);
            });
        });
    }
    // the short last group (its slot-0 fragments are in odA and fx); the
    // reads of its last slot fetch fragments nothing uses
    if (tail_slots <= 2) {
        slot(odA, odB, J1{}, none);
        slot(odB, odA, J1{}, none);
    } else if (NSPLIT == 3 && tail_slots == 3) {
        slot(odA, odB, J1{}, none);
        slot(odB, odA, J2{}, none);
        slot(odA, odB, J2{}, none);
    }

    // ---- the four phases' sums of each column set, in a fixed order
    // (p0 + p2) + (p1 + p3), through LDS (idle after the barrier): phases 2
    // and 3 park their blocks and phases 0 and 1 add them; then phase 0
    // keeps k-block 0 and phase 1 k-block 1, each parks the other k-block
    // and adds the one parked for it, and stores its rows of the partial.
    // A parked block is [4][64 lanes] of 16-byte pieces (4 consecutive
    // accumulator rows); the lane holds column l32 of its block, rows
    // 8*(r/4) + 4*(lane/32) + r%4.
    constexpr int NT_ = KB * NCB;  // this set's blocks
    constexpr int SET_BASE = CB0 == 0 ? 0 : 2 * KB * Cf::NCB_A * TILE_BYTES;
    f32x4 *const lds4 = (f32x4 *)smem + lane;
    auto part = [&](int h) { return lds4 + (SET_BASE + h * NT_ * TILE_BYTES) / 16; };
    auto park = [&](f32x4 *p, int t, const f32x16 &v) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 4; ++q) p[(t * 4 + q) * 64] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    };
    auto add = [&](const f32x4 *p, int t, f32x16 &v) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);  // one block at a time
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 u = p[(t * 4 + q) * 64];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] += u[e];
        }
    };
    __syncthreads();  // every wave is done with the buffers
    if (phase >= 2) {
#pragma unroll
        for (int t = 0; t < NT_; ++t) park(part(phase - 2), t, acc[t / NCB][t % NCB]);
    }
    __syncthreads();
    if (phase < 2) {
#pragma unroll
        for (int t = 0; t < NT_; ++t) add(part(phase), t, acc[t / NCB][t % NCB]);
    }
    __syncthreads();
    // (the k-block indices are compile-time: a runtime index would put the
    // accumulators in scratch memory)
    auto keep = [&](auto kb_c) __attribute__((always_inline)) {  // park the other k-block
        constexpr int KEEP = decltype(kb_c)::value;
#pragma unroll
        for (int i = 0; i < NCB; ++i) park(part(KEEP), i, acc[1 - KEEP][i]);
    };
    auto finish = [&](auto kb_c) __attribute__((always_inline)) {  // add the parked one, store
        constexpr int KEEP = decltype(kb_c)::value;
        float *const out = (float *)a.out + (size_t)band * a.part_stride + colh * (CB_WG * 32);
#pragma unroll
        for (int i = 0; i < NCB; ++i) {
            f32x16 &v = acc[KEEP][i];
            add(part(1 - KEEP), i, v);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                __builtin_nontemporal_store(
                    v[r], &out[(size_t)(KEEP * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3)) * NCOLS + (CB0 + i) * 32 + l32]);
        }
    };
    if (phase == 0) keep(IntC<0>{});
    if (phase == 1) keep(IntC<1>{});
    __syncthreads();
    if (phase == 0) finish(IntC<0>{});
    if (phase == 1) finish(IntC<1>{});
    if constexpr (DB) {
        // the bias-gradient partial of the band: lanes l32 and l32 + 32 hold
        // the two pixel halves of a channel; the four phases' sums are added
        // in phase order through LDS
        float *dbs = (float *)smem;  // [PHASES][CH]
        __syncthreads();             // every wave is done with the parked blocks
        if (DBW && colh == 0) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const float v = dbacc[kb] + __shfl_xor(dbacc[kb], 32);
                if (lhi == 0) dbs[phase * CH + kb * 32 + l32] = v;
            }
        }
        __syncthreads();
        if (colh == 0 && wave == 0) {
            float s = dbs[lane];
#pragma unroll
            for (int p = 1; p < PHASES; ++p) s += dbs[p * CH + lane];
            ((float *)a.out)[(size_t)band * a.part_stride + (size_t)CH * NCOLS + lane] = s;
        }
    }
}

template <class E, bool DB, int NSPLIT>
__global__ __launch_bounds__(512) void wgrad_band_kernel(const WgradBandArgs a)
{
    using Cf = wb::Cfg<NSPLIT>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::LDS_BYTES];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // waves 0-3 (one per SIMD) and 4-7 (the second of each SIMD) take the two column sets
    if (wave < wb::PHASES)
        wgrad_band_wave<E, DB, NSPLIT, Cf::NCB_A, 0>(a, smem, wave, lane);
    else
        wgrad_band_wave<E, DB, NSPLIT, Cf::NCB_B, Cf::NCB_A>(a, smem, wave, lane);
}

bool wgrad_band_supported(int R, int S, int C, int K, int dil, int Q)
{
    return R == wb::R && S == wb::S && C == wb::CH && K == wb::CH && dil == wb::DIL && Q >= 1 && Q <= wb::QMAX;
}

template <class E, bool DB>
static void launch_wgrad_band_e(const WgradBandArgs &a, hipStream_t st)
{
    if (a.nsplit == 3)
        wgrad_band_kernel<E, DB, 3><<<dim3((unsigned)(3 * a.nbands)), wb::NT, 0, st>>>(a);
    else
        wgrad_band_kernel<E, DB, 2><<<dim3((unsigned)(2 * a.N * a.chunks_per_img)), wb::NT, 0, st>>>(a);
}

hipError_t launch_wgrad_band(int dtype, const WgradBandArgs &a, hipStream_t st)
{
    if (a.nsplit != 2 && a.nsplit != 3) return hipErrorInvalidValue;
    switch (dtype) {
    case CONV2D_DTYPE_F16:
        if (a.with_db)
            launch_wgrad_band_e<EF16, true>(a, st);
        else
            launch_wgrad_band_e<EF16, false>(a, st);
        break;
    case CONV2D_DTYPE_BF16:
        if (a.with_db)
            launch_wgrad_band_e<EBF16, true>(a, st);
        else
            launch_wgrad_band_e<EBF16, false>(a, st);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cnv

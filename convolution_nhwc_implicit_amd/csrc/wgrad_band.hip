// wgrad_band.hip -- stride-1 weight gradient with dy and x rows resident in
// LDS and transposing LDS reads (gfx950).
//
// dw[k][r][s][c] = sum over output pixels (p,q) of dy[p,q,k] * x[p-ph+r*d, q-pw+s*d, c]
// is a GEMM with rows k, columns (r,s,c) and a reduction over pixels.  Both
// operands arrive pixel-major (NHWC), while an MFMA operand needs eight
// consecutive reduction elements (pixels) per lane.  gfx950's
// ds_read_b64_tr_b16 gives exactly that from a pixel-major tile: in each group
// of 16 lanes, lane L points at 4 channels of pixel L/4 and lane i receives
// channel i of the 4 pixels.  So dy and x rows are copied into LDS as they are,
// every input byte once (plus the halo rows), and all R*S tap shifts of x are
// just different read addresses.
//
// Rows are laid out with the padded pitch XW = Q + dil*(S-1) in both LDS
// buffers: dy gets XW - Q zero pixels after each row, so output pixel
// (p, q) sits at v = p*XW + q and its tap (r, s) of x at v + r*dil*XW +
// s*dil.  Every address is then linear in v: a 16-pixel step moves every
// read by the same 2 KB (an immediate offset), the few padding pixels add
// zeros, and the main loop needs no per-step index arithmetic.
//
// A workgroup (12 waves, three per SIMD) owns a band of output rows of one
// image and all K x R*S*C outputs.  Output blocks are 32x32 (32x32x16 MFMA,
// fp32 accumulators): wave w owns k-block w/6 and the three column blocks
// 3*(w%6)..+2 (which share one tap row r), over every pixel of the band.  The
// band is walked in groups of GR output rows; each group's dy rows and its
// GR + halo x rows are brought by direct-to-LDS loads (buffer_load ... lds;
// pixels outside the image and the padding come from the buffer range check
// as zeros) into one of two buffers, while the previous group is computed
// from the other.  Each workgroup writes its fp32 partial sums; the split-K
// reduction adds the workgroups' partials in workgroup order.
//
// 16-byte channel chunks of pixel v are stored with chunk bit 2 flipped
// when bit 1 of v is set: the transposing reads of 4 consecutive pixels x
// 32 channels then cover all 64 LDS banks.
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
constexpr int NT = 768;          // 12 waves
constexpr int WAVES = NT / 64;
constexpr int CH = 64;           // C = K = 64 channels, 128 bytes per pixel
constexpr int PIXB = CH * 2;
constexpr int GR = 4;            // output rows per group
constexpr int R = 3, S = 3, DIL = 1;
constexpr int HALO = DIL * (R - 1);
constexpr int NCOLB = R * S * CH / 32;   // 18 column blocks of 32 in all
constexpr int CB_WG = NCOLB / 2;         // a workgroup computes one half of them
constexpr int WAVE_CB = 3;               // column blocks per wave
constexpr int WAVE_KB = 2;               // k-blocks per wave (all of K = 64)
constexpr int NACC = WAVE_KB * WAVE_CB;
constexpr int WSETS = CB_WG / WAVE_CB;   // 3 waves cover the workgroup's columns ...
constexpr int PHASES = WAVES / WSETS;    // ... and 4 such sets split the 16-pixel steps (t mod 4)
constexpr int BODY = 4;                  // steps per straight-line body (per phase)
// buffer capacities in pixels (whole 1 KB direct-to-LDS blocks of 8 pixels),
// sized for Q <= QMAX: a group covers steps*16 virtual pixels of dy (steps a
// multiple of PHASES*BODY) and those plus the tap shifts of x
constexpr int QMAX = 56;
constexpr int DCAP = 256;        // >= 16 * round_up(ceil(GR*(QMAX+2)/16), PHASES*BODY)
constexpr int XCAP = 376;        // >= DCAP + HALO*(QMAX+2) + DIL*(S-1)
constexpr int D_BYTES = DCAP * PIXB, X_BYTES = XCAP * PIXB;
constexpr int BUF_BYTES = D_BYTES + X_BYTES;
constexpr int LDS_BYTES = 2 * BUF_BYTES;
constexpr int PARK_WAVE = 64 * NACC * 16 * 4;  // one wave's accumulators
static_assert(CB_WG == WSETS * WAVE_CB && WAVES == WSETS * PHASES && PHASES == 4, "3 x 4 waves");
static_assert(2 * WSETS * PARK_WAVE <= LDS_BYTES, "two phases' accumulators fit in LDS");
static_assert(DCAP % 8 == 0 && XCAP % 8 == 0, "whole 1 KB blocks");
static_assert(LDS_BYTES <= 163840, "fits in the 160 KB LDS");

template <int V>
struct IntC {
    static constexpr int value = V;
};
__device__ inline int swz_chunk(int chunk, int v) { return chunk ^ (((v >> 1) & 1) << 2); }
}  // namespace wb


template <class E>
__global__ __launch_bounds__(768, 1) void wgrad_band_kernel(const WgradBandArgs a)
{
    using namespace wb;
    using elem = typename E::elem;
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroup -> (band, column half).  Workgroups are dealt to the 8 XCDs
    // in turn, so the two halves of a band go 8 apart: same XCD, and the
    // second one's row loads hit that XCD's L2.
    int band, colh;
    if (a.xcd_pairs) {
        const int bid = blockIdx.x;
        colh = (bid >> 3) & 1;
        band = (bid & 7) + 8 * (bid >> 4);
    } else {
        colh = blockIdx.x & 1;
        band = blockIdx.x >> 1;
    }
    const int img = band / a.chunks_per_img;
    const int chunk = band - img * a.chunks_per_img;
    const int p_start = chunk * a.rows_per_wg;
    const int p_end = min(p_start + a.rows_per_wg, a.P);
    const int nrows = p_end - p_start;  // >= 1 by construction of the grid
    const int Q = a.Q, XW = a.xw;
    const int h_base = p_start - a.pad_h;  // input row of x band row 0

    // ---- loads.  Group g covers band rows [g*GR, g*GR + GR): dy virtual
    // pixels [0, DCAP) and x virtual pixels [0, XCAP) of its buffer, 1 KB
    // block b going to wave b % WAVES.  Lane i of a block fills stored chunk
    // i%8 of pixel 8*blk + i/8, i.e. source chunk swz_chunk(i%8, pixel).
    const u32x4 x_rs = make_buf_rsrc((const elem *)a.x + (size_t)img * a.H * a.W * CH, (uint32_t)(a.H * a.W * CH * 2));
    const u32x4 d_rs =
        make_buf_rsrc((const elem *)a.dy + ((size_t)img * a.P + p_start) * Q * CH, (uint32_t)(nrows * Q * CH * 2));
    // The pixel a lane moves in each of its wave's blocks is the same in every
    // group (buffers start at a group's first row), so its (row, column) in
    // the group is computed once, row << 8 | column in 16 bits, two blocks
    // per register: block wave + WAVES*j in bits 16*(j%2) of rc[j/2].  Bit 1
    // of the pixel index, which sets the chunk swizzle, is bit 1 of lane/8
    // (blocks are 8 pixels).
    constexpr int DBLK = DCAP / 8, NBLK = (DCAP + XCAP) / 8;
    constexpr int MAXB = (NBLK + WAVES - 1) / WAVES;  // blocks per wave
    static_assert(XCAP < 256 * 6 && QMAX + 2 < 256, "row and column fit in 8 bits");
    uint32_t rc[(MAXB + 1) / 2] = {};
#pragma unroll
    for (int jb = 0; jb < MAXB; ++jb) {
        const int b = wave + WAVES * jb;
        const int v = (b < DBLK ? b : b - DBLK) * 8 + (lane >> 3);
        const int row = (int)fdiv((uint32_t)v, a.div_xw);
        rc[jb / 2] |= (((uint32_t)row << 8) | (uint32_t)(v - row * XW)) << (16 * (jb & 1));
    }
    const int lane_chunk16 = swz_chunk(lane & 7, lane >> 3) * 16;  // byte offset of the chunk in its pixel
    const uint32_t lds0 = lds_addr(smem);
    auto dma_group = [&](int g) {
        const int d0 = g * GR;
        if (d0 >= nrows) return;
        const int ndy = min(GR, nrows - d0);  // dy rows of the group
        const int nx = ndy + HALO;            // x rows it reads
        const uint32_t buf = lds0 + (uint32_t)((g & 1) * BUF_BYTES);  // LDS byte address
#pragma unroll
        for (int jb = 0; jb < MAXB; ++jb) {
            const int b = wave + WAVES * jb;  // wave-uniform
            if (b >= NBLK) break;
            const uint32_t e = rc[jb / 2] >> (16 * (jb & 1));
            const int row = (int)((e >> 8) & 0xffu), col = (int)(e & 0xffu);
            unsigned voff = kBufOOB;
            if (b < DBLK) {
                if (row < ndy && col < Q) voff = (unsigned)(((d0 + row) * Q + col) * PIXB + lane_chunk16);
                dma16(d_rs, buf + b * 1024, voff);
            } else {
                const int h = h_base + d0 + row, w = col - a.pad_w;
                if (row < nx && (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W)
                    voff = (unsigned)((h * a.W + w) * PIXB + lane_chunk16);
                dma16(x_rs, buf + b * 1024, voff);
            }
        }
    };

    dma_group(0);
    wait_vm_all();
    __syncthreads();
    dma_group(1);

    // ---- per-wave roles: both k-blocks, column blocks cb0..cb0+2 of the
    // workgroup's half (all of one tap row r: column block cb is tap cb/2 =
    // (r, s), channel half cb&1), and the steps t = phase (mod 4)
    const int phase = wave / WSETS;
    const int cb0 = colh * CB_WG + WAVE_CB * (wave % WSETS);
    const int tap_r = (cb0 >> 1) / S;
    const int l32 = lane & 31, lhi = lane >> 5;

    // ---- per-lane read offsets (first step of this phase in a buffer).
    // Read rd of a step covers pixels v = 16*t + 8*lhi + 4*rd + 0..3; this
    // lane points at pixel v + L/4.  Read rd = 1 and later steps move every
    // read by a multiple of 4 pixels, which keeps bit 1 of the pixel index and
    // so the swizzle: they are constant byte offsets (4 pixels = 512 B) from
    // the rd = 0 offsets of the body's first step.
    auto dy_off = [&](int ln, int rd, int kb) {
        const int L_ = ln & 15, g_ = (ln >> 4) & 1, h_ = ln >> 5;
        const int c_ = 16 * g_ + 4 * (L_ & 3);
        const int v = 16 * phase + 8 * h_ + 4 * rd + (L_ >> 2);
        return v * PIXB + swz_chunk(kb * 4 + (c_ >> 3), v) * 16 + (c_ & 7) * 2;
    };
    auto x_off = [&](int ln, int rd, int i) {
        const int L_ = ln & 15, g_ = (ln >> 4) & 1, h_ = ln >> 5;
        const int c_ = 16 * g_ + 4 * (L_ & 3);
        const int v = 16 * phase + 8 * h_ + 4 * rd + (L_ >> 2);
        const int cb = cb0 + i, tap_s = (cb >> 1) - tap_r * S;
        const int xv = v + tap_r * DIL * XW + tap_s * DIL;
        return D_BYTES + xv * PIXB + swz_chunk((cb & 1) * 4 + (c_ >> 3), xv) * 16 + (c_ & 7) * 2;
    };

    f32x16 acc[WAVE_KB][WAVE_CB];
#pragma unroll
    for (int kb = 0; kb < WAVE_KB; ++kb)
#pragma unroll
        for (int n = 0; n < WAVE_CB; ++n) acc[kb][n] = f32x16{};
    // bias gradient (with_db): the first column set of each phase in the
    // first column half adds up the dy values its fragments hold (every dy
    // pixel of the band exactly once); lane holds channel 32*kb + l32, the
    // pixels of half lhi of each step
    const bool dbw = a.with_db && colh == 0 && wave % WSETS == 0;  // wave-uniform
    float dbacc[WAVE_KB] = {};

    typedef __attribute__((address_space(3))) unsigned char lds_u8;  // 32-bit LDS addresses
    auto tr = [](const lds_u8 *p) -> s16x4 {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    };
    // one step's fragments as raw 64-bit halves: [2*kb + rd] dy, [4 + 2*i + rd] x
    typedef s16x4 Frag[2 * WAVE_KB + 2 * WAVE_CB];
    // lane addresses of a body's first step; step k (k-th of this phase) adds
    // k*PHASES*2 KB, which the reads take as an immediate offset (the empty
    // asm keeps the compiler from re-associating base + offset + k*8 KB into
    // one register per step)
    constexpr int STEPB = PHASES * 16 * PIXB;
    constexpr int RDB = 4 * PIXB;  // read rd = 1: 4 pixels further
    // The offsets are recomputed per body from an opaque copy of the lane id
    // (holding them across the loop would cost registers the fragments need).
    const lds_u8 *ad[WAVE_KB], *ax[WAVE_CB];
    auto set_body = [&](const lds_u8 *base) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int kb = 0; kb < WAVE_KB; ++kb) {
            ad[kb] = base + dy_off(ln, 0, kb);
            asm volatile("" : "+v"(ad[kb]));
        }
#pragma unroll
        for (int i = 0; i < WAVE_CB; ++i) {
            ax[i] = base + x_off(ln, 0, i);
            asm volatile("" : "+v"(ax[i]));
        }
    };
    auto load_step = [&](Frag &f, int k) {
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
#pragma unroll
            for (int kb = 0; kb < WAVE_KB; ++kb) f[2 * kb + rd] = tr(ad[kb] + rd * RDB + k * STEPB);
#pragma unroll
            for (int i = 0; i < WAVE_CB; ++i) f[2 * WAVE_KB + 2 * i + rd] = tr(ax[i] + rd * RDB + k * STEPB);
        }
    };
    auto join = [](s16x4 lo, s16x4 hi) -> u32x4 {
        const uint2 l = __builtin_bit_cast(uint2, lo), h = __builtin_bit_cast(uint2, hi);
        return u32x4{l.x, l.y, h.x, h.y};
    };
    // MFMAs [m0, m1) of a step (kb-major over the WAVE_KB x WAVE_CB blocks)
    auto mma = [&](const Frag &f, int m0, int m1) {
#pragma unroll
        for (int kb = 0; kb < WAVE_KB; ++kb) {
            const u32x4 fa = join(f[2 * kb], f[2 * kb + 1]);
#pragma unroll
            for (int i = 0; i < WAVE_CB; ++i) {
                const int m = kb * WAVE_CB + i;
                if (m >= m0 && m < m1)
                    acc[kb][i] =
                        Mfma32w<E>::run(fa, join(f[2 * WAVE_KB + 2 * i], f[2 * WAVE_KB + 2 * i + 1]), acc[kb][i]);
            }
        }
    };

    // Steps run in straight-line bodies of BODY (of one phase): the reads of
    // step k+1 are issued right after the first MFMA of step k (so that MFMA
    // waits for step k's reads alone), and nothing is in flight across
    // bodies.  Steps past the group's pixels read zero dy
    // pixels.
    const int ngroups = (nrows + GR - 1) / GR;
    for (int g = 0; g < ngroups; ++g) {
        const unsigned char *buf = smem + (g & 1) * BUF_BYTES;
        const int nbody = a.steps_per_group / (PHASES * BODY);
        for (int bd = 0; bd < nbody; ++bd) {
            set_body((const lds_u8 *)buf + bd * BODY * STEPB);
            Frag f[BODY];
            load_step(f[0], 0);
#pragma unroll
            for (int k = 0; k < BODY; ++k) {
                // step k's first MFMA, then step k+1's reads, then the rest:
                // the first MFMA waits for step k's reads alone
                __builtin_amdgcn_sched_barrier(0);
                mma(f[k], 0, 1);
                __builtin_amdgcn_sched_barrier(0);
                if (k + 1 < BODY) load_step(f[k + 1], k + 1);
                __builtin_amdgcn_sched_barrier(0);
                mma(f[k], 1, NACC);
                if (dbw) {
#pragma unroll
                    for (int kb = 0; kb < WAVE_KB; ++kb)
#pragma unroll
                        for (int rd = 0; rd < 2; ++rd) {
                            const uint2 u = __builtin_bit_cast(uint2, f[k][2 * kb + rd]);
                            dbacc[kb] = DotOne<E>::add(u.x, dbacc[kb]);
                            dbacc[kb] = DotOne<E>::add(u.y, dbacc[kb]);
                        }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_vm_all();     // the next group's rows
        __syncthreads();   // every wave is done with this group's buffer
        dma_group(g + 2);  // into the buffer this group used
    }

    // ---- the four phases' sums, in a fixed order (p0 + p2) + (p1 + p3),
    // through LDS (the buffers are idle now).  Step 1: phases 2 and 3 park
    // all their accumulators, phases 0 and 1 add them.  Step 2: phase 0
    // keeps k-block 0 and phase 1 k-block 1; each parks the other block and
    // adds the one parked for it, then stores its rows of the partial tile.
    // A parked block set is [blocks*4][64 lanes] of 16-byte pieces (4
    // consecutive accumulator rows).
    constexpr int PARK_HALF = PARK_WAVE / WAVE_KB;  // one k-block's accumulators
    const int ws_ = wave % WSETS;
    auto slot = [&](int s, int bytes) { return (f32x4 *)(smem + s * bytes) + lane; };
    // park / add k-blocks [KB0, KB0 + NKB) (compile-time, so acc stays in registers)
    auto park = [&](f32x4 *p, auto kb0_c, auto nkb_c) {
        constexpr int KB0 = decltype(kb0_c)::value, NKB = decltype(nkb_c)::value;
#pragma unroll
        for (int kb = KB0; kb < KB0 + NKB; ++kb)
#pragma unroll
            for (int i = 0; i < WAVE_CB; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16 &v = acc[kb][i];
                    p[(((kb - KB0) * WAVE_CB + i) * 4 + q) * 64] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
                }
    };
    auto add = [&](const f32x4 *p, auto kb0_c, auto nkb_c) {
        constexpr int KB0 = decltype(kb0_c)::value, NKB = decltype(nkb_c)::value;
#pragma unroll
        for (int kb = KB0; kb < KB0 + NKB; ++kb)
#pragma unroll
            for (int i = 0; i < WAVE_CB; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 t = p[(((kb - KB0) * WAVE_CB + i) * 4 + q) * 64];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[kb][i][4 * q + e] += t[e];
                }
    };
    // the partial tile's rows k = 32*KB + 0..31 in this wave's columns: lane
    // holds column l32, rows 8*(r/4) + 4*(lane/32) + r%4 of each block
    auto store = [&](auto kb_c) {
        constexpr int KB = decltype(kb_c)::value;
        constexpr int NCOLS = R * S * CH;
        constexpr int TCOLS = CB_WG * 32;
        float *out = (float *)a.out + (size_t)band * a.part_stride + colh * TCOLS;
#pragma unroll
        for (int i = 0; i < WAVE_CB; ++i) {
            const int col = (WAVE_CB * ws_ + i) * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int k = KB * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);
                out[(size_t)k * NCOLS + col] = acc[KB][i][r];
            }
        }
    };
    using I0 = wb::IntC<0>;
    using I1 = wb::IntC<1>;
    using I2 = wb::IntC<2>;
    if (phase >= 2) park(slot((phase - 2) * WSETS + ws_, PARK_WAVE), I0{}, I2{});
    __syncthreads();
    if (phase < 2) add(slot(phase * WSETS + ws_, PARK_WAVE), I0{}, I2{});
    __syncthreads();
    if (phase == 0) park(slot(ws_, PARK_HALF), I1{}, I1{});
    if (phase == 1) park(slot(WSETS + ws_, PARK_HALF), I0{}, I1{});
    __syncthreads();
    if (phase == 0) {
        add(slot(WSETS + ws_, PARK_HALF), I0{}, I1{});
        store(I0{});
    }
    if (phase == 1) {
        add(slot(ws_, PARK_HALF), I1{}, I1{});
        store(I1{});
    }
    if (a.with_db) {  // uniform: the barriers are reached by every wave
        // the bias-gradient partial of the band: lanes l32 and l32 + 32 of a
        // summing wave hold the two pixel halves of a channel; the four
        // phases' sums are added in phase order through LDS
        float *dbs = (float *)smem;  // [PHASES][CH]
        __syncthreads();             // every wave is done with the slots
        if (dbw) {
#pragma unroll
            for (int kb = 0; kb < WAVE_KB; ++kb) {
                const float v = dbacc[kb] + __shfl_xor(dbacc[kb], 32);
                if (lhi == 0) dbs[phase * CH + kb * 32 + l32] = v;
            }
        }
        __syncthreads();
        if (colh == 0 && wave == 0) {
            constexpr int NCOLS = R * S * CH;
            float s = dbs[lane];
#pragma unroll
            for (int p = 1; p < PHASES; ++p) s += dbs[p * CH + lane];
            ((float *)a.out)[(size_t)band * a.part_stride + (size_t)CH * NCOLS + lane] = s;
        }
    }
}

// Steps of 16 pixels per group for output width Q, rounded up to whole
// bodies; 0 if the group does not fit the buffers.
int wgrad_band_steps(int Q)
{
    const int xw = Q + wb::DIL * (wb::S - 1);
    int steps = (wb::GR * xw + 15) / 16;
    constexpr int unit = wb::PHASES * wb::BODY;
    steps = (steps + unit - 1) / unit * unit;
    if (steps * 16 > wb::DCAP || steps * 16 + wb::HALO * xw + wb::DIL * (wb::S - 1) > wb::XCAP) return 0;
    return steps;
}

bool wgrad_band_supported(int R, int S, int C, int K, int dil, int Q)
{
    return R == wb::R && S == wb::S && C == wb::CH && K == wb::CH && dil == wb::DIL && Q % 4 == 0 &&
           Q <= wb::QMAX && Q >= 4 && wgrad_band_steps(Q) > 0;
}

hipError_t launch_wgrad_band(int dtype, const WgradBandArgs &a, hipStream_t st)
{
    dim3 grid((unsigned)(2 * a.N * a.chunks_per_img));  // two column halves per band
    switch (dtype) {
    case CONV2D_DTYPE_F16: wgrad_band_kernel<EF16><<<grid, wb::NT, 0, st>>>(a); break;
    case CONV2D_DTYPE_BF16: wgrad_band_kernel<EBF16><<<grid, wb::NT, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cnv

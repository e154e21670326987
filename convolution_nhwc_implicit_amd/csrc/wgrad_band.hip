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
// every input byte once, and all R*S tap shifts of x are just different read
// addresses.
//
// A workgroup (12 waves, three per SIMD) owns a band of output rows of one
// image and all K x R*S*C outputs.  Output blocks are 32x32 (32x32x16 MFMA,
// fp32 accumulators): wave w owns k-block w/6 and the three column blocks
// 3*(w%6)..+2, over every pixel of the band.  Rows stream through two LDS
// rings (dy: 2 groups of 4 rows, x: 4 rows + halo + 4 prefetched rows); the
// next group's rows are loaded into registers while the current one is
// computed.  Each workgroup writes its fp32 partial sums; the split-K
// reduction adds the workgroups' partials in workgroup order.
//
// 16-byte channel chunks of pixel `col` are stored with chunk bit 2 flipped
// when bit 1 of col is set: the transposing reads of 4 consecutive pixels x
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
constexpr int CH = 64;           // C = K = 64 channels, 128 bytes per pixel
constexpr int PIXB = CH * 2;
constexpr int GR = 4;            // output rows per group
constexpr int R = 3, S = 3, DIL = 1;
constexpr int HALO = DIL * (R - 1);
constexpr int XSLOTS = 2 * GR + HALO;
constexpr int DSLOTS = 2 * GR;
constexpr int QMAX = 56;         // widest output row handled (sizes the prefetch)
constexpr int XW_MAX = QMAX + DIL * (S - 1);
constexpr int X_BYTES = XSLOTS * XW_MAX * PIXB;
constexpr int D_BYTES = DSLOTS * QMAX * PIXB;
constexpr int ZERO_BYTES = PIXB;
constexpr int LDS_BYTES = X_BYTES + D_BYTES + ZERO_BYTES;
constexpr int NCOLB = R * S * CH / 32;   // 18 column blocks of 32 (static check below)
constexpr int WAVE_CB = 3;               // column blocks per wave
static_assert(NCOLB == 6 * WAVE_CB, "six waves x three column blocks per k-block");
static_assert(LDS_BYTES <= 163840, "fits in the 160 KB LDS");
// Row loading: a group brings GR dy rows and GR x rows; each of these 2*GR rows
// is moved by NT/(2*GR) threads, thread t owning channel chunk t%8 of columns
// (t % TPR)/8 + i*COLS_STEP.
constexpr int TPR = NT / (2 * GR);               // 96 threads per row
constexpr int COLS_STEP = TPR / 8;               // 12 columns apart
constexpr int PRE_CPT = (XW_MAX + COLS_STEP - 1) / COLS_STEP;  // chunks per thread
static_assert(TPR % 8 == 0, "whole pixels per thread stride");

__device__ inline int swz_chunk(int chunk, int col) { return chunk ^ (((col >> 1) & 1) << 2); }
}  // namespace wb

template <class E>
__global__ __launch_bounds__(768, 1) void wgrad_band_kernel(const WgradBandArgs a)
{
    using namespace wb;
    using elem = typename E::elem;
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
    unsigned char *xring = smem;
    unsigned char *dring = smem + X_BYTES;
    unsigned char *zpix = smem + X_BYTES + D_BYTES;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int img = blockIdx.x / a.chunks_per_img;
    const int chunk = blockIdx.x - img * a.chunks_per_img;
    const int p_start = chunk * a.rows_per_wg;
    const int p_end = min(p_start + a.rows_per_wg, a.P);
    const int nrows = p_end - p_start;  // >= 1 by construction of the grid
    const int Q = a.Q;
    const int XW = Q + DIL * (S - 1);
    const int xslotb = XW * PIXB, dslotb = Q * PIXB;
    const int h_base = p_start - a.pad_h;  // input row of x band row 0
    const int w_base = -a.pad_w;           // input column of x ring column 0
    const elem *x = (const elem *)a.x + (size_t)img * a.H * a.W * CH;
    const elem *dy = (const elem *)a.dy + ((size_t)img * a.P + p_start) * Q * CH;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    if (tid < ZERO_BYTES / 16) *(u32x4 *)(zpix + tid * 16) = zero;

    // ---- row loading (see TPR / COLS_STEP).  Thread t moves chunk my_j of
    // columns my_col0 + i*COLS_STEP of row my_row of the group's new rows:
    // rows 0..GR-1 are dy rows, GR..2GR-1 are x rows.
    const int my_row = tid / TPR, my_j = tid % 8;
    const int my_col0 = (tid % TPR) / 8;
    const bool my_is_dy = my_row < GR;
    const int my_rr = my_is_dy ? my_row : my_row - GR;
    const int my_w = my_is_dy ? Q : XW;  // pixels in the row
    u32x4 pre[PRE_CPT];
    auto fetch = [&](int drow0, int xrow0) {
        const int br = (my_is_dy ? drow0 : xrow0) + my_rr;
        const int h = h_base + br;
        const bool row_ok = my_is_dy ? br < nrows : (unsigned)h < (unsigned)a.H;
        const elem *rowsrc = my_is_dy ? dy + (size_t)br * Q * CH : x + (size_t)h * a.W * CH;
#pragma unroll
        for (int i = 0; i < PRE_CPT; ++i) {
            const int col = my_col0 + i * COLS_STEP;
            const int w = my_is_dy ? col : w_base + col;
            const bool ok = row_ok && col < my_w && (unsigned)w < (unsigned)(my_is_dy ? Q : a.W);
            pre[i] = ok ? *(const u32x4 *)(rowsrc + (size_t)w * CH + my_j * 8) : zero;
        }
    };
    auto store = [&](int drow0, int xrow0) {
        const int br = (my_is_dy ? drow0 : xrow0) + my_rr;
        unsigned char *rowdst = my_is_dy ? dring + (br % DSLOTS) * dslotb : xring + (br % XSLOTS) * xslotb;
#pragma unroll
        for (int i = 0; i < PRE_CPT; ++i) {
            const int col = my_col0 + i * COLS_STEP;
            if (col < my_w) *(u32x4 *)(rowdst + col * PIXB + swz_chunk(my_j, col) * 16) = pre[i];
        }
    };

    // prologue: x halo rows [0, HALO) (the x-row threads load them, HALO <= GR),
    // then group 0: dy rows [0, GR), x rows [HALO, HALO + GR)
    if (!my_is_dy && my_rr < HALO) {
        fetch(0, 0);
        store(0, 0);
    }
    fetch(0, HALO);
    store(0, HALO);
    __syncthreads();

    // ---- per-wave roles
    const int kb = wave / 6;
    const int cb0 = WAVE_CB * (wave % 6);
    const int l32 = lane & 31, g16 = l32 >> 4, L = lane & 15, lhi = lane >> 5;
    const int cin = 16 * g16 + 4 * (L & 3);      // channel offset inside a 32-channel block
    const int cchunk = cin >> 3, cbyte = (cin & 7) * 2;
    // column block -> (tap row r, tap column s, channel half): tap = cb / 2
    int cb_r[WAVE_CB], cb_s[WAVE_CB], cb_chunk[WAVE_CB];
#pragma unroll
    for (int i = 0; i < WAVE_CB; ++i) {
        const int cb = cb0 + i, tap = cb >> 1;
        cb_r[i] = tap / S;
        cb_s[i] = tap - cb_r[i] * S;
        cb_chunk[i] = (cb & 1) * 4 + cchunk;
    }

    f32x16 acc[WAVE_CB];
#pragma unroll
    for (int n = 0; n < WAVE_CB; ++n) acc[n] = f32x16{};

    const int band_pix = nrows * Q;
    const int nsteps = (band_pix + 15) / 16;
    const int steps_per_group = GR * Q / 16;  // Q % 4 == 0
    const int ngroups = (nrows + GR - 1) / GR;

    auto tr = [](const unsigned char *p) -> s16x4 {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    };

    // ---- per-lane read state.  Lane reads pixels f and f + 4 of each 16-pixel
    // step (f = 16*t + 8*lhi + L/4).  Pixels only ever move by multiples of 4
    // (16 per step, -Q on a row wrap, Q % 4 == 0), so each read's channel
    // swizzle is fixed: its byte offsets inside a pixel are precomputed, and
    // only the column and the ring rows are updated per step.
    int pq[2], prr[2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
        pq[rd] = 8 * lhi + 4 * rd + (L >> 2);
        prr[rd] = 0;
        while (pq[rd] >= Q) {
            pq[rd] -= Q;
            ++prr[rd];
        }
    }
    int aoff[2], boff[2][WAVE_CB];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
        aoff[rd] = swz_chunk(kb * 4 + cchunk, pq[rd]) * 16 + cbyte;
#pragma unroll
        for (int i = 0; i < WAVE_CB; ++i) {
            // tap column shift plus the swizzled chunk of the shifted pixel;
            // the current column pq is added per step
            const int col = pq[rd] + cb_s[i] * DIL;
            boff[rd][i] = cb_s[i] * DIL * PIXB + swz_chunk(cb_chunk[i], col) * 16 + cbyte;
        }
    }
    // byte offsets of each read inside the ring (without the column pq*PIXB):
    // dy row prr; x row prr + r_i*DIL of column block i.  Static indices only
    // (a register array indexed by a runtime value becomes a select chain),
    // recomputed on a row wrap.
    int doff[2], xoff[2][WAVE_CB];
    auto set_rows = [&](int rd) {
        doff[rd] = X_BYTES + (prr[rd] % DSLOTS) * dslotb + aoff[rd];
#pragma unroll
        for (int i = 0; i < WAVE_CB; ++i)
            xoff[rd][i] = ((prr[rd] + cb_r[i] * DIL) % XSLOTS) * xslotb + boff[rd][i];
    };
    set_rows(0);
    set_rows(1);
    auto advance = [&]() {
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            pq[rd] += 16;
            if (pq[rd] >= Q) {
                do {
                    pq[rd] -= Q;
                    ++prr[rd];
                } while (pq[rd] >= Q);
                set_rows(rd);
            }
        }
    };
    const int zoff = X_BYTES + D_BYTES + cbyte;  // the zero pixel
    auto load_step = [&](u32x4 &fa, u32x4 (&fb)[WAVE_CB]) {
        s16x4 ra[2], rb[WAVE_CB][2];
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            const bool ok = prr[rd] < nrows;
            const int qb = pq[rd] * PIXB;
            ra[rd] = tr(smem + (ok ? doff[rd] + qb : zoff));
#pragma unroll
            for (int i = 0; i < WAVE_CB; ++i) rb[i][rd] = tr(smem + (ok ? xoff[rd][i] + qb : zoff));
        }
        const uint2 alo = __builtin_bit_cast(uint2, ra[0]), ahi = __builtin_bit_cast(uint2, ra[1]);
        fa = u32x4{alo.x, alo.y, ahi.x, ahi.y};
#pragma unroll
        for (int i = 0; i < WAVE_CB; ++i) {
            const uint2 lo = __builtin_bit_cast(uint2, rb[i][0]), hi = __builtin_bit_cast(uint2, rb[i][1]);
            fb[i] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
    };
    auto mma = [&](const u32x4 &fa, const u32x4 (&fb)[WAVE_CB]) {
#pragma unroll
        for (int i = 0; i < WAVE_CB; ++i) acc[i] = Mfma32w<E>::run(fa, fb[i], acc[i]);
    };

    for (int g = 0; g < ngroups; ++g) {
        const bool more = g + 1 < ngroups;
        if (more) fetch((g + 1) * GR, (g + 1) * GR + HALO);
        const int t0 = g * steps_per_group;
        const int t1 = min(t0 + steps_per_group, nsteps);
        for (int t = t0; t < t1; ++t) {
            u32x4 fa, fb[WAVE_CB];
            load_step(fa, fb);
            advance();
            mma(fa, fb);
        }
        if (more) store((g + 1) * GR, (g + 1) * GR + HALO);  // slots of rows the previous group used
        __syncthreads();
    }

    // ---- the workgroup's fp32 partials [K][R*S*C]; 32x32 block layout: lane
    // holds column (lane & 31), rows 8*(r/4) + 4*(lane/32) + r%4
    {
        constexpr int NCOLS = R * S * CH;
        float *out = (float *)a.out + (size_t)blockIdx.x * a.part_stride;
#pragma unroll
        for (int i = 0; i < WAVE_CB; ++i) {
            const int col = (cb0 + i) * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int k = kb * 32 + 8 * (r >> 2) + 4 * lhi + (r & 3);
                out[(size_t)k * NCOLS + col] = acc[i][r];
            }
        }
    }
}

bool wgrad_band_supported(int R, int S, int C, int K, int dil, int Q)
{
    return R == wb::R && S == wb::S && C == wb::CH && K == wb::CH && dil == wb::DIL && Q % 4 == 0 &&
           Q <= wb::QMAX && Q >= 4;
}

hipError_t launch_wgrad_band(int dtype, const WgradBandArgs &a, hipStream_t st)
{
    dim3 grid((unsigned)(a.N * a.chunks_per_img));
    switch (dtype) {
    case CONV2D_DTYPE_F16: wgrad_band_kernel<EF16><<<grid, wb::NT, 0, st>>>(a); break;
    case CONV2D_DTYPE_BF16: wgrad_band_kernel<EBF16><<<grid, wb::NT, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cnv

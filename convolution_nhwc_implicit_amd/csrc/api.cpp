// api.cpp -- the C ABI of the conv2d library: argument validation, planning
// (kernel, tile, split-K, dgrad stride phases, workspace layout) and launches
// on the caller's stream.
//
// Dispatch rule (after the burn CubeCL conv dispatch, conv_forward_nhwc /
// conv_weight_backward / conv_data_backward): groups > 1 runs the direct
// kernels; groups == 1 runs the implicit GEMM for all three passes, including
// strided dgrad (which that dispatch sends to a fallback).  Every check runs
// before anything is enqueued, and an unsupported case is reported, never run
// on another algorithm.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "conv2d_nhwc.h"
#include "internal.h"

using namespace cnv;

namespace {

constexpr long long kMaxElems = (1LL << 31) - 1;
constexpr int kNumCUs = 256;  // MI355X

struct Dims {
    long long N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, G, P, Q, Cg, Kg;
};

int validate(const conv2d_problem_t *p, Dims *d)
{
    if (!p) return CONV2D_ERR_INVALID_ARGUMENT;
    if (p->n < 1 || p->c < 1 || p->h < 1 || p->w < 1 || p->k < 1 || p->r < 1 || p->s < 1)
        return CONV2D_ERR_INVALID_ARGUMENT;
    if (p->pad_h < 0 || p->pad_w < 0 || p->stride_h < 1 || p->stride_w < 1 || p->dil_h < 1 ||
        p->dil_w < 1 || p->groups < 1)
        return CONV2D_ERR_INVALID_ARGUMENT;
    if (p->c % p->groups || p->k % p->groups) return CONV2D_ERR_INVALID_ARGUMENT;
    const long long span_h = (long long)p->dil_h * (p->r - 1) + 1;
    const long long span_w = (long long)p->dil_w * (p->s - 1) + 1;
    const long long ph = (long long)p->h + 2LL * p->pad_h, pw = (long long)p->w + 2LL * p->pad_w;
    if (ph < span_h || pw < span_w) return CONV2D_ERR_INVALID_ARGUMENT;
    d->N = p->n; d->C = p->c; d->H = p->h; d->W = p->w; d->K = p->k; d->R = p->r; d->S = p->s;
    d->ph = p->pad_h; d->pw = p->pad_w; d->sh = p->stride_h; d->sw = p->stride_w;
    d->dh = p->dil_h; d->dw = p->dil_w; d->G = p->groups;
    d->P = (ph - span_h) / p->stride_h + 1;
    d->Q = (pw - span_w) / p->stride_w + 1;
    d->Cg = d->C / d->G;
    d->Kg = d->K / d->G;
    return CONV2D_OK;
}

// Sizes the kernels index with 32-bit arithmetic.
bool fits_32bit(const Dims &d)
{
    return d.N * d.H * d.W * d.C <= kMaxElems && d.N * d.P * d.Q * d.K <= kMaxElems &&
           d.K * d.R * d.S * d.Cg <= kMaxElems && d.N * d.P * d.Q <= kMaxElems &&
           d.N * d.H * d.W <= kMaxElems && d.sh * (d.P + 1) + d.dh * d.R + d.H < (1LL << 28) &&
           d.sw * (d.Q + 1) + d.dw * d.S + d.W < (1LL << 28);
}

int elem_size(int dtype) { return dtype == CONV2D_DTYPE_I8 ? 1 : 2; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- dgrad stride phases ---------------------------------------------------
// Input row h is reached by tap r from output row p = (h + pad - r*dil)/stride
// when that division is exact.  For rows h = ph + stride*i of one phase the
// valid taps form an arithmetic progression r0, r0 + step, ... with
// step = stride / gcd(stride, dil), and the source row is i + o with
// o = (ph + pad - r*dil) / stride, which falls by lcm(stride, dil)/stride per tap.
struct AxisPhase {
    int extent;  // rows of the input in this phase
    int r0, step, ntap;
    int o0, dstep;
};

AxisPhase axis_phase(int ph, int extent_full, int stride, int pad, int dil, int R)
{
    AxisPhase a;
    a.extent = ph < extent_full ? (extent_full - 1 - ph) / stride + 1 : 0;
    int g = stride, t = dil;
    while (t) {
        int u = g % t;
        g = t;
        t = u;
    }
    a.step = stride / g;
    a.r0 = -1;
    for (int r = 0; r < R && r < stride; ++r)
        if (((ph + pad - r * dil) % stride + stride) % stride == 0) {
            a.r0 = r;
            break;
        }
    if (a.r0 < 0) {
        a.ntap = 0;
        a.r0 = 0;
        a.o0 = 0;
        a.dstep = 0;
        return a;
    }
    a.ntap = (R - 1 - a.r0) / a.step + 1;
    a.o0 = (ph + pad - a.r0 * dil) / stride;  // exact
    a.dstep = -(a.step * dil) / stride;       // exact
    return a;
}

// dgrad on the implicit GEMM reads the filter as it is (transposing LDS
// reads of B) unless a stride phase has GEMM-K rows longer than this: there
// the reads (two 8-byte reads per fragment instead of one 16-byte read) cost
// more than re-laying the filter out first (measured: 16x57x57x96 -> 192,
// 5x5 s2 d2, 4800-long rows, 57.7 against 50.5 us; 1x1 64x56x56x256 -> 64,
// 256-long rows, 26.8 against 29.0 us).
constexpr int kDgradTransMaxK = 2048;

// 1x1 stride-1 problems without padding (fprop and dgrad, 16-bit types, no
// linear combination) whose GEMM-K and output channel counts the pointwise
// kernel takes.
bool pointwise_eligible(const Dims &d, int dtype, int op, bool axpby)
{
    if (axpby || d.G != 1 || d.R != 1 || d.S != 1 || d.sh != 1 || d.sw != 1 || d.ph != 0 || d.pw != 0) return false;
    const long long gk = op == CONV2D_OP_FPROP ? d.C : d.K, nout = op == CONV2D_OP_FPROP ? d.K : d.C;
    const long long npix = d.N * d.H * d.W;
    if (npix * gk * 2 > kBufMaxBytes || gk * nout * 2 > kBufMaxBytes) return false;
    return pointwise_supported(dtype, (int)gk, (int)nout);
}
// wgrad of the same problems when K and C are 64, 128 or 256 with K*C <=
// 16384 (the pointwise wgrad kernel), and its pixels per slice: whole groups
// of 64, short enough for 32-bit offsets into the slice.
bool pointwise_wgrad_eligible(const Dims &d, int dtype)
{
    if (d.G != 1 || d.R != 1 || d.S != 1 || d.sh != 1 || d.sw != 1 || d.ph != 0 || d.pw != 0) return false;
    return pointwise_wgrad_supported(dtype, (int)d.K, (int)d.C);
}
long long pointwise_wgrad_pps(const Dims &d, int splits)
{
    const long long npix = d.N * d.H * d.W;
    return ((npix + splits - 1) / splits + 63) / 64 * 64;
}
bool pointwise_wgrad_fits(const Dims &d, int splits)
{
    const long long npix = d.N * d.H * d.W;
    return npix < (1LL << 32) && pointwise_wgrad_pps(d, splits) * 2 * std::max(d.K, d.C) < (1LL << 31);
}
// One slice per CU, and at least 8 groups of 64 pixels per slice.
int choose_pointwise_wgrad_splits(const Dims &d)
{
    const long long npix = d.N * d.H * d.W;
    return (int)std::max(1LL, std::min((long long)kNumCUs, npix / 512));
}
bool dgrad_relayout(const Dims &d)
{
    long long kmax = 0;
    for (int py = 0; py < d.sh; ++py)
        for (int px = 0; px < d.sw; ++px) {
            AxisPhase ay = axis_phase(py, (int)d.H, (int)d.sh, (int)d.ph, (int)d.dh, (int)d.R);
            AxisPhase ax = axis_phase(px, (int)d.W, (int)d.sw, (int)d.pw, (int)d.dw, (int)d.S);
            if (ay.extent == 0 || ax.extent == 0) continue;
            kmax = std::max(kmax, (long long)ay.ntap * ax.ntap * d.Kg);
        }
    return kmax > kDgradTransMaxK;
}

constexpr size_t kNoBuf = ~(size_t)0;

// Output epilogue of a pass (conv2d_epilogue_t, checked): out = alpha * result
// + beta * c; wgrad may store fp32.
struct Epi {
    bool axpby = false;  // alpha != 1 or beta != 0
    float alpha = 1.0f, beta = 0.0f;
    const void *c = nullptr;
    bool out_f32 = false;
    void *db = nullptr;  // wgrad: bias gradient output
};

struct Plan {
    int op, dtype;
    int kernel;  // 1 implicit GEMM, 2 direct
    int tile, num_tiles, split_k, phases;
    size_t ws_bytes;
    Dims d;
    // Channel counts that are not whole 16-byte vectors (groups == 1): the
    // pass runs as `inner` on copies padded with zero channels, kept in the
    // workspace after the inner pass's own (offsets, or kNoBuf when the
    // tensor is used in place).  fprop: act = x, out = y; dgrad: act = dx,
    // out = dy; wgrad: act = x, out = dy; filt = the padded filter (w or dw).
    bool padded;
    int tile_shift;  // the padded path's tiles follow the few-channel kernel's: inner tile = tile - tile_shift
    conv2d_problem_t inner;
    size_t inner_ws, off_act, off_out, off_filt, off_bias;
};

int choose_igemm_tile(long long m_total, long long ngemm)
{
    // Prefer the widest N tile the problem fills; shrink M until the grid has
    // enough workgroups for 256 CUs.  With a 64-wide N, 64 x 64 tiles unless
    // they would make more than 16 workgroups per CU (measured: the 1x1
    // 64x56x56x256 -> 64 dgrad takes 28 us on 64 x 64 against 33 us on
    // 128 x 64; larger grids gain nothing from the smaller tile).
    if (ngemm <= 32) return 4;  // 64 x 32
    auto tiles = [&](int t) {
        TileShape s = igemm_tile_shape(t);
        return ((m_total + s.bm - 1) / s.bm) * ((ngemm + s.bn - 1) / s.bn);
    };
    if (ngemm >= 128 && ngemm % 128 == 0 && tiles(1) >= 2 * kNumCUs) return 1;  // 128 x 128
    if (tiles(0) >= 2 * kNumCUs && tiles(2) > 16 * kNumCUs) return 0;           // 128 x 64
    return 2;                                                                      // 64 x 64
}

// Stride-1 problems whose source channel count and filter the band kernel
// is built for keep the filter and a ring of input rows in LDS.
bool band_eligible(const Dims &d, int dtype, long long cin, long long src_h, long long src_w, long long ngemm,
                   long long dst_h, long long dst_w)
{
    // buffer offsets are 32-bit: one source image, one output image and the
    // filter stay under 1 GiB
    const long long e = elem_size(dtype);
    return d.G == 1 && d.sh == 1 && d.sw == 1 && d.dh == d.dw &&
           band_supported(dtype, (int)d.R, (int)d.S, (int)cin, (int)d.dh) && src_h * src_w * cin * e < (1LL << 30) &&
           dst_h * dst_w * ngemm * e < (1LL << 30) && d.R * d.S * cin * ngemm * e < (1LL << 30);
}

constexpr int kBandTile = 5;  // tile index of the band kernel (algo tile 6)
constexpr int kPwTile = 5;    // 1x1 problems (never band-eligible): the pointwise kernel in that place
constexpr int kWinoTile = 6;  // fprop: Winograd F(2x2,3x3) (algo tile 7), only when asked for

// Winograd F(2x2, 3x3): a band-eligible problem (stride 1, 3x3, dilation 1,
// buffer sizes) whose source has 64 channels and whose output channels are a
// multiple of 16: fprop (x -> y), or dgrad (dy -> dx, the forward
// convolution of dy padded by 2 - pad, so pad <= 2).  Never the library's
// own choice: its rounding differs from the direct sum's.
bool wino_eligible(const Dims &d, int dtype, int op)
{
    if (op == CONV2D_OP_FPROP) return wino_supported(dtype, (int)d.R, (int)d.S, (int)d.C, (int)d.dh) && d.K % 16 == 0;
    return wino_supported(dtype, (int)d.R, (int)d.S, (int)d.K, (int)d.dh) && d.C % 16 == 0 && d.ph <= 2 &&
           d.pw <= 2;
}

// Patch kernel: the lattice of source rows and columns the taps read, the
// output tile (TP lattice rows x TQ columns, at most 128 pixels) and its
// patch of lattice pixels, which must fit in LDS beside the filter rings.
// fprop reads x on the lattice of step gcd(stride, dil).  dgrad applies when
// the stride divides the dilation on both axes: dx is nonzero only on the
// rows h = -pad (mod stride) (likewise columns), where it is a stride-1
// correlation of dy with the flipped filter (dilation dil/stride).  nb:
// output channels per workgroup in blocks of 32; u: 16-channel steps per
// filter super-step.  Returns false when the kernel does not apply.
bool patch_layout(int op, const Dims &d, int dtype, PatchArgs *pa, int *nb_out)
{
    if (d.G != 1 || (dtype != CONV2D_DTYPE_F16 && dtype != CONV2D_DTYPE_BF16)) return false;
    if (op != CONV2D_OP_FPROP && op != CONV2D_OP_DGRAD) return false;
    const bool dg = op == CONV2D_OP_DGRAD;
    const long long SC = dg ? d.K : d.C, OC = dg ? d.C : d.K;
    if (SC % 16 || OC % 32) return false;
    auto gcd = [](long long u, long long v) {
        while (v) {
            const long long r = u % v;
            u = v;
            v = r;
        }
        return u;
    };
    // source lattice, output lattice and extents per axis
    long long gh, gw, sh1, sw1, dh1, dw1, padh, padw, ogh = 1, ogw = 1, oh0 = 0, ow0 = 0, LP, LQ, SH, SW;
    if (!dg) {
        gh = gcd(d.sh, d.dh);
        gw = gcd(d.sw, d.dw);
        sh1 = d.sh / gh; sw1 = d.sw / gw; dh1 = d.dh / gh; dw1 = d.dw / gw;
        padh = d.ph; padw = d.pw;
        LP = d.P; LQ = d.Q; SH = d.H; SW = d.W;
    } else {
        if (d.dh % d.sh || d.dw % d.sw) return false;
        auto axis = [](long long s, long long dil, long long pad, long long R, long long extent, long long *o0,
                       long long *n, long long *pe) {
            *o0 = ((-pad) % s + s) % s;               // first row h >= 0 with h + pad = 0 (mod s)
            *n = extent > *o0 ? (extent - *o0 + s - 1) / s : 0;
            *pe = (R - 1) * (dil / s) - (*o0 + pad) / s;  // padding of the flipped stride-1 correlation
        };
        axis(d.sh, d.dh, d.ph, d.R, d.H, &oh0, &LP, &padh);
        axis(d.sw, d.dw, d.pw, d.S, d.W, &ow0, &LQ, &padw);
        if (LP == 0 || LQ == 0) return false;
        ogh = d.sh; ogw = d.sw;
        gh = gw = 1; sh1 = sw1 = 1;
        dh1 = d.dh / d.sh; dw1 = d.dw / d.sw;
        SH = d.P; SW = d.Q;
    }
    const long long cpp = SC / 8;
    const long long PP = cpp % 2 ? cpp : cpp + 1;
    // Candidates: pixel blocks of 32 per workgroup (mb = 4 or 2), output
    // channels per workgroup (32*nb, nb | OC/32), the filter stream's
    // super-step (fprop: u 16-channel steps, u | SC/16; dgrad: 1) and ring
    // depth (fprop: set by nb and u; dgrad: 8 or 4).  Each takes the most
    // output rows whose patch fits beside its rings; the cheapest by a simple
    // model wins: rounds of 256 workgroups times (the main loop's cycles per
    // wave, steps * mb * nb MFMAs at about 12 cycles each per wave, plus a
    // prologue and epilogue of about 6000 + 600 * mb * nb cycles); ties go to
    // the larger tiles and deeper rings.
    const long long steps = d.R * d.S * (SC / 16);
    long long best = -1, TP = 0, TQ = 0, PW = 0;
    int nb = 0, u = 0, nsb = 0, mb = 0;
    for (int mbc : {4, 2}) {
        const long long tq = std::min<long long>(LQ, 32 * mbc);
        const long long tp_max = std::min<long long>(LP, 32 * mbc / tq);
        const long long pw = (tq - 1) * sw1 + (d.S - 1) * dw1 + 1;
        for (int nbc : {3, 2, 1}) {
            if (OC % (32 * nbc)) continue;
            for (int uc : {4, 2, 1}) {
                if ((SC / 16) % uc || (dg && uc != 1)) continue;
                for (int sc : {8, 4}) {
                    if (!dg && sc == 4) continue;  // one ring depth per (nb, u) for fprop
                    const int ns = dg ? sc : patch_ring_stages(nbc, uc);
                    const long long budget = patch_lds_bytes() - 4LL * ns * nbc * uc * 1024;
                    long long tp = tp_max;
                    for (; tp > 0; --tp) {
                        const long long ph = (tp - 1) * sh1 + (d.R - 1) * dh1 + 1;
                        if ((ph * pw * PP + 63) / 64 * 1024 <= budget) break;
                    }
                    if (tp == 0) continue;
                    const long long wgs = d.N * ((LP + tp - 1) / tp) * ((LQ + tq - 1) / tq) * (OC / (32 * nbc));
                    const long long cost = (wgs + kNumCUs - 1) / kNumCUs *
                                           (steps * mbc * nbc * 12 + 6000 + 600 * mbc * nbc);
                    if (best < 0 || cost < best) {
                        best = cost;
                        TP = tp;
                        TQ = tq;
                        PW = pw;
                        nb = nbc;
                        u = uc;
                        nsb = ns;
                        mb = mbc;
                    }
                }
            }
        }
    }
    if (TP == 0) return false;
    const long long PH = (TP - 1) * sh1 + (d.R - 1) * dh1 + 1;
    if (pa) {
        pa->N = (int)d.N; pa->H = (int)SH; pa->W = (int)SW; pa->SC = (int)SC;
        pa->OH = (int)(dg ? d.H : d.P); pa->OW = (int)(dg ? d.W : d.Q); pa->OC = (int)OC;
        pa->P = (int)LP; pa->Q = (int)LQ; pa->R = (int)d.R; pa->S = (int)d.S;
        pa->gh = (int)gh; pa->gw = (int)gw; pa->pad_h = (int)padh; pa->pad_w = (int)padw;
        pa->sh1 = (int)sh1; pa->sw1 = (int)sw1; pa->dh1 = (int)dh1; pa->dw1 = (int)dw1;
        pa->ogh = (int)ogh; pa->ogw = (int)ogw; pa->oh0 = (int)oh0; pa->ow0 = (int)ow0;
        pa->TP = (int)TP; pa->TQ = (int)TQ;
        pa->tiles_q = (int)((LQ + TQ - 1) / TQ);
        pa->tiles_img = (int)((LP + TP - 1) / TP) * pa->tiles_q;
        pa->PH = (int)PH; pa->PW = (int)PW; pa->PP = (int)PP;
        pa->patch_slots = (int)(PH * PW * PP);
        pa->div_pp = make_fastdiv((uint32_t)PP);
        pa->div_pw = make_fastdiv((uint32_t)PW);
        pa->div_tq = make_fastdiv((uint32_t)TQ);
        pa->nb = nb;
        pa->u = u;
        pa->nsb = nsb;
        pa->mb = mb;
    }
    if (nb_out) *nb_out = nb;
    return true;
}

// Stride-1 wgrad with the filter shape and channel counts the wgrad band
// kernel is built for.
bool wgrad_band_eligible(const Dims &d, int dtype)
{
    return d.G == 1 && d.sh == 1 && d.sw == 1 && d.dh == d.dw && dtype != CONV2D_DTYPE_I8 &&
           wgrad_band_supported((int)d.R, (int)d.S, (int)d.C, (int)d.K, (int)d.dh, (int)d.Q);
}

constexpr int kWgradBandTile = 2;  // wgrad tile index of the band kernel (algo tile 3), after the generic ones

// Bands of the wgrad band kernel, about one workgroup per CU: bands within
// one image, two workgroups (column halves) each, or 85 bands of the stacked
// rows of all images, three workgroups (filter rows) each (255 workgroups,
// fp32 partials of 85 slices).  The split with the lower estimated time, from
// a model fitted to measured passes on one MI355X (64x56x56x64 -> 64 at
// N = 64, 96 and 128): per unit of band work (the 28 x 58 pixel steps of a
// column half of N = 64) 14.7 us with halves, 17.6 us with filter rows (more
// fragment reads per MFMA); 0.5 us per MB of partials (stored, then read by
// the reduce); 4.0 and 3.1 us of fixed cost.  Halves that need a second
// round of workgroups pay their band work twice.  Filter rows only with at
// least 4 rows a band.
struct WgradBandLayout {
    int nsplit;
    int rows, chunks;      // nsplit = 2: rows per band, bands per image
    int nbands;            // partial slices
};
WgradBandLayout wgrad_band_layout(const Dims &d)
{
    WgradBandLayout h = {};
    long long c = (kNumCUs / 2 + d.N - 1) / d.N;
    c = std::max(1LL, std::min(c, d.P));
    h.nsplit = 2;
    h.rows = (int)((d.P + c - 1) / c);
    h.chunks = (int)((d.P + h.rows - 1) / h.rows);
    h.nbands = (int)(d.N * h.chunks);

    const long long rows_total = d.N * d.P;
    const long long nb3 = kNumCUs / 3;
    // x is read through one 32-bit buffer range over the images a band touches
    const long long rows3 = (rows_total + nb3 - 1) / nb3;
    const long long band_imgs = (rows3 + d.P - 1) / d.P + 1;
    if (rows3 < 4 || rows_total >= (1LL << 30) ||  // (the model is fitted to bands of 42 rows and more)
        (unsigned long long)(band_imgs * d.H * d.W * d.C * 2) > kBufMaxBytes)
        return h;
    const double unit = 28.0 * 58.0, xw = (double)(d.Q + d.dw * (d.S - 1));
    const double part_mb = (double)(d.K * d.R * d.S * d.C) * 4.0 / 1e6;  // one slice
    const long long rounds = (2LL * h.nbands + kNumCUs - 1) / kNumCUs;
    const double t_halves = 14.7 * (double)rounds * h.rows * xw / unit + 0.5 * part_mb * h.nbands + 4.0;
    const double t_rows = 17.6 * (double)rows3 * xw * (2.0 / 3.0) / unit + 0.5 * part_mb * (double)nb3 + 3.1;
    if (t_rows >= t_halves) return h;
    WgradBandLayout l = {};
    l.nsplit = 3;
    l.nbands = (int)nb3;
    return l;
}

// Few-channel fprop (fewchan.hip): the window layout of each filter row
// (delta elements before its S*C taps, Lw elements in all), the padded input
// row in LDS (image element 0 at element `left`, room on the right for the
// last pixel's window) and the output rows per workgroup: about two
// workgroups per CU, as long as the rows and the staging fit 64 KB of LDS.
// Returns false when the kernel does not apply.
bool fewchan_layout(const Dims &d, int dtype, FewArgs *f)
{
    if (d.G != 1 || !fewchan_supported(dtype, (int)d.C, (int)d.K, (int)d.S, (int)d.sw, (int)d.dw, (int)d.W))
        return false;
    const long long e = elem_size(dtype);
    if (e * d.N * d.H * d.W * d.C > kBufMaxBytes) return false;
    const long long SC = d.S * d.C;
    const long long delta = (d.pw * d.C) & 1;
    const long long lw = (delta + SC + 7) / 8 * 8;
    const int nst = fewchan_steps((int)d.R, (int)lw);
    if (!nst) return false;
    const long long left = (d.pw * d.C + delta + 7) / 8 * 8;
    const long long win0 = left - d.pw * d.C - delta;  // window start of pixel 0
    const long long emax = win0 + (d.Q - 1) * d.sw * d.C + lw - 1;
    const long long pitch_e = (std::max(left + d.W * d.C, emax + 1) + 7) / 8 * 8;
    const long long pitch = pitch_e * 2;
    // the filter as it is (whole 1 KB blocks, and room for window reads up to
    // lw elements past it), then the output staging of the four waves
    const long long stage = std::max((d.K * d.R * SC * e + 2 * lw + 1023) / 1024 * 1024, 4LL * 32 * (2 * d.K + 16));
    auto buf_for = [&](long long rows) { return ((rows - 1) * d.sh + (d.R - 1) * d.dh + 1) * pitch; };
    constexpr long long kLds = 65536 - 1024;  // the last 1 KB holds the bias
    long long rows = std::max(1LL, std::min(d.P, d.N * d.P / (2 * kNumCUs)));
    while (rows > 1 && (buf_for(rows) + 1023) / 1024 * 1024 + stage > kLds) --rows;
    const long long buf = (buf_for(rows) + 1023) / 1024 * 1024;
    if (buf + stage > kLds) return false;
    if (!f) return true;
    f->N = (int)d.N; f->H = (int)d.H; f->WC = (int)(d.W * d.C); f->P = (int)d.P; f->Q = (int)d.Q;
    f->K = (int)d.K; f->R = (int)d.R; f->SC = (int)SC;
    f->pad_h = (int)d.ph; f->sh = (int)d.sh; f->dh = (int)d.dh;
    f->rows_per_wg = (int)rows;
    f->bands = (int)((d.P + rows - 1) / rows);
    f->nrows = (int)((rows - 1) * d.sh + (d.R - 1) * d.dh + 1);
    f->pitch = (int)pitch;
    f->cpr = (int)(pitch_e / 8);
    f->left = (int)left;
    f->delta = (int)delta;
    f->lw = (int)lw;
    f->win0 = (int)win0;
    f->qstep = (int)(d.sw * d.C);
    f->buf_bytes = (int)buf;
    f->stage_bytes = (int)stage;
    f->x_bytes = (uint32_t)(e * d.N * d.H * d.W * d.C);
    f->div_cpr = make_fastdiv((uint32_t)f->cpr);
    f->div_q = make_fastdiv((uint32_t)d.Q);
    for (int j = 0; j < kFewMaxSteps; ++j)
        for (int h = 0; h < 2; ++h) {
            const long long t0 = 8LL * (2 * j + h), r = t0 / lw, kk0 = t0 - r * lw;
            FewStep &st = f->step[j];
            const bool rok = j < nst && r < d.R;
            st.fbase[h] = rok ? (int)(r * SC + kk0 - delta) : 0;
            st.coff[h] = rok ? (uint32_t)(r * d.dh * pitch + kk0 * 2) : 0u;
            for (int p = 0; p < 4; ++p) {
                uint32_t m = 0;
                for (int k = 0; k < 2; ++k) {
                    const long long sc = kk0 + 2 * p + k - delta;
                    if (rok && sc >= 0 && sc < SC) m |= 0xffffu << (16 * k);
                }
                st.mask[h][p] = m;
            }
        }
    return true;
}

// Few-channel wgrad (fewchan_wgrad.hip): the window layout of each filter
// row (delta makes the even pixels' windows 8-byte aligned; when sw*C is 2
// mod 4 the odd pixels read a copy of the rows shifted by 4 bytes), the
// group buffers (two output rows a group, two buffers in the kernel's LDS)
// and the bands: about one workgroup per CU.  Returns false when the kernel
// does not apply.
bool fewchan_wgrad_layout(const Dims &d, int dtype, FewWgradArgs *f)
{
    if (d.G != 1 ||
        !fewchan_wgrad_supported(dtype, (int)d.C, (int)d.K, (int)d.S, (int)d.sw, (int)d.dw, (int)d.W))
        return false;
    const long long e = elem_size(dtype);
    if (e * d.N * d.H * d.W * d.C > kBufMaxBytes || e * d.N * d.P * d.Q * d.K > kBufMaxBytes) return false;
    const long long SC = d.S * d.C;
    const long long delta = (4 - (d.pw * d.C) % 4) % 4;
    const long long lw = (delta + SC + 3) / 4 * 4;
    long long ncb = (d.R * lw + 31) / 32;
    if (ncb > 6) return false;
    ncb = std::max(ncb, 2LL);
    const long long left = (d.pw * d.C + delta + 7) / 8 * 8;
    const long long win0 = left - d.pw * d.C - delta;  // a multiple of 4
    const long long qstep = d.sw * d.C;
    const bool odd_shift = qstep % 4 == 2;
    const long long spc = (d.Q + 31) / 32, dq = 32 * spc;
    const long long emax = win0 + (dq - 1) * qstep + lw - 1;
    const long long pitch_e = (std::max(left + d.W * d.C, emax + 3) + 7) / 8 * 8;
    const long long pitch = 2 * pitch_e, cpr = pitch_e / 8;
    long long grw = 2, nxr = 0, nblk_dy = 0, nblk_x = 0, xa = 0, xb = 0, buf = 0;
    for (; grw >= 1; --grw) {
        nxr = (grw - 1) * d.sh + (d.R - 1) * d.dh + 1;
        nblk_dy = grw * dq / 8;
        nblk_x = (nxr * cpr + 63) / 64;
        xa = nblk_x * 1024;
        xb = odd_shift ? (nxr * pitch + 16 + 1023) / 1024 * 1024 : 0;
        buf = nblk_dy * 1024 + xa + xb;
        if (2 * buf <= fewchan_wgrad_lds_bytes()) break;
    }
    if (grw < 1) return false;
    if (!f) return true;
    const long long rows = std::max(1LL, std::min(d.P, (d.N * d.P + kNumCUs / 2) / kNumCUs));
    f->N = (int)d.N; f->H = (int)d.H; f->WC = (int)(d.W * d.C); f->P = (int)d.P; f->Q = (int)d.Q;
    f->R = (int)d.R; f->SC = (int)SC;
    f->pad_h = (int)d.ph; f->sh = (int)d.sh; f->dh = (int)d.dh;
    f->rows_per_wg = (int)rows;
    f->bands = (int)((d.P + rows - 1) / rows);
    f->grw = (int)grw;
    f->spc = (int)spc;
    f->dq = (int)dq;
    f->lw = (int)lw;
    f->delta = (int)delta;
    f->win0 = (int)win0;
    f->qstep = (int)qstep;
    f->nxr = (int)nxr;
    f->pitch = (int)pitch;
    f->cpr = (int)cpr;
    f->left = (int)left;
    f->odd_shift = odd_shift ? 1 : 0;
    f->nblk_dy = (int)nblk_dy;
    f->nblk_x = (int)nblk_x;
    f->xa_off = (int)(nblk_dy * 1024);
    f->xb_off = (int)(nblk_dy * 1024 + xa);
    f->buf_bytes = (int)buf;
    f->xcopy_chunks = (int)(nxr * pitch / 16);
    f->ncb = (int)ncb;
    f->ncba = (int)((ncb + 1) / 2);
    f->x_bytes = (uint32_t)(e * d.N * d.H * d.W * d.C);
    f->dy_bytes = (uint32_t)(e * d.N * d.P * d.Q * d.K);
    f->part_stride = splitk_stride(d.K * d.R * SC);
    f->div_cpr = make_fastdiv((uint32_t)cpr);
    return true;
}

// Few-channel dgrad (fewchan_dgrad.hip): the dy offsets a 2x2 output block
// reads (over both stride phases of each axis), the ring of dy rows, and
// the bands of super-rows: about one workgroup per CU.  Returns false when
// the kernel does not apply.
static void fewchan_dgrad_offsets(long long pad, long long R, long long *lo, long long *n)
{
    long long mn = 1LL << 40, mx = -(1LL << 40);
    for (long long a = 0; a < 2; ++a)
        for (long long r = 0; r < R; ++r) {
            const long long t = a + pad - r;
            if (((t % 2) + 2) % 2) continue;
            mn = std::min(mn, t / 2);
            mx = std::max(mx, t / 2);
        }
    *lo = mn;
    *n = mx - mn + 1;
}
bool fewchan_dgrad_layout(const Dims &d, int dtype, FewDgradArgs *f)
{
    if (d.G != 1 || !fewchan_dgrad_supported(dtype, (int)d.C, (int)d.K, (int)d.sh, (int)d.sw, (int)d.dh, (int)d.dw,
                                             (int)d.W))
        return false;
    const long long e = elem_size(dtype);
    if (e * d.N * d.H * d.W * d.C > kBufMaxBytes || e * d.N * d.P * d.Q * d.K > kBufMaxBytes) return false;
    long long dp_min, ndh, dq_min, ndw;
    fewchan_dgrad_offsets(d.ph, d.R, &dp_min, &ndh);
    fewchan_dgrad_offsets(d.pw, d.S, &dq_min, &ndw);
    const long long mx = fewchan_dgrad_max_offsets();
    if (ndh < 2 || ndh > mx || ndw < 2 || ndw > mx) return false;
    const long long HS = (d.H + 1) / 2, WS = (d.W + 1) / 2;
    const long long nblk_r = (WS + 15) / 16;
    const long long rsl = (16 * nblk_r + ndw - 1 + 7) / 8 * 8;  // pixel slots of a dy row in LDS
    const long long rowb = rsl * 128;
    const long long nslot = ndh + 3;
    const long long ring = nslot * rowb;
    const long long filt = (d.K * d.R * d.S * d.C * e + 1023) / 1024 * 1024;
    const long long stage_wave = 2 * 32 * d.C * e;
    const long long bmat = 2 * ndh * ndw * 64 * 16;  // the B fragments
    if (ring + filt + bmat + 8 * stage_wave > fewchan_dgrad_lds_bytes()) return false;
    if (!f) return true;
    const long long rows = std::max(1LL, std::min(HS, (d.N * HS + kNumCUs / 2) / kNumCUs));
    f->N = (int)d.N; f->H = (int)d.H; f->W = (int)d.W; f->C = (int)d.C; f->P = (int)d.P; f->Q = (int)d.Q;
    f->R = (int)d.R; f->S = (int)d.S;
    f->pad_h = (int)d.ph; f->pad_w = (int)d.pw;
    f->HS = (int)HS; f->WS = (int)WS;
    f->rows_per_wg = (int)rows;
    f->bands = (int)((HS + rows - 1) / rows);
    f->nblk_r = (int)nblk_r;
    f->dp_min = (int)dp_min; f->ndh = (int)ndh; f->dq_min = (int)dq_min; f->ndw = (int)ndw;
    f->rsl = (int)rsl; f->rowb = (int)rowb; f->nslot = (int)nslot;
    f->ring_bytes = (int)ring; f->filt_bytes = (int)filt; f->stage_wave = (int)stage_wave;
    f->dy_bytes = (uint32_t)(e * d.N * d.P * d.Q * d.K);
    return true;
}

int choose_wgrad_splits(long long tiles, long long npix, long long min_steps)
{
    // about three workgroups per CU, at least min_steps main-loop steps per
    // slice; with few tiles per slice, from 8 slices on a multiple of 8, so
    // that every XCD gets as many slices (the kernels then put all tiles of a
    // slice on one XCD)
    const long long steps = (npix + kWgradPixStep - 1) / kWgradPixStep;
    const long long cap = std::max(1LL, steps / min_steps);
    long long s = std::min((3 * kNumCUs) / std::max(1LL, tiles), cap);
    if (tiles <= kWgradXcdTiles && s >= 8) {
        const long long r = (s + 4) / 8 * 8;
        s = r <= cap ? r : s / 8 * 8;
    }
    return (int)std::max(1LL, std::min(s, 4096LL));
}

int choose_direct_splits(long long outputs, long long npix)
{
    long long s = (256LL * 1024) / std::max(1LL, outputs);
    s = std::min(s, std::max(1LL, npix / 64));
    return (int)std::max(1LL, std::min(s, 4096LL));
}

int choose_direct_tiled_splits(long long wgs_per_slice, long long npix)
{
    // about two workgroups per CU, slices of at least 64 pixels
    long long s = (2 * kNumCUs) / std::max(1LL, wgs_per_slice);
    s = std::min(s, std::max(1LL, npix / 64));
    return (int)std::max(1LL, std::min(s, 4096LL));
}

int make_plan(int op, const conv2d_problem_t *prob, int dtype, const conv2d_algo_t *algo, const Epi &ep,
              Plan *pl);

// Work units of the depthwise wgrad kernel: strips of cols output columns of
// one output row.
static long long depthwise_units(const Dims &d)
{
    const int cols = direct_depthwise_wgrad_cols((int)d.N, (int)d.H, (int)d.W, (int)d.C, (int)d.P, (int)d.Q, (int)d.R, (int)d.S,
                                               (int)d.sw, (int)d.dw);
    return d.N * d.P * ((d.Q + cols - 1) / cols);
}

// depthwise wgrad: at most two workgroups per CU, at least 64 pixels per slice
int choose_direct_depthwise_splits(const Dims &d)
{
    const int cols = direct_depthwise_wgrad_cols((int)d.N, (int)d.H, (int)d.W, (int)d.C, (int)d.P, (int)d.Q, (int)d.R, (int)d.S,
                                               (int)d.sw, (int)d.dw);
    return (int)std::max(1LL, std::min(2LL * kNumCUs, depthwise_units(d) * cols / 64));
}

// Plan of a groups == 1 problem whose C or K is not a multiple of vec: the
// inner problem has both rounded up to vec; the workspace holds the inner
// pass's own workspace, then the padded copies the pass needs.
int plan_padded(int op, const conv2d_problem_t *prob, int dtype, const conv2d_algo_t *algo, const Epi &ep, int vec,
                Plan *pl)
{
    const Dims d = pl->d;
    conv2d_problem_t in = *prob;
    in.c = (int)((d.C + vec - 1) / vec * vec);
    in.k = (int)((d.K + vec - 1) / vec * vec);
    Plan ip;
    int st = make_plan(op, &in, dtype, algo, ep, &ip);
    if (st) return st;
    *pl = ip;
    pl->d = d;
    pl->padded = true;
    pl->inner = in;
    pl->inner_ws = ip.ws_bytes;
    const size_t e = (size_t)elem_size(dtype);
    const long long Cp = in.c, Kp = in.k;
    const bool pad_c = Cp != d.C, pad_k = Kp != d.K;
    size_t off = round_up(ip.ws_bytes, 256);
    auto take = [&](long long elems, size_t esz) {
        const size_t o = off;
        off += round_up((size_t)elems * esz, 256);
        return o;
    };
    pl->off_filt = take(Kp * d.R * d.S * Cp, ep.out_f32 ? 4 : e);
    if (op == CONV2D_OP_FPROP) {
        if (pad_c) pl->off_act = take(d.N * d.H * d.W * Cp, e);
        if (pad_k) pl->off_out = take(d.N * d.P * d.Q * Kp, e);
        if (pad_k) pl->off_bias = take(Kp, dtype == CONV2D_DTYPE_I8 ? 4 : e);
    } else {
        if (pad_c) pl->off_act = take(d.N * d.H * d.W * Cp, e);
        if (pad_k) pl->off_out = take(d.N * d.P * d.Q * Kp, e);
    }
    pl->ws_bytes = off;
    return CONV2D_OK;
}

int make_plan(int op, const conv2d_problem_t *prob, int dtype, const conv2d_algo_t *algo, const Epi &ep,
              Plan *pl)
{
    int st = validate(prob, &pl->d);
    if (st) return st;
    const Dims &d = pl->d;
    if (op != CONV2D_OP_FPROP && op != CONV2D_OP_DGRAD && op != CONV2D_OP_WGRAD)
        return CONV2D_ERR_INVALID_ARGUMENT;
    if (dtype != CONV2D_DTYPE_F16 && dtype != CONV2D_DTYPE_BF16 && dtype != CONV2D_DTYPE_I8)
        return CONV2D_ERR_UNSUPPORTED;
    if (dtype == CONV2D_DTYPE_I8 && op != CONV2D_OP_FPROP) return CONV2D_ERR_UNSUPPORTED;
    if (!fits_32bit(d)) return CONV2D_ERR_UNSUPPORTED;
    if (algo && (algo->tile < 0 || algo->split_k < 0)) return CONV2D_ERR_INVALID_ARGUMENT;
    if ((ep.axpby || ep.out_f32) && dtype == CONV2D_DTYPE_I8) return CONV2D_ERR_UNSUPPORTED;
    if (ep.out_f32 && op != CONV2D_OP_WGRAD) return CONV2D_ERR_INVALID_ARGUMENT;
    // the wgrad epilogue runs in the split-K reduce: partials even for one slice
    const bool wparts = ep.axpby || ep.out_f32;
    pl->op = op;
    pl->dtype = dtype;
    pl->split_k = 1;
    pl->phases = 1;
    pl->ws_bytes = 0;
    pl->tile = 0;
    pl->padded = false;
    pl->tile_shift = 0;
    pl->off_act = pl->off_out = pl->off_filt = pl->off_bias = kNoBuf;

    // implicit GEMM: 128-bit chunks of channels along GEMM-K and GEMM-N;
    // other channel counts run on zero-padded copies
    const int vec = dtype == CONV2D_DTYPE_I8 ? 16 : 8;
    if (d.G == 1 && (d.C % vec || d.K % vec)) {
        // fprop and wgrad with few input channels: tile 0 is the
        // few-channel kernel (the default), the padded path's tiles follow it
        FewWgradArgs fw;
        const bool fewk = op == CONV2D_OP_FPROP   ? !ep.axpby && fewchan_layout(d, dtype, nullptr)
                          : op == CONV2D_OP_WGRAD ? fewchan_wgrad_layout(d, dtype, &fw)
                                                  : !ep.axpby && fewchan_dgrad_layout(d, dtype, nullptr);
        if (!fewk) return plan_padded(op, prob, dtype, algo, ep, vec, pl);
        conv2d_algo_t ia = algo ? *algo : conv2d_algo_t{0, 0};
        const bool few = ia.tile <= 1;
        ia.tile = few ? 0 : ia.tile - 1;
        Plan pp;
        pp.d = d;
        st = plan_padded(op, prob, dtype, &ia, ep, vec, &pp);
        if (!few) {
            if (st) return st;
            *pl = pp;
            pl->tile += 1;
            pl->num_tiles += 1;
            pl->tile_shift = 1;
            return CONV2D_OK;
        }
        pl->kernel = 4;
        pl->tile = 0;
        pl->num_tiles = 1 + (st ? 0 : pp.num_tiles);
        if (op == CONV2D_OP_WGRAD) {  // one fp32 partial per band, then the split-K reduce
            pl->split_k = (int)(d.N * fw.bands);
            pl->ws_bytes = round_up((size_t)pl->split_k * (size_t)fw.part_stride * sizeof(float), 256);
        }
        return CONV2D_OK;
    }

    // grouped problems whose channels per group come in 128-bit chunks: the
    // implicit GEMM, one GEMM per group (grid.y = groups x N tiles); the
    // direct kernels follow its tiles in the table
    const bool grouped_gemm = d.G > 1 && d.Cg % vec == 0 && d.Kg % vec == 0 &&
                              (op != CONV2D_OP_WGRAD || dtype != CONV2D_DTYPE_I8);
    const int n_gemm = grouped_gemm ? (op == CONV2D_OP_WGRAD ? wgrad_num_tiles() : igemm_num_tiles()) : 0;
    // direct kernels (groups > 1): tile 0 one thread per output; tile 1 the
    // depthwise kernels (groups = C = K) or the LDS-tiled dot-product kernels
    // (16-bit types, channel counts in 16-byte vectors, staging fits LDS)
    int n_direct = 0;
    bool dwise = false;
    if (d.G > 1) {
        dwise = direct_depthwise_ok(dtype, (int)d.C, (int)d.Cg, (int)d.Kg, (int)d.R, (int)d.S);
        const bool tiled = dwise || (op == CONV2D_OP_WGRAD
                                         ? direct_wgrad_tiled_ok(dtype, (int)d.Cg, (int)d.Kg)
                                         : direct_tiled_rows(op == CONV2D_OP_DGRAD, dtype, (int)d.R, (int)d.S,
                                                             (int)d.W, (int)d.Q, (int)d.Cg, (int)d.Kg) > 0);
        n_direct = tiled ? 2 : 1;
    }
    if (d.G > 1 && (!grouped_gemm || (algo && algo->tile > n_gemm))) {
        pl->kernel = 2;
        pl->num_tiles = n_gemm + n_direct;
        if (algo && algo->tile > pl->num_tiles) return CONV2D_ERR_UNSUPPORTED;
        pl->tile = (algo && algo->tile) ? algo->tile - 1 - n_gemm : n_direct - 1;
        if (op == CONV2D_OP_WGRAD) {
            const long long outputs = d.K * d.R * d.S * d.Cg;
            const long long npix = d.N * d.P * d.Q;
            const bool dwk = pl->tile == 1 && dwise;  // one workgroup per pixel slice, always partials
            const long long wgs = dwk        ? 1
                                  : pl->tile ? direct_wgrad_tiled_wgs((int)d.R, (int)d.S, (int)d.Cg, (int)d.Kg,
                                                                      (int)d.G)
                                             : 0;
            int s = (algo && algo->split_k) ? algo->split_k
                    : dwk                   ? choose_direct_depthwise_splits(d)
                    : pl->tile              ? choose_direct_tiled_splits(wgs, npix)
                                            : choose_direct_splits(outputs, npix);
            if (s > 65535) return CONV2D_ERR_UNSUPPORTED;
            pl->split_k = s;
            if (s > 1 || wparts || dwk)
                pl->ws_bytes = round_up((size_t)s * splitk_stride(outputs) * sizeof(float), 256);
        }
        return CONV2D_OK;
    }

    pl->kernel = 1;
    {
        // operands are read through 32-bit buffer offsets
        const unsigned long long e = (unsigned long long)elem_size(dtype);
        if (e * d.N * d.H * d.W * d.C > kBufMaxBytes || e * d.N * d.P * d.Q * d.K > kBufMaxBytes ||
            e * d.K * d.R * d.S * d.C > kBufMaxBytes)
            return CONV2D_ERR_UNSUPPORTED;
    }
    if (op == CONV2D_OP_WGRAD) {
        const bool wband = wgrad_band_eligible(d, dtype);
        // 1x1 problems (never band-eligible): the pointwise wgrad kernel in
        // the band kernel's place, the default whatever the split count
        const bool pww = pointwise_wgrad_eligible(d, dtype);
        pl->num_tiles = wgrad_num_tiles() + (wband || pww ? 1 : 0) + n_direct;
        if (algo && algo->tile > pl->num_tiles) return CONV2D_ERR_UNSUPPORTED;
        if (pww && (!(algo && algo->tile) || algo->tile - 1 == kWgradBandTile)) {
            const int s = (algo && algo->split_k) ? algo->split_k : choose_pointwise_wgrad_splits(d);
            if (s > 65535 || !pointwise_wgrad_fits(d, s)) return CONV2D_ERR_UNSUPPORTED;
            pl->kernel = 5;
            pl->tile = kWgradBandTile;
            pl->split_k = s;
            pl->ws_bytes = round_up((size_t)s * splitk_stride(d.K * d.C + (ep.db ? d.K : 0)) * sizeof(float), 256);
            return CONV2D_OK;
        }
        // default: the band kernel when it applies and no split count is forced
        const bool use_band = algo && algo->tile ? algo->tile - 1 == kWgradBandTile
                                                  : wband && !(algo && algo->split_k);
        const long long ncols = d.R * d.S * d.Cg;  // per group
        if (use_band) {
            pl->tile = kWgradBandTile;
            pl->split_k = wgrad_band_layout(d).nbands;
            // with the bias gradient each slice also holds the band's K dy column sums
            const long long per = d.K * ncols + (ep.db ? d.K : 0);
            pl->ws_bytes = round_up((size_t)pl->split_k * splitk_stride(per) * sizeof(float), 256);
            return CONV2D_OK;
        }
        // default: 128 x 128 tiles when they give the chip at least 16 tiles,
        // else the 64 x 64 kernel, whose extra tiles need fewer slices (and
        // fewer fp32 partials) on small problems
        const TileShape big = wgrad_tile_shape(0);
        const long long big_tiles = d.G * ((d.Kg + big.bm - 1) / big.bm) * ((ncols + big.bn - 1) / big.bn);
        pl->tile = (algo && algo->tile) ? algo->tile - 1 : (big_tiles >= 16 ? 0 : 1);
        if (pl->tile == kWgradBandTile) return CONV2D_ERR_UNSUPPORTED;
        TileShape ts = wgrad_tile_shape(pl->tile);
        const long long tiles = d.G * ((d.Kg + ts.bm - 1) / ts.bm) * ((ncols + ts.bn - 1) / ts.bn);
        const long long npix = d.N * d.P * d.Q;
        int s = (algo && algo->split_k) ? algo->split_k : choose_wgrad_splits(tiles, npix, pl->tile == 0 ? 2 : 8);
        if (s > 65535) return CONV2D_ERR_UNSUPPORTED;
        pl->split_k = s;
        // with the bias gradient, tile 0 carries dy's column sums in its slices
        const bool gdb = ep.db && pl->tile == 0;
        if (s > 1 || wparts || gdb)
            pl->ws_bytes = round_up((size_t)s * splitk_stride(d.K * ncols + (gdb ? d.K : 0)) * sizeof(float), 256);
        return CONV2D_OK;
    }
    // the band kernels have no linear-combination epilogue
    const bool band = !ep.axpby && (op == CONV2D_OP_FPROP ? band_eligible(d, dtype, d.C, d.H, d.W, d.K, d.P, d.Q)
                                                          : band_eligible(d, dtype, d.K, d.P, d.Q, d.C, d.H, d.W));
    const bool wino = band && wino_eligible(d, dtype, op);
    const bool pw = pointwise_eligible(d, dtype, op, ep.axpby);  // 1x1: never with band
    int patch_nb = 1;
    // the patch kernel's tile follows the others; the default for filters
    // with more than one tap when its grid takes at most two workgroups per
    // CU (each workgroup pays for loading its patch and adding its four
    // partial tiles, which many small tiles would repeat)
    PatchArgs pa;
    const bool patch = !ep.axpby && patch_layout(op, d, dtype, &pa, &patch_nb);
    const int patch_tile = igemm_num_tiles() + (band ? 1 : 0) + (wino ? 1 : 0) + (pw ? 1 : 0);
    const bool patch_default =
        patch && !band && !pw && d.R * d.S > 1 && d.N * pa.tiles_img * (pa.OC / (32 * patch_nb)) <= 2 * kNumCUs;
    pl->num_tiles = igemm_num_tiles() + (band ? 1 : 0) + (wino ? 1 : 0) + (pw ? 1 : 0) + (patch ? 1 : 0) + n_direct;
    if (algo && algo->tile > pl->num_tiles) return CONV2D_ERR_UNSUPPORTED;
    if (op == CONV2D_OP_FPROP) {
        pl->tile = (algo && algo->tile) ? algo->tile - 1
                   : pw               ? kPwTile
                   : band             ? kBandTile
                   : patch_default    ? patch_tile
                                      : choose_igemm_tile(d.N * d.P * d.Q, d.Kg);
        if (pl->tile == kWinoTile && wino) pl->kernel = 3;
        if (pw && pl->tile == kPwTile) pl->kernel = 5;
        if (patch && pl->tile == patch_tile) pl->kernel = 6;
        return CONV2D_OK;
    }
    // dgrad
    pl->tile = (algo && algo->tile) ? algo->tile - 1
               : pw               ? kPwTile
               : band             ? kBandTile
               : patch_default    ? patch_tile
                                  : -1;
    if (patch && pl->tile == patch_tile) {
        pl->kernel = 6;
        return CONV2D_OK;
    }
    if (d.sh * d.sw > kMaxPhases) return CONV2D_ERR_UNSUPPORTED;
    pl->phases = (int)(d.sh * d.sw);
    if (pl->tile < 0) pl->tile = choose_igemm_tile(d.N * d.H * d.W / pl->phases, d.Cg);
    if (pw && pl->tile == kPwTile) {
        pl->kernel = 5;
        return CONV2D_OK;
    }
    // the band kernel reads the filter as it is, and so does the implicit
    // GEMM unless its GEMM-K rows are long (then a re-laid-out copy);
    // Winograd takes its transform
    if (pl->tile == kWinoTile) {
        pl->kernel = 3;
        pl->ws_bytes = round_up((size_t)16 * d.C * d.K * elem_size(dtype), 256);
    } else if (pl->tile != kBandTile && dgrad_relayout(d)) {
        pl->ws_bytes = round_up((size_t)d.R * d.S * d.C * d.Kg * elem_size(dtype), 256);
    }
    return CONV2D_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CONV2D_OK : CONV2D_ERR_DEVICE; }

// Copy rows x src_cols of src (row pitch src_ld) into dst (dst_rows x
// dst_cols, pitch dst_ld), zero-filling what src does not cover.
hipError_t repack(int esz, const void *src, long long src_rows, long long src_cols, long long src_ld, void *dst,
                  long long dst_rows, long long dst_cols, long long dst_ld, hipStream_t s)
{
    RepackArgs a;
    a.src = src; a.dst = dst;
    a.src_rows = src_rows; a.dst_rows = dst_rows;
    a.src_cols = (int)src_cols; a.src_ld = (int)src_ld; a.dst_cols = (int)dst_cols; a.dst_ld = (int)dst_ld;
    return launch_repack(esz, a, s);
}

void fill_phase_common(Phase &ph, int tile)
{
    TileShape ts = igemm_tile_shape(tile);
    ph.tiles_m = (int)(((long long)ph.m_total + ts.bm - 1) / ts.bm);
    ph.div_mj = make_fastdiv((uint32_t)std::max(1, ph.mj));
    ph.div_mimj = make_fastdiv((uint32_t)std::max(1LL, (long long)ph.mi * ph.mj));
}

// Rows of one image per band workgroup: enough workgroups for every CU.
void band_rows(BandArgs &b, long long other_wgs)
{
    long long chunks = (kNumCUs + b.N * other_wgs - 1) / (b.N * other_wgs);
    chunks = std::max(1LL, std::min(chunks, (long long)b.P));
    b.rows_per_wg = (int)((b.P + chunks - 1) / chunks);
    b.chunks_per_img = (b.P + b.rows_per_wg - 1) / b.rows_per_wg;
}

// Stride-1 convolution src [N][H][W][cin] -> dst [N][P][Q][ngemm] on the band kernel.
int run_band(int dtype, const Dims &d, int cin, const void *src, int H, int W, const void *bmat, int flip,
             const void *bias, int relu, double requant_m, void *dst, int P, int Q, int ngemm, int pad_h,
             int pad_w, hipStream_t s)
{
    BandArgs b;
    memset(&b, 0, sizeof(b));
    b.src = src; b.bmat = bmat; b.bias = bias; b.dst = dst;
    b.N = (int)d.N; b.H = H; b.W = W; b.P = P; b.Q = Q; b.ngemm = ngemm;
    b.pad_h = pad_h; b.pad_w = pad_w; b.flip = flip; b.relu = relu; b.requant_m = requant_m;
    const int seg = 64 - (int)(d.dw * (d.S - 1));
    const int gn = (ngemm + 63) / 64, gq = (Q + seg - 1) / seg;
    band_rows(b, (long long)gn * gq);
    return hip_status(launch_band(dtype, (int)d.R, (int)d.S, cin, (int)d.dh, b, gn, gq, s));
}

// Winograd launch: batches of 2 output rows x 64 columns over a persistent
// grid of about one workgroup per CU across the 64-channel slices, a multiple
// of 8 (one share per XCD) when there are that many batches.
int run_wino(int dtype, const Dims &d, WinoArgs &wa, hipStream_t s)
{
    wa.tile_rows = (wa.P + 1) / 2;
    wa.tiles_q = (wa.Q + 63) / 64;
    const long long batches = d.N * wa.tile_rows * wa.tiles_q;
    if (batches > INT32_MAX) return CONV2D_ERR_UNSUPPORTED;
    wa.batches = (int)batches;
    const long long slices = (wa.ngemm + 63) / 64;
    long long gx = std::max(1LL, (long long)kNumCUs / slices);
    gx = std::min(gx, batches);
    if (gx >= 8) gx -= gx % 8;
    return hip_status(launch_wino_fprop(dtype, wa, (int)gx, s));
}

}  // namespace

// Bias gradient: column sums of dy [N*P*Q][K] over row slices, about two
// workgroups per CU and at least 64 rows per slice, then the split-K reduce.
static int bias_grad_plan(const conv2d_problem_t *prob, int dtype, Dims *d, int *splits, size_t *ws)
{
    int st = validate(prob, d);
    if (st) return st;
    if (dtype != CONV2D_DTYPE_F16 && dtype != CONV2D_DTYPE_BF16) return CONV2D_ERR_UNSUPPORTED;
    const long long rows = d->N * d->P * d->Q;
    if (rows * d->K > kMaxElems) return CONV2D_ERR_UNSUPPORTED;
    const long long cb = ((d->K + 7) / 8 + kColsumVecsPerWg - 1) / kColsumVecsPerWg;
    long long s = std::min(std::max(1LL, 2LL * kNumCUs / cb), std::max(1LL, rows / 64));
    s = std::min(s, 65535LL);
    *splits = (int)s;
    *ws = round_up((size_t)s * splitk_stride(d->K) * sizeof(float), 256);
    return CONV2D_OK;
}

// ---- scratch of the no-allocation wgrad entry point -------------------------
// For callers that cannot allocate, the wgrad partials go to this file-scope
// device array instead of a caller workspace.  Every device the library runs
// on holds its own copy (CONV2D_NOALLOC_SCRATCH_BYTES) until the process
// ends.  The array's name is a host-side stand-in, not a device address: its
// address on a device comes from hipGetSymbolAddress with that device
// current, taken once per device and kept in scratch_ptr; only that pointer
// is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[CONV2D_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
static void *scratch_ptr[kMaxDevices];
static std::mutex scratch_mu;

// The scratch address on the device the stream belongs to (the current device
// for the null stream).
static int scratch_for_stream(hipStream_t s, void **out)
{
    int cur = -1, dev = -1;
    if (hipGetDevice(&cur) != hipSuccess) return CONV2D_ERR_DEVICE;
    dev = cur;
    if (s && hipStreamGetDevice(s, &dev) != hipSuccess) return CONV2D_ERR_DEVICE;
    if (dev < 0 || dev >= kMaxDevices) return CONV2D_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return CONV2D_ERR_DEVICE;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return CONV2D_ERR_DEVICE;
        if (e != hipSuccess || !p) return CONV2D_ERR_DEVICE;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return CONV2D_OK;
}

extern "C" {

const char *conv2d_status_string(int status)
{
    switch (status) {
    case CONV2D_OK: return "ok";
    case CONV2D_ERR_INVALID_ARGUMENT: return "invalid argument";
    case CONV2D_ERR_UNSUPPORTED: return "unsupported problem, dtype or alignment";
    case CONV2D_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case CONV2D_ERR_DEVICE: return "device (HIP) error";
    case CONV2D_ERR_SCRATCH_LIMIT:
        return "the pass needs more scratch than the no-allocation entry point's static buffer holds";
    default: return "unknown status";
    }
}

int conv2d_output_size(const conv2d_problem_t *prob, int *P, int *Q)
{
    Dims d;
    int st = validate(prob, &d);
    if (st) return st;
    if (P) *P = (int)d.P;
    if (Q) *Q = (int)d.Q;
    return CONV2D_OK;
}

int conv2d_workspace_size(int op, const conv2d_problem_t *prob, int dtype, const conv2d_algo_t *algo,
                          size_t *bytes)
{
    if (!bytes) return CONV2D_ERR_INVALID_ARGUMENT;
    Plan pl;
    int st = make_plan(op, prob, dtype, algo, Epi(), &pl);
    if (st) return st;
    *bytes = pl.ws_bytes;
    return CONV2D_OK;
}

int conv2d_plan_info(int op, const conv2d_problem_t *prob, int dtype, const conv2d_algo_t *algo,
                     conv2d_plan_info_t *info)
{
    if (!info) return CONV2D_ERR_INVALID_ARGUMENT;
    Plan pl;
    int st = make_plan(op, prob, dtype, algo, Epi(), &pl);
    if (st) return st;
    info->kernel = pl.kernel;
    info->tile = pl.tile;
    info->num_tiles = pl.num_tiles;
    info->split_k = pl.split_k;
    info->phases = pl.phases;
    info->workspace_bytes = pl.ws_bytes;
    return CONV2D_OK;
}

static int fprop_run(const conv2d_problem_t *prob, int dtype, const void *x, const void *w, const void *bias,
                     int relu, double act_scale, double w_scale, double out_scale, const Epi &ep, void *y,
                     void *workspace, size_t workspace_bytes, const conv2d_algo_t *algo, void *stream)
{
    Plan pl;
    int st = make_plan(CONV2D_OP_FPROP, prob, dtype, algo, ep, &pl);
    if (st) return st;
    if (!x || !w || !y) return CONV2D_ERR_INVALID_ARGUMENT;
    if (relu != 0 && relu != 1) return CONV2D_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return CONV2D_ERR_UNSUPPORTED;
    const size_t bias_align = dtype == CONV2D_DTYPE_I8 ? 4 : 2;
    if (bias && ((uintptr_t)bias % bias_align)) return CONV2D_ERR_UNSUPPORTED;
    double m = 0.0;
    if (dtype == CONV2D_DTYPE_I8) {
        const double sc[3] = {act_scale, w_scale, out_scale};
        for (double s : sc)
            if (!(s > 0.0) || !(s < 1e300)) return CONV2D_ERR_INVALID_ARGUMENT;
        m = act_scale * w_scale / out_scale;  // double, left to right
    }
    if (workspace_bytes < pl.ws_bytes) return CONV2D_ERR_WORKSPACE_TOO_SMALL;
    if (pl.ws_bytes && (!workspace || !aligned16(workspace))) return CONV2D_ERR_INVALID_ARGUMENT;
    const Dims &d = pl.d;
    hipStream_t s = (hipStream_t)stream;

    if (pl.kernel == 4) {
        FewArgs f;
        memset(&f, 0, sizeof(f));
        if (!fewchan_layout(d, dtype, &f)) return CONV2D_ERR_UNSUPPORTED;
        f.x = x; f.w = w; f.bias = bias; f.y = y; f.relu = relu;
        return hip_status(launch_fewchan_fprop(dtype, f, s));
    }
    if (pl.kernel == 5 && !pl.padded) {  // (a padded plan carries its inner plan's kernel)
        PwArgs p;
        memset(&p, 0, sizeof(p));
        p.src = x; p.w = w; p.bias = bias; p.dst = y;
        p.npix = (int)(d.N * d.H * d.W); p.gk = (int)d.C; p.nout = (int)d.K;
        p.src_bytes = (long long)p.npix * d.C * 2; p.w_bytes = d.K * d.C * 2;
        p.relu = relu;
        return hip_status(launch_pointwise(dtype, p, s));
    }

    if (pl.padded) {
        unsigned char *wsb = (unsigned char *)workspace;
        const int e = elem_size(dtype);
        const long long Cp = pl.inner.c, Kp = pl.inner.k, npix = d.N * d.P * d.Q;
        const void *xp = x, *bp = bias;
        conv2d_algo_t ia;
        if (pl.tile_shift && algo) {
            ia = *algo;
            ia.tile -= pl.tile_shift;
            algo = &ia;
        }
        void *yp = y;
        if (pl.off_act != kNoBuf) {
            xp = wsb + pl.off_act;
            if (repack(e, x, d.N * d.H * d.W, d.C, d.C, (void *)xp, d.N * d.H * d.W, Cp, Cp, s) != hipSuccess)
                return CONV2D_ERR_DEVICE;
        }
        if (repack(e, w, d.K * d.R * d.S, d.C, d.C, wsb + pl.off_filt, Kp * d.R * d.S, Cp, Cp, s) != hipSuccess)
            return CONV2D_ERR_DEVICE;
        Epi ei = ep;
        if (pl.off_out != kNoBuf) {
            yp = wsb + pl.off_out;
            if (bias) {
                bp = wsb + pl.off_bias;
                if (repack(dtype == CONV2D_DTYPE_I8 ? 4 : e, bias, 1, d.K, d.K, (void *)bp, 1, Kp, Kp, s) != hipSuccess)
                    return CONV2D_ERR_DEVICE;
            }
            if (ep.c) {  // C padded into the padded output, which the inner pass reads and overwrites
                if (repack(e, ep.c, npix, d.K, d.K, yp, npix, Kp, Kp, s) != hipSuccess) return CONV2D_ERR_DEVICE;
                ei.c = yp;
            }
        }
        st = fprop_run(&pl.inner, dtype, xp, wsb + pl.off_filt, bp, relu, act_scale, w_scale, out_scale, ei, yp,
                       workspace, pl.inner_ws, algo, stream);
        if (st || pl.off_out == kNoBuf) return st;
        return hip_status(repack(e, yp, npix, d.K, Kp, y, npix, d.K, d.K, s));
    }

    if (pl.kernel == 2) {
        DirectArgs a{};
        a.a = x; a.b = w; a.bias = bias; a.out = y;
        a.N = (int)d.N; a.H = (int)d.H; a.W = (int)d.W; a.C = (int)d.C; a.K = (int)d.K;
        a.R = (int)d.R; a.S = (int)d.S; a.P = (int)d.P; a.Q = (int)d.Q;
        a.pad_h = (int)d.ph; a.pad_w = (int)d.pw; a.sh = (int)d.sh; a.sw = (int)d.sw;
        a.dh = (int)d.dh; a.dw = (int)d.dw; a.G = (int)d.G; a.Cg = (int)d.Cg; a.Kg = (int)d.Kg;
        a.relu = relu; a.requant_m = m; a.splits = 1;
        a.axpby = ep.axpby; a.alpha = ep.alpha; a.beta = ep.beta; a.cmat = ep.c;
        a.total = d.N * d.P * d.Q * d.K;
        if (pl.tile == 1 && direct_depthwise_ok(dtype, a.C, a.Cg, a.Kg, a.R, a.S)) {
            a.depthwise = 1;
        } else if (pl.tile == 1) {
            a.tiled = 1;
            a.rows = direct_tiled_rows(0, dtype, a.R, a.S, a.W, a.Q, a.Cg, a.Kg);
        }
        return hip_status(launch_direct_fprop(dtype, a, s));
    }

    if (pl.kernel == 6 && !pl.padded) {
        PatchArgs pa;
        memset(&pa, 0, sizeof(pa));
        if (!patch_layout(CONV2D_OP_FPROP, d, dtype, &pa, nullptr)) return CONV2D_ERR_UNSUPPORTED;
        pa.src = x; pa.filt = w; pa.bias = bias; pa.dst = y; pa.relu = relu;
        return hip_status(launch_patch(dtype, pa, false, s));
    }
    if (pl.tile == kBandTile)
        return run_band(dtype, d, (int)d.C, x, (int)d.H, (int)d.W, w, 0, bias, relu, m, y, (int)d.P, (int)d.Q,
                        (int)d.K, (int)d.ph, (int)d.pw, s);
    if (pl.tile == kWinoTile) {
        WinoArgs wa;
        memset(&wa, 0, sizeof(wa));
        wa.src = x; wa.w = w; wa.u = nullptr; wa.bias = bias; wa.dst = y;
        wa.N = (int)d.N; wa.H = (int)d.H; wa.W = (int)d.W; wa.P = (int)d.P; wa.Q = (int)d.Q;
        wa.ngemm = (int)d.K; wa.pad_h = (int)d.ph; wa.pad_w = (int)d.pw; wa.relu = relu;
        return run_wino(dtype, d, wa, s);
    }

    IgemmArgs a;
    memset(&a, 0, sizeof(a));
    a.src = x; a.bmat = w; a.bias = bias; a.dst = y;
    a.b_elems = d.K * d.R * d.S * d.Cg;
    a.nimg = (int)d.N; a.hs = (int)d.H; a.ws = (int)d.W; a.cs = (int)d.C;
    a.ngemm = (int)d.K;
    a.cg = (int)d.Cg; a.kg = (int)d.Kg;
    a.ho = (int)d.P; a.wo = (int)d.Q; a.osh = 1; a.osw = 1;
    a.gsh = (int)d.sh; a.gsw = (int)d.sw;
    a.relu = relu; a.requant_m = m;
    a.axpby = ep.axpby; a.alpha = ep.alpha; a.beta = ep.beta; a.cmat = ep.c;
    a.nphases = 1;
    Phase &ph = a.ph[0];
    ph.mi = (int)d.P; ph.mj = (int)d.Q; ph.oh0 = 0; ph.ow0 = 0;
    ph.th0 = -(int)d.ph; ph.tw0 = -(int)d.pw; ph.tdh = (int)d.dh; ph.tdw = (int)d.dw;
    ph.ntr = (int)d.R; ph.nts = (int)d.S;
    ph.kgemm = (int)(d.R * d.S * d.Cg);
    ph.m_total = (uint32_t)(d.N * d.P * d.Q);
    ph.b_off = 0;
    fill_phase_common(ph, pl.tile);
    TileShape ts = igemm_tile_shape(pl.tile);
    a.ntiles_g = (int)((d.Kg + ts.bn - 1) / ts.bn);
    return hip_status(launch_igemm(dtype, pl.tile, a, ph.tiles_m, (int)d.G * a.ntiles_g, s));
}

static int dgrad_run(const conv2d_problem_t *prob, int dtype, const void *dy, const void *w, const Epi &ep,
                     void *dx, void *workspace, size_t workspace_bytes, const conv2d_algo_t *algo, void *stream)
{
    Plan pl;
    int st = make_plan(CONV2D_OP_DGRAD, prob, dtype, algo, ep, &pl);
    if (st) return st;
    if (!dy || !w || !dx) return CONV2D_ERR_INVALID_ARGUMENT;
    if (!aligned16(dy) || !aligned16(w) || !aligned16(dx)) return CONV2D_ERR_UNSUPPORTED;
    if (workspace_bytes < pl.ws_bytes) return CONV2D_ERR_WORKSPACE_TOO_SMALL;
    if (pl.ws_bytes && (!workspace || !aligned16(workspace))) return CONV2D_ERR_INVALID_ARGUMENT;
    const Dims &d = pl.d;
    hipStream_t s = (hipStream_t)stream;

    if (pl.kernel == 4) {
        FewDgradArgs f;
        memset(&f, 0, sizeof(f));
        if (!fewchan_dgrad_layout(d, dtype, &f)) return CONV2D_ERR_UNSUPPORTED;
        f.dy = dy; f.w = w; f.dx = dx;
        return hip_status(launch_fewchan_dgrad(dtype, f, s));
    }
    if (pl.kernel == 5 && !pl.padded) {  // (a padded plan carries its inner plan's kernel)
        PwArgs p;
        memset(&p, 0, sizeof(p));
        p.src = dy; p.w = w; p.bias = nullptr; p.dst = dx;
        p.npix = (int)(d.N * d.H * d.W); p.gk = (int)d.K; p.nout = (int)d.C;
        p.src_bytes = (long long)p.npix * d.K * 2; p.w_bytes = d.K * d.C * 2;
        p.trans = 1;
        return hip_status(launch_pointwise(dtype, p, s));
    }
    if (pl.kernel == 6 && !pl.padded) {  // (a padded plan carries its inner plan's kernel)
        PatchArgs pa;
        memset(&pa, 0, sizeof(pa));
        if (!patch_layout(CONV2D_OP_DGRAD, d, dtype, &pa, nullptr)) return CONV2D_ERR_UNSUPPORTED;
        pa.src = dy; pa.filt = w; pa.bias = nullptr; pa.dst = dx; pa.relu = 0;
        return hip_status(launch_patch(dtype, pa, true, s));
    }

    if (pl.padded) {
        unsigned char *wsb = (unsigned char *)workspace;
        const int e = elem_size(dtype);
        const long long Cp = pl.inner.c, Kp = pl.inner.k, npix = d.N * d.P * d.Q, nin = d.N * d.H * d.W;
        const void *dyp = dy;
        void *dxp = dx;
        conv2d_algo_t ia;
        if (pl.tile_shift && algo) {
            ia = *algo;
            ia.tile -= pl.tile_shift;
            algo = &ia;
        }
        if (pl.off_out != kNoBuf) {
            dyp = wsb + pl.off_out;
            if (repack(e, dy, npix, d.K, d.K, (void *)dyp, npix, Kp, Kp, s) != hipSuccess) return CONV2D_ERR_DEVICE;
        }
        if (repack(e, w, d.K * d.R * d.S, d.C, d.C, wsb + pl.off_filt, Kp * d.R * d.S, Cp, Cp, s) != hipSuccess)
            return CONV2D_ERR_DEVICE;
        Epi ei = ep;
        if (pl.off_act != kNoBuf) {
            dxp = wsb + pl.off_act;
            if (ep.c) {  // C padded into the padded dx, which the inner pass reads and overwrites
                if (repack(e, ep.c, nin, d.C, d.C, dxp, nin, Cp, Cp, s) != hipSuccess) return CONV2D_ERR_DEVICE;
                ei.c = dxp;
            }
        }
        st = dgrad_run(&pl.inner, dtype, dyp, wsb + pl.off_filt, ei, dxp, workspace, pl.inner_ws, algo, stream);
        if (st || pl.off_act == kNoBuf) return st;
        return hip_status(repack(e, dxp, nin, d.C, Cp, dx, nin, d.C, d.C, s));
    }

    if (pl.kernel == 2) {
        DirectArgs a{};
        a.a = dy; a.b = w; a.out = dx;
        a.N = (int)d.N; a.H = (int)d.H; a.W = (int)d.W; a.C = (int)d.C; a.K = (int)d.K;
        a.R = (int)d.R; a.S = (int)d.S; a.P = (int)d.P; a.Q = (int)d.Q;
        a.pad_h = (int)d.ph; a.pad_w = (int)d.pw; a.sh = (int)d.sh; a.sw = (int)d.sw;
        a.dh = (int)d.dh; a.dw = (int)d.dw; a.G = (int)d.G; a.Cg = (int)d.Cg; a.Kg = (int)d.Kg;
        a.splits = 1;
        a.axpby = ep.axpby; a.alpha = ep.alpha; a.beta = ep.beta; a.cmat = ep.c;
        a.total = d.N * d.H * d.W * d.C;
        if (pl.tile == 1 && direct_depthwise_ok(dtype, a.C, a.Cg, a.Kg, a.R, a.S)) {
            a.depthwise = 1;
        } else if (pl.tile == 1) {
            a.tiled = 1;
            a.rows = direct_tiled_rows(1, dtype, a.R, a.S, a.W, a.Q, a.Cg, a.Kg);
        }
        return hip_status(launch_direct_dgrad(dtype, a, s));
    }

    if (pl.tile == kWinoTile) {  // the forward Winograd kernel on dy, with the flipped, transposed filter
        WinoArgs wa;
        memset(&wa, 0, sizeof(wa));
        wa.src = dy; wa.w = w; wa.u = workspace; wa.bias = nullptr; wa.dst = dx;
        wa.N = (int)d.N; wa.H = (int)d.P; wa.W = (int)d.Q; wa.P = (int)d.H; wa.Q = (int)d.W;
        wa.ngemm = (int)d.C; wa.pad_h = (int)(2 - d.ph); wa.pad_w = (int)(2 - d.pw); wa.relu = 0;
        return run_wino(dtype, d, wa, s);
    }
    if (pl.tile == kBandTile)  // stride 1: every tap, filter read reversed and transposed
        return run_band(dtype, d, (int)d.K, dy, (int)d.P, (int)d.Q, w, 1, nullptr, 0, 0.0, dx, (int)d.H, (int)d.W,
                        (int)d.C, (int)(d.dh * (d.R - 1) - d.ph), (int)(d.dw * (d.S - 1) - d.pw), s);

    // One GEMM per stride phase (h mod sh, w mod sw), one launch for all.
    // B is the filter as it lies in memory, read transposed in LDS, or for
    // long GEMM-K rows a copy re-laid out per phase by a first kernel.
    const bool relayout = dgrad_relayout(d);
    PrepArgs pa;
    memset(&pa, 0, sizeof(pa));
    pa.w = w; pa.wt = workspace;
    pa.K = (int)d.K; pa.R = (int)d.R; pa.S = (int)d.S; pa.C = (int)d.C;
    pa.Kg = (int)d.Kg; pa.Cg = (int)d.Cg;
    IgemmArgs a;
    memset(&a, 0, sizeof(a));
    a.src = dy; a.bias = nullptr; a.dst = dx;
    if (relayout) {
        a.bmat = workspace;
        a.b_elems = d.R * d.S * d.C * d.Kg;
    } else {
        a.bmat = w;
        a.b_elems = d.K * d.R * d.S * d.Cg;
        a.b_trans = 1; a.filt_r = (int)d.R; a.filt_s = (int)d.S;
    }
    a.nimg = (int)d.N; a.hs = (int)d.P; a.ws = (int)d.Q; a.cs = (int)d.K;
    a.ngemm = (int)d.C;
    a.cg = (int)d.Kg; a.kg = (int)d.Cg;  // one GEMM per group: Kg dy channels in, Cg dx channels out
    a.ho = (int)d.H; a.wo = (int)d.W; a.osh = (int)d.sh; a.osw = (int)d.sw;
    a.gsh = 1; a.gsw = 1;
    a.relu = 0;
    a.axpby = ep.axpby; a.alpha = ep.alpha; a.beta = ep.beta; a.cmat = ep.c;
    long long off = 0;
    int nph = 0, max_tiles = 0;
    for (int py = 0; py < d.sh; ++py)
        for (int px = 0; px < d.sw; ++px) {
            AxisPhase ay = axis_phase(py, (int)d.H, (int)d.sh, (int)d.ph, (int)d.dh, (int)d.R);
            AxisPhase ax = axis_phase(px, (int)d.W, (int)d.sw, (int)d.pw, (int)d.dw, (int)d.S);
            if (ay.extent == 0 || ax.extent == 0) continue;
            Phase &ph = a.ph[nph];
            ph.mi = ay.extent; ph.mj = ax.extent; ph.oh0 = py; ph.ow0 = px;
            ph.th0 = ay.o0; ph.tw0 = ax.o0; ph.tdh = ay.dstep; ph.tdw = ax.dstep;
            ph.ntr = ay.ntap; ph.nts = ax.ntap;
            ph.kgemm = (int)(ay.ntap * ax.ntap * d.Kg);
            ph.m_total = (uint32_t)(d.N * ay.extent * ax.extent);
            ph.r0 = ay.r0; ph.rstep = ay.step; ph.s0 = ax.r0; ph.sstep = ax.step;
            ph.b_off = off;
            fill_phase_common(ph, pl.tile);
            max_tiles = std::max(max_tiles, ph.tiles_m);
            PrepPhase &pp = pa.ph[nph];
            pp.r0 = ay.r0; pp.rstep = ay.step; pp.ntr = ay.ntap;
            pp.s0 = ax.r0; pp.sstep = ax.step; pp.nts = ax.ntap;
            pp.off = off;
            const long long elems = d.C * ay.ntap * ax.ntap * d.Kg;
            pa.max_elems = (int)std::max<long long>(pa.max_elems, elems);
            off += elems;
            ++nph;
        }
    a.nphases = nph;
    pa.nphases = nph;
    if (nph == 0) return CONV2D_OK;
    if (relayout && launch_dgrad_prep(dtype, pa, s) != hipSuccess) return CONV2D_ERR_DEVICE;
    TileShape ts = igemm_tile_shape(pl.tile);
    a.ntiles_g = (int)((d.Cg + ts.bn - 1) / ts.bn);
    return hip_status(launch_igemm(dtype, pl.tile, a, max_tiles, (int)d.G * a.ntiles_g, s));
}

static int wgrad_run(const conv2d_problem_t *prob, int dtype, const void *x, const void *dy, const Epi &ep,
                     void *dw, void *workspace, size_t workspace_bytes, const conv2d_algo_t *algo, void *stream)
{
    Plan pl;
    int st = make_plan(CONV2D_OP_WGRAD, prob, dtype, algo, ep, &pl);
    if (st) return st;
    if (!x || !dy || !dw) return CONV2D_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dw)) return CONV2D_ERR_UNSUPPORTED;
    if (workspace_bytes < pl.ws_bytes) return CONV2D_ERR_WORKSPACE_TOO_SMALL;
    if (pl.ws_bytes && (!workspace || !aligned16(workspace))) return CONV2D_ERR_INVALID_ARGUMENT;
    const Dims &d = pl.d;
    hipStream_t s = (hipStream_t)stream;
    const uint32_t npix = (uint32_t)(d.N * d.P * d.Q);
    // the epilogue (alpha, beta, fp32 output) runs in the split-K reduce
    const bool to_parts = ep.axpby || ep.out_f32;
    const bool reduce = pl.split_k > 1 || to_parts;
    void *out = reduce ? workspace : dw;
    const ReduceEpi re{ep.alpha, ep.beta, ep.axpby ? ep.c : nullptr, ep.out_f32 ? 1 : 0, nullptr, 0};

    if (pl.kernel == 4) {
        FewWgradArgs f;
        memset(&f, 0, sizeof(f));
        if (!fewchan_wgrad_layout(d, dtype, &f)) return CONV2D_ERR_UNSUPPORTED;
        f.x = x; f.dy = dy; f.out = workspace;
        if (launch_fewchan_wgrad(dtype, f, s) != hipSuccess) return CONV2D_ERR_DEVICE;
        return hip_status(launch_splitk_reduce(dtype, (const float *)workspace, pl.split_k, d.K * d.R * d.S * d.C,
                                               f.part_stride, dw, &re, s));
    }

    if (pl.padded) {
        unsigned char *wsb = (unsigned char *)workspace;
        const int e = elem_size(dtype);
        const long long Cp = pl.inner.c, Kp = pl.inner.k, nin = d.N * d.H * d.W;
        const void *xp = x, *dyp = dy;
        conv2d_algo_t ia;
        if (pl.tile_shift && algo) {
            ia = *algo;
            ia.tile -= pl.tile_shift;
            algo = &ia;
        }
        if (pl.off_act != kNoBuf) {
            xp = wsb + pl.off_act;
            if (repack(e, x, nin, d.C, d.C, (void *)xp, nin, Cp, Cp, s) != hipSuccess) return CONV2D_ERR_DEVICE;
        }
        if (pl.off_out != kNoBuf) {
            dyp = wsb + pl.off_out;
            if (repack(e, dy, npix, d.K, d.K, (void *)dyp, npix, Kp, Kp, s) != hipSuccess) return CONV2D_ERR_DEVICE;
        }
        void *dwp = wsb + pl.off_filt;
        const int eo = ep.out_f32 ? 4 : e;  // element size of dw (and C)
        Epi ei = ep;
        ei.db = nullptr;  // the bias gradient of the padded problem is not the caller's
        if (ep.c) {  // C padded into the padded dw, which the inner pass reads and overwrites
            if (repack(eo, ep.c, d.K * d.R * d.S, d.C, d.C, dwp, Kp * d.R * d.S, Cp, Cp, s) != hipSuccess)
                return CONV2D_ERR_DEVICE;
            ei.c = dwp;
        }
        st = wgrad_run(&pl.inner, dtype, xp, dyp, ei, dwp, workspace, pl.inner_ws, algo, stream);
        if (st) return st;
        // the first K*R*S rows of the padded [Kp][R][S][Cp] filter are k < K
        return hip_status(repack(eo, dwp, Kp * d.R * d.S, Cp, Cp, dw, d.K * d.R * d.S, d.C, d.C, s));
    }

    if (pl.kernel == 2) {
        DirectArgs a{};
        a.a = x; a.b = dy; a.out = out;
        a.N = (int)d.N; a.H = (int)d.H; a.W = (int)d.W; a.C = (int)d.C; a.K = (int)d.K;
        a.R = (int)d.R; a.S = (int)d.S; a.P = (int)d.P; a.Q = (int)d.Q;
        a.pad_h = (int)d.ph; a.pad_w = (int)d.pw; a.sh = (int)d.sh; a.sw = (int)d.sw;
        a.dh = (int)d.dh; a.dw = (int)d.dw; a.G = (int)d.G; a.Cg = (int)d.Cg; a.Kg = (int)d.Kg;
        a.splits = pl.split_k;
        a.npix = npix;
        a.pix_per_split = (npix + pl.split_k - 1) / pl.split_k;
        a.total = d.K * d.R * d.S * d.Cg;
        a.part_stride = splitk_stride(a.total);
        a.depthwise = pl.tile == 1 && direct_depthwise_ok(dtype, a.C, a.Cg, a.Kg, a.R, a.S);
        a.tiled = pl.tile == 1 && !a.depthwise;
        a.to_parts = to_parts || a.depthwise;
        if (a.depthwise) {
            a.out = workspace;  // the depthwise kernel always writes partials
            const int cols = direct_depthwise_wgrad_cols(a.N, a.H, a.W, a.C, a.P, a.Q, a.R, a.S, a.sw, a.dw);
            a.npix = (uint32_t)depthwise_units(d);
            a.pix_per_split = (a.npix + pl.split_k - 1) / pl.split_k;
            a.div_q = make_fastdiv((uint32_t)((a.Q + cols - 1) / cols));
            a.div_p = make_fastdiv((uint32_t)a.P);
        }
        hipError_t e = launch_direct_wgrad(dtype, a, s);
        if (e != hipSuccess || !(reduce || a.depthwise)) return hip_status(e);
        return hip_status(
            launch_splitk_reduce(dtype, (const float *)workspace, pl.split_k, a.total, a.part_stride, dw, &re, s));
    }

    if (pl.kernel == 5 && !pl.padded) {  // (a padded plan carries its inner plan's kernel)
        PwWgradArgs p;
        memset(&p, 0, sizeof(p));
        p.x = x; p.dy = dy; p.out = workspace;
        p.npix = npix;
        p.K = (int)d.K; p.C = (int)d.C;
        p.splits = pl.split_k;
        p.pix_per_split = (int)pointwise_wgrad_pps(d, pl.split_k);
        p.with_db = ep.db != nullptr;  // the bias gradient rides along in the slices
        const long long kc = d.K * d.C;
        p.part_stride = splitk_stride(kc + (p.with_db ? d.K : 0));
        if (launch_pointwise_wgrad(dtype, p, s) != hipSuccess) return CONV2D_ERR_DEVICE;
        ReduceEpi rp = re;
        if (p.with_db) {
            rp.out2 = ep.db;
            rp.count1 = kc;
        }
        return hip_status(launch_splitk_reduce(dtype, (const float *)workspace, pl.split_k,
                                               kc + (p.with_db ? d.K : 0), p.part_stride, dw, &rp, s));
    }

    if (pl.tile == kWgradBandTile) {
        WgradBandArgs b;
        memset(&b, 0, sizeof(b));
        b.x = x; b.dy = dy; b.out = workspace;
        b.N = (int)d.N; b.H = (int)d.H; b.W = (int)d.W; b.P = (int)d.P; b.Q = (int)d.Q;
        b.pad_h = (int)d.ph; b.pad_w = (int)d.pw;
        const WgradBandLayout bl = wgrad_band_layout(d);
        b.nsplit = bl.nsplit;
        b.rows_per_wg = bl.rows;
        b.chunks_per_img = bl.chunks;
        b.nbands = bl.nbands;
        b.rows_total = (int)(d.N * d.P);
        b.band_f = (3 * bl.nbands) / 24;
        b.div_p = make_fastdiv((uint32_t)d.P);
        const long long kcols = d.K * d.R * d.S * d.C;
        b.with_db = ep.db != nullptr;  // the bias gradient rides along in the slices
        b.part_stride = splitk_stride(kcols + (b.with_db ? d.K : 0));
        b.xw = (int)(d.Q + d.dw * (d.S - 1));
        b.div_xw = make_fastdiv((uint32_t)b.xw);
        b.xcd_pairs = bl.nsplit == 2 && (d.N * b.chunks_per_img) % 8 == 0;
        hipError_t e = launch_wgrad_band(dtype, b, s);
        if (e != hipSuccess) return CONV2D_ERR_DEVICE;
        ReduceEpi rb = re;
        if (b.with_db) {
            rb.out2 = ep.db;
            rb.count1 = kcols;
        }
        return hip_status(launch_splitk_reduce(dtype, (const float *)workspace, pl.split_k,
                                               kcols + (b.with_db ? d.K : 0), b.part_stride, dw, &rb, s));
    }

    WgradArgs a;
    memset(&a, 0, sizeof(a));
    a.x = x; a.dy = dy; a.out = out;
    a.N = (int)d.N; a.H = (int)d.H; a.W = (int)d.W; a.C = (int)d.C; a.K = (int)d.K;
    a.R = (int)d.R; a.S = (int)d.S; a.P = (int)d.P; a.Q = (int)d.Q;
    a.pad_h = (int)d.ph; a.pad_w = (int)d.pw; a.sh = (int)d.sh; a.sw = (int)d.sw;
    a.dh = (int)d.dh; a.dw = (int)d.dw;
    a.ncols = (int)(d.R * d.S * d.Cg);  // per group
    a.Kg = (int)d.Kg; a.Cg = (int)d.Cg;
    a.mtiles_g = (int)((d.Kg + wgrad_tile_shape(pl.tile).bm - 1) / wgrad_tile_shape(pl.tile).bm);
    a.npix = npix;
    // slices are whole main-loop steps
    const uint32_t steps = (npix + kWgradPixStep - 1) / kWgradPixStep;
    a.pix_per_split = ((steps + pl.split_k - 1) / pl.split_k) * kWgradPixStep;
    a.splits = pl.split_k;
    a.part_stride = splitk_stride((long long)d.K * a.ncols);
    a.div_Q = make_fastdiv((uint32_t)d.Q);
    a.div_PQ = make_fastdiv((uint32_t)(d.P * d.Q));
    a.div_C = make_fastdiv((uint32_t)d.Cg);
    a.div_S = make_fastdiv((uint32_t)d.S);
    a.to_parts = to_parts;
    a.with_db = ep.db && pl.tile == 0;
    if (a.with_db) {  // dy's column sums ride along in the slices: always partials
        a.to_parts = 1;
        a.out = workspace;
        a.part_stride = splitk_stride((long long)d.K * a.ncols + d.K);
    }
    hipError_t e = launch_wgrad(dtype, pl.tile, a, s);
    if (e != hipSuccess || !(reduce || a.with_db)) return hip_status(e);
    ReduceEpi rg = re;
    if (a.with_db) {
        rg.out2 = ep.db;
        rg.count1 = (long long)d.K * a.ncols;
    }
    return hip_status(launch_splitk_reduce(dtype, (const float *)workspace, pl.split_k,
                                           (long long)d.K * a.ncols + (a.with_db ? d.K : 0), a.part_stride, dw,
                                           &rg, s));
}

// conv2d_epilogue_t -> Epi, with its checks (before anything is enqueued)
static int make_epi(const conv2d_epilogue_t *e, int op, Epi *ep)
{
    *ep = Epi();
    if (!e) return CONV2D_OK;
    if (!(std::fabs(e->alpha) < 1e30) || !(std::fabs(e->beta) < 1e30)) return CONV2D_ERR_INVALID_ARGUMENT;
    if (e->out_f32 != 0 && e->out_f32 != 1) return CONV2D_ERR_INVALID_ARGUMENT;
    if (e->out_f32 && op != CONV2D_OP_WGRAD) return CONV2D_ERR_INVALID_ARGUMENT;
    ep->alpha = (float)e->alpha;
    ep->beta = (float)e->beta;
    ep->axpby = ep->alpha != 1.0f || ep->beta != 0.0f;
    ep->out_f32 = e->out_f32 != 0;
    if (ep->beta != 0.0f) {
        if (!e->c) return CONV2D_ERR_INVALID_ARGUMENT;
        if (!aligned16(e->c)) return CONV2D_ERR_UNSUPPORTED;
        ep->c = e->c;
    }
    if (e->db) {
        if (op != CONV2D_OP_WGRAD) return CONV2D_ERR_INVALID_ARGUMENT;
        if (!aligned16(e->db)) return CONV2D_ERR_UNSUPPORTED;
        ep->db = e->db;
    }
    return CONV2D_OK;
}

// Workspace of wgrad_ex: the pass's own, then (with db, unless the wgrad band
// kernel sums dy in its own slices) the bias-gradient partials at the next
// 256-byte boundary.  *fused tells which.
static int wgrad_ex_workspace(const conv2d_problem_t *prob, int dtype, const conv2d_algo_t *algo, const Epi &ep,
                              size_t *pass_bytes, size_t *total, bool *fused)
{
    Plan pl;
    int st = make_plan(CONV2D_OP_WGRAD, prob, dtype, algo, ep, &pl);
    if (st) return st;
    *pass_bytes = pl.ws_bytes;
    *total = pl.ws_bytes;
    *fused = ep.db && !pl.padded &&
             ((pl.kernel == 1 && (pl.tile == kWgradBandTile || pl.tile == 0)) || pl.kernel == 5);
    if (ep.db && !*fused) {
        Dims d;
        int splits;
        size_t bws;
        st = bias_grad_plan(prob, dtype, &d, &splits, &bws);
        if (st) return st;
        *total = round_up(pl.ws_bytes, 256) + bws;
    }
    return CONV2D_OK;
}

int conv2d_workspace_size_ex(int op, const conv2d_problem_t *prob, int dtype, const conv2d_algo_t *algo,
                             const conv2d_epilogue_t *epi, size_t *bytes)
{
    if (!bytes) return CONV2D_ERR_INVALID_ARGUMENT;
    Epi ep;
    int st = make_epi(epi, op, &ep);
    if (st) return st;
    if (op == CONV2D_OP_WGRAD) {
        size_t pass;
        bool fused;
        return wgrad_ex_workspace(prob, dtype, algo, ep, &pass, bytes, &fused);
    }
    Plan pl;
    st = make_plan(op, prob, dtype, algo, ep, &pl);
    if (st) return st;
    *bytes = pl.ws_bytes;
    return CONV2D_OK;
}

int conv2d_fprop(const conv2d_problem_t *prob, int dtype, const void *x, const void *w, const void *bias,
                 int relu, double act_scale, double w_scale, double out_scale, void *y, void *workspace,
                 size_t workspace_bytes, const conv2d_algo_t *algo, void *stream)
{
    return fprop_run(prob, dtype, x, w, bias, relu, act_scale, w_scale, out_scale, Epi(), y, workspace,
                     workspace_bytes, algo, stream);
}

int conv2d_dgrad(const conv2d_problem_t *prob, int dtype, const void *dy, const void *w, void *dx,
                 void *workspace, size_t workspace_bytes, const conv2d_algo_t *algo, void *stream)
{
    return dgrad_run(prob, dtype, dy, w, Epi(), dx, workspace, workspace_bytes, algo, stream);
}

int conv2d_wgrad(const conv2d_problem_t *prob, int dtype, const void *x, const void *dy, void *dw,
                 void *workspace, size_t workspace_bytes, const conv2d_algo_t *algo, void *stream)
{
    return wgrad_run(prob, dtype, x, dy, Epi(), dw, workspace, workspace_bytes, algo, stream);
}

int conv2d_wgrad_noalloc(const conv2d_problem_t *prob, int dtype, const void *x, const void *dy, void *dw,
                         const conv2d_algo_t *algo, void *stream)
{
    Plan pl;
    int st = make_plan(CONV2D_OP_WGRAD, prob, dtype, algo, Epi(), &pl);
    if (st) return st;
    if (pl.ws_bytes > (size_t)CONV2D_NOALLOC_SCRATCH_BYTES) return CONV2D_ERR_SCRATCH_LIMIT;
    void *ws = nullptr;
    if (pl.ws_bytes) {
        st = scratch_for_stream((hipStream_t)stream, &ws);
        if (st) return st;
    }
    return wgrad_run(prob, dtype, x, dy, Epi(), dw, ws, pl.ws_bytes ? (size_t)CONV2D_NOALLOC_SCRATCH_BYTES : 0,
                     algo, stream);
}

int conv2d_fprop_ex(const conv2d_problem_t *prob, int dtype, const void *x, const void *w, const void *bias,
                    int relu, const conv2d_epilogue_t *epi, void *y, void *workspace, size_t workspace_bytes,
                    const conv2d_algo_t *algo, void *stream)
{
    Epi ep;
    int st = make_epi(epi, CONV2D_OP_FPROP, &ep);
    if (st) return st;
    if (dtype == CONV2D_DTYPE_I8) return CONV2D_ERR_UNSUPPORTED;
    return fprop_run(prob, dtype, x, w, bias, relu, 1.0, 1.0, 1.0, ep, y, workspace, workspace_bytes, algo, stream);
}

int conv2d_dgrad_ex(const conv2d_problem_t *prob, int dtype, const void *dy, const void *w,
                    const conv2d_epilogue_t *epi, void *dx, void *workspace, size_t workspace_bytes,
                    const conv2d_algo_t *algo, void *stream)
{
    Epi ep;
    int st = make_epi(epi, CONV2D_OP_DGRAD, &ep);
    if (st) return st;
    return dgrad_run(prob, dtype, dy, w, ep, dx, workspace, workspace_bytes, algo, stream);
}

int conv2d_bias_grad_workspace_size(const conv2d_problem_t *prob, int dtype, size_t *bytes)
{
    if (!bytes) return CONV2D_ERR_INVALID_ARGUMENT;
    Dims d;
    int splits;
    return bias_grad_plan(prob, dtype, &d, &splits, bytes);
}

int conv2d_bias_grad(const conv2d_problem_t *prob, int dtype, const void *dy, void *db, int out_f32,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    Dims d;
    int splits;
    size_t ws;
    int st = bias_grad_plan(prob, dtype, &d, &splits, &ws);
    if (st) return st;
    if (!dy || !db || (out_f32 != 0 && out_f32 != 1)) return CONV2D_ERR_INVALID_ARGUMENT;
    if (!aligned16(dy) || !aligned16(db)) return CONV2D_ERR_UNSUPPORTED;
    if (workspace_bytes < ws) return CONV2D_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace || !aligned16(workspace)) return CONV2D_ERR_INVALID_ARGUMENT;
    const uint32_t rows = (uint32_t)(d.N * d.P * d.Q);
    ColsumArgs a;
    a.src = dy;
    a.parts = (float *)workspace;
    a.rows = rows;
    a.rows_per_split = (rows + splits - 1) / splits;
    a.K = (int)d.K;
    a.vec = d.K % 8 == 0;
    a.part_stride = splitk_stride(d.K);
    hipStream_t s = (hipStream_t)stream;
    if (launch_colsum(dtype, a, splits, s) != hipSuccess) return CONV2D_ERR_DEVICE;
    const ReduceEpi re{1.0f, 0.0f, nullptr, out_f32, nullptr, 0};
    return hip_status(launch_splitk_reduce(dtype, a.parts, splits, d.K, a.part_stride, db, &re, s));
}

int conv2d_wgrad_ex(const conv2d_problem_t *prob, int dtype, const void *x, const void *dy,
                    const conv2d_epilogue_t *epi, void *dw, void *workspace, size_t workspace_bytes,
                    const conv2d_algo_t *algo, void *stream)
{
    Epi ep;
    int st = make_epi(epi, CONV2D_OP_WGRAD, &ep);
    if (st) return st;
    if (!ep.db) return wgrad_run(prob, dtype, x, dy, ep, dw, workspace, workspace_bytes, algo, stream);
    // with the bias gradient: check everything of both parts before enqueuing either
    size_t pass, total;
    bool fused;
    st = wgrad_ex_workspace(prob, dtype, algo, ep, &pass, &total, &fused);
    if (st) return st;
    if (fused) return wgrad_run(prob, dtype, x, dy, ep, dw, workspace, workspace_bytes, algo, stream);
    if (!x || !dy || !dw) return CONV2D_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dw)) return CONV2D_ERR_UNSUPPORTED;
    if (workspace_bytes < total) return CONV2D_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace || !aligned16(workspace)) return CONV2D_ERR_INVALID_ARGUMENT;
    Epi en = ep;
    en.db = nullptr;  // the bias gradient runs on its own below
    st = wgrad_run(prob, dtype, x, dy, en, dw, pass ? workspace : nullptr, pass, algo, stream);
    if (st) return st;
    unsigned char *bws = (unsigned char *)workspace + round_up(pass, 256);
    return conv2d_bias_grad(prob, dtype, dy, ep.db, ep.out_f32 ? 1 : 0, bws, total - round_up(pass, 256), stream);
}

}  // extern "C"

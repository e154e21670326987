// internal.h -- types shared by the host planner (api.cpp) and the HIP kernel
// launchers of the conv2d library.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "conv2d_nhwc.h"

namespace cnv {

// Unsigned division by an invariant divisor d (1 <= d < 2^31) for dividends
// n < 2^31: q = (umulhi(n, m) + n) >> s with s = ceil(log2 d) and
// m = floor(2^32 * (2^s - d) / d) + 1 (Granlund & Montgomery, "Division by
// invariant integers using multiplication", 1994).  Replaces the slow integer
// divide in per-element index decomposition.
struct FastDiv {
    uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.s = s;
    f.m = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1);
    return f;
}

__host__ __device__ inline uint32_t fdiv(uint32_t n, const FastDiv &f)
{
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t t = __umulhi(n, f.m);
#else
    uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);
#endif
    return (t + n) >> f.s;
}

// ---------------------------------------------------------------------------
// Implicit GEMM (fprop, and dgrad per stride phase).
//
// The GEMM is D[m][n] = sum_kk A[m][kk] * B[n][kk] with
//   m  = output pixel of an output sub-grid (image, i, j),
//   n  = output channel,
//   kk = (tap tr, tap ts, source channel c), c innermost,
//   A[m][kk] = src[image][i*gsh + th0 + tr*tdh][j*gsw + tw0 + ts*tdw][c]
//              (zero outside the source image: implicit padding),
//   B        = a dense row-major [ngemm][kgemm] matrix.
// fprop: src = x, B = w ([K][R*S*C]), one phase covering all of y.
// dgrad: src = dy, B = the filter re-laid out per stride phase; each phase is
//   the sub-grid of dx rows h = oh0 + i*osh (and columns likewise) that the
//   same set of taps reaches.
// ---------------------------------------------------------------------------
constexpr int kMaxPhases = 16;
// Largest operand (bytes) the implicit-GEMM kernels read through 32-bit
// buffer offsets; kBufOOBFar lies past it.
constexpr unsigned long long kBufMaxBytes = 0xffffff00ull;

struct Phase {
    int mi, mj;       // sub-grid extent
    int oh0, ow0;     // first output row / column of the sub-grid
    int th0, tw0;     // source row / column of tap (0,0) at sub-grid origin
    int tdh, tdw;     // source offset per tap index
    int ntr, nts;     // taps per axis
    int kgemm;        // ntr * nts * cs
    int tiles_m;      // ceil(m_total / BM)
    uint32_t m_total; // nimg * mi * mj
    long long b_off;  // element offset of this phase's B matrix
    FastDiv div_mj, div_mimj;
    // dgrad with the filter read as it is (IgemmArgs.b_trans): filter tap
    // (r0 + jr*rstep, s0 + js*sstep) for tap index (jr, js)
    int r0, rstep, s0, sstep;
};

struct IgemmArgs {
    const void *src;
    const void *bmat;
    long long b_elems; // elements of bmat (all phases)
    const void *bias;  // [ngemm]; element type (float paths) or int32 (int8)
    void *dst;
    int nimg, hs, ws, cs;  // source image (cs: channels per pixel)
    int ngemm;
    // groups (fprop): GEMM-K runs over cg channels per tap starting at
    // g*cg, GEMM-N over kg output channels starting at g*kg; grid.y =
    // groups * ntiles_g.  Dense: cg = cs, kg = ngemm, ntiles_g = grid.y.
    int cg, kg, ntiles_g;
    int ho, wo;            // full output image extent
    int osh, osw;          // output step of the sub-grid
    int gsh, gsw;          // source step per sub-grid step
    int relu;
    double requant_m;      // int8 only
    // out = alpha * acc + beta * cmat (+ bias), cmat laid out like dst (float paths)
    int axpby;
    float alpha, beta;
    const void *cmat;
    int nphases;
    // dgrad: B is the filter w[K][R][S][C] itself (no re-layout pass): its
    // GEMM-K rows (tap, dy channel) are staged as they lie in w, dx channels
    // along the row, and the fragments are read with transposing LDS reads
    int b_trans, filt_r, filt_s;
    Phase ph[kMaxPhases];
};

struct TileShape {
    int bm, bn;
};

int igemm_num_tiles();
TileShape igemm_tile_shape(int tile);
hipError_t launch_igemm(int dtype, int tile, const IgemmArgs &a, int grid_m, int grid_n,
                        hipStream_t st);

// ---------------------------------------------------------------------------
// Patch kernel (patch.hip): the workgroup's source patch in LDS.  Along each
// axis the source rows a convolution reads lie on a lattice of step
// g = gcd(stride, dil) (lattice row i is source row g*i - pad); on it the
// convolution has stride sh1 = stride / g and dilation dh1 = dil / g.  A
// workgroup computes TP x TQ output lattice pixels (TP*TQ <= 128) of one
// image and 32*nb output channels from PH x PW lattice pixels held at a pitch
// of PP 16-byte slots (PP odd, PP >= SC/8); TP*TQ <= 32*mb.  Output lattice pixel (p, q) is
// destination pixel (oh0 + ogh*p, ow0 + ogw*q).
// fprop: src = x (SC = C), dst = y, lattice extents P x Q, ogh = ogw = 1.
// dgrad (stride dividing dilation): src = dy (SC = K, g = 1, sh1 = 1,
//   dh1 = dil/stride, pad = the flipped filter's), dst = dx (OC = C), ogh =
//   the stride; the dx pixels off the lattice are written as zeros.
// groups == 1, SC % 16 == 0, OC % (32*nb) == 0.
// ---------------------------------------------------------------------------
struct PatchArgs {
    const void *src;
    const void *filt;  // w [K][R][S][C]
    const void *bias;  // fprop: [K] or null
    void *dst;
    int N, H, W, SC;   // source tensor
    int OH, OW, OC;    // destination tensor
    int P, Q;          // output lattice extents
    int R, S;
    int gh, gw, pad_h, pad_w, sh1, sw1, dh1, dw1;
    int ogh, ogw, oh0, ow0;
    int TP, TQ, tiles_q, tiles_img;
    int PH, PW, PP, patch_slots;
    int relu;
    int nb, u, nsb, mb;  // output-channel blocks, super-step, ring depth, pixel blocks (2 or 4)
    FastDiv div_pp, div_pw, div_tq;
};
// u: 16-channel steps per super-step of the filter stream (1, 2 or 4;
// divides SC/16); nsb: filter ring stages per wave (fprop:
// patch_ring_stages(nb, u); dgrad: u = 1 and 4 or 8 stages)
int patch_ring_stages(int nb, int u);
int patch_lds_bytes();
hipError_t launch_patch(int dtype, const PatchArgs &a, bool dgrad, hipStream_t st);

// ---------------------------------------------------------------------------
// Stride-1 band kernel (band.hip): filter in registers, a ring of input rows
// in LDS.  src [N][H][W][CIN] -> dst [N][P][Q][ngemm] with
// P = H + 2*pad_h - dil*(R-1) (likewise Q); pad_h / pad_w may be negative.
// Without flip, bmat is the fprop filter [ngemm][R][S][CIN]; with flip it is
// the filter w[CIN][R][S][ngemm] of a dgrad, read with its taps reversed and
// its two channel axes swapped.
// ---------------------------------------------------------------------------
struct BandArgs {
    const void *src;
    const void *bmat;
    const void *bias;
    void *dst;
    int N, H, W, P, Q, ngemm;
    int pad_h, pad_w;
    int flip, relu;
    double requant_m;  // int8: output code = requant(acc + bias) with this multiplier
    int rows_per_wg, chunks_per_img;
};
bool band_supported(int dtype, int R, int S, int cin, int dil);
hipError_t launch_band(int dtype, int R, int S, int cin, int dil, const BandArgs &a, int grid_n, int grid_q,
                       hipStream_t st);

// ---------------------------------------------------------------------------
// Winograd F(2x2, 3x3) fprop (wino.hip): stride 1, 3x3, 64 input channels,
// src [N][H][W][64], filter w [ngemm][3][3][64], dst [N][P][Q][ngemm],
// ngemm % 16 == 0.  Batches of 32 tiles (2 output rows x 64 columns):
// tile_rows = ceil(P/2), tiles_q = ceil(Q/64), batches = N*tile_rows*tiles_q.
// ---------------------------------------------------------------------------
struct WinoArgs {
    const void *src;
    const void *w;  // filter [ngemm][3][3][64] (fprop) or [64][3][3][ngemm] (dgrad)
    void *u;        // dgrad: workspace for the transformed filter U[16][ngemm][64]; null for fprop
    const void *bias;
    void *dst;
    int N, H, W, P, Q, ngemm;
    int pad_h, pad_w;
    int relu;
    int tile_rows, tiles_q, batches;
};
bool wino_supported(int dtype, int R, int S, int cin, int dil);
hipError_t launch_wino_fprop(int dtype, const WinoArgs &a, int grid_x, hipStream_t st);


// 1x1 stride-1 convolution without padding as a streaming GEMM over the
// pixels (fprop; dgrad with the filter read transposed): src [npix][gk] ->
// dst [npix][nout].  fprop: w [nout][gk], bias [nout] or NULL; dgrad (trans):
// w [gk][nout], no bias.
struct PwArgs {
    const void *src;
    const void *w;
    const void *bias;
    void *dst;
    long long src_bytes, w_bytes;  // both under 2^31 (32-bit buffer offsets)
    int npix, gk, nout;
    int trans, relu;
};
bool pointwise_supported(int dtype, int gk, int nout);
int pointwise_nwg(int gk, int nout);  // output channels per workgroup, 0 if none fits
int pointwise_pixels_per_wg(int gk);
hipError_t launch_pointwise(int dtype, const PwArgs &a, hipStream_t st);

// pointwise_wgrad.hip: 1x1 stride-1 weight gradient, one workgroup per pixel
// slice holding the whole K x C tile; fp32 partial per slice ([K][C], then K
// dy column sums with_db), summed by the split-K reduce
struct PwWgradArgs {
    const void *x, *dy;
    void *out;
    uint32_t npix;
    int pix_per_split;  // a multiple of 64
    int splits;
    long long part_stride;
    int K, C;
    int with_db;
};
bool pointwise_wgrad_supported(int dtype, int K, int C);
hipError_t launch_pointwise_wgrad(int dtype, const PwWgradArgs &a, hipStream_t st);

// Re-lays the filter w[K][R][S][C/G] out as one [C][taps*K/G] matrix per
// dgrad stride phase, for the implicit GEMM on long GEMM-K rows (taps of the phase in (jr, js) order, the dx channel's
// group's dy channels innermost).
struct PrepPhase {
    int r0, rstep, ntr;
    int s0, sstep, nts;
    long long off;  // element offset in the output buffer
};
struct PrepArgs {
    const void *w;
    void *wt;
    int K, R, S, C;
    int Kg, Cg;     // per group (dense: K, C); dx channel c reads the Kg dy channels of its group
    int nphases;
    int max_elems;  // largest C*ntr*nts*K over phases
    PrepPhase ph[kMaxPhases];
};
hipError_t launch_dgrad_prep(int dtype, const PrepArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// wgrad implicit GEMM: D[k][col] = sum over output pixels of
//   dy[pix][k] * x[gather(pix, tap(col))][chan(col)],  col = (r, s, c).
// Pixels are cut into `splits` contiguous slices of pix_per_split pixels; each
// slice writes fp32 partials [splits][K][ncols] (or the final dw when
// splits == 1), reduced in slice order by launch_splitk_reduce.
// ---------------------------------------------------------------------------
struct WgradArgs {
    const void *x;
    const void *dy;
    void *out;
    int N, H, W, C, K, R, S, P, Q;
    int pad_h, pad_w, sh, sw, dh, dw;
    int ncols;            // R*S*C
    uint32_t npix;        // N*P*Q
    uint32_t pix_per_split;
    int splits;
    long long part_stride;  // elements between consecutive slices' partials
    FastDiv div_Q, div_PQ, div_C, div_S;
    int to_parts;           // fp32 partials even for one split
    int with_db;            // wgrad_kernel (tile 0): also dy's column sums at [K*ncols, +K) of each slice
    // groups: one GEMM per group, rows g*Kg + (0..Kg-1), columns (r, s, c')
    // over the group's Cg channels (ncols = R*S*Cg, div_C divides by Cg);
    // grid.x = groups * mtiles_g.  Dense: Kg = K, Cg = C.
    int Kg, Cg, mtiles_g;
};

int wgrad_num_tiles();
TileShape wgrad_tile_shape(int tile);
constexpr int kWgradPixStep = 64;  // pixels per main-loop step
constexpr int kWgradXcdTiles = 8;  // up to this many tiles per pixel slice, a slice's tiles share an XCD
hipError_t launch_wgrad(int dtype, int tile, const WgradArgs &a, hipStream_t st);
// Epilogue of the split-K sum t: out = alpha * t + beta * c (c laid out like
// out, NULL when beta == 0), stored as fp32 when out_f32, else rounded once.
struct ReduceEpi {
    float alpha, beta;
    const void *c;
    int out_f32;
    // elements [count1, count) go to out2[i - count1] with no alpha/beta/c
    // (the bias gradient reduced with the weight gradient); count1 % 4 == 0
    void *out2;
    long long count1;
};
hipError_t launch_splitk_reduce(int dtype, const float *parts, int splits, long long count,
                                long long stride, void *out, const ReduceEpi *epi, hipStream_t st);
// Elements between consecutive slices' partials: count rounded up to 4.
inline long long splitk_stride(long long count) { return (count + 3) / 4 * 4; }

// Column sums of a row-major [rows][K] fp16/bf16 matrix into fp32 partials,
// one per row slice: parts[z*part_stride + k] = sum over rows r of slice z of
// src[r][k], in a fixed order (wgrad.hip, colsum_kernel).  The bias gradient
// is this over dy viewed as [N*P*Q][K], then the split-K reduce.
struct ColsumArgs {
    const void *src;
    float *parts;
    uint32_t rows, rows_per_split;
    int K;
    int vec;                // K % 8 == 0: 16-byte row pieces (src 16-byte aligned)
    long long part_stride;
};
constexpr int kColsumVecsPerWg = 256;  // 8-column vectors per workgroup (grid.y = column blocks)
hipError_t launch_colsum(int dtype, const ColsumArgs &a, int splits, hipStream_t st);

// ---------------------------------------------------------------------------
// Stride-1 3x3 wgrad band kernel (wgrad_band.hip): dy and x pixels in LDS,
// transposing LDS reads.  nsplit workgroups per band of output rows, each
// with 1/nsplit of the R*S*C columns: nsplit = 2 (column halves), bands of
// rows_per_wg rows of one image, chunks_per_img per image; nsplit = 3 (one
// filter row each), nbands bands of the stacked rows of all images (row
// n*P + p), band b = rows [b*rows_total/nbands, (b+1)*rows_total/nbands).
// Band b's fp32 partial [K][R*S*C] goes to
// out + b * part_stride.
// ---------------------------------------------------------------------------
struct WgradBandArgs {
    const void *x;
    const void *dy;
    void *out;
    int N, H, W, P, Q;
    int pad_h, pad_w;
    int nsplit;
    int rows_per_wg, chunks_per_img;  // nsplit = 2
    int nbands, rows_total, band_f;   // nsplit = 3; band_f = (3 * nbands) / 24
    FastDiv div_p;                    // nsplit = 3: divides by P
    long long part_stride;
    int xw;              // padded row pitch Q + dil*(S-1)
    FastDiv div_xw;
    int xcd_pairs;        // bands a multiple of 8: the two column halves of a band share an XCD
    int with_db;          // also the band's dy column sums at [K*R*S*C, +K) of its slice
};
bool wgrad_band_supported(int R, int S, int C, int K, int dil, int Q);
hipError_t launch_wgrad_band(int dtype, const WgradBandArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// Few-channel fprop (fewchan.hip): groups == 1, C not a multiple of 8,
// stride_w*C even, dil_w == 1, K = 32 or 64, fp16/bf16.  Each filter row's
// S*C taps are read as a window of lw elements (a multiple of 8) starting
// delta elements before them.  A workgroup computes rows_per_wg output rows
// of one image from nrows padded input rows in LDS (pitch bytes each, cpr
// 16-byte chunks, the image row's first element at element `left`).
// ---------------------------------------------------------------------------
// Per reduction step j and lane half h (chunk c = 2*j + h, t0 = 8*c in filter
// row r = t0 / Lw at window position kk0 = t0 % Lw): the filter element
// offset within an output channel's R*S*C (r*S*C + kk0 - delta), the masks of
// the chunk's valid 16-bit halves (kk0 + i - delta in [0, S*C), r < R), and
// the chunk's byte offset from a pixel's window start in LDS (r*dh rows down,
// kk0 elements on).  Chunks past the filter: mask 0, offsets 0.
constexpr int kFewMaxSteps = 16;
struct FewStep {
    int fbase[2];
    uint32_t mask[2][4];
    uint32_t coff[2];
};
struct FewArgs {
    const void *x, *w, *bias;
    void *y;
    int N, H, WC, P, Q, K, R, SC;
    int pad_h, sh, dh;
    int relu;
    int rows_per_wg, bands;   // output rows per workgroup, workgroups per image
    int nrows, pitch, cpr, left;
    int delta, lw;
    int win0, qstep;          // window start of pixel q: element win0 + q*qstep of its row
    int buf_bytes, stage_bytes;
    uint32_t x_bytes;
    FastDiv div_cpr, div_q;
    FewStep step[kFewMaxSteps];
};
bool fewchan_supported(int dtype, int C, int K, int S, int sw, int dw, int W);
int fewchan_steps(int R, int lw);  // reduction steps of the kernel built for R*lw, 0 if none
hipError_t launch_fewchan_fprop(int dtype, const FewArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// Few-channel wgrad (fewchan_wgrad.hip): groups == 1, C not a multiple of 8,
// stride_w*C even, dil_w == 1, W*C % 8 == 0, K == 64, fp16/bf16.  Column t of
// the window layout is window position t % lw of filter row t / lw, i.e. tap
// s*C + c = t % lw - delta.  A workgroup owns rows_per_wg output rows of one
// image, taken grw at a time; buffer g & 1 (buf_bytes) holds a group's dy
// rows (dq pixel slots each, 128 bytes a pixel), its nxr input rows at xa_off
// (pitch bytes each, image element 0 at element `left`) and, when odd_shift,
// the same rows shifted by 4 bytes at xb_off.  Each workgroup writes the fp32
// partial [K][R*S*C] of its band at out + blockIdx.x * part_stride.
// ---------------------------------------------------------------------------
struct FewWgradArgs {
    const void *x, *dy;
    void *out;
    int N, H, WC, P, Q, R, SC;
    int pad_h, sh, dh;
    int rows_per_wg, bands, grw;
    int spc, dq;              // steps per class and row, dy pixel slots per row (32 * spc)
    int lw, delta, win0, qstep;
    int nxr, pitch, cpr, left;
    int odd_shift;            // the odd pixels' windows are read from the shifted copy
    int nblk_dy, nblk_x;      // 1 KB loads per group
    int xa_off, xb_off, buf_bytes, xcopy_chunks;
    int ncb, ncba;            // column blocks, and those of the first set
    uint32_t x_bytes, dy_bytes;
    long long part_stride;
    FastDiv div_cpr;
};
bool fewchan_wgrad_supported(int dtype, int C, int K, int S, int sw, int dw, int W);
int fewchan_wgrad_lds_bytes();
hipError_t launch_fewchan_wgrad(int dtype, const FewWgradArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// Few-channel dgrad (fewchan_dgrad.hip): groups == 1, C <= 4 (not a multiple
// of 8), stride 2, dilation 1, K == 64, W*C % 8 == 0, fp16/bf16.  Super-pixel
// (i, j) = the 2x2 output pixels (2i + a, 2j + b); it reads dy pixels
// (i + dp, j + dq) for dp in [dp_min, dp_min + ndh), dq likewise (ndh and
// ndw in 2..4).  A workgroup owns rows_per_wg super-rows of one image (HS = ceil(H/2)
// of them, WS = ceil(W/2) super-pixels each, nblk_r blocks of 16); its dy rows
// sit in a ring of nslot rows of rsl pixel slots (rowb bytes).
// ---------------------------------------------------------------------------
struct FewDgradArgs {
    const void *dy, *w;
    void *dx;
    int N, H, W, C, P, Q, R, S;
    int pad_h, pad_w;
    int HS, WS, rows_per_wg, bands, nblk_r;
    int dp_min, ndh, dq_min, ndw;
    int rsl, rowb, nslot, ring_bytes, filt_bytes, stage_wave;
    uint32_t dy_bytes;
};
bool fewchan_dgrad_supported(int dtype, int C, int K, int sh, int sw, int dh, int dw, int W);
int fewchan_dgrad_lds_bytes();
int fewchan_dgrad_max_offsets();
hipError_t launch_fewchan_dgrad(int dtype, const FewDgradArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// Direct convolution for groups > 1: one thread per output element, fp32
// (int32 for int8) accumulation in a fixed (r, s, channel) order.
// ---------------------------------------------------------------------------
struct DirectArgs {
    const void *a;     // fprop: x   dgrad: dy   wgrad: x
    const void *b;     // fprop: w   dgrad: w    wgrad: dy
    const void *bias;
    void *out;         // y / dx / (dw or fp32 partials)
    int N, H, W, C, K, R, S, P, Q;
    int pad_h, pad_w, sh, sw, dh, dw, G, Cg, Kg;
    int relu;
    double requant_m;
    int splits;
    long long part_stride;  // wgrad: elements between slices' partials
    uint32_t npix;          // wgrad: N*P*Q (depthwise: work units, direct_depthwise_wgrad_cols)
    uint32_t pix_per_split; // wgrad: pixels (depthwise: work units) per slice
    long long total;        // output elements (per split for wgrad)
    int tiled;              // use the LDS-tiled kernel (direct_tiled_rows / direct_wgrad_tiled_ok)
    int rows;               // fprop / dgrad tiled: output rows per workgroup
    // fprop / dgrad: out = alpha * conv + beta * cmat (+ bias), cmat laid out
    // like out, when axpby; wgrad: fp32 partials even for one split when to_parts
    int axpby;
    float alpha, beta;
    const void *cmat;
    int to_parts;
    int depthwise;          // groups = C = K: the depthwise kernels (direct_depthwise_ok)
    FastDiv div_q, div_p;   // depthwise wgrad: work units per output row, and P
};
// Output rows per workgroup of the LDS-tiled direct fprop (op 0) / dgrad
// (op 1) kernel for 16-bit types, or 0 if it does not apply.
int direct_tiled_rows(int op, int dtype, int R, int S, int W, int Q, int Cg, int Kg);
bool direct_wgrad_tiled_ok(int dtype, int Cg, int Kg);
bool direct_depthwise_ok(int dtype, int C, int Cg, int Kg, int R, int S);
// Output columns per work unit of the depthwise wgrad kernel (1: one pixel).
int direct_depthwise_wgrad_cols(int N, int H, int W, int C, int P, int Q, int R, int S, int sw, int dw);
long long direct_wgrad_tiled_wgs(int R, int S, int Cg, int Kg, int G);  // workgroups per pixel slice
hipError_t launch_direct_fprop(int dtype, const DirectArgs &a, hipStream_t st);
hipError_t launch_direct_dgrad(int dtype, const DirectArgs &a, hipStream_t st);
hipError_t launch_direct_wgrad(int dtype, const DirectArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// Row re-layout (repack.hip): dst[r][c] = (r < src_rows && c < src_cols) ?
// src[r][c] : 0 for r < dst_rows, c < dst_cols; rows are src_ld / dst_ld
// elements apart.  Element size 1, 2 or 4 bytes.
struct RepackArgs {
    const void *src;
    void *dst;
    long long src_rows, dst_rows;
    int src_cols, src_ld, dst_cols, dst_ld;
};
hipError_t launch_repack(int esz, const RepackArgs &a, hipStream_t st);

}  // namespace cnv

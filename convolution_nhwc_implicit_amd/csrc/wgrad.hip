// wgrad.hip -- weight-gradient implicit GEMM for gfx950, the fixed-order
// split-K reduction, and column sums (bias gradient).
//
// dw[k][r][s][c] = sum over output pixels (n,p,q) of
//                  dy[n,p,q,k] * x[n, p*sh-ph+r*dh, q*sw-pw+s*dw, c].
// As a GEMM: rows k, columns (r,s,c), reduction over the N*P*Q pixels -- the
// very long GEMM-K the TVM CUTLASS wgrad pull request names as the reason
// split-K is needed.  The reduction over pixels is cut into contiguous slices;
// each slice writes fp32 partials and a second kernel sums them in slice
// order (the CUTLASS notebook's "parallel" split-K, with a fixed order instead
// of atomics, so results are identical run to run).  Accumulation is fp32
// throughout, as the TVM pull request requires for wgrad.
//
// A workgroup computes a 128 x 128 tile (dy channels x columns) over its
// slice, 32 pixels per stage.  Both operands arrive pixel-major (NHWC) by
// direct-to-LDS loads, one 256-byte LDS row per pixel: dy rows are 128
// consecutive channels, x rows are gathered 16-byte pieces (8 channels of one
// tap each; C % 8 == 0).  The MFMA wants 8 consecutive pixels of one channel
// per lane, which the transposing LDS read ds_read_b64_tr_b16 delivers from
// the pixel-major rows, so no registers or VALU work go into re-laying the
// operands out.  16-byte chunk c of row r is stored at chunk c ^ 2*(r % 4):
// the 4 rows of a transposing read then fall on different banks.  Three
// stages in flight (two loading while one is computed), four waves in a 2 x 2
// arrangement of 64 x 64 wave tiles (2 x 2 blocks of 32x32x16 MFMA).
#include "device_common.h"

namespace cnv {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 (the fragment reads of wgrad_kernel)
__device__ inline s16x4 tr16(const unsigned char *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
// Workgroup -> (row tile gx = group * mtiles_g + row tile, column tile nt,
// pixel slice z) of the generic wgrad kernels.  With few tiles per slice
// (T = gxn * gyn <= kWgradXcdTiles) the tiles of a slice, which read the
// same dy and x pixels, share an XCD's L2: the grid is one-dimensional,
// workgroups are dealt to the 8 XCDs in turn, and workgroup 8q + u takes
// tile q % T of slice u + 8 * (q / T) (slices past the last -- the grid is
// rounded up to 8 of them -- have no work).  Otherwise the grid is
// (gxn, gyn, slices).
struct WgradTileId {
    int gx, nt, z;
};
__device__ inline WgradTileId wgrad_tile_id(int gxn, int gyn)
{
    const int T = gxn * gyn;
    if (T > kWgradXcdTiles) return WgradTileId{(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
    const int L = blockIdx.x, u = L & 7, q = L >> 3, qt = q / T;
    const int t = q - qt * T, nt = t / gxn;
    return WgradTileId{t - nt * gxn, nt, u + 8 * qt};
}
inline dim3 wgrad_grid(int gxn, int gyn, int splits)
{
    if (gxn * gyn > kWgradXcdTiles) return dim3((unsigned)gxn, (unsigned)gyn, (unsigned)splits);
    return dim3((unsigned)(gxn * gyn * ((splits + 7) / 8 * 8)));
}

template <class E>
struct Mfma32x16 {
    __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c)
    {
        if constexpr (E::kDtype == CONV2D_DTYPE_F16)
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                           c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <class E>
__global__ __launch_bounds__(256) void wgrad_kernel(const WgradArgs a)
{
    constexpr int BM = 128, BN = 128, SP = 32, NSTAGE = 3;
    constexpr int ROWB = 256;
    constexpr int TILE = SP * ROWB;      // 8 KB: 8 direct-to-LDS blocks of 4 rows
    constexpr int STAGE = 2 * TILE;      // dy tile, then x tile
    constexpr int PER = 4;               // direct-to-LDS loads per wave and stage
    using elem = typename E::elem;
    static_assert(SP * 2 == kWgradPixStep, "slices are whole pairs of stages");

    __shared__ __attribute__((aligned(16))) unsigned char smem[NSTAGE * STAGE];

    const WgradTileId id = wgrad_tile_id(a.K / a.Kg * a.mtiles_g, (a.ncols + BN - 1) / BN);
    if (id.z >= a.splits) return;  // the whole workgroup
    const int nt = id.nt, z = id.z;
    const int gi = id.gx / a.mtiles_g, mt = id.gx - gi * a.mtiles_g;  // group, row tile in it
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    const uint32_t pbeg = (uint32_t)z * a.pix_per_split;
    uint32_t pend = pbeg + a.pix_per_split;
    if (pend > a.npix || pend < pbeg) pend = a.npix;
    const int KT = pend > pbeg ? (int)((pend - pbeg + SP - 1) / SP) : 0;

    // ---- direct-to-LDS loads.  Wave w fills blocks w and w + 4 of each tile;
    // lane i fills row 4*blk + i/16, stored chunk i%16, i.e. logical chunk lc.
    const int lc = (lane & 15) ^ (2 * ((lane >> 4) & 3));
    const uint32_t lds0 = lds_addr(smem);
    const u32x4 dy_rs = make_buf_rsrc(a.dy, (uint32_t)((size_t)a.npix * a.K * sizeof(elem)));
    const u32x4 x_rs = make_buf_rsrc(a.x, (uint32_t)((size_t)a.N * a.H * a.W * a.C * sizeof(elem)));
    // dy: channel k of this lane's chunk (whole chunk valid or not, Kg % 8 == 0)
    const int kl = mt * BM + 8 * lc;  // within the group
    const bool kval = kl < a.Kg;
    const int k = gi * a.Kg + kl;
    // x: column (tap, channel of the group) of this lane's chunk
    const int col = nt * BN + 8 * lc;
    const bool cval = col < a.ncols;
    const uint32_t tap = fdiv((uint32_t)(cval ? col : 0), a.div_C);
    const int cch = gi * a.Cg + (cval ? col : 0) - (int)tap * a.Cg;
    const uint32_t tr = fdiv(tap, a.div_S);
    const int hoff = (int)tr * a.dh - a.pad_h;
    const int woff = ((int)tap - (int)tr * a.S) * a.dw - a.pad_w;
    // the lane's pixel in each of its two blocks: pixel index and (n, p, q),
    // advanced by SP per stage in mixed radix (Q, P)
    const uint32_t PQ = (uint32_t)a.P * (uint32_t)a.Q;
    const uint32_t dn = SP / PQ, dp = (SP / (uint32_t)a.Q) % (uint32_t)a.P, dq = SP % (uint32_t)a.Q;
    uint32_t pix[2], pn[2], pp[2], pq[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        pix[t] = pbeg + 4 * (wave + 4 * t) + (lane >> 4);
        const uint32_t v = pix[t] < a.npix ? pix[t] : 0;
        pn[t] = fdiv(v, a.div_PQ);
        const uint32_t rem = v - pn[t] * PQ;
        pp[t] = fdiv(rem, a.div_Q);
        pq[t] = rem - pp[t] * (uint32_t)a.Q;
    }
    auto dma_stage = [&](int kt) {
        const uint32_t base = lds0 + (uint32_t)((kt % NSTAGE) * STAGE);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bool ok = pix[t] < pend;
            const uint32_t blk = (uint32_t)(wave + 4 * t) * 1024;
            dma16(dy_rs, base + blk,
                  (ok && kval) ? (uint32_t)(((size_t)pix[t] * a.K + k) * sizeof(elem)) : kBufOOBFar);
            const int h = (int)pp[t] * a.sh + hoff, w = (int)pq[t] * a.sw + woff;
            const bool okx = ok && cval && (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W;
            dma16(x_rs, base + TILE + blk,
                  okx ? (uint32_t)(((((size_t)pn[t] * a.H + h) * a.W + w) * a.C + cch) * sizeof(elem)) : kBufOOBFar);
            // the lane's pixel of the next stage
            pix[t] += SP;
            pq[t] += dq;
            const uint32_t c1 = pq[t] >= (uint32_t)a.Q;
            if (c1) pq[t] -= a.Q;
            pp[t] += dp + c1;
            const uint32_t c2 = pp[t] >= (uint32_t)a.P;
            if (c2) pp[t] -= a.P;
            pn[t] += dn + c2;
        }
    };

    // ---- fragments by transposing reads: lane l gets column l%32 of a 32-wide
    // block (dy channel or x column) for pixels 8*(l/32) + 0..7 of a 16-pixel
    // k-step; in each 16-lane group lane L addresses row L/4, columns
    // 4*(L%4)..+3 of a 4 x 16 piece.
    const int fcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // column offset in a 32-wide block
    const int frow = 8 * (lane >> 5) + ((lane & 15) >> 2);      // pixel row in a k-step (+4: second read)
    auto frag = [&](const unsigned char *tile, int colb, int ks) -> u32x4 {
        const int c = colb + fcol;  // first of this lane's 4 columns
        const int r0 = 16 * ks + frow, r1 = r0 + 4;
        const int ch = c >> 3, cb = (c & 7) * 2;
        const uint2 lo = __builtin_bit_cast(uint2, tr16(tile + r0 * ROWB + ((ch ^ (2 * (r0 & 3))) << 4) + cb));
        const uint2 hi = __builtin_bit_cast(uint2, tr16(tile + r1 * ROWB + ((ch ^ (2 * (r1 & 3))) << 4) + cb));
        return u32x4{lo.x, lo.y, hi.x, hi.y};
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    // bias gradient (with_db): the waves of the first column tile's left
    // half add up the dy values their fragments hold (every dy element of
    // the slice once); lane holds channel wm*64 + 32*i + l%32
    const bool dbw = a.with_db && nt == 0 && wn == 0;  // wave-uniform
    const bool idle = mt * BM + wm * 64 >= a.Kg;        // wave-uniform
    float dbacc[2] = {0.0f, 0.0f};

#pragma unroll
    for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
        if (s0 < KT) dma_stage(s0);
    // The main loop; a wave whose 64 rows all lie past the group's K (the
    // last row tile of K = 192, say) runs it without the MFMA work, only
    // loading and meeting the barriers, and leaves its SIMD to the other
    // workgroups' waves.  (Two copies of the loop: a branch inside it around
    // the MFMAs costs registers.)
    auto main_loop = [&](auto compute_c) __attribute__((always_inline)) {
        for (int kt = 0; kt < KT; ++kt) {
            // stage kt has landed when at most the younger stage's loads remain
            if (kt + 1 < KT)
                wait_vm_n<PER * (NSTAGE - 2)>();
            else
                wait_vm_n<0>();
            __syncthreads();  // every wave's loads of stage kt are visible; stage kt-1 is consumed
            if (kt + NSTAGE - 1 < KT) dma_stage(kt + NSTAGE - 1);
            if constexpr (decltype(compute_c)::value) {
                const unsigned char *ta = smem + (kt % NSTAGE) * STAGE;
                const unsigned char *tb = ta + TILE;
#pragma unroll
                for (int ks = 0; ks < SP / 16; ++ks) {
                    u32x4 fa[2], fb[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i) fa[i] = frag(ta, wm * 64 + 32 * i, ks);
#pragma unroll
                    for (int j = 0; j < 2; ++j) fb[j] = frag(tb, wn * 64 + 32 * j, ks);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j) acc[i][j] = Mfma32x16<E>::run(fa[i], fb[j], acc[i][j]);
                    if (dbw) {
#pragma unroll
                        for (int i = 0; i < 2; ++i)
#pragma unroll
                            for (int q = 0; q < 4; ++q) dbacc[i] = DotOne<E>::add(fa[i][q], dbacc[i]);
                    }
                }
            }
        }
    };
    if (idle)
        main_loop(std::integral_constant<bool, false>{});
    else
        main_loop(std::integral_constant<bool, true>{});
    if (dbw) {
        // lanes l and l + 32 hold the two pixel halves of a channel
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float v = dbacc[i] + __shfl_xor(dbacc[i], 32);
            const int kl2 = mt * BM + wm * 64 + 32 * i + lane;
            if (lane < 32 && kl2 < a.Kg)
                ((float *)a.out)[(size_t)z * a.part_stride + (size_t)a.K * a.ncols + gi * a.Kg + kl2] = v;
        }
    }

    // result block layout: lane holds column l%32, rows 8*(e/4) + 4*(l/32) + e%4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = nt * BN + wn * 64 + 32 * j + (lane & 31);
            if (c >= a.ncols) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int kl2 = mt * BM + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (kl2 >= a.Kg) continue;
                const int kk = gi * a.Kg + kl2;
                if (a.splits == 1 && !a.to_parts)
                    ((elem *)a.out)[(size_t)kk * a.ncols + c] = E::from_f32(acc[i][j][e]);
                else
                    ((float *)a.out)[(size_t)z * a.part_stride + (size_t)kk * a.ncols + c] = acc[i][j][e];
            }
        }
}

// Small problems: 64 x 64 tiles, 64 pixels per step.  Each thread loads two
// neighbouring pixels' 8-channel chunks of dy and x into registers and
// interleaves them into channel-major LDS rows (pixels innermost), which the
// 16x16x32 MFMA reads directly.  More tiles per problem than the 128 x 128
// kernel, so fewer slices (and fewer partials) fill the chip.
template <class E, int BM, int BN>
__global__ __launch_bounds__(256) void wgrad_interleave_kernel(const WgradArgs a)
{
    constexpr int NT = 256;
    constexpr int BKP = kWgradPixStep;  // pixels per step
    constexpr int ROWB = BKP * 2 + 16;  // LDS row: 64 pixels of 2 bytes + pad
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int PAIRS = BKP / 2;      // 32 pixel pairs per step
    constexpr int ACH = BM / 8, BCH = BN / 8;  // 8-wide channel chunks per step
    static_assert(PAIRS * ACH == NT && PAIRS * BCH == NT, "one A and one B chunk pair per thread");
    constexpr int WTM = BM / 2, WTN = BN / 2;  // 2x2 waves
    constexpr int FM = WTM / 16, FN = WTN / 16;
    using elem = typename E::elem;

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

    const WgradTileId id = wgrad_tile_id(a.K / a.Kg * a.mtiles_g, (a.ncols + BN - 1) / BN);
    if (id.z >= a.splits) return;  // the whole workgroup
    const int nt = id.nt, z = id.z;
    const int gi = id.gx / a.mtiles_g, mt = id.gx - gi * a.mtiles_g;  // group, row tile in it
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int pp = tid % PAIRS, ch = tid / PAIRS;

    // this thread's dy chunk: channels k0..k0+7 (of the group's Kg)
    const int k0 = gi * a.Kg + mt * BM + ch * 8;
    const bool kval = mt * BM + ch * 8 < a.Kg;
    // this thread's x chunk: columns col0..col0+7, all in one tap (Cg % 8 == 0)
    const int col0 = nt * BN + ch * 8;
    const bool cval = col0 < a.ncols;
    const uint32_t tap = fdiv((uint32_t)(cval ? col0 : 0), a.div_C);
    const int cch = gi * a.Cg + (cval ? col0 : 0) - (int)tap * a.Cg;
    const uint32_t tr = fdiv(tap, a.div_S);
    const int ts = (int)tap - (int)tr * a.S;
    const int hoff = (int)tr * a.dh - a.pad_h;
    const int woff = ts * a.dw - a.pad_w;

    const uint32_t pbeg = (uint32_t)z * a.pix_per_split;
    uint32_t pend = pbeg + a.pix_per_split;
    if (pend > a.npix || pend < pbeg) pend = a.npix;
    const int KT = pend > pbeg ? (int)((pend - pbeg + BKP - 1) / BKP) : 0;

    const elem *dy = (const elem *)a.dy;
    const elem *x = (const elem *)a.x;
    const uint32_t PQ = (uint32_t)a.P * (uint32_t)a.Q;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 rdy[2], rx[2];

    auto gload = [&](int kt) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint32_t pix = pbeg + (uint32_t)kt * BKP + 2 * pp + e;
            const bool ok = pix < pend;
            rdy[e] = (ok && kval) ? *(const u32x4 *)(dy + (size_t)pix * a.K + k0) : zero;
            bool okx = ok && cval;
            const uint32_t n = fdiv(ok ? pix : 0, a.div_PQ);
            const uint32_t rem = (ok ? pix : 0) - n * PQ;
            const uint32_t p = fdiv(rem, a.div_Q);
            const uint32_t q = rem - p * a.Q;
            const int h = (int)p * a.sh + hoff;
            const int w = (int)q * a.sw + woff;
            okx = okx && (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W;
            rx[e] = okx ? *(const u32x4 *)(x + (((size_t)n * a.H + h) * a.W + w) * a.C + cch) : zero;
        }
    };
    // interleave the two pixels: LDS row = channel, 32-bit word = (pixel 2pp, pixel 2pp+1)
    auto sstore = [&](int stage) {
        unsigned char *base = smem + stage * STAGE;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a0 = rdy[0][j], a1 = rdy[1][j];
            *(uint32_t *)(base + (ch * 8 + 2 * j) * ROWB + pp * 4) = (a0 & 0xFFFFu) | (a1 << 16);
            *(uint32_t *)(base + (ch * 8 + 2 * j + 1) * ROWB + pp * 4) = (a0 >> 16) | (a1 & 0xFFFF0000u);
            const uint32_t b0 = rx[0][j], b1 = rx[1][j];
            *(uint32_t *)(base + (BM + ch * 8 + 2 * j) * ROWB + pp * 4) = (b0 & 0xFFFFu) | (b1 << 16);
            *(uint32_t *)(base + (BM + ch * 8 + 2 * j + 1) * ROWB + pp * 4) = (b0 >> 16) | (b1 & 0xFFFF0000u);
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int frag_row = lane & 15, frag_k = (lane >> 4) * 16;
    if (KT > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < KT) gload(kt + 1);
            const unsigned char *base = smem + cur * STAGE;
#pragma unroll
            for (int ks = 0; ks < BKP * 2 / 64; ++ks) {
                u32x4 fa[FM], fb[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    fa[i] = *(const u32x4 *)(base + (wm * WTM + i * 16 + frag_row) * ROWB + ks * 64 + frag_k);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    fb[j] = *(const u32x4 *)(base + (BM + wn * WTN + j * 16 + frag_row) * ROWB + ks * 64 + frag_k);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = E::mfma(fa[i], fb[j], acc[i][j]);
            }
            if (kt + 1 < KT) sstore(cur ^ 1);
            __syncthreads();
        }
    }

    // result block layout: lane holds column (lane & 15), rows 4*(lane >> 4) + r
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = nt * BN + wn * WTN + j * 16 + (lane & 15);
            if (col >= a.ncols) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kl = mt * BM + wm * WTM + i * 16 + (lane >> 4) * 4 + r;
                if (kl >= a.Kg) continue;
                const int k = gi * a.Kg + kl;
                if (a.splits == 1 && !a.to_parts)
                    ((elem *)a.out)[(size_t)k * a.ncols + col] = E::from_f32(acc[i][j][r]);
                else
                    ((float *)a.out)[(size_t)z * a.part_stride + (size_t)k * a.ncols + col] = acc[i][j][r];
            }
        }
}

// tile 0: the transposing-read kernel (128 x 128), tile 1: the interleaving
// kernel (64 x 64)
int wgrad_num_tiles() { return 2; }
TileShape wgrad_tile_shape(int tile)
{
    return tile == 0 ? TileShape{128, 128} : TileShape{64, 64};
}

hipError_t launch_wgrad(int dtype, int tile, const WgradArgs &a, hipStream_t st)
{
    if (tile < 0 || tile >= wgrad_num_tiles()) return hipErrorInvalidValue;
    const TileShape ts = wgrad_tile_shape(tile);
    if (a.mtiles_g != (a.Kg + ts.bm - 1) / ts.bm || a.K % a.Kg) return hipErrorInvalidValue;
    const dim3 grid(wgrad_grid(a.K / a.Kg * a.mtiles_g, (a.ncols + ts.bn - 1) / ts.bn, a.splits));
    switch (dtype) {
    case CONV2D_DTYPE_F16:
        if (tile == 0)
            wgrad_kernel<EF16><<<grid, 256, 0, st>>>(a);
        else
            wgrad_interleave_kernel<EF16, 64, 64><<<grid, 256, 0, st>>>(a);
        break;
    case CONV2D_DTYPE_BF16:
        if (tile == 0)
            wgrad_kernel<EBF16><<<grid, 256, 0, st>>>(a);
        else
            wgrad_interleave_kernel<EBF16, 64, 64><<<grid, 256, 0, st>>>(a);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// out[i] = round(sum over slices z of parts[z*stride + i]) in fp32, in a fixed
// order: the slices are split into NCLS classes z % NCLS; each class is summed
// in ascending z, then the class sums are added in ascending class order.
// A workgroup owns 4*256/NCLS consecutive elements: thread (class c, lane e)
// reads elements 4e..4e+3 of every slice of class c with 128-bit loads, and
// the class sums meet in LDS.  NCLS is 16 (256 contiguous bytes of a slice
// per class) unless there are few elements and many slices, where 64 classes
// keep more loads in flight; the choice depends only on count and splits.
// stride is a multiple of 4 and at least count; the last workgroup's lanes
// past count read inside the slice padding and store nothing.
// ---------------------------------------------------------------------------
template <class E, int NCLS>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *parts, int splits, long long count,
                                                            long long stride, void *out_, const ReduceEpi epi)
{
    using elem = typename E::elem;
    constexpr int NL = 256 / NCLS;  // lanes per class
    __shared__ f32x4 part[NCLS][NL];
    const int cls = threadIdx.x / NL, e = threadIdx.x % NL;
    const long long i = (long long)blockIdx.x * (4 * NL) + e * 4;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if (i < stride) {
        const float *p = parts + i;
        // eight slices of the class in flight; past the last slice a load
        // gives +0, which leaves the sum unchanged
        for (int z = cls; z < splits; z += 8 * NCLS) {
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = z + u * NCLS < splits ? *(const f32x4 *)(p + (size_t)(z + u * NCLS) * stride)
                                             : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                s[0] += v[u][0];
                s[1] += v[u][1];
                s[2] += v[u][2];
                s[3] += v[u][3];
            }
        }
    }
    part[cls][e] = s;
    __syncthreads();
    if (cls == 0 && i < count) {
        f32x4 t = part[0][e];
        for (int c = 1; c < NCLS; ++c) {
            const f32x4 v = part[c][e];
            t[0] += v[0];
            t[1] += v[1];
            t[2] += v[2];
            t[3] += v[3];
        }
        // [0, count1) (all of it without out2) -> out with the linear
        // combination; [count1, count) -> out2 as is
        const bool second = epi.out2 && i >= epi.count1;
        const long long base = second ? epi.count1 : 0;
        const long long end = (epi.out2 && !second) ? epi.count1 : count;
        if (!second && (epi.alpha != 1.0f || epi.beta != 0.0f)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float c = 0.0f;
                if (epi.c && i + j < end)
                    c = epi.out_f32 ? ((const float *)epi.c)[i + j] : E::to_f32(((const elem *)epi.c)[i + j]);
                t[j] = epi.alpha * t[j] + epi.beta * c;
            }
        }
        const long long o0 = i - base, n = end - base;  // o0 % 4 == 0
        if (epi.out_f32) {
            float *out = (float *)(second ? epi.out2 : out_);
            if (o0 + 4 <= n) {
                *(f32x4 *)(out + o0) = t;
            } else {
                for (int j = 0; j < 4 && o0 + j < n; ++j) out[o0 + j] = t[j];
            }
        } else {
            elem *out = (elem *)(second ? epi.out2 : out_);
            elem o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = E::from_f32(t[j]);
            if (o0 + 4 <= n) {
                *(uint2 *)(out + o0) = *(const uint2 *)o;
            } else {
                for (int j = 0; j < 4 && o0 + j < n; ++j) out[o0 + j] = o[j];
            }
        }
    }
}

hipError_t launch_splitk_reduce(int dtype, const float *parts, int splits, long long count,
                                long long stride, void *out, const ReduceEpi *epi, hipStream_t st)
{
    if (stride % 4 || stride < count) return hipErrorInvalidValue;
    if (count == 0) return hipSuccess;
    const ReduceEpi e = epi ? *epi : ReduceEpi{1.0f, 0.0f, nullptr, 0, nullptr, 0};
    if (e.out2 && (e.count1 % 4 || e.count1 <= 0 || e.count1 >= count)) return hipErrorInvalidValue;
    const bool wide = (count + 63) / 64 < 256 && splits >= 128;  // fewer workgroups than CUs
    const unsigned blocks = (unsigned)(wide ? (count + 15) / 16 : (count + 63) / 64);
    switch (dtype) {
    case CONV2D_DTYPE_F16:
        if (wide)
            splitk_reduce_kernel<EF16, 64><<<blocks, 256, 0, st>>>(parts, splits, count, stride, out, e);
        else
            splitk_reduce_kernel<EF16, 16><<<blocks, 256, 0, st>>>(parts, splits, count, stride, out, e);
        break;
    case CONV2D_DTYPE_BF16:
        if (wide)
            splitk_reduce_kernel<EBF16, 64><<<blocks, 256, 0, st>>>(parts, splits, count, stride, out, e);
        else
            splitk_reduce_kernel<EBF16, 16><<<blocks, 256, 0, st>>>(parts, splits, count, stride, out, e);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Column sums (bias gradient).  Workgroup (z, y) takes rows [z*rows_per_split,
// ...) and the 8-column vectors [256*y, 256*y + ncv).  Thread (row lane rl,
// vector cv) adds rows rl, rl + nrl, ... of the slice in ascending order in
// fp32; the nrl lane sums of a column are then added in lane order through
// LDS, and the workgroup writes one fp32 partial per column.  A wave reads
// whole consecutive rows, 16 bytes a lane (K % 8 == 0), else element by
// element.
// ---------------------------------------------------------------------------
template <class E, bool VEC>
__global__ __launch_bounds__(256) void colsum_kernel(const ColsumArgs a)
{
    using elem = typename E::elem;
    __shared__ float red[256][8];
    const int K8 = (a.K + 7) / 8, cb = blockIdx.y * kColsumVecsPerWg;
    const int ncv = min(K8 - cb, kColsumVecsPerWg), nrl = 256 / ncv;
    const int tid = threadIdx.x, cv = tid % ncv, rl = tid / ncv;
    const int k0 = (cb + cv) * 8;
    const uint32_t r0 = blockIdx.x * a.rows_per_split;
    uint32_t r1 = r0 + a.rows_per_split;
    if (r1 > a.rows || r1 < r0) r1 = a.rows;
    float s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = 0.0f;
    if (rl < nrl) {
        const elem *src = (const elem *)a.src + k0;
        uint32_t r = r0 + rl;
        if (VEC) {
            // eight rows in flight per step (rows past the slice read as
            // zeros, which leave the sums unchanged); each added in order
            for (; r < r1; r += 8 * (uint32_t)nrl) {
                u32x4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    v[u] = r + u * nrl < r1 ? *(const u32x4 *)(src + (size_t)(r + u * nrl) * a.K)
                                            : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int j = 0; j < 8; ++j) s[j] += E::to_f32((elem)(w[j >> 1] >> (16 * (j & 1))));
                }
            }
        } else {
            for (; r < r1; r += nrl) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (k0 + j < a.K) s[j] += E::to_f32(src[(size_t)r * a.K + j]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) red[tid][j] = s[j];
    __syncthreads();
    float *part = a.parts + (size_t)blockIdx.x * a.part_stride;
    for (int o = tid; o < ncv * 8; o += 256) {
        const int oc = o >> 3, j = o & 7, k = (cb + oc) * 8 + j;
        float sum = 0.0f;
        for (int l = 0; l < nrl; ++l) sum += red[l * ncv + oc][j];
        if (k < a.K) part[k] = sum;
    }
}

hipError_t launch_colsum(int dtype, const ColsumArgs &a, int splits, hipStream_t st)
{
    if (a.K < 1 || splits < 1 || (a.vec && a.K % 8)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)splits, (unsigned)(((a.K + 7) / 8 + kColsumVecsPerWg - 1) / kColsumVecsPerWg));
    switch (dtype) {
    case CONV2D_DTYPE_F16:
        if (a.vec)
            colsum_kernel<EF16, true><<<grid, 256, 0, st>>>(a);
        else
            colsum_kernel<EF16, false><<<grid, 256, 0, st>>>(a);
        break;
    case CONV2D_DTYPE_BF16:
        if (a.vec)
            colsum_kernel<EBF16, true><<<grid, 256, 0, st>>>(a);
        else
            colsum_kernel<EBF16, false><<<grid, 256, 0, st>>>(a);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cnv

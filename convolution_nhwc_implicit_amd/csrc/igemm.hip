// igemm.hip -- implicit-GEMM convolution kernel for gfx950 (fprop, and dgrad
// one stride phase per grid z-slice).
//
// The convolution is a GEMM whose A operand is gathered on the fly from the
// NHWC source tensor, with no im2col buffer (the tensorcore Conv2D page's
// "Strategy" materialises one; its "Conv2D vs GEMM tradeoffs" note on the
// scratch size is the cost this kernel avoids).  Each 16-byte chunk of a GEMM
// row is 8 (16-bit types) or 16 (int8) consecutive channels of one filter tap,
// so every global load is a 128-bit load of contiguous NHWC memory or zero for
// a padding tap.  Tiles arrive in LDS by direct-to-LDS loads into a ring of
// three stages (two k-steps in flight while the third is computed; padding
// reads zeros through the buffer range check) and feed 16x16x32 (f16/bf16)
// or 16x16x64 (int8) MFMA with fp32 / int32 accumulation.  The
// epilogue (bias, ReLU, int8 requantisation, rounding) is fused and the tile
// leaves through LDS as 128-bit stores.
//
// The CUTLASS Python Conv2d notebook's "Tile Description" section is the
// model for the tile table: every entry must give the same result.
#include "device_common.h"

namespace cnv {

template <int BM_, int BN_, int BKB_, int WM_, int WN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BKB = BKB_, WM = WM_, WN = WN_;
};

// tile table (index = conv2d_algo_t.tile - 1)
using T0 = Tile<128, 64, 128, 2, 2>;
using T1 = Tile<128, 128, 64, 2, 2>;
using T2 = Tile<64, 64, 128, 2, 2>;
using T3 = Tile<256, 64, 64, 4, 1>;
using T4 = Tile<64, 32, 128, 4, 1>;

// s_waitcnt with vmcnt = N (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ inline void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// TB (dgrad, 16-bit types): the B tile is staged as BK rows (tap, dy
// channel) of BN dx channels straight from w[K][R][S][C], 16-byte chunks of
// row k swizzled by btswz(k), and read with ds_read_b64_tr_b16.
template <int BROWCH>
__device__ inline int btswz(int row)
{
    const int b3 = ((row >> 3) & 1) << 1;
    if constexpr (BROWCH == 4) return b3;
    if constexpr (BROWCH == 8) return (((row >> 1) & 1) << 2) | b3;
    return ((row & 3) << 2) | b3;
}

template <class E, class TL, bool TB>
__global__ __launch_bounds__(256) void igemm_kernel(const IgemmArgs a)
{
    constexpr int NT = 256;
    constexpr int BM = TL::BM, BN = TL::BN, BKB = TL::BKB;
    constexpr int CH = BKB / 16;        // 16-byte chunks per tile row per k-step
    constexpr int EPC = E::EPC;
    constexpr int BK = CH * EPC;        // GEMM-K elements per k-step
    constexpr int RB = 64 / CH;         // tile rows per 1 KB direct-to-LDS block
    constexpr int SH = CH == 8 ? 1 : 2; // chunk swizzle: stored slot = chunk ^ ((row >> SH) & (CH - 1))
    constexpr int A_BLK = BM / RB / 4;  // blocks per wave and stage
    constexpr int B_BLK = BN / RB / 4;
    constexpr int PER = A_BLK + B_BLK;  // direct-to-LDS loads per wave and stage
    constexpr int NSTAGE = 3;
    constexpr int WTM = BM / TL::WM, WTN = BN / TL::WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int KSUB = BKB / 64;      // MFMAs along K per k-step
    constexpr int STAGE = (BM + BN) * BKB;
    static_assert(TL::WM * TL::WN == 4, "four waves");
    static_assert(CH == 4 || CH == 8, "64- or 128-byte tile rows");
    static_assert((BM / RB) % 4 == 0 && (BN / RB) % 4 == 0 && A_BLK > 0 && B_BLK > 0, "whole blocks per wave");
    constexpr int BROWCH = BN / 8;      // TB: 16-byte chunks per B row
    constexpr int RPB = 64 / BROWCH;    // TB: B rows per 1 KB block
    static_assert(!TB || (EPC == 8 && (BROWCH == 4 || BROWCH == 8 || BROWCH == 16) && 4 * B_BLK * RPB == BK),
                  "transposed B: 16-bit types, 32- to 128-wide N tiles");
    using elem = typename E::elem;
    using acc_t = typename E::acc;
    constexpr int OSZ = (int)sizeof(elem);
    constexpr int CROWB = BN * OSZ + 16;
    static_assert(BM * CROWB <= NSTAGE * STAGE, "epilogue tile fits in LDS");

    __shared__ __attribute__((aligned(16))) unsigned char smem[NSTAGE * STAGE];

    const Phase &ph = a.ph[blockIdx.z];
    const int mt = blockIdx.x;
    if (mt >= ph.tiles_m) return;
    // N tile ntl of group gi: output channels gi*kg + ntl*BN + (0..BN-1), of
    // which the first kg - ntl*BN exist
    const int gi = blockIdx.y / a.ntiles_g, ntl = blockIdx.y - gi * a.ntiles_g;
    const int ncol0 = gi * a.kg + ntl * BN;       // first output channel of the tile
    const int nvalid = min(BN, a.kg - ntl * BN);  // channels of the tile in the group
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / TL::WN, wn = wave % TL::WN;

    const int hs = a.hs, ws = a.ws, cs = a.cs;
    const uint32_t mi_mj = (uint32_t)ph.mi * (uint32_t)ph.mj;

    // ---- operand tiles arrive by direct-to-LDS loads (buffer_load ... lds):
    // wave w fills blocks w, w+4, ... of a stage's A rows and B rows; lane i
    // of a block fills stored slot i % CH of block row i / CH, which holds
    // logical chunk kc = (i % CH) ^ swizzle(row).  For every block a wave
    // fills, the swizzle of its rows depends on the lane alone, so each lane
    // moves the same GEMM-K chunk kc of all its rows.
    const int brow = lane / CH;  // row inside a block
    const int kc = (lane % CH) ^ (((RB * wave + brow) >> SH) & (CH - 1));
    const u32x4 a_rs = make_buf_rsrc(a.src, (uint32_t)((size_t)a.nimg * hs * ws * cs * sizeof(elem)));
    const u32x4 b_rs = make_buf_rsrc(a.bmat, (uint32_t)(a.b_elems * sizeof(elem)));
    const uint32_t lds0 = lds_addr(smem);

    // per lane: A rows (image base, source coordinates of tap (0,0))
    uint32_t a_img[A_BLK];
    int a_ih[A_BLK], a_iw[A_BLK];
#pragma unroll
    for (int t = 0; t < A_BLK; ++t) {
        const int row = RB * (wave + 4 * t) + brow;
        const uint32_t m = (uint32_t)mt * BM + row;
        if (m < ph.m_total) {
            const uint32_t n = fdiv(m, ph.div_mimj);
            const uint32_t rem = m - n * mi_mj;
            const uint32_t ii = fdiv(rem, ph.div_mj);
            const uint32_t jj = rem - ii * ph.mj;
            a_img[t] = n * (uint32_t)(hs * ws);
            a_ih[t] = (int)ii * a.gsh + ph.th0;
            a_iw[t] = (int)jj * a.gsw + ph.tw0;
        } else {
            a_img[t] = 0;
            a_ih[t] = -(1 << 29);  // never inside the image
            a_iw[t] = -(1 << 29);
        }
    }
    // per lane: B rows (element offset of the row, or -1 past ngemm)
    long long b_row[B_BLK];
    // TB: per block t, the lane's B row is GEMM-K index (tap (bjr, bjs), dy
    // channel bk) and its chunk column bcol (dx channel within the group),
    // or -1 past the tile's valid channels
    int bk[B_BLK], bjs[B_BLK], bjr[B_BLK], bcol[B_BLK];
#pragma unroll
    for (int t = 0; t < B_BLK; ++t) {
        if constexpr (!TB) {
            const int nl = RB * (wave + 4 * t) + brow;
            b_row[t] = nl < nvalid ? ph.b_off + (long long)(ncol0 + nl) * ph.kgemm : -1;
        } else {
            const int row = RPB * (wave + 4 * t) + lane / BROWCH;  // B row in the stage
            const int cs = (lane % BROWCH) ^ btswz<BROWCH>(row);   // source chunk of the stored one
            bcol[t] = 8 * cs < nvalid ? ntl * BN + 8 * cs : -1;
            bk[t] = row;
            bjs[t] = 0;
            bjr[t] = 0;
        }
    }
    auto normalize_b = [&](int t) {
        while (bk[t] >= a.cg) {
            bk[t] -= a.cg;
            if (++bjs[t] == ph.nts) {
                bjs[t] = 0;
                ++bjr[t];
            }
        }
    };
    if constexpr (TB) {
#pragma unroll
        for (int t = 0; t < B_BLK; ++t) normalize_b(t);
    }

    // ---- GEMM-K position of this lane's chunk: (tap tr, tap ts, channel c)
    int c = kc * EPC, tr = 0, ts = 0, kk = kc * EPC;
    auto normalize = [&]() {
        while (c >= a.cg) {
            c -= a.cg;
            if (++ts == ph.nts) {
                ts = 0;
                ++tr;
            }
        }
    };
    normalize();

    const int KT = (ph.kgemm + BK - 1) / BK;
    // issue stage kt's loads into buffer kt % NSTAGE, then advance the chunk
    auto dma_stage = [&](int kt) {
        const uint32_t base = lds0 + (uint32_t)((kt % NSTAGE) * STAGE);  // LDS byte address
        const bool kval = tr < ph.ntr;
#pragma unroll
        for (int t = 0; t < A_BLK; ++t) {
            const int h = a_ih[t] + tr * ph.tdh;
            const int w = a_iw[t] + ts * ph.tdw;
            const bool ok = kval && (unsigned)h < (unsigned)hs && (unsigned)w < (unsigned)ws;
            const uint32_t voff = ok ? ((a_img[t] + (uint32_t)(h * ws + w)) * (uint32_t)cs + (uint32_t)(gi * a.cg + c)) * sizeof(elem)
                                     : kBufOOBFar;
            dma16(a_rs, base + (wave + 4 * t) * 1024, voff);
        }
#pragma unroll
        for (int t = 0; t < B_BLK; ++t) {
            if constexpr (!TB) {
                const uint32_t voff =
                    (kval && b_row[t] >= 0) ? (uint32_t)((b_row[t] + kk) * (long long)sizeof(elem)) : kBufOOBFar;
                dma16(b_rs, base + BM * BKB + (wave + 4 * t) * 1024, voff);
            } else {
                // w[gi*Kg + k][r][s][col]
                const int r = ph.r0 + bjr[t] * ph.rstep, s = ph.s0 + bjs[t] * ph.sstep;
                const bool ok = bjr[t] < ph.ntr && bcol[t] >= 0;
                const uint32_t voff =
                    ok ? (uint32_t)((((gi * a.cg + bk[t]) * a.filt_r + r) * a.filt_s + s) * a.kg + bcol[t]) *
                             (uint32_t)sizeof(elem)
                       : kBufOOBFar;
                dma16(b_rs, base + BM * BKB + (wave + 4 * t) * 1024, voff);
                bk[t] += BK;
                normalize_b(t);
            }
        }
        c += BK;
        kk += BK;
        normalize();
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

    // fragment reads: row (lane & 15) of a 16-row block, logical chunk
    // 4*ks + lane/16, at its swizzled slot (the swizzle of rows 16q + r is
    // that of r)
    const int frag_row = lane & 15;
    const int fswz = (frag_row >> SH) & (CH - 1);
    int fofs[KSUB];
#pragma unroll
    for (int ks = 0; ks < KSUB; ++ks) fofs[ks] = frag_row * BKB + (((4 * ks + (lane >> 4)) ^ fswz) << 4);
    // TB: ds_read_b64_tr_b16 -- in each group of 16 lanes, lane L points at
    // row L/4, columns 4*(L%4)..+3 of a 4 x 16 tile and receives column L of
    // the 4 rows.  Lane group q reads B rows 32*ks + 8q + 4t + L/4 (t = 0, 1:
    // the fragment's 8 k values), columns n0 + 4*(L%4) of block j; the row's
    // swizzle depends on the lane only (rows move by multiples of 4 and 32).
    int bofs[FN];
    if constexpr (TB) {
        const int L = lane & 15, rl = 8 * (lane >> 4) + (L >> 2);
        const int sw = btswz<BROWCH>(rl);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int chunk = (wn * WTN + j * 16) / 8 + ((L & 3) >> 1);
            bofs[j] = BM * BKB + rl * BN * 2 + ((chunk ^ sw) << 4) + (L & 1) * 8;
        }
    }

#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < KT) dma_stage(s);
    for (int kt = 0; kt < KT; ++kt) {
        // stage kt has landed when at most the younger stages' loads remain
        const int younger = min(NSTAGE - 2, KT - 1 - kt);
        if (younger >= 1)
            wait_vm<PER * (NSTAGE - 2)>();
        else
            wait_vm<0>();
        __syncthreads();  // every wave's loads of stage kt are visible; stage kt-1 is consumed
        if (kt + NSTAGE - 1 < KT) dma_stage(kt + NSTAGE - 1);
        const unsigned char *base = smem + (kt % NSTAGE) * STAGE;
#pragma unroll
        for (int ks = 0; ks < KSUB; ++ks) {
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = *(const u32x4 *)(base + (wm * WTM + i * 16) * BKB + fofs[ks]);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (!TB) {
                    fb[j] = *(const u32x4 *)(base + (BM + wn * WTN + j * 16) * BKB + fofs[ks]);
                } else {
                    typedef short s16x4 __attribute__((ext_vector_type(4)));
                    uint2 h[2];
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        h[t] = __builtin_bit_cast(
                            uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) s16x4 *)(base + bofs[j] +
                                                                                    (32 * ks + 4 * t) * BN * 2)));
                    fb[j] = u32x4{h[0].x, h[0].y, h[1].x, h[1].y};
                }
            }
            // filter fragment as the MFMA's A operand, pixels as B: each lane
            // of a result block then holds 4 consecutive channels of a pixel
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = E::mfma(fb[j], fa[i], acc[i][j]);
        }
    }
    __syncthreads();  // the stage buffers become the epilogue tile

    // ---- fused epilogue: acc -> (bias, ReLU | requant) -> LDS tile -> HBM
    // MFMA 16x16 result layout (A = channels, B = pixels): lane holds pixel
    // (lane & 15) and channels 4*(lane >> 4) + 0..3 of each 16x16 block, so
    // a lane packs its 4 channels of a pixel into one LDS write.  ngemm is a
    // multiple of 8 (16 for int8), so those 4 channels are all in range or
    // all past it.  fprop writes one output image in pixel order, where the
    // address of GEMM row m is m*ngemm (contig); dgrad phases decompose m.
    const bool contig = ph.oh0 == 0 && ph.ow0 == 0 && a.osh == 1 && a.osw == 1 && ph.mi == a.ho && ph.mj == a.wo;
    auto out_offset = [&](uint32_t m) -> size_t {
        if (contig) return (size_t)m * a.ngemm;
        const uint32_t n = fdiv(m, ph.div_mimj);
        const uint32_t rem = m - n * mi_mj;
        const uint32_t ii = fdiv(rem, ph.div_mj);
        const uint32_t jj = rem - ii * ph.mj;
        const int oh = ph.oh0 + (int)ii * a.osh, ow = ph.ow0 + (int)jj * a.osw;
        return (((size_t)n * a.ho + oh) * a.wo + ow) * a.ngemm;
    };
    const int prow = lane & 15, cq = 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = wn * WTN + j * 16 + cq;
        const int n = ncol0 + col;
        const bool nok = col < nvalid;
        if constexpr (E::kDtype == CONV2D_DTYPE_I8) {
            int b[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) b[r] = (a.bias && nok) ? ((const int32_t *)a.bias)[n + r] : 0;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WTM + i * 16 + prow;
                uint32_t word = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int v = acc[i][j][r] + b[r];
                    if (a.relu && v < 0) v = 0;
                    word |= (uint32_t)(uint8_t)requant_i8(v, a.requant_m) << (8 * r);
                }
                *(uint32_t *)(smem + row * CROWB + col) = word;
            }
        } else {
            float b[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) b[r] = (a.bias && nok) ? E::to_f32(((const elem *)a.bias)[n + r]) : 0.0f;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WTM + i * 16 + prow;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r];
                if (a.axpby) {
                    // linear combination with C at these output elements
                    float c[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    const uint32_t m = (uint32_t)mt * BM + row;
                    if (a.cmat && nok && m < ph.m_total) {
                        const uint2 cv = *(const uint2 *)((const elem *)a.cmat + out_offset(m) + n);
                        const uint32_t cw[2] = {cv.x, cv.y};
#pragma unroll
                        for (int r = 0; r < 4; ++r) c[r] = E::to_f32((elem)(cw[r >> 1] >> (16 * (r & 1))));
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = a.alpha * v[r] + a.beta * c[r];
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] += b[r];
                uint2 p;
                if (a.relu) {
                    p.x = out_pair<E, true>(v[0], v[1]);
                    p.y = out_pair<E, true>(v[2], v[3]);
                } else {
                    p.x = out_pair<E, false>(v[0], v[1]);
                    p.y = out_pair<E, false>(v[2], v[3]);
                }
                *(uint2 *)(smem + row * CROWB + col * OSZ) = p;
            }
        }
    }
    __syncthreads();

    constexpr int OCH = BN * OSZ / 16;  // 16-byte chunks per output row
    constexpr int EPO = 16 / OSZ;       // elements per output chunk
    elem *dst = (elem *)a.dst;
    for (int id = tid; id < BM * OCH; id += NT) {
        const int row = id / OCH, cc = id % OCH;
        const uint32_t m = (uint32_t)mt * BM + row;
        if (m >= ph.m_total || cc * EPO >= nvalid) continue;
        __builtin_nontemporal_store(*(const u32x4 *)(smem + row * CROWB + cc * 16),
                                    (u32x4 *)(dst + out_offset(m) + ncol0 + cc * EPO));
    }
}

int igemm_num_tiles() { return 5; }

TileShape igemm_tile_shape(int tile)
{
    switch (tile) {
    case 0: return {T0::BM, T0::BN};
    case 1: return {T1::BM, T1::BN};
    case 2: return {T2::BM, T2::BN};
    case 3: return {T3::BM, T3::BN};
    default: return {T4::BM, T4::BN};
    }
}

template <class E, bool TB>
static hipError_t launch_e(int tile, const IgemmArgs &a, int gm, int gn, hipStream_t st)
{
    dim3 grid((unsigned)gm, (unsigned)gn, (unsigned)a.nphases);
    switch (tile) {
    case 0: igemm_kernel<E, T0, TB><<<grid, 256, 0, st>>>(a); break;
    case 1: igemm_kernel<E, T1, TB><<<grid, 256, 0, st>>>(a); break;
    case 2: igemm_kernel<E, T2, TB><<<grid, 256, 0, st>>>(a); break;
    case 3: igemm_kernel<E, T3, TB><<<grid, 256, 0, st>>>(a); break;
    case 4: igemm_kernel<E, T4, TB><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_igemm(int dtype, int tile, const IgemmArgs &a, int grid_m, int grid_n, hipStream_t st)
{
    switch (dtype) {
    case CONV2D_DTYPE_F16:
        return a.b_trans ? launch_e<EF16, true>(tile, a, grid_m, grid_n, st)
                         : launch_e<EF16, false>(tile, a, grid_m, grid_n, st);
    case CONV2D_DTYPE_BF16:
        return a.b_trans ? launch_e<EBF16, true>(tile, a, grid_m, grid_n, st)
                         : launch_e<EBF16, false>(tile, a, grid_m, grid_n, st);
    case CONV2D_DTYPE_I8:
        if (a.b_trans) return hipErrorInvalidValue;
        return launch_e<EI8, false>(tile, a, grid_m, grid_n, st);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// dgrad filter re-layout: for each stride phase, wt[c][tap][k] =
// w[g*Kg + k][r0 + jr*rstep][s0 + js*sstep][c - g*Cg] with tap = jr*nts + js
// and g = c / Cg the dx channel's group (one group: w[k][r][s][c]).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dgrad_prep_kernel(const PrepArgs a)
{
    const PrepPhase &p = a.ph[blockIdx.y];
    const int ntap = p.ntr * p.nts;
    const int total = a.C * ntap * a.Kg;
    const T *w = (const T *)a.w;
    T *wt = (T *)a.wt + p.off;
    for (int idx = blockIdx.x * 256 + threadIdx.x; idx < total; idx += gridDim.x * 256) {
        const int k = idx % a.Kg;  // dy channel within the group
        const int t = idx / a.Kg;
        const int tap = t % ntap;
        const int c = t / ntap;    // dx channel
        const int g = c / a.Cg;
        const int r = p.r0 + (tap / p.nts) * p.rstep;
        const int s = p.s0 + (tap % p.nts) * p.sstep;
        wt[idx] = w[((((size_t)g * a.Kg + k) * a.R + r) * a.S + s) * a.Cg + (c - g * a.Cg)];
    }
}

hipError_t launch_dgrad_prep(int dtype, const PrepArgs &a, hipStream_t st)
{
    (void)dtype;  // f16 and bf16 are both 2-byte copies
    if (a.max_elems <= 0) return hipSuccess;
    int blocks = (a.max_elems + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    dgrad_prep_kernel<uint16_t><<<dim3(blocks, a.nphases), 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace cnv

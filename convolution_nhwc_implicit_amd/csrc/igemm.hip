// igemm.hip -- implicit-GEMM convolution kernel for gfx950 (fprop, and dgrad
// one stride phase per grid z-slice).
//
// The convolution is a GEMM whose A operand is gathered on the fly from the
// NHWC source tensor, with no im2col buffer (the tensorcore Conv2D page's
// "Strategy" materialises one; its "Conv2D vs GEMM tradeoffs" note on the
// scratch size is the cost this kernel avoids).  Each 16-byte chunk of a GEMM
// row is 8 (16-bit types) or 16 (int8) consecutive channels of one filter tap,
// so every global load is a 128-bit load of contiguous NHWC memory or zero for
// a padding tap.  Tiles are staged in LDS in two buffers and fed to 16x16x32
// (f16/bf16) or 16x16x64 (int8) MFMA with fp32 / int32 accumulation.  The
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

template <class E, class TL>
__global__ __launch_bounds__(256) void igemm_kernel(const IgemmArgs a)
{
    constexpr int NT = 256;
    constexpr int BM = TL::BM, BN = TL::BN, BKB = TL::BKB;
    constexpr int CH = BKB / 16;        // 16-byte chunks per tile row per k-step
    constexpr int EPC = E::EPC;
    constexpr int BK = CH * EPC;        // GEMM-K elements per k-step
    constexpr int ROWB = BKB + 16;      // padded LDS row: conflict-free 128-bit reads
    constexpr int A_CH = BM * CH / NT;  // A chunks per thread
    constexpr int B_TOT = BN * CH;
    constexpr int B_CH = (B_TOT + NT - 1) / NT;
    constexpr int WTM = BM / TL::WM, WTN = BN / TL::WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int KSUB = BKB / 64;      // MFMAs along K per k-step
    constexpr int STAGE = (BM + BN) * ROWB;
    static_assert(TL::WM * TL::WN == 4, "four waves");
    static_assert((BM * CH) % NT == 0 && NT % CH == 0, "chunk mapping");
    using elem = typename E::elem;
    using acc_t = typename E::acc;
    constexpr int OSZ = (int)sizeof(elem);
    constexpr int CROWB = BN * OSZ + 16;
    static_assert(BM * CROWB <= 2 * STAGE, "epilogue tile fits in LDS");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

    const Phase &ph = a.ph[blockIdx.z];
    const int mt = blockIdx.x;
    if (mt >= ph.tiles_m) return;
    const int nt = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / TL::WN, wn = wave % TL::WN;
    const int kc = tid % CH;

    const elem *src = (const elem *)a.src;
    const int hs = a.hs, ws = a.ws, cs = a.cs;
    const uint32_t mi_mj = (uint32_t)ph.mi * (uint32_t)ph.mj;

    // ---- per-thread A rows: image base and source coordinates of tap (0,0)
    const elem *a_base[A_CH];
    int a_ih[A_CH], a_iw[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int row = (tid + i * NT) / CH;
        const uint32_t m = (uint32_t)mt * BM + row;
        if (m < ph.m_total) {
            const uint32_t n = fdiv(m, ph.div_mimj);
            const uint32_t rem = m - n * mi_mj;
            const uint32_t ii = fdiv(rem, ph.div_mj);
            const uint32_t jj = rem - ii * ph.mj;
            a_base[i] = src + (size_t)n * hs * ws * cs;
            a_ih[i] = (int)ii * a.gsh + ph.th0;
            a_iw[i] = (int)jj * a.gsw + ph.tw0;
        } else {
            a_base[i] = src;
            a_ih[i] = -(1 << 29);  // never inside the image
            a_iw[i] = -(1 << 29);
        }
    }
    // ---- per-thread B rows
    const elem *b_ptr[B_CH];
    bool b_ok[B_CH];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
        const int id = tid + i * NT;
        const int row = id / CH;
        const int n = nt * BN + row;
        b_ok[i] = (id < B_TOT) && (n < a.ngemm);
        b_ptr[i] = (const elem *)a.bmat + ph.b_off + (b_ok[i] ? (size_t)n * ph.kgemm + kc * EPC : 0);
    }

    // ---- GEMM-K position of this thread's chunk: (tap tr, tap ts, channel c)
    int c = kc * EPC, tr = 0, ts = 0;
    auto normalize = [&]() {
        while (c >= cs) {
            c -= cs;
            if (++ts == ph.nts) {
                ts = 0;
                ++tr;
            }
        }
    };
    normalize();

    const int KT = (ph.kgemm + BK - 1) / BK;
    u32x4 ra[A_CH], rb[B_CH];
    const u32x4 zero = {0u, 0u, 0u, 0u};

    auto gload = [&](int kt) {
        const bool kval = tr < ph.ntr;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int h = a_ih[i] + tr * ph.tdh;
            const int w = a_iw[i] + ts * ph.tdw;
            const bool ok = kval && (unsigned)h < (unsigned)hs && (unsigned)w < (unsigned)ws;
            ra[i] = ok ? *(const u32x4 *)(a_base[i] + ((size_t)(h * ws + w) * cs + c)) : zero;
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i)
            rb[i] = (b_ok[i] && kval) ? *(const u32x4 *)(b_ptr[i] + (size_t)kt * BK) : zero;
    };
    auto sstore = [&](int stage) {
        unsigned char *base = smem + stage * STAGE;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int row = (tid + i * NT) / CH;
            *(u32x4 *)(base + row * ROWB + kc * 16) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int id = tid + i * NT;
            if (id < B_TOT) {
                const int row = id / CH;
                *(u32x4 *)(base + (BM + row) * ROWB + kc * 16) = rb[i];
            }
        }
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

    const int frag_row = lane & 15;
    const int frag_k = (lane >> 4) * 16;
    if (KT > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < KT) {
                c += BK;
                normalize();
                gload(kt + 1);
            }
            const unsigned char *base = smem + cur * STAGE;
#pragma unroll
            for (int ks = 0; ks < KSUB; ++ks) {
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

    // ---- fused epilogue: acc -> (bias, ReLU | requant) -> element -> LDS tile
    // MFMA 16x16 result layout: lane holds column (lane & 15) and rows
    // 4*(lane >> 4) + 0..3 of each 16x16 block.
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = wn * WTN + j * 16 + (lane & 15);
        const int n = nt * BN + col;
        const bool nok = n < a.ngemm;
        if constexpr (E::kDtype == CONV2D_DTYPE_I8) {
            const int b = (a.bias && nok) ? ((const int32_t *)a.bias)[n] : 0;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = wm * WTM + i * 16 + (lane >> 4) * 4 + r;
                    int v = acc[i][j][r] + b;
                    if (a.relu && v < 0) v = 0;
                    *(int8_t *)(smem + row * CROWB + col) = requant_i8(v, a.requant_m);
                }
        } else {
            const float b = (a.bias && nok) ? E::to_f32(((const elem *)a.bias)[n]) : 0.0f;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = wm * WTM + i * 16 + (lane >> 4) * 4 + r;
                    *(elem *)(smem + row * CROWB + col * OSZ) =
                        E::from_f32(bias_relu_f32(acc[i][j][r], b, a.relu));
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
        const int n0 = nt * BN + cc * EPO;
        if (m >= ph.m_total || n0 >= a.ngemm) continue;
        const uint32_t n = fdiv(m, ph.div_mimj);
        const uint32_t rem = m - n * mi_mj;
        const uint32_t ii = fdiv(rem, ph.div_mj);
        const uint32_t jj = rem - ii * ph.mj;
        const int oh = ph.oh0 + (int)ii * a.osh;
        const int ow = ph.ow0 + (int)jj * a.osw;
        *(u32x4 *)(dst + (((size_t)n * a.ho + oh) * a.wo + ow) * a.ngemm + n0) =
            *(const u32x4 *)(smem + row * CROWB + cc * 16);
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

template <class E>
static hipError_t launch_e(int tile, const IgemmArgs &a, int gm, int gn, hipStream_t st)
{
    dim3 grid((unsigned)gm, (unsigned)gn, (unsigned)a.nphases);
    switch (tile) {
    case 0: igemm_kernel<E, T0><<<grid, 256, 0, st>>>(a); break;
    case 1: igemm_kernel<E, T1><<<grid, 256, 0, st>>>(a); break;
    case 2: igemm_kernel<E, T2><<<grid, 256, 0, st>>>(a); break;
    case 3: igemm_kernel<E, T3><<<grid, 256, 0, st>>>(a); break;
    case 4: igemm_kernel<E, T4><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_igemm(int dtype, int tile, const IgemmArgs &a, int grid_m, int grid_n, hipStream_t st)
{
    switch (dtype) {
    case CONV2D_DTYPE_F16: return launch_e<EF16>(tile, a, grid_m, grid_n, st);
    case CONV2D_DTYPE_BF16: return launch_e<EBF16>(tile, a, grid_m, grid_n, st);
    case CONV2D_DTYPE_I8: return launch_e<EI8>(tile, a, grid_m, grid_n, st);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// dgrad filter re-layout: for each stride phase, wt[c][tap][k] =
// w[k][r0 + jr*rstep][s0 + js*sstep][c] with tap = jr*nts + js.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dgrad_prep_kernel(const PrepArgs a)
{
    const PrepPhase &p = a.ph[blockIdx.y];
    const int ntap = p.ntr * p.nts;
    const int total = a.C * ntap * a.K;
    const T *w = (const T *)a.w;
    T *wt = (T *)a.wt + p.off;
    for (int idx = blockIdx.x * 256 + threadIdx.x; idx < total; idx += gridDim.x * 256) {
        const int k = idx % a.K;
        const int t = idx / a.K;
        const int tap = t % ntap;
        const int c = t / ntap;
        const int r = p.r0 + (tap / p.nts) * p.rstep;
        const int s = p.s0 + (tap % p.nts) * p.sstep;
        wt[idx] = w[(((size_t)k * a.R + r) * a.S + s) * a.C + c];
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

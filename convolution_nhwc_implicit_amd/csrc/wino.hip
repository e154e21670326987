// wino.hip -- Winograd F(2x2, 3x3) for stride-1 3x3 layers with 64 input
// channels, on 16x16x32 MFMAs (gfx950): fprop, and dgrad as the forward
// convolution of dy (64 channels) with the filter's taps reversed and its
// channel axes swapped, padded by 2 - pad.
//
// The tensorcore "Conv2D" page ("What's not done in v0.1") names a Winograd
// path for 3x3 stride-1 layers as a later priority.  F(2x2, 3x3) (Lavin and
// Gray's minimal filtering) computes each 2x2 output block from a 4x4 input
// tile d and each 3x3 filter g as
//
//     Y = A^T [ sum_c (G g G^T) (.) (B^T d B) ] A,
//
// 16 products per block instead of 36: 16 independent GEMMs, one per
// transformed point xi = (a, b), each over the input channels, of
// U_xi [K x C] by V_xi [C x tiles].
//
// Work split.  A workgroup (8 waves, two per SIMD) holds 64 output channels
// and walks batches of 32 tiles (2 output rows x 64 output columns).  Wave w
// owns output channels 16*(w%4) .. +15 and tiles 16*(w/4) .. +15 for all 16
// points: sixteen 16x16 accumulators, so the inverse transform needs no
// exchange between lanes (a lane holds one tile and four channels of each).
//
//   * U: the wave's 16 channels x 64 input channels x 16 points in fp16
//     are 32 A fragments of 16 bytes a lane (128 VGPRs), computed once per
//     workgroup from the filter (in fp32, rounded once) and kept in registers
//     for every batch; only V goes through LDS.  The grid is persistent (one
//     workgroup per CU and channel slice) so the filter is transformed once
//     per CU.
//   * V is double-buffered in LDS (2 x 64 KB): each batch step forms the next
//     batch's V, then runs this batch's MFMAs and epilogue, one barrier per
//     batch, so the two waves of a SIMD overlap transform and MFMA work.
//   * V: thread (tile t, channels 4j..4j+3) reads its 4x4 input window from
//     HBM/L2 (8-byte loads; padding from the buffer range check), forms
//     B^T d B in fp32 two channels at a time, rounds once and writes V into
//     LDS as [point][tile][channel], the 16-byte channel chunks of tile t
//     XOR-swizzled by t/2 so the MFMA's B-fragment reads (16 tiles, one
//     chunk) cover all 64 banks.
//   * Epilogue: A^T M A in fp32 per lane, + bias, ReLU, one rounding; each
//     lane stores its four channels (8 bytes) of four output pixels.
//
// fp16 only (bf16's 8-bit significand would leave rms_scaled near 4e-3).
// Numerics differ from the direct convolution: U and V are rounded to fp16
// before the products, so each product carries up to ~2 units
// of that type's rounding of the transformed terms.  Integer-valued data
// small enough that U (quarter-integers) and V are exact give exactly the
// direct result.
#include "device_common.h"

namespace cnv {

typedef unsigned v2u32 __attribute__((ext_vector_type(2)));
template <bool B>
struct BoolConst {
    static constexpr bool value = B;
};

namespace wn {
constexpr int NT = 512;
constexpr int CIN = 64;                 // input channels: two 32-channel MFMA steps
constexpr int BK = 64;                  // output channels per workgroup (4 waves x 16)
constexpr int TB = 32;                  // tiles per batch: 2 output rows x 64 output columns
constexpr int XI = 16;                  // transformed points
constexpr int VROW = CIN * 2;           // bytes of one (point, tile) row of V
constexpr int V_BYTES = XI * TB * VROW;  // 64 KB
}  // namespace wn

// dgrad: the transformed filter of the equivalent forward convolution of dy,
// whose filter is w'[c][r][s][k] = w[k][2-r][2-s][c] (taps reversed, channel
// axes swapped): U[xi][c][k] = (G w'_ck G^T)[xi] for every dx channel
// c < ngemm and dy channel k < 64, in fp32, rounded once, into the workspace.
// One thread per (k, c), c fastest, so the filter reads are coalesced.
template <class E>
__global__ __launch_bounds__(256) void wino_dgrad_filter_kernel(const void *w, void *u, int ngemm)
{
    using elem = typename E::elem;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= ngemm * wn::CIN) return;
    const int k = i / ngemm, c = i - k * ngemm;
    const elem *wk = (const elem *)w + (size_t)k * 9 * ngemm + c;
    float g[3][3];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int s = 0; s < 3; ++s) g[r][s] = E::to_f32(wk[((2 - r) * 3 + (2 - s)) * ngemm]);
    float t[4][3];  // G g
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        t[0][s] = g[0][s];
        t[1][s] = 0.5f * (g[0][s] + g[1][s] + g[2][s]);
        t[2][s] = 0.5f * (g[0][s] - g[1][s] + g[2][s]);
        t[3][s] = g[2][s];
    }
    elem *uo = (elem *)u + (size_t)c * wn::CIN + k;
    const size_t pstride = (size_t)ngemm * wn::CIN;  // between points
#pragma unroll
    for (int r = 0; r < 4; ++r) {  // (G g) G^T
        uo[(4 * r + 0) * pstride] = E::from_f32(t[r][0]);
        uo[(4 * r + 1) * pstride] = E::from_f32(0.5f * (t[r][0] + t[r][1] + t[r][2]));
        uo[(4 * r + 2) * pstride] = E::from_f32(0.5f * (t[r][0] - t[r][1] + t[r][2]));
        uo[(4 * r + 3) * pstride] = E::from_f32(t[r][2]);
    }
}

// UWS: U comes ready from the workspace (dgrad) instead of being formed from
// the filter in the prologue (fprop).
template <class E, bool UWS>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void wino_fprop_kernel(
    const WinoArgs a)
{
    using elem = typename E::elem;
    __shared__ __attribute__((aligned(16))) unsigned char vbuf[2 * wn::V_BYTES];  // V double-buffered
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave & 3, tg = wave >> 2;
    const int k0 = blockIdx.y * wn::BK;

    // ---- U fragments (A operand): point xi = 4a + b, channel step cs; lane
    // holds output channel kr = k0 + 16kg + (lane & 15) and input channels
    // 32cs + 8(lane >> 4) + 0..7.  U = G g G^T with G = [1 0 0; h h h; h -h h;
    // 0 0 1], h = 1/2, computed in fp32 and rounded once.
    u32x4 uf[wn::XI][2];
    if constexpr (UWS) {
        // U[xi][k][c] from the workspace, one 16-byte load per fragment
        const int kr = k0 + 16 * kg + (lane & 15);
        const bool kok = kr < a.ngemm;
        const elem *uk = (const elem *)a.u + (size_t)(kok ? kr : 0) * wn::CIN + 8 * (lane >> 4);
#pragma unroll
        for (int xi = 0; xi < wn::XI; ++xi)
#pragma unroll
            for (int cs = 0; cs < 2; ++cs)
                uf[xi][cs] = kok ? *(const u32x4 *)(uk + (size_t)xi * a.ngemm * wn::CIN + 32 * cs) : u32x4{0, 0, 0, 0};
    } else {
        const int kr = k0 + 16 * kg + (lane & 15);
        const bool kok = kr < a.ngemm;
        const elem *wk = (const elem *)a.w + (size_t)(kok ? kr : 0) * 9 * wn::CIN;
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
            const int c0 = 32 * cs + 8 * (lane >> 4);
            // the 8 channels of each tap: one 16-byte load per tap
            u32x4 gv[9];
#pragma unroll
            for (int tap = 0; tap < 9; ++tap)
                gv[tap] = kok ? *(const u32x4 *)(wk + tap * wn::CIN + c0) : u32x4{0, 0, 0, 0};
            uint32_t packed[wn::XI][4];
#pragma unroll
            for (int hp = 0; hp < 4; ++hp) {  // channel pairs c0 + 2hp, +1
                float u[2][wn::XI];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    float g[3][3];
#pragma unroll
                    for (int r = 0; r < 3; ++r)
#pragma unroll
                        for (int s = 0; s < 3; ++s)
                            g[r][s] = E::to_f32((elem)(gv[r * 3 + s][hp] >> (16 * e)));
                    float t[4][3];  // G g
#pragma unroll
                    for (int s = 0; s < 3; ++s) {
                        t[0][s] = g[0][s];
                        t[1][s] = 0.5f * (g[0][s] + g[1][s] + g[2][s]);
                        t[2][s] = 0.5f * (g[0][s] - g[1][s] + g[2][s]);
                        t[3][s] = g[2][s];
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {  // (G g) G^T
                        u[e][4 * r + 0] = t[r][0];
                        u[e][4 * r + 1] = 0.5f * (t[r][0] + t[r][1] + t[r][2]);
                        u[e][4 * r + 2] = 0.5f * (t[r][0] - t[r][1] + t[r][2]);
                        u[e][4 * r + 3] = t[r][2];
                    }
                }
#pragma unroll
                for (int xi = 0; xi < wn::XI; ++xi)
                    packed[xi][hp] = (uint32_t)E::from_f32(u[0][xi]) | ((uint32_t)E::from_f32(u[1][xi]) << 16);
            }
#pragma unroll
            for (int xi = 0; xi < wn::XI; ++xi)
                uf[xi][cs] = u32x4{packed[xi][0], packed[xi][1], packed[xi][2], packed[xi][3]};
        }
    }
    // bias of the lane's accumulator rows: channels k0 + 16kg + 4(lane >> 4) + i
    const int kq = k0 + 16 * kg + 4 * (lane >> 4);
    const bool kq_ok = kq < a.ngemm;  // ngemm % 16 == 0: all four or none
    float bias_v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) bias_v[i] = (a.bias && kq_ok) ? E::to_f32(((const elem *)a.bias)[kq + i]) : 0.0f;

    // ---- batches: b -> image n, tile row tr (output rows 2tr, 2tr+1),
    // segment ts (output columns 64ts ..).  With a grid that is a multiple of
    // 8, the workgroups of one XCD (blockIdx.x % 8) take consecutive batches,
    // whose input windows overlap by two rows, so the overlap hits that
    // XCD's L2.
    const int G = gridDim.x;
    const int L = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int per_img = a.tile_rows * a.tiles_q;
    const size_t img_in = (size_t)a.H * a.W * wn::CIN, img_out = (size_t)a.P * a.Q * a.ngemm;

    // transform thread: tile tt, channels 4jc .. 4jc+3
    const int tt = tid >> 4, jc = tid & 15;
    // V row (point xi, tile t) at (xi*TB + t)*VROW; logical 16-byte chunk
    // ch of tile t stored at chunk ch ^ ((t >> 1) & 7)
    const int vw_off = tt * wn::VROW + (((jc >> 1) ^ ((tt >> 1) & 7)) << 4) + (jc & 1) * 8;
    const int tm = 16 * tg + (lane & 15);  // the MFMA lane's tile
    const int vr_off = tm * wn::VROW;
    const int vr_swz = (tm >> 1) & 7;

    // ---- input window of batch bb (thread: tile tt, channels 4jc..): 16
    // 8-byte loads into raw, issued one batch ahead so that their latency
    // overlaps the previous batch's MFMAs and epilogue
    uint2 raw[4][4];
    auto load_windows = [&](int bb) {
        const int n = bb / per_img, rem = bb - n * per_img;
        const int tr = rem / a.tiles_q, ts = rem - tr * a.tiles_q;
        const int p0 = 2 * tr, q0 = 64 * ts;
        const __amdgpu_buffer_rsrc_t src_rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const elem *)a.src + (size_t)n * img_in), (short)0, (int)(img_in * sizeof(elem)), 0x00020000);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = p0 - a.pad_h + i;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int w = q0 + 2 * tt - a.pad_w + j;
                const bool ok = (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W;
                const uint32_t off = ok ? (uint32_t)(((h * a.W + w) * wn::CIN + 4 * jc) * (int)sizeof(elem)) : kBufOOB;
                raw[i][j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(src_rs, off, 0, 0));
            }
        }
    };
    // ---- V = B^T d B of this thread's tile and 4 channels, into buffer vb:
    // two channels at a time in fp32, each pair rounded once by one packed
    // conversion.  B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1].
    auto transform = [&](unsigned char *vb) {
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
            float v[2][wn::XI];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float d[4][4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        d[i][j] = E::to_f32((elem)(((hp ? raw[i][j].y : raw[i][j].x) >> (16 * e)) & 0xffffu));
                float t[4][4];  // B^T d
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    t[0][j] = d[0][j] - d[2][j];
                    t[1][j] = d[1][j] + d[2][j];
                    t[2][j] = d[2][j] - d[1][j];
                    t[3][j] = d[1][j] - d[3][j];
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {  // (B^T d) B
                    v[e][4 * r + 0] = t[r][0] - t[r][2];
                    v[e][4 * r + 1] = t[r][1] + t[r][2];
                    v[e][4 * r + 2] = t[r][2] - t[r][1];
                    v[e][4 * r + 3] = t[r][1] - t[r][3];
                }
            }
#pragma unroll
            for (int xi = 0; xi < wn::XI; ++xi)
                *(uint32_t *)(vb + xi * wn::TB * wn::VROW + vw_off + 4 * hp) = Pack2<E>::cvt(f2v{v[0][xi], v[1][xi]});
        }
    };
    if (L < a.batches) {
        load_windows(L);
        transform(vbuf);
        if (L + G < a.batches) load_windows(L + G);
    }
    __syncthreads();  // the first batch's V is complete

    for (int b = L, it = 0; b < a.batches; b += G, ++it) {
        const int n = b / per_img, rem = b - n * per_img;
        const int tr = rem / a.tiles_q, ts = rem - tr * a.tiles_q;
        const int p0 = 2 * tr, q0 = 64 * ts;

        // the next batch's V into the other buffer, then this batch's MFMAs
        if (b + G < a.batches) {
            transform(vbuf + ((it + 1) & 1) * wn::V_BYTES);
            if (b + 2 * G < a.batches) load_windows(b + 2 * G);  // raw is free again
        }
        const unsigned char *vcur = vbuf + (it & 1) * wn::V_BYTES;

        // ---- 16 GEMMs: M_xi [16 channels x 16 tiles] over 64 input channels
        f32x4 acc[wn::XI];
#pragma unroll
        for (int xi = 0; xi < wn::XI; ++xi) {
            acc[xi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
                const int ch = ((4 * cs + (lane >> 4)) ^ vr_swz) << 4;
                const u32x4 vf = *(const u32x4 *)(vcur + xi * wn::TB * wn::VROW + vr_off + ch);
                acc[xi] = E::mfma(uf[xi][cs], vf, acc[xi]);
            }
        }

        // ---- Y = A^T M A, A^T = [1 1 1 0; 0 1 -1 -1]; + bias, ReLU, round
        const __amdgpu_buffer_rsrc_t dst_rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((elem *)a.dst + (size_t)n * img_out), (short)0, (int)(img_out * sizeof(elem)), 0x00020000);
        float y[2][2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float rr[2][4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                rr[0][c] = acc[c][i] + acc[4 + c][i] + acc[8 + c][i];
                rr[1][c] = acc[4 + c][i] - acc[8 + c][i] - acc[12 + c][i];
            }
#pragma unroll
            for (int yy = 0; yy < 2; ++yy) {
                y[yy][0][i] = rr[yy][0] + rr[yy][1] + rr[yy][2] + bias_v[i];
                y[yy][1][i] = rr[yy][1] - rr[yy][2] - rr[yy][3] + bias_v[i];
            }
        }
        auto store = [&](auto relu_c) {
            constexpr bool RELU = decltype(relu_c)::value;
#pragma unroll
            for (int yy = 0; yy < 2; ++yy)
#pragma unroll
                for (int xx = 0; xx < 2; ++xx) {
                    const int p = p0 + yy, q = q0 + 2 * tm + xx;
                    const bool ok = kq_ok && p < a.P && q < a.Q;
                    const uint2 v{out_pair<E, RELU>(y[yy][xx][0], y[yy][xx][1]),
                                  out_pair<E, RELU>(y[yy][xx][2], y[yy][xx][3])};
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(v2u32, v), dst_rs,
                        ok ? (uint32_t)(((p * a.Q + q) * a.ngemm + kq) * (int)sizeof(elem)) : kBufOOB, 0, 0);
                }
        };
        if (a.relu)
            store(BoolConst<true>{});
        else
            store(BoolConst<false>{});
        // the next batch's V is complete; this batch's buffer is free for the
        // batch after next
        __syncthreads();
    }
}

// fp16 only: with bf16's 8-bit significand, the one rounding of U and V
// before the products leaves rms_scaled near 4e-3 on Gaussian data, above the
// 1e-3 every other path meets, so bf16 problems are not offered this tile.
bool wino_supported(int dtype, int R, int S, int cin, int dil)
{
    return dtype == CONV2D_DTYPE_F16 && R == 3 && S == 3 && dil == 1 && cin == wn::CIN;
}

hipError_t launch_wino_fprop(int dtype, const WinoArgs &a, int grid_x, hipStream_t st)
{
    dim3 grid((unsigned)grid_x, (unsigned)((a.ngemm + wn::BK - 1) / wn::BK));
    const unsigned fblocks = (unsigned)((a.ngemm * wn::CIN + 255) / 256);
    switch (dtype) {
    case CONV2D_DTYPE_F16:
        if (a.u) {
            wino_dgrad_filter_kernel<EF16><<<fblocks, 256, 0, st>>>(a.w, a.u, a.ngemm);
            wino_fprop_kernel<EF16, true><<<grid, wn::NT, 0, st>>>(a);
        } else {
            wino_fprop_kernel<EF16, false><<<grid, wn::NT, 0, st>>>(a);
        }
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cnv

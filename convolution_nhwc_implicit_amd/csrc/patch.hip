// patch.hip -- implicit-GEMM fprop with the workgroup's whole input patch
// resident in LDS (gfx950), for strided and dilated filters.
//
// y[n,p,q,k] = sum over taps (r,s) and channels c of
//   x[n, p*sh - ph + r*dh, q*sw - pw + s*dw, c] * w[k,r,s,c]
// (the definition on the CUTLASS Conv2d notebook's fprop example and the
// tensorcore Conv2D page's "Surface").  Along each axis the input rows a
// convolution touches lie on a lattice: with g = gcd(stride, dilation),
// row = p*stride + r*dil - pad is always -pad plus a multiple of g.  Indexing
// the lattice (lattice row i <-> input row g*i - pad), the convolution is one
// with stride s/g and dilation d/g on it; for stride 2 and dilation 2 it is a
// stride-1, dilation-1 convolution over the even input pixels.
//
// A workgroup owns TP x TQ output pixels (at most 128: four blocks of 32
// pixels) of one image and BN = 32*NB output channels.  The lattice pixels
// its taps read (PH x PW of them, with all C channels) arrive once, by
// direct-to-LDS loads, at a pitch of an odd number of 16-byte slots per pixel
// so that 16 consecutive pixels of a fragment read fall on 16 different
// 16-byte bank groups; pixels outside the image read as zeros through the
// buffer range check.  Every filter tap is then an address shift into this
// patch: the generic implicit GEMM's per-tap re-gather of the input through
// L2 (25 reads of each input pixel for a 5x5 filter) becomes one read.
//
// The reduction (taps x channels, in steps of 16 channels) is split four
// ways: wave w (one per SIMD) takes the steps j = w (mod 4) and holds the
// whole 128 x BN tile as 4 x NB accumulator blocks of 32x32x16 MFMAs (fp32).
// Each wave streams the filter rows of its own steps through a private ring
// of NSB stages (direct-to-LDS loads NSB-1 steps ahead, no workgroup barrier
// in the main loop) and reads the next step's fragments during the current
// step's MFMAs.  At the end the four waves' partial tiles are added through
// LDS in a fixed order (wave 0 + wave 1 + wave 2 + wave 3), so the result
// does not depend on timing; wave w keeps pixel block w, adds the bias,
// applies ReLU, rounds once to the output type and stores whole 16-byte
// pieces of output rows.
#include "device_common.h"

namespace cnv {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <class E>
struct PkMfma;
template <>
struct PkMfma<EF16> {
    __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                       0, 0, 0);
    }
};
template <>
struct PkMfma<EBF16> {
    __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                        c, 0, 0, 0);
    }
};

namespace pk {
constexpr int NT = 256;         // four waves, one per SIMD
constexpr int WAVES = 4;
constexpr int MB = 4;           // pixel blocks of 32 per workgroup
// filter ring stages per wave: about 24 KB of filter rows, 3 to 8 stages
constexpr int ring_stages(int nb, int u)
{
    const int s = 24 / (nb * u);
    return s < 3 ? 3 : s > 8 ? 8 : s;
}
constexpr int LDS_BYTES = 160 * 1024;

template <int V>
struct IntC {
    static constexpr int value = V;
};
template <int B, int E, class F>
__device__ __attribute__((always_inline)) inline void static_for(F &&f)
{
    if constexpr (B < E) {
        f(IntC<B>{});
        static_for<B + 1, E>(f);
    }
}
}  // namespace pk

int patch_ring_bytes(int nb, int u) { return pk::WAVES * pk::ring_stages(nb, u) * nb * u * 1024; }
int patch_lds_bytes() { return pk::LDS_BYTES; }

template <class E, int NB, int U>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void patch_fprop_kernel(const PatchArgs a)
{
    using namespace pk;
    using elem = typename E::elem;
    constexpr int BN = 32 * NB;
    constexpr int NSB = ring_stages(NB, U);
    constexpr int RING = WAVES * NSB * NB * U * 1024;
    constexpr int STAGE_B = NB * U * 1024;  // one super-step of filter rows: BN rows x 16*U channels
    constexpr int SWS = U == 1 ? 3 : U == 2 ? 2 : 1;
    static_assert(U == 1 || U == 2 || U == 4, "super-steps of 1, 2 or 4 channel steps");
    static_assert(12 * NB * 4096 <= LDS_BYTES, "the parked partial tiles fit in LDS");
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bid = blockIdx.x;
    const int nt = blockIdx.y;
    const int img = bid / a.tiles_img;
    const int t = bid - img * a.tiles_img;
    const int tp = t / a.tiles_q, tq = t - tp * a.tiles_q;
    const int p0 = tp * a.TP, q0 = tq * a.TQ;
    const int i0 = p0 * a.sh1, j0 = q0 * a.sw1;  // lattice row / column of patch pixel (0, 0)
    const int CB = a.C >> 4;                     // 16-channel steps per tap
    const int RS = a.R * a.S;
    const int nsuper = RS * CB / U;
    const int nss = (nsuper - wave + WAVES - 1) / WAVES;  // this wave's super-steps J = wave + 4*I

    // the bias values this lane adds in the epilogue, loaded now so that
    // their latency hides behind the main loop
    float bias_v[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        bias_v[nb] = a.bias ? E::to_f32(((const elem *)a.bias)[nt * BN + nb * 32 + (lane & 31)]) : 0.0f;

    const uint32_t lds0 = lds_addr(smem);
    const uint32_t patch_lds = lds0 + RING;
    const uint32_t ring_lds = lds0 + (uint32_t)(wave * NSB * STAGE_B);

    // ---- the patch: slot z (16 bytes) = chunk z % PP of lattice pixel z / PP
    const u32x4 x_rs = make_buf_rsrc((const elem *)a.src + (size_t)img * a.H * a.W * a.C,
                                     (uint32_t)((size_t)a.H * a.W * a.C * sizeof(elem)));
    {
        const int nblk = (a.patch_slots + 63) >> 6;
        const int cpp = a.C >> 3;  // 16-byte chunks of a pixel
        for (int b = wave; b < nblk; b += WAVES) {
            const int z = b * 64 + lane;
            const int pix = (int)fdiv((uint32_t)z, a.div_pp), ch = z - pix * a.PP;
            const int pi = (int)fdiv((uint32_t)pix, a.div_pw), pj = pix - pi * a.PW;
            const int h = a.gh * (i0 + pi) - a.pad_h, w = a.gw * (j0 + pj) - a.pad_w;
            const bool in = z < a.patch_slots && ch < cpp && (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W;
            dma16(x_rs, patch_lds + (uint32_t)(b * 1024),
                  in ? (uint32_t)(h * a.W + w) * (uint32_t)(a.C * (int)sizeof(elem)) + (uint32_t)(ch * 16) : kBufOOB);
        }
    }

    // ---- this wave's filter ring.  The reduction runs in super-steps of U
    // consecutive 16-channel steps of one tap (U divides C/16), so that a
    // super-step's filter rows are 32*U contiguous bytes each; wave w takes
    // the super-steps J = w (mod 4).  Super-step I of the wave sits in stage
    // I % NSB: NB blocks of 32 filter rows x 2U chunks, chunk c of row n at
    // slot 2U*n + (c ^ swz(n)), so that the 16 lanes of a fragment read hit
    // 16 different 16-byte bank groups.  Each block arrives as U
    // direct-to-LDS loads of 32/U rows.
    const u32x4 w_rs = make_buf_rsrc((const elem *)a.filt + (size_t)nt * BN * RS * a.C,
                                     (uint32_t)((size_t)BN * RS * a.C * sizeof(elem)));
    auto swz = [](int n) { return (n >> SWS) & (2 * U - 1); };
    uint32_t dl_off[U];  // per load h of a block: this lane's row and chunk
#pragma unroll
    for (int h = 0; h < U; ++h) {
        const int n = h * (32 / U) + lane / (2 * U);
        const int c = (lane % (2 * U)) ^ swz(n);
        dl_off[h] = (uint32_t)((n * RS * a.C + c * 8) * (int)sizeof(elem));
    }
    const uint32_t dblk_off = (uint32_t)(32 * RS * a.C * (int)sizeof(elem));
    // DMA cursor: super-step index, its tap and first channel step
    int d_i = 0, d_tap = 0, d_cb = wave * U;
    while (d_cb >= CB) {
        d_cb -= CB;
        ++d_tap;
    }
    auto dma_super = [&]() __attribute__((always_inline)) {
        const uint32_t st = ring_lds + (uint32_t)((d_i % NSB) * STAGE_B);
        const bool in = d_i < nss;
        const uint32_t base = (uint32_t)((d_tap * a.C + d_cb * 16) * (int)sizeof(elem));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int h = 0; h < U; ++h)
                dma16(w_rs, st + (nb * U + h) * 1024, in ? base + dl_off[h] + nb * dblk_off : kBufOOB);
        ++d_i;
        d_cb += WAVES * U;
        while (d_cb >= CB) {
            d_cb -= CB;
            ++d_tap;
        }
    };
#pragma unroll 1
    for (int k = 0; k < NSB - 1; ++k) dma_super();

    // ---- fragment addresses.  A (pixels): lane L reads 8 channels
    // (chunk L/32 of the step) of pixel L%32 of its block; B (filter rows):
    // lane L reads chunk 2u + L/32 of filter row L%32 of each block.
    typedef __attribute__((address_space(3))) unsigned char lds_u8;
    const lds_u8 *const lds_base = (const lds_u8 *)smem;
    int a_off[MB];
    const int npix = a.TP * a.TQ;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = mb * 32 + (lane & 31);
        int pix = 0;
        if (m < npix) {
            const int pr = (int)fdiv((uint32_t)m, a.div_tq), pq = m - pr * a.TQ;
            pix = pr * a.sh1 * a.PW + pq * a.sw1;
        }
        a_off[mb] = RING + pix * a.PP * 16 + (lane >> 5) * 16;
    }
    int b_off[U];
    {
        const int n = lane & 31;
#pragma unroll
        for (int u = 0; u < U; ++u)
            b_off[u] = wave * NSB * STAGE_B + (2 * U * n + ((2 * u + (lane >> 5)) ^ swz(n))) * 16;
    }

    // read cursor: super-step I's tap (r, s) and first channel step
    int r_i = 0, r_r = 0, r_s = 0, r_cb = wave * U;
    while (r_cb >= CB) {
        r_cb -= CB;
        if (++r_s == a.S) {
            r_s = 0;
            ++r_r;
        }
    }
    const int tap_rb = a.dh1 * a.PW * a.PP * 16, tap_sb = a.dw1 * a.PP * 16;
    typedef u32x4 Frag[MB + NB];
    // step u of the current super-step; the cursor moves on after u = U-1
    auto read_step = [&](Frag &f, auto u_c) __attribute__((always_inline)) {
        constexpr int UU = decltype(u_c)::value;
        const int toff = r_r * tap_rb + r_s * tap_sb + (r_cb + UU) * 32;
        const int soff = (r_i % NSB) * STAGE_B;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            f[mb] = *(const __attribute__((address_space(3))) u32x4 *)(lds_base + a_off[mb] + toff);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            f[MB + nb] =
                *(const __attribute__((address_space(3))) u32x4 *)(lds_base + b_off[UU] + soff + nb * U * 1024);
        if constexpr (UU == U - 1) {
            ++r_i;
            r_cb += WAVES * U;
            while (r_cb >= CB) {
                r_cb -= CB;
                if (++r_s == a.S) {
                    r_s = 0;
                    ++r_r;
                }
            }
        }
    };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};
    auto mfma_step = [&](const Frag &f) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = PkMfma<E>::run(f[mb], f[MB + nb], acc[mb][nb]);
    };

    // the patch (issued before the ring's first stages) has landed once at
    // most the ring's loads are outstanding; then every wave's share is visible
    wait_vm_n<(NSB - 1) * NB * U>();
    __syncthreads();

    // Step t of the wave (super-step t / U, step u = t % U) is computed from
    // one fragment set while step t + 1 is read into the other.  Before the
    // read of a super-step's first step, its loads are waited for; after the
    // MFMAs of a super-step's first step, the loads of super-step I + NSB - 1
    // go to the stage super-step I - 1 used, whose fragments are consumed.
    constexpr int WAITN = (U == 1 ? NSB - 3 : NSB - 2) * NB * U;
    Frag f0, f1;
    wait_vm_n<(NSB - 2) * NB * U>();
    read_step(f0, IntC<0>{});
    const int ns = nss * U;  // this wave's steps
    constexpr int BODY = U == 1 ? 2 : U;
    int t0 = 0;
    auto one = [&](Frag &cur, Frag &nxt, auto b_c, bool live) __attribute__((always_inline)) {
        constexpr int BB = decltype(b_c)::value;
        constexpr int UU = BB % U;
        if constexpr (UU == U - 1) wait_vm_n<WAITN>();
        read_step(nxt, IntC<(UU + 1) % U>{});
        if (live) mfma_step(cur);
        if constexpr (UU == 0) dma_super();
    };
#pragma unroll 1
    for (; t0 + BODY < ns; t0 += BODY) {
        static_for<0, BODY>([&](auto b_c) __attribute__((always_inline)) {
            constexpr int BB = decltype(b_c)::value;
            if constexpr (BB % 2 == 0)
                one(f0, f1, b_c, true);
            else
                one(f1, f0, b_c, true);
        });
    }
    // the last BODY steps or fewer (every wave has at least one unless ns == 0)
    static_for<0, BODY>([&](auto b_c) __attribute__((always_inline)) {
        constexpr int BB = decltype(b_c)::value;
        if (t0 + BB < ns) {
            if constexpr (BB % 2 == 0)
                mfma_step(f0);
            else
                mfma_step(f1);
        }
        if constexpr (BB + 1 < BODY) {
            if (t0 + BB + 1 < ns) {
                if constexpr ((BB + 1) % U == 0) wait_vm_n<0>();
                if constexpr (BB % 2 == 0)
                    read_step(f1, IntC<(BB + 1) % U>{});
                else
                    read_step(f0, IntC<(BB + 1) % U>{});
            }
        }
    });

    // ---- the four waves' partial tiles, added in wave order through LDS.
    // Wave w keeps pixel block w; it parks its other blocks in slot
    // (block, source wave) = 3*block + (w < block ? w : w - 1).  A parked
    // 32x32 block is [4][64 lanes] of 16-byte pieces.
    wait_vm_all();
    __syncthreads();
    f32x4 *const park = (f32x4 *)smem + lane;
    auto slot_of = [](int blk, int src) { return 3 * blk + (src < blk ? src : src - 1); };
    static_for<0, MB>([&](auto mb_c) __attribute__((always_inline)) {
        constexpr int MBC = decltype(mb_c)::value;
        if (wave != MBC) {
            const int sl = slot_of(MBC, wave);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16 &v = acc[MBC][nb];
                    park[((sl * NB + nb) * 4 + q) * 64] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
                }
        }
    });
    __syncthreads();
    f32x16 tot[NB];
    static_for<0, MB>([&](auto mb_c) __attribute__((always_inline)) {
        constexpr int MBC = decltype(mb_c)::value;
        if (wave == MBC) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                static_for<0, WAVES>([&](auto src_c) __attribute__((always_inline)) {
                    constexpr int SRC = decltype(src_c)::value;
                    f32x16 v;
                    if constexpr (SRC == MBC) {
                        v = acc[MBC][nb];
                    } else {
                        const int sl = 3 * MBC + (SRC < MBC ? SRC : SRC - 1);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const f32x4 u = park[((sl * NB + nb) * 4 + q) * 64];
                            v[4 * q] = u[0];
                            v[4 * q + 1] = u[1];
                            v[4 * q + 2] = u[2];
                            v[4 * q + 3] = u[3];
                        }
                    }
                    if constexpr (SRC == 0)
                        tot[nb] = v;
                    else
                        tot[nb] += v;
                });
            }
        }
    });
    __syncthreads();  // every wave is done with the parked blocks

    // ---- epilogue: bias, ReLU, one rounding; staged per wave as 32 rows of
    // BN values (row pitch BN*2 + 16 bytes), then stored as 16-byte pieces
    constexpr int ROWB = BN * 2 + 16;
    unsigned char *const stage = smem + wave * 32 * ROWB;
    const int n_l = lane & 31;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float bv = bias_v[nb];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int m = 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            const float v = bias_relu_f32(tot[nb][j], bv, a.relu);
            *(elem *)(stage + m * ROWB + (nb * 32 + n_l) * 2) = E::from_f32(v);
        }
    }
    constexpr int CPR = BN / 8;  // 16-byte pieces per staged row
#pragma unroll
    for (int u = 0; u < 32 * CPR / 64; ++u) {
        const int idx = u * 64 + lane;
        const int row = idx / CPR, ch = idx - row * CPR;
        const int m = wave * 32 + row;
        if (m < npix) {
            const int pr = (int)fdiv((uint32_t)m, a.div_tq), pq = m - pr * a.TQ;
            const int p = p0 + pr, q = q0 + pq;
            if (p < a.P && q < a.Q) {
                const u32x4 v = *(const u32x4 *)(stage + row * ROWB + ch * 16);
                elem *dst = (elem *)a.dst + ((size_t)(img * a.P + p) * a.Q + q) * a.K + nt * BN + ch * 8;
                __builtin_nontemporal_store(v, (u32x4 *)dst);
            }
        }
    }
}

hipError_t launch_patch_fprop(int dtype, int nb, int u, const PatchArgs &a, hipStream_t st)
{
    dim3 grid((unsigned)(a.N * a.tiles_img), (unsigned)(a.K / (32 * nb)));
#define PK_LAUNCH(E_, NB_, U_) patch_fprop_kernel<E_, NB_, U_><<<grid, pk::NT, 0, st>>>(a)
#define PK_U(E_, NB_)                          \
    do {                                       \
        if (u == 1) PK_LAUNCH(E_, NB_, 1);     \
        else if (u == 2) PK_LAUNCH(E_, NB_, 2); \
        else PK_LAUNCH(E_, NB_, 4);            \
    } while (0)
#define PK_NB(E_)                   \
    do {                            \
        if (nb == 1) PK_U(E_, 1);   \
        else if (nb == 2) PK_U(E_, 2); \
        else PK_U(E_, 3);           \
    } while (0)
    if (u != 1 && u != 2 && u != 4) return hipErrorInvalidValue;
    if (dtype == CONV2D_DTYPE_F16)
        PK_NB(EF16);
    else if (dtype == CONV2D_DTYPE_BF16)
        PK_NB(EBF16);
    else
        return hipErrorInvalidValue;
#undef PK_NB
#undef PK_U
#undef PK_LAUNCH
    return hipGetLastError();
}

}  // namespace cnv

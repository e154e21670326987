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
//
// dgrad (DG) runs the same kernel when the stride divides the dilation on
// each axis.  dx[h] = sum over taps r of dy[p] w[r] with p*s - pad + r*d = h
// then has solutions only for h = -pad (mod s), and on those rows
// (h = h0 + s*a) it is a stride-1 correlation of dy with the filter's taps
// reversed, its two channel axes swapped, dilation d/s and padding
// (R-1)*d/s - (h0+pad)/s.  The filter rows (16*U dy channels of one tap,
// the workgroup's dx channels contiguous) stream through the rings as they
// lie in w and come out of LDS transposed by ds_read_b64_tr_b16.  The
// workgroup also writes the zeros of the dx rows and columns between its
// lattice rows and columns, so that every dx element is written once.
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

int patch_ring_stages(int nb, int u) { return pk::ring_stages(nb, u); }
int patch_lds_bytes() { return pk::LDS_BYTES; }

template <class E, int NB, int U, bool DG, int NSB, int MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void patch_kernel(const PatchArgs a)
{
    using namespace pk;
    static_assert(MB == 2 || MB == 4, "two or four pixel blocks of 32 per workgroup");
    using elem = typename E::elem;
    constexpr int BN = 32 * NB;
    static_assert(NSB >= 3 && (NSB - 1) * NB * U < 64, "ring depth within the load counter's range");
    constexpr int RING = WAVES * NSB * NB * U * 1024;
    constexpr int STAGE_B = NB * U * 1024;  // one super-step of filter rows: BN rows x 16*U channels
    constexpr int SWS = U == 1 ? 3 : U == 2 ? 2 : 1;
    static_assert(U == 1 || U == 2 || U == 4, "super-steps of 1, 2 or 4 channel steps");
    static_assert(3 * MB * NB * 4096 <= LDS_BYTES, "the parked partial tiles fit in LDS");
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
    const int CB = a.SC >> 4;                    // 16-channel steps per tap
    const int nsuper = a.R * a.S * CB / U;
    const int nss = (nsuper - wave + WAVES - 1) / WAVES;  // this wave's super-steps J = wave + 4*I

    // the bias values this lane adds in the epilogue, loaded now so that
    // their latency hides behind the main loop
    float bias_v[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        bias_v[nb] = (!DG && a.bias) ? E::to_f32(((const elem *)a.bias)[nt * BN + nb * 32 + (lane & 31)]) : 0.0f;

    const uint32_t lds0 = lds_addr(smem);
    const uint32_t patch_lds = lds0 + RING;
    const uint32_t ring_lds = lds0 + (uint32_t)(wave * NSB * STAGE_B);

    // ---- the patch: slot z (16 bytes) = chunk z % PP of lattice pixel z / PP
    const u32x4 x_rs = make_buf_rsrc((const elem *)a.src + (size_t)img * a.H * a.W * a.SC,
                                     (uint32_t)((size_t)a.H * a.W * a.SC * sizeof(elem)));
    {
        const int nblk = (a.patch_slots + 63) >> 6;
        const int cpp = a.SC >> 3;  // 16-byte chunks of a pixel
        for (int b = wave; b < nblk; b += WAVES) {
            const int z = b * 64 + lane;
            const int pix = (int)fdiv((uint32_t)z, a.div_pp), ch = z - pix * a.PP;
            const int pi = (int)fdiv((uint32_t)pix, a.div_pw), pj = pix - pi * a.PW;
            const int h = a.gh * (i0 + pi) - a.pad_h, w = a.gw * (j0 + pj) - a.pad_w;
            const bool in = z < a.patch_slots && ch < cpp && (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W;
            dma16(x_rs, patch_lds + (uint32_t)(b * 1024),
                  in ? (uint32_t)(h * a.W + w) * (uint32_t)(a.SC * (int)sizeof(elem)) + (uint32_t)(ch * 16) : kBufOOB);
        }
    }

    // ---- this wave's filter ring.  The reduction runs in super-steps of U
    // consecutive 16-channel steps of one tap (U divides SC/16), so that a
    // super-step's filter rows are long contiguous pieces; wave w takes the
    // super-steps J = w (mod 4), super-step I of the wave in stage I % NSB.
    // fprop: NB blocks of 32 filter rows (output channels) x 2U chunks,
    //   chunk c of row n at slot 2U*n + (c ^ swz(n)), so that the 16 lanes of
    //   a fragment read hit 16 different 16-byte bank groups; each block
    //   arrives as U direct-to-LDS loads of 32/U rows.
    // dgrad: 16*U rows (dy channels) of BN dx channels as they lie in w,
    //   chunk c of row k at position c ^ swzb(k) (BN = 64: rows 128 bytes
    //   apart would put rows k and k + 2 on the same banks), read with
    //   ds_read_b64_tr_b16; slot z of the stage is filled by lane z % 64 of
    //   load z / 64.
    const int RS = a.R * a.S;
    const u32x4 w_rs = DG ? make_buf_rsrc((const elem *)a.filt + (size_t)nt * BN,
                                          (uint32_t)(((size_t)a.SC * RS * a.OC - (size_t)nt * BN) * sizeof(elem)))
                          : make_buf_rsrc((const elem *)a.filt + (size_t)nt * BN * RS * a.SC,
                                          (uint32_t)((size_t)BN * RS * a.SC * sizeof(elem)));
    auto swz = [](int n) { return (n >> SWS) & (2 * U - 1); };
    auto swzb = [](int k) { return BN == 64 ? ((k >> 1) & 1) * 4 : 0; };
    constexpr int NLD = NB * U;  // loads per super-step
    uint32_t dl_off[NLD];        // per load: this lane's row and chunk
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
        if constexpr (DG) {
            const int z = j * 64 + lane;
            const int k = z / (BN / 8), c = (z % (BN / 8)) ^ swzb(z / (BN / 8));
            dl_off[j] = (uint32_t)((k * RS * a.OC + c * 8) * (int)sizeof(elem));
        } else {
            const int nb = j / U, h = j % U;
            const int n = h * (32 / U) + lane / (2 * U);
            const int c = (lane % (2 * U)) ^ swz(n);
            dl_off[j] = (uint32_t)(((nb * 32 + n) * RS * a.SC + c * 8) * (int)sizeof(elem));
        }
    }
    // DMA cursor: super-step index, its tap and first channel step
    int d_i = 0, d_tap = 0, d_cb = wave * U;
    while (d_cb >= CB) {
        d_cb -= CB;
        ++d_tap;
    }
    auto dma_super = [&]() __attribute__((always_inline)) {
        const uint32_t st = ring_lds + (uint32_t)((d_i % NSB) * STAGE_B);
        const bool in = d_i < nss;
        // dgrad: dy channels 16*d_cb.. of the tap reversed in both axes
        const uint32_t base =
            DG ? (uint32_t)((d_cb * 16 * RS * a.OC + (RS - 1 - d_tap) * a.OC) * (int)sizeof(elem))
               : (uint32_t)((d_tap * a.SC + d_cb * 16) * (int)sizeof(elem));
#pragma unroll
        for (int j = 0; j < NLD; ++j) dma16(w_rs, st + j * 1024, in ? base + dl_off[j] : kBufOOB);
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
    // fprop: per step u of a super-step; dgrad: per 32-column block (the
    // row of read rd of step u is 16u + 4rd past it)
    constexpr int NBO = DG ? NB : U;
    int b_off[NBO];
    if constexpr (DG) {
        const int L = lane & 15;
        const int k0 = 8 * (lane >> 5) + (L >> 2);
        const int c0 = 16 * ((lane >> 4) & 1) + 4 * (L & 3);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            b_off[nb] = wave * NSB * STAGE_B + k0 * (BN * 2) + (((nb * 32 + c0) / 8) ^ swzb(k0)) * 16 + (c0 % 8) * 2;
    } else {
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
        for (int nb = 0; nb < NB; ++nb) {
            if constexpr (DG) {
                typedef short s16x4 __attribute__((ext_vector_type(4)));
                auto tr = [&](int off) {
                    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                         (__attribute__((address_space(3))) s16x4 *)(lds_base + off)));
                };
                const uint2 lo = tr(b_off[nb] + soff + (16 * UU) * (BN * 2));
                const uint2 hi = tr(b_off[nb] + soff + (16 * UU + 4) * (BN * 2));
                f[MB + nb] = u32x4{lo.x, lo.y, hi.x, hi.y};
            } else {
                f[MB + nb] =
                    *(const __attribute__((address_space(3))) u32x4 *)(lds_base + b_off[UU] + soff + nb * U * 1024);
            }
        }
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
    // the last BODY steps or fewer: a step past the wave's last computes with
    // zero fragments (adding exact zeros), so that no MFMA is conditional
    // (a branch around MFMAs makes the compiler keep the accumulators in
    // memory across it)
    static_for<0, BODY>([&](auto b_c) __attribute__((always_inline)) {
        constexpr int BB = decltype(b_c)::value;
        Frag &cur = BB % 2 == 0 ? f0 : f1;
        if (t0 + BB >= ns) {
#pragma unroll
            for (int k = 0; k < MB + NB; ++k) cur[k] = u32x4{0, 0, 0, 0};
        }
        mfma_step(cur);
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
    // Block (mb, nb) of the tile is owned by wave (nb % (4/MB))*MB + mb (MB =
    // 4: wave w owns pixel block w; MB = 2: waves 0 and 1 own the even
    // channel blocks of pixel blocks 0 and 1, waves 2 and 3 the odd ones).
    // The other waves park their partial of it in slot 3*(mb*NB + nb) +
    // (src < owner ? src : src - 1); the owner adds the four partials in
    // wave order.  A parked 32x32 block is [4][64 lanes] of 16-byte pieces.
    wait_vm_all();
    __syncthreads();
    f32x4 *const park = (f32x4 *)smem + lane;
    constexpr int NSPLIT = WAVES / MB;
    static_for<0, MB * NB>([&](auto b_c) __attribute__((always_inline)) {
        constexpr int BB = decltype(b_c)::value, MBC = BB / NB, NBC = BB % NB;
        constexpr int OWN = (NBC % NSPLIT) * MB + MBC;
        if (wave != OWN) {
            const int sl = 3 * BB + (wave < OWN ? wave : wave - 1);
            const f32x16 &v = acc[MBC][NBC];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                park[(sl * 4 + q) * 64] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        }
    });
    __syncthreads();
    static_for<0, MB * NB>([&](auto b_c) __attribute__((always_inline)) {
        constexpr int BB = decltype(b_c)::value, MBC = BB / NB, NBC = BB % NB;
        constexpr int OWN = (NBC % NSPLIT) * MB + MBC;
        if (wave == OWN) {
            f32x16 s;
            static_for<0, WAVES>([&](auto src_c) __attribute__((always_inline)) {
                constexpr int SRC = decltype(src_c)::value;
                f32x16 v;
                if constexpr (SRC == OWN) {
                    v = acc[MBC][NBC];
                } else {
                    constexpr int SL = 3 * BB + (SRC < OWN ? SRC : SRC - 1);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 u = park[(SL * 4 + q) * 64];
                        v[4 * q] = u[0];
                        v[4 * q + 1] = u[1];
                        v[4 * q + 2] = u[2];
                        v[4 * q + 3] = u[3];
                    }
                }
                if constexpr (SRC == 0)
                    s = v;
                else
                    s += v;
            });
            acc[MBC][NBC] = s;
        }
    });
    __syncthreads();  // every wave is done with the parked blocks

    // ---- epilogue: bias, ReLU, one rounding of the wave's own blocks
    // (pixel block wave % MB), staged as 32 rows of BN values (row pitch
    // BN*2 + 16 bytes, each block at its channel offset), then stored as
    // 16-byte pieces of output rows
    constexpr int ROWB = BN * 2 + 16;
    unsigned char *const stage = smem + wave * 32 * ROWB;
    const int n_l = lane & 31;
    const int mb_w = wave % MB;
    static_for<0, MB * NB>([&](auto b_c) __attribute__((always_inline)) {
        constexpr int BB = decltype(b_c)::value, MBC = BB / NB, NBC = BB % NB;
        constexpr int OWN = (NBC % NSPLIT) * MB + MBC;
        if (wave == OWN) {
            // (the empty asm, different in every block, keeps the compiler
            // from merging the blocks' branches into one that indexes the
            // accumulators by the wave number, which would put them in
            // scratch memory)
            asm volatile("; epilogue block %0" ::"n"(BB));
            const float bv = bias_v[NBC];
            static_for<0, 16>([&](auto j_c) __attribute__((always_inline)) {
                constexpr int J = decltype(j_c)::value;
                const int m = 8 * (J >> 2) + 4 * (lane >> 5) + (J & 3);
                const float v = bias_relu_f32(acc[MBC][NBC][J], bv, a.relu);
                *(elem *)(stage + m * ROWB + (NBC * 32 + n_l) * 2) = E::from_f32(v);
            });
        }
    });
    constexpr int CPR = BN / 8;  // 16-byte pieces per staged row
#pragma unroll
    for (int u = 0; u < 32 * CPR / 64; ++u) {
        const int idx = u * 64 + lane;
        const int row = idx / CPR, ch = idx - row * CPR;
        const int m = mb_w * 32 + row;
        const bool mine = MB == 4 || (ch / 4) % NSPLIT == wave / MB;  // the piece's channel block is this wave's
        if (mine && m < npix) {
            const int pr = (int)fdiv((uint32_t)m, a.div_tq), pq = m - pr * a.TQ;
            const int p = p0 + pr, q = q0 + pq;
            if (p < a.P && q < a.Q) {
                const u32x4 v = *(const u32x4 *)(stage + row * ROWB + ch * 16);
                const int oh = a.oh0 + a.ogh * p, ow = a.ow0 + a.ogw * q;
                elem *dst = (elem *)a.dst + ((size_t)(img * a.OH + oh) * a.OW + ow) * a.OC + nt * BN + ch * 8;
                __builtin_nontemporal_store(v, (u32x4 *)dst);
            }
        }
    }
    if constexpr (DG) {
        // zeros of the dx rows and columns of this tile's range that lie off
        // the lattice; the first and last tiles of an axis also take the
        // rows (columns) before the first and after the last lattice row
        if (a.ogh > 1 || a.ogw > 1) {
            const int hlo = tp == 0 ? 0 : a.oh0 + a.ogh * p0;
            const int hhi = p0 + a.TP >= a.P ? a.OH : a.oh0 + a.ogh * (p0 + a.TP);
            const int wlo = tq == 0 ? 0 : a.ow0 + a.ogw * q0;
            const int whi = q0 + a.TQ >= a.Q ? a.OW : a.ow0 + a.ogw * (q0 + a.TQ);
            const int nw = whi - wlo, cpr = BN / 8;
            const int total = (hhi - hlo) * nw * cpr;
            for (int idx = threadIdx.x; idx < total; idx += NT) {
                const int pix = idx / cpr, ch = idx - pix * cpr;
                const int h = hlo + pix / nw, w = wlo + pix % nw;
                const bool on = h >= a.oh0 && (h - a.oh0) % a.ogh == 0 && w >= a.ow0 && (w - a.ow0) % a.ogw == 0;
                if (!on) {
                    elem *dst = (elem *)a.dst + ((size_t)(img * a.OH + h) * a.OW + w) * a.OC + nt * BN + ch * 8;
                    __builtin_nontemporal_store(u32x4{0, 0, 0, 0}, (u32x4 *)dst);
                }
            }
        }
    }
}

template <class E, int NB, int U, bool DG, int NSB, int MB>
static void launch_one(dim3 grid, hipStream_t st, const PatchArgs &a)
{
    patch_kernel<E, NB, U, DG, NSB, MB><<<grid, pk::NT, 0, st>>>(a);
}

template <class E, int NB, int MB>
static void launch_nb(int u, int nsb, bool dgrad, dim3 grid, hipStream_t st, const PatchArgs &a)
{
    if (dgrad) {
        if (nsb == 4)
            launch_one<E, NB, 1, true, 4, MB>(grid, st, a);
        else
            launch_one<E, NB, 1, true, 8, MB>(grid, st, a);
    } else if (u == 1) {
        launch_one<E, NB, 1, false, pk::ring_stages(NB, 1), MB>(grid, st, a);
    } else if (u == 2) {
        launch_one<E, NB, 2, false, pk::ring_stages(NB, 2), MB>(grid, st, a);
    } else {
        launch_one<E, NB, 4, false, pk::ring_stages(NB, 4), MB>(grid, st, a);
    }
}

template <class E>
static void launch_e(int nb, int u, int nsb, int mb, bool dgrad, dim3 grid, hipStream_t st, const PatchArgs &a)
{
    if (mb == 4) {
        if (nb == 1) launch_nb<E, 1, 4>(u, nsb, dgrad, grid, st, a);
        else if (nb == 2) launch_nb<E, 2, 4>(u, nsb, dgrad, grid, st, a);
        else launch_nb<E, 3, 4>(u, nsb, dgrad, grid, st, a);
    } else {
        if (nb == 1) launch_nb<E, 1, 2>(u, nsb, dgrad, grid, st, a);
        else if (nb == 2) launch_nb<E, 2, 2>(u, nsb, dgrad, grid, st, a);
        else launch_nb<E, 3, 2>(u, nsb, dgrad, grid, st, a);
    }
}

// fprop: super-steps of u = 1, 2 or 4 channel steps, ring_stages(nb, u)
// stages; dgrad (filter rows contiguous at any u): u = 1, 4 or 8 stages.
// mb: pixel blocks of 32 per workgroup (2 or 4).
hipError_t launch_patch(int dtype, const PatchArgs &a, bool dgrad, hipStream_t st)
{
    const int nb = a.nb, u = a.u, nsb = a.nsb, mb = a.mb;
    if (nb < 1 || nb > 3 || (mb != 2 && mb != 4)) return hipErrorInvalidValue;
    if (dgrad ? (u != 1 || (nsb != 4 && nsb != 8)) : (u != 1 && u != 2 && u != 4)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(a.N * a.tiles_img), (unsigned)(a.OC / (32 * nb)));
    if (dtype == CONV2D_DTYPE_F16)
        launch_e<EF16>(nb, u, nsb, mb, dgrad, grid, st, a);
    else if (dtype == CONV2D_DTYPE_BF16)
        launch_e<EBF16>(nb, u, nsb, mb, dgrad, grid, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace cnv

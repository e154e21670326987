// band.hip -- stride-1 implicit-GEMM convolution with the filter held in
// registers and a ring of input rows in LDS filled by direct-to-LDS loads
// (gfx950).
//
// For a stride-1 convolution every input pixel feeds R*S output pixels.  This
// kernel keeps a band of input rows in LDS and forms all R*S tap-shifted
// operand fragments from it, so each input byte leaves HBM once per
// workgroup (plus the R-1 halo rows).  A workgroup (8 waves, two per SIMD)
// walks a contiguous range of output rows of one image, four rows per group:
//
//   * GEMM: rows = 32 output channels per wave (the A operand, the filter),
//     columns = 64 output pixels of one row (two 32x32x16 MFMA blocks), K =
//     (tap, channel).  The two waves of an output row take the two 32-channel
//     halves of the workgroup's 64 channels;
//   * the wave's 32 x (R*S*CIN) filter slice lives in VGPRs for the whole
//     kernel, so the only LDS reads in the main loop are the pixel fragments
//     (half of what reading both operands from LDS would cost);
//   * input rows arrive through buffer_load ... lds (no register staging):
//     padding comes from the buffer range check, which returns zeros.  The
//     rows of group g+1 are in flight while group g is computed; a group's
//     slots are refilled with the rows of group g+2 right after its barrier;
//   * results (bias, ReLU and rounding applied) are staged in LDS, over the
//     filter staging area that only the prologue uses, and each wave stores
//     its own results from there as 64-byte half pixels (four lanes each):
//     stores straight from the accumulators would be 8-byte pieces, four
//     times as many memory requests;
//   * the LDS has 64 four-byte banks and serves 16 lanes of a 128-bit read per
//     cycle.  A 128-byte pixel covers half of the banks, so the 16-byte channel
//     chunks of pixel `col` are XOR-swizzled by col/2: any 16 consecutive
//     pixels of a fragment (at any tap shift) then hit all 64 banks.
//
// int8 (the quantised fprop) runs the same data movement: a pixel of 128
// int8 channels is the 128 bytes of 64 fp16 ones, and the 32x32x32 int8 MFMA
// takes 16 bytes a lane like the 32x32x16 fp16 one, so only the MFMA, the
// int32 accumulators (started at the int32 bias) and the epilogue (ReLU,
// requantisation in fp64, 64 bytes per staged pixel) differ.  CIN counts
// 2-byte units.
//
// The same kernel runs stride-1 dgrad (TRANS): the source is dy, the padding
// is dil*(R-1) - pad, and the filter w[K][R][S][C] is read with its taps
// reversed and K and C swapped.  The swap is done while the filter is copied
// from LDS into registers, with the transposing read ds_read_b64_tr_b16, so
// dgrad needs no separate re-layout pass.
#include "device_common.h"

namespace cnv {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <class E>
struct Mfma32;
template <>
struct Mfma32<EF16> {
    using acc = f32x16;
    __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <>
struct Mfma32<EBF16> {
    using acc = f32x16;
    __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <>
struct Mfma32<EI8> {
    using acc = i32x16;
    __device__ static inline i32x16 run(u32x4 a, u32x4 b, i32x16 c)
    {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b),
                                                      c, 0, 0, 0);
    }
};

namespace band {
__device__ inline s16x4 tr16(const unsigned char *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

template <int R, int S, int CIN, int DIL, bool TRANS>
struct BandCfg {
    static constexpr int NT = 512;
    static constexpr int WAVES = NT / 64;
    static constexpr int GR = WAVES / 2;                // output rows per group (two waves each)
    static constexpr int BN = 64;                       // output channels per workgroup
    static constexpr int HALO_R = DIL * (R - 1);
    static constexpr int HALO_S = DIL * (S - 1);
    static constexpr int NSLOT = 2 * GR + HALO_R;       // ring rows: current group + halo + next group
    static constexpr int RCOLS = 64;                    // input columns per ring row
    static constexpr int SEG = RCOLS - HALO_S;          // output columns per workgroup
    static constexpr int NCH = CIN / 8;                 // 16-byte chunks per pixel
    static constexpr int PIXB = CIN * 2;
    static constexpr int SLOTB = RCOLS * PIXB;
    static constexpr int KG = R * S * CIN;              // GEMM-K
    static constexpr int C16 = CIN / 16;                // k16 steps per tap
    static constexpr int KSTEPS = KG / 16;
    static constexpr int PF = 3;                        // pixel-fragment reads in flight (k16 steps)
    // Fragments of the last output columns of a segment read up to HALO_S
    // pixels past a ring row (those outputs are discarded); the tail pad keeps
    // the reads of the last slot inside the ring.
    static constexpr int RING_BYTES = NSLOT * SLOTB + HALO_S * PIXB;
    // Filter staging (prologue only): FROWS rows of FROWE elements plus a pad
    // that makes the fragment reads conflict-free: 16 bytes for the 128-bit
    // reads of fprop (row stride = 36 banks mod 64), 64 bytes for the
    // transposing 64-bit reads of dgrad (48 banks mod 64).
    static constexpr int FROWS = TRANS ? CIN : BN;
    static constexpr int FROWE = R * S * (TRANS ? BN : CIN);
    static constexpr int FROWB = FROWE * 2 + (TRANS ? 64 : 16);
    static constexpr int FROWCH = FROWB / 16;
    static constexpr int FILT_BYTES = FROWS * FROWB;
    static constexpr int FBLOCKS = FROWS * FROWCH / 64;  // 1 KB direct-to-LDS blocks
    // Output staging (after the prologue, over the filter staging): GR rows
    // x RCOLS pixels x BN channels.
    static constexpr int OSTAGE_BYTES = GR * SLOTB;
    static constexpr int STAGE_BYTES = FILT_BYTES > OSTAGE_BYTES ? FILT_BYTES : OSTAGE_BYTES;
    static constexpr int BIAS_BYTES = BN * 4;
    static constexpr int LDS_BYTES = RING_BYTES + STAGE_BYTES + BIAS_BYTES;
    static_assert(CIN == 64 && BN == 64, "pixels of 8 chunks, two 32-channel halves");
    static_assert(BN * 2 == PIXB, "a staged output pixel has the layout of a ring pixel");
    static_assert(RCOLS * NCH == 64 * WAVES, "one 1 KB block of each ring row per wave");
    static_assert(FROWS * FROWCH % 64 == 0, "the filter staging is whole 1 KB blocks");
    static_assert(FROWE == KG, "filter staging rows hold one GEMM-K row");
    static_assert(LDS_BYTES <= 163840, "fits in the 160 KB LDS");
};
}  // namespace band

template <class E, int R, int S, int CIN, int DIL, bool TRANS>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void band_kernel(const BandArgs a)
{
    using C = band::BandCfg<R, S, CIN, DIL, TRANS>;
    using elem = typename E::elem;
    using acc_t = typename Mfma32<E>::acc;
    constexpr bool I8 = E::kDtype == CONV2D_DTYPE_I8;
    static_assert(!(I8 && TRANS), "int8 is fprop only");
    constexpr int EPC16 = 16 / (int)sizeof(elem);  // output channels per 16-byte chunk
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_BYTES];
    unsigned char *ring = smem;
    unsigned char *filt = smem + C::RING_BYTES;    // prologue only
    unsigned char *ostage = smem + C::RING_BYTES;  // after the prologue
    float *bias_s = (float *)(smem + C::RING_BYTES + C::STAGE_BYTES);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
    const int img = blockIdx.x / a.chunks_per_img;
    const int chunk = blockIdx.x - img * a.chunks_per_img;
    const int p_start = chunk * a.rows_per_wg;
    const int p_end = min(p_start + a.rows_per_wg, a.P);
    if (p_start >= p_end) return;  // whole workgroup
    const int nrows = p_end - p_start;
    const int n0 = blockIdx.y * C::BN;
    const int q0 = blockIdx.z * C::SEG;
    const int h_base = p_start - a.pad_h;  // input row of ring row 0
    const int w_base = q0 - a.pad_w;       // input column of ring column 0

    // ---- ring rows by direct-to-LDS loads.  Wave w moves pixels 8w..8w+7 of
    // each row (one 1 KB block); lane i fills stored chunk i%8 of pixel
    // 8w + i/8, i.e. source chunk (i%8) ^ swizzle(pixel).
    const unsigned char *src_img = (const unsigned char *)a.src + (size_t)img * a.H * a.W * C::PIXB;
    const u32x4 src_rs = make_buf_rsrc(src_img, (uint32_t)(a.H * a.W * C::PIXB));
    const unsigned row_bytes = (unsigned)(a.W * CIN * 2);
    auto lane_src = [&](int blk) -> int {  // byte offset in a source row, or -1 past the row
        const int col = 8 * blk + (lane >> 3);
        const int j = (lane & 7) ^ ((col >> 1) & 7);
        const int w = w_base + col;
        return (unsigned)w < (unsigned)a.W ? (w * CIN + j * 8) * 2 : -1;
    };
    const int my_off = lane_src(wave);
    const uint32_t ring0 = lds_addr(ring);  // LDS byte address of the ring
    auto dma_row = [&](int rr, int blk, int off) {
        const int h = h_base + rr;
        const bool ok = off >= 0 && (unsigned)h < (unsigned)a.H;
        dma16(src_rs, ring0 + (uint32_t)((rr % C::NSLOT) * C::SLOTB + blk * 1024),
              ok ? (unsigned)h * row_bytes + (unsigned)off : kBufOOB);
    };
    // group g reads ring rows [g*GR, g*GR + GR + HALO_R); it brings the rows
    // past the previous group's (all of them for g = 0)
    auto group_rows = [&](int g, int &r0, int &r1) {
        r0 = g == 0 ? 0 : g * C::GR + C::HALO_R;
        r1 = min((g + 1) * C::GR + C::HALO_R, nrows + C::HALO_R);
    };
    // The first half of the waves (the "leading waves") are older: they win
    // the MFMA arbitration against the second half (the "trailing waves") on
    // their SIMD and finish each group's MFMAs first.  So the leading waves
    // start a group's MFMAs right after its barrier, and the trailing waves
    // first store the previous group's results and issue the row loads of
    // the group after next (blocks w and w ^ PW of every ring row), which
    // they wait for before the next barrier.
    constexpr int PW = C::WAVES / 2;
    const bool lead = wave < PW;
    const int off2 = lane_src(wave ^ PW);
    auto dma_group = [&](int g) {
        int r0, r1;
        group_rows(g, r0, r1);
        for (int rr = r0; rr < r1; ++rr) {
            dma_row(rr, wave, my_off);
            dma_row(rr, wave ^ PW, off2);
        }
    };

    // ---- prologue: the filter tile, then group 0's rows (every wave a
    // share).  The filter is read into registers as soon as it has landed,
    // while the rows are still on their way.
    int nrow0;
    {
        const int fbytes = (TRANS ? CIN * R * S * a.ngemm : a.ngemm * C::KG) * 2;
        const u32x4 w_rs = make_buf_rsrc(a.bmat, (uint32_t)fbytes);
        for (int b = wave; b < C::FBLOCKS; b += C::WAVES) {
            const int p = b * 64 + lane;
            const int row = p / C::FROWCH, col = p - row * C::FROWCH;
            unsigned voff = kBufOOB;
            if (col < C::FROWE / 8) {
                if (!TRANS) {
                    // row = output channel, col = (tap, channel chunk)
                    if (n0 + row < a.ngemm) voff = (unsigned)(((n0 + row) * C::KG + col * 8) * 2);
                } else {
                    // row = k (dy channel), col = (tap, chunk of the dx channel slice)
                    const int tap = col / (C::BN / 8), c = n0 + (col - tap * (C::BN / 8)) * 8;
                    if (c < a.ngemm) voff = (unsigned)(((row * R * S + tap) * a.ngemm + c) * 2);
                }
            }
            dma16(w_rs, lds_addr(filt + b * 1024), voff);
        }
        int r0, r1;
        group_rows(0, r0, r1);
        for (int rr = r0; rr < r1; ++rr) dma_row(rr, wave, my_off);
        nrow0 = r1 - r0;
    }
    // loads complete in issue order: with only the row loads outstanding,
    // this wave's share of the filter is in LDS
    static_assert(C::GR + C::HALO_R <= 6, "row loads of group 0 the wait below covers");
    switch (nrow0) {
    case 6: wait_vm_n<6>(); break;
    case 5: wait_vm_n<5>(); break;
    case 4: wait_vm_n<4>(); break;
    case 3: wait_vm_n<3>(); break;
    case 2: wait_vm_n<2>(); break;
    case 1: wait_vm_n<1>(); break;
    default: wait_vm_all(); break;
    }
    __syncthreads();  // the filter staging is complete
    // ---- the wave's filter fragments (A operand): rows n0 + 32*nb + 0..31,
    // k16 step ks = tap*C16 + c16; lane holds row l32, k = 8*lhi + 0..7
    const int nb = wave & 1, l32 = lane & 31, lhi = lane >> 5;
    u32x4 fr[C::KSTEPS];
    if (!TRANS) {
        const unsigned char *fp = filt + (nb * 32 + l32) * C::FROWB + lhi * 16;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) fr[ks] = *(const u32x4 *)(fp + ks * 32);
    } else {
        // ds_read_b64_tr_b16: in each group of 16 lanes, lane L points at
        // row L/4, columns 4*(L%4)..+3 of a 4 x 16 tile; lane i receives
        // column i of the 4 rows.  Rows are k, columns the dx channels.
        const int L = lane & 15, g16 = l32 >> 4;
        const unsigned char *fp = filt + (L >> 2) * C::FROWB + (nb * 32 + g16 * 16 + 4 * (L & 3)) * 2;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            const int tap = ks / C::C16, c16 = ks - tap * C::C16;
            const int stap = R * S - 1 - tap;
            const int kb = 16 * c16 + 8 * lhi;
            const uint2 lo = __builtin_bit_cast(uint2, band::tr16(fp + kb * C::FROWB + stap * C::BN * 2));
            const uint2 hi = __builtin_bit_cast(uint2, band::tr16(fp + (kb + 4) * C::FROWB + stap * C::BN * 2));
            fr[ks] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
    }

    {
        // the bias in the accumulator layout, [nb][lhi][16]: entry i of a
        // lane's acc holds channel 32*nb + 8*(i/4) + 4*lhi + i%4
        if (tid < C::BN) {
            const int i = tid & 15, lh = (tid >> 4) & 1, hb = tid >> 5;
            const int ch = n0 + 32 * hb + 8 * (i >> 2) + 4 * lh + (i & 3);
            if constexpr (I8)
                ((int32_t *)bias_s)[tid] = (a.bias && ch < a.ngemm) ? ((const int32_t *)a.bias)[ch] : 0;
            else
                bias_s[tid] = (a.bias && ch < a.ngemm) ? E::to_f32(((const elem *)a.bias)[ch]) : 0.0f;
        }
        wait_vm_all();    // group 0's rows
        __syncthreads();  // rows and bias visible; every wave holds its filter fragments
        if (!lead) dma_group(1);  // into slots group 0 does not read
    }

    // ---- pixel fragments (B operand): output column mb*32 + l32 at tap
    // column s reads ring column mb*32 + l32 + s*DIL, channel chunk
    // 2*c16 + lhi, stored at chunk (2*c16 + lhi) ^ swizzle.  The byte offset
    // inside a row is t_off[s] ^ (c16 << 5) (+ 32 pixels for mb = 1, which
    // keeps the swizzle).
    int t_off[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int col = l32 + s * DIL;
        t_off[s] = col * C::PIXB + ((lhi ^ ((col >> 1) & 7)) << 4);
    }

    const int ngroups = (nrows + C::GR - 1) / C::GR;
    // A wave's unit of a group: output row pr (of the band) and its blocks
    // [c0, c0 + 32*nblk) of 32 columns, for the channel half nb.  In a whole
    // group the two waves of each row take the two channel halves over both
    // column blocks; a group with at most GR/2 rows (the last group of a
    // band) gives each wave one block, so all waves work on it.
    struct Unit {
        int pr, slot, c0, nblk;
        bool active;
    };
    auto unit = [&](int g) {
        const int rows_g = min(C::GR, nrows - g * C::GR);
        Unit u;
        if (rows_g <= C::GR / 2) {
            u.slot = (wave >> 1) & (C::GR / 2 - 1);
            u.c0 = 32 * (wave / C::GR);
            u.nblk = 1;
        } else {
            u.slot = wave >> 1;
            u.c0 = 0;
            u.nblk = 2;
        }
        u.pr = g * C::GR + u.slot;
        u.active = u.slot < rows_g;
        return u;
    };
    // Output stores use 32-bit offsets from the start of the output image
    // (its size is checked on the host); stores past a row's valid pixels or
    // channels go to an offset past the range, which the range check drops.
    const __amdgpu_buffer_rsrc_t dst_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((elem *)a.dst + (size_t)img * a.P * a.Q * a.ngemm), (short)0,
        (int)((size_t)a.P * a.Q * a.ngemm * sizeof(elem)), 0x00020000);

    // ---- epilogue, part 1: ReLU, round, into the staging row of the unit
    // as [pixel][channel] with the ring's chunk swizzle.  Lane holds pixel
    // c0 + mb*32 + l32, channels 32*nb + 8*j + 4*lhi + 0..3 in
    // acc[mb][4j..4j+3]: 8 bytes, half lhi of chunk 4nb+j.  Each wave stages
    // and stores its own pixels, so no wave waits on another for its
    // results.
    acc_t acc[2];
    auto epilogue = [&](const Unit &u, auto relu_c) {
        constexpr bool RELU = decltype(relu_c)::value;
        unsigned char *stage = ostage + u.slot * C::SLOTB;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            if (mb >= u.nblk) break;
            const int px = u.c0 + mb * 32 + l32;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t v[2];
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    v[t] = out_pair<E, RELU>(acc[mb][4 * j + 2 * t], acc[mb][4 * j + 2 * t + 1]);
                const int chunk = (4 * nb + j) ^ ((px >> 1) & 7);
                *(uint2 *)(stage + px * C::PIXB + chunk * 16 + lhi * 8) = uint2{v[0], v[1]};
            }
        }
    };
    // int8: lane's 4 channels -> ReLU, requantise (fp64), 4 bytes at byte
    // 8*(j&1) + 4*lhi of logical chunk 2*nb + j/2 (16 channels a chunk)
    auto epilogue_i8 = [&](const Unit &u) {
        unsigned char *stage = ostage + u.slot * C::SLOTB;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            if (mb >= u.nblk) break;
            const int px = u.c0 + mb * 32 + l32;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t word = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int v = (int)acc[mb][4 * j + r];
                    if (a.relu && v < 0) v = 0;
                    word |= (uint32_t)(uint8_t)requant_i8(v, a.requant_m) << (8 * r);
                }
                const int chunk = (2 * nb + (j >> 1)) ^ ((px >> 1) & 7);
                *(uint32_t *)(stage + px * C::PIXB + chunk * 16 + 8 * (j & 1) + 4 * lhi) = word;
            }
        }
    };
    auto stage_rows = [&](const Unit &u) {
        if constexpr (I8)
            epilogue_i8(u);
        else if (a.relu)
            epilogue(u, band::BoolC<true>{});
        else
            epilogue(u, band::BoolC<false>{});
    };
    // ---- epilogue, part 2: the wave's 16-byte chunks back from the staging
    // (its own writes: LDS runs a wave's accesses in order) and out, four
    // lanes (64 contiguous bytes) per pixel for fp16/bf16, two for int8.
    // fp16/bf16 lane order: pixels {2u, 2u+1, 2u+8, 2u+9} of a quarter-wave
    // cover all 64 banks under the swizzle.
    auto store_rows = [&](const Unit &u) {
        const unsigned char *stage = ostage + u.slot * C::SLOTB;
        const int qrow = (p_start + u.pr) * a.Q + q0;  // wave-uniform
        asm volatile("" ::: "memory");  // the reads stay after the staging writes
        constexpr int LPP = I8 ? 2 : 4;  // lanes per pixel
        constexpr int PPI = 64 / LPP;    // pixels per store instruction
#pragma unroll
        for (int t = 0; t < C::RCOLS / PPI; ++t) {
            if (t * PPI >= 32 * u.nblk) break;
            const int uu = lane / LPP, c = lane % LPP;
            const int px = u.c0 + (I8 ? PPI * t + uu : 16 * t + (uu & 1) + 8 * ((uu >> 1) & 1) + 2 * (uu >> 2));
            const int chunk = LPP * nb + c;
            const u32x4 v = *(const u32x4 *)(stage + px * C::PIXB + ((chunk ^ ((px >> 1) & 7)) << 4));
            const int ch = n0 + chunk * EPC16;
            const bool ok = px < C::SEG && q0 + px < a.Q && ch < a.ngemm;
            __builtin_amdgcn_raw_buffer_store_b128(
                v, dst_rs, ok ? (uint32_t)(((qrow + px) * a.ngemm + ch) * (int)sizeof(elem)) : kBufOOB, 0, 2);
        }
    };
    // The trailing waves stage and store group g's results after the barrier
    // that ends the group, while the leading waves already run group g+1's
    // MFMAs; the leading waves stage theirs right after their MFMAs, while
    // the trailing waves still run their own.
    for (int g = 0; g < ngroups; ++g) {
        if (!lead && g > 0) {
            const Unit up = unit(g - 1);
            if (up.active) {
                stage_rows(up);
                store_rows(up);
            }
        }
        const Unit u = unit(g);
        if (u.active) {
            // the accumulators start at the bias (zero for dgrad)
            acc[0] = *(const acc_t *)(bias_s + (nb * 2 + lhi) * 16);
            acc[1] = acc[0];
            int rowb[R];
#pragma unroll
            for (int r = 0; r < R; ++r) rowb[r] = ((u.pr + r * DIL) % C::NSLOT) * C::SLOTB;
            const int cb = u.c0 * C::PIXB;  // the unit's first column (keeps the swizzle)
            auto mma = [&](auto two_c) {
                constexpr int NB = decltype(two_c)::value ? 2 : 1;
                u32x4 P[C::KSTEPS][NB];
                auto ld = [&](int ks) {
                    const int tap = ks / C::C16, c16 = ks - tap * C::C16;
                    const int r = tap / S, s = tap - r * S;
                    const unsigned char *p = ring + rowb[r] + cb + (t_off[s] ^ (c16 << 5));
#pragma unroll
                    for (int mb = 0; mb < NB; ++mb) P[ks][mb] = *(const u32x4 *)(p + mb * 32 * C::PIXB);
                };
#pragma unroll
                for (int ks = 0; ks < C::PF; ++ks) ld(ks);
#pragma unroll
                for (int ks = 0; ks < C::KSTEPS; ++ks) {
                    if (ks + C::PF < C::KSTEPS) ld(ks + C::PF);
#pragma unroll
                    for (int mb = 0; mb < NB; ++mb) acc[mb] = Mfma32<E>::run(fr[ks], P[ks][mb], acc[mb]);
                    // keep the reads PF steps ahead of their MFMAs (the
                    // scheduler would otherwise sink each read down to its use)
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            if (u.nblk == 2)
                mma(band::BoolC<true>{});
            else
                mma(band::BoolC<false>{});
        }
        if (lead) {
            if (u.active) {
                stage_rows(u);
                store_rows(u);
            }
        } else {
            wait_vm_all();  // the next group's rows (and this wave's older stores)
        }
        __syncthreads();  // every wave is done with this group's rows
        if (!lead) dma_group(g + 2);  // into the slots of the rows only this group read
    }
    if (!lead) {
        const Unit up = unit(ngroups - 1);
        if (up.active) {
            stage_rows(up);
            store_rows(up);
        }
    }
}

bool band_supported(int dtype, int R, int S, int cin, int dil)
{
    // pixels of 128 bytes: 64 fp16/bf16 channels, or 128 int8 ones
    return R == 3 && S == 3 && dil == 1 && (dtype == CONV2D_DTYPE_I8 ? cin == 128 : cin == 64);
}

hipError_t launch_band(int dtype, int R, int S, int cin, int dil, const BandArgs &a, int grid_n, int grid_q,
                       hipStream_t st)
{
    if (!band_supported(dtype, R, S, cin, dil)) return hipErrorInvalidValue;
    dim3 grid((unsigned)(a.N * a.chunks_per_img), (unsigned)grid_n, (unsigned)grid_q);
    const bool t = a.flip != 0;
    switch (dtype) {
    case CONV2D_DTYPE_F16:
        if (t)
            band_kernel<EF16, 3, 3, 64, 1, true><<<grid, 512, 0, st>>>(a);
        else
            band_kernel<EF16, 3, 3, 64, 1, false><<<grid, 512, 0, st>>>(a);
        break;
    case CONV2D_DTYPE_BF16:
        if (t)
            band_kernel<EBF16, 3, 3, 64, 1, true><<<grid, 512, 0, st>>>(a);
        else
            band_kernel<EBF16, 3, 3, 64, 1, false><<<grid, 512, 0, st>>>(a);
        break;
    case CONV2D_DTYPE_I8:
        if (t) return hipErrorInvalidValue;
        band_kernel<EI8, 3, 3, 64, 1, false><<<grid, 512, 0, st>>>(a);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cnv

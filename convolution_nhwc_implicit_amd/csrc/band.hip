// band.hip -- stride-1 implicit-GEMM convolution with the whole filter and a
// ring of input rows resident in LDS (gfx950).
//
// For a stride-1 convolution every input pixel feeds R*S output pixels.  The
// generic implicit-GEMM kernel gathers each GEMM row from memory once per tap;
// this kernel instead keeps a band of input rows in LDS and forms all R*S
// tap-shifted operand fragments from it, so each input byte leaves HBM once.
// The filter ([Ngemm-tile 64][R*S*CIN]) stays in LDS for the life of the
// workgroup, which walks a contiguous range of output rows of one image:
//
//   * a group is 8 output rows; each of the 8 waves (two per SIMD) owns one
//     row x 64 output columns x 64 output channels (a 64x64 tile of 32x32x16
//     MFMA blocks, fp32 accumulators);
//   * the LDS ring holds the 8 + dil*(R-1) input rows the group reads; while a
//     group is computed, the 8 input rows of the next group are loaded into
//     registers;
//   * when the group is done, the 8 ring slots only it used take each wave's
//     finished output row (bias, ReLU, rounding applied), which then leaves as
//     fully coalesced 128-bit stores; the prefetched rows go into the same
//     slots afterwards;
//   * the LDS has 64 four-byte banks and serves 16 lanes of a 128-bit read per
//     cycle.  A 128-byte pixel covers half of the banks, so the 16-byte channel
//     chunks of pixel `col` are XOR-swizzled by col/2: any 16 consecutive
//     pixels of an operand fragment (at any tap shift) then hit all 64 banks.
//     Filter rows are padded by 16 bytes, which does the same for them.
//
// The same kernel runs stride-1 dgrad: the source is dy, the padding is
// dil*(R-1) - pad, and the filter (re-laid out as [C][R*S*K]) is read with its
// taps reversed.
#include "device_common.h"

namespace cnv {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <class E>
struct Mfma32;
template <>
struct Mfma32<EF16> {
    __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <>
struct Mfma32<EBF16> {
    __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <int R, int S, int CIN, int DIL>
struct BandCfg {
    static constexpr int NT = 512;
    static constexpr int GROUP_ROWS = 8;                // output rows per group = waves
    static constexpr int BN = 64;                       // output channels per workgroup
    static constexpr int HALO_R = DIL * (R - 1);
    static constexpr int HALO_S = DIL * (S - 1);
    static constexpr int NSLOT = GROUP_ROWS + HALO_R;   // ring rows
    static constexpr int RCOLS = 64;                    // input columns per ring row
    static constexpr int SEG = RCOLS - HALO_S;          // output columns per workgroup
    static constexpr int NCH = CIN / 8;                 // 16-byte chunks per pixel
    static constexpr int PIXB = CIN * 2;
    static constexpr int SLOTB = RCOLS * PIXB;
    static constexpr int KG = R * S * CIN;              // GEMM-K
    static constexpr int FROWB = KG * 2 + 16;           // padded filter row
    static constexpr int FILT_BYTES = BN * FROWB;
    // Fragments of the last output columns of a segment read up to HALO_S
    // pixels past a ring row (those outputs are discarded); the tail pad keeps
    // the reads of the last slot inside the allocation.
    static constexpr int RING_BYTES = NSLOT * SLOTB + HALO_S * PIXB;
    static constexpr int LDS_BYTES = FILT_BYTES + RING_BYTES;
    static constexpr int ROW_CHUNKS = RCOLS * NCH;
    static constexpr int NEW_CHUNKS = GROUP_ROWS * ROW_CHUNKS;
    static constexpr int CPR = ROW_CHUNKS / NT;         // chunks per thread per ring row
    static constexpr int NEW_CPT = GROUP_ROWS * CPR;    // prefetch chunks per thread
    static constexpr int SWZ = (NCH >= 8 ? 8 : NCH) - 1;  // applied to col / 2
    static_assert(ROW_CHUNKS % NT == 0, "a ring row is a whole number of chunks per thread");
    static constexpr int OUT_PIXB = BN * 2;             // staged output pixel (BN channels)
    static_assert(SEG * OUT_PIXB <= SLOTB, "a wave's output row fits in one ring slot");
    static_assert(CIN % 16 == 0, "k16 steps stay inside one tap");
    static_assert(LDS_BYTES <= 163840, "fits in the 160 KB LDS");
};

template <class E, int R, int S, int CIN, int DIL>
__global__ __launch_bounds__(512, 1) void band_kernel(const BandArgs a)
{
    using C = BandCfg<R, S, CIN, DIL>;
    using elem = typename E::elem;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_BYTES];
    unsigned char *filt = smem;
    unsigned char *ring = smem + C::FILT_BYTES;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int img = blockIdx.x / a.chunks_per_img;
    const int chunk = blockIdx.x - img * a.chunks_per_img;
    const int p_start = chunk * a.rows_per_wg;
    const int p_end = min(p_start + a.rows_per_wg, a.P);
    if (p_start >= p_end) return;
    const int n0 = blockIdx.y * C::BN;
    const int q0 = blockIdx.z * C::SEG;
    const int h_base = p_start - a.pad_h;  // input row of ring row 0
    const int w_base = q0 - a.pad_w;       // input column of ring column 0

    const elem *src = (const elem *)a.src + (size_t)img * a.H * a.W * CIN;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    // ---- ring rows.  Thread t always moves the same (column, channel chunk)
    // positions of a row: chunk t + i*256 of the row's RCOLS*NCH chunks, so
    // a row costs CPR loads per thread and the addresses are a base plus
    // compile-time offsets.
    const int my_j = tid % C::NCH;
    const int my_col = tid / C::NCH;  // + i * (NT / NCH) for the i-th chunk of a row
    constexpr int COL_STEP = C::NT / C::NCH;
    const elem *my_src = src + (size_t)my_j * 8;
    const int my_swz = ((my_j ^ ((my_col >> 1) & C::SWZ)) * 16) + my_col * C::PIXB;
    static_assert(((COL_STEP >> 1) & C::SWZ) == 0 && COL_STEP % 2 == 0, "column step keeps the swizzle phase");
    auto load_row_chunk = [&](int hrel, int i) -> u32x4 {
        const int h = h_base + hrel, w = w_base + my_col + i * COL_STEP;
        if ((unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W)
            return *(const u32x4 *)(my_src + ((size_t)h * a.W + w) * CIN);
        return zero;
    };
    auto ring_chunk = [&](int hrel, int i) -> u32x4 * {
        return (u32x4 *)(ring + (hrel % C::NSLOT) * C::SLOTB + my_swz + i * COL_STEP * C::PIXB);
    };
    u32x4 pre[C::NEW_CPT];
    auto prefetch = [&](int r0) {
#pragma unroll
        for (int rr = 0; rr < C::GROUP_ROWS; ++rr)
#pragma unroll
            for (int i = 0; i < C::CPR; ++i) pre[rr * C::CPR + i] = load_row_chunk(r0 + rr, i);
    };
    auto commit = [&](int r0) {
#pragma unroll
        for (int rr = 0; rr < C::GROUP_ROWS; ++rr)
#pragma unroll
            for (int i = 0; i < C::CPR; ++i) *ring_chunk(r0 + rr, i) = pre[rr * C::CPR + i];
    };

    // ---- prologue: the filter tile (taps reversed for dgrad), the halo rows
    // and group 0's rows are all requested before any of them is waited for
    constexpr int F_CHUNKS = C::BN * C::KG / 8;
    constexpr int F_CPT = (F_CHUNKS + C::NT - 1) / C::NT;
    {
        u32x4 freg[F_CPT];
#pragma unroll
        for (int i = 0; i < F_CPT; ++i) {
            const int id = tid + i * C::NT;
            const int n = id / (C::KG / 8), kc = id - n * (C::KG / 8);
            const int tap = kc / (CIN / 8), cc = kc - tap * (CIN / 8);
            const int stap = a.flip ? (R * S - 1 - tap) : tap;
            freg[i] = zero;
            if (id < F_CHUNKS && n0 + n < a.ngemm)
                freg[i] = *(const u32x4 *)((const elem *)a.bmat + (size_t)(n0 + n) * C::KG + stap * CIN + cc * 8);
        }
        u32x4 hreg[C::HALO_R * C::CPR > 0 ? C::HALO_R * C::CPR : 1];
#pragma unroll
        for (int rr = 0; rr < C::HALO_R; ++rr)
#pragma unroll
            for (int i = 0; i < C::CPR; ++i) hreg[rr * C::CPR + i] = load_row_chunk(rr, i);
        prefetch(C::HALO_R);
#pragma unroll
        for (int i = 0; i < F_CPT; ++i) {
            const int id = tid + i * C::NT;
            const int n = id / (C::KG / 8), kc = id - n * (C::KG / 8);
            if (id < F_CHUNKS) *(u32x4 *)(filt + n * C::FROWB + kc * 16) = freg[i];
        }
#pragma unroll
        for (int rr = 0; rr < C::HALO_R; ++rr)
#pragma unroll
            for (int i = 0; i < C::CPR; ++i) *ring_chunk(rr, i) = hreg[rr * C::CPR + i];
        commit(C::HALO_R);
    }
    __syncthreads();

    const int ngroups = (p_end - p_start + C::GROUP_ROWS - 1) / C::GROUP_ROWS;
    const int l32 = lane & 31, lhi = lane >> 5;
    const unsigned char *fbase = filt + l32 * C::FROWB + lhi * 16;
    float bias_v[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int ch = n0 + n * 32 + l32;
        bias_v[n] = (a.bias && ch < a.ngemm) ? E::to_f32(((const elem *)a.bias)[ch]) : 0.0f;
    }

    for (int g = 0; g < ngroups; ++g) {
        const bool more = g + 1 < ngroups;
        if (more) prefetch((g + 1) * C::GROUP_ROWS + C::HALO_R);

        // the output row of this wave (relative to p_start)
        const int pr = g * C::GROUP_ROWS + wave;
        const bool active = p_start + pr < p_end;
        f32x16 acc[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n) acc[m][n] = f32x16{};
        if (active) {
            // Taps in a rolled loop, the CIN/16 channel steps of a tap
            // unrolled.  Two fragment buffers: while the MFMAs of one step
            // issue, the reads of the next step are interleaved between them
            // (one LDS read per MFMA); the first step of the next tap is read
            // during the last step of this one (at the last tap it re-reads
            // the same tap, so every read stays unconditional).
            constexpr int C16 = CIN / 16;
            static_assert(C16 % 2 == 0, "even channel steps per tap");
            u32x4 fa0[2], fb0[2], fa1[2], fb1[2];
            auto load_frags = [&](int tap, int c16, u32x4 (&A)[2], u32x4 (&Bf)[2]) {
                const int r = tap / S, sx = tap - r * S;
                const unsigned char *rowp = ring + ((pr + r * DIL) % C::NSLOT) * C::SLOTB;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int col = h * 32 + l32 + sx * DIL;
                    A[h] = *(const u32x4 *)(rowp + col * C::PIXB +
                                            (((2 * c16 + lhi) ^ ((col >> 1) & C::SWZ)) << 4));
                }
                const unsigned char *fp = fbase + tap * CIN * 2 + c16 * 32;
                Bf[0] = *(const u32x4 *)(fp);
                Bf[1] = *(const u32x4 *)(fp + 32 * C::FROWB);
            };
            auto mma = [&](const u32x4 (&A)[2], const u32x4 (&Bf)[2], bool interleave) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int n = 0; n < 2; ++n) acc[m][n] = Mfma32<E>::run(A[m], Bf[n], acc[m][n]);
                if (interleave) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);  // one LDS read
                        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // one MFMA
                    }
                }
            };
            load_frags(0, 0, fa0, fb0);
#pragma unroll 1
            for (int tap = 0; tap < R * S; ++tap) {
                const int next = tap + 1 < R * S ? tap + 1 : tap;
#pragma unroll
                for (int c16 = 0; c16 < C16; c16 += 2) {
                    load_frags(tap, c16 + 1, fa1, fb1);
                    mma(fa0, fb0, true);
                    if (c16 + 2 < C16)
                        load_frags(tap, c16 + 2, fa0, fb0);
                    else
                        load_frags(next, 0, fa0, fb0);
                    mma(fa1, fb1, true);
                }
            }
        }
        __syncthreads();  // every wave is done reading this group's ring rows

        // ---- epilogue: bias, ReLU, round, staged in the ring slot of input
        // row pr (used by this group only) as [column][channel]; 32x32 block
        // layout: lane holds channel (lane & 31), columns 8*(i/4) + 4*(lane/32) + i%4
        unsigned char *stage = ring + (pr % C::NSLOT) * C::SLOTB;
        if (active) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int chl = n * 32 + l32;
                const float b = bias_v[n];
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int ql = m * 32 + 8 * (i >> 2) + 4 * lhi + (i & 3);
                        *(elem *)(stage + ql * C::OUT_PIXB + chl * 2) =
                            E::from_f32(bias_relu_f32(acc[m][n][i], b, a.relu));
                    }
            }
        }
        __syncthreads();
        // read the staged row back (SEG columns x BN channels, 16 bytes per
        // lane), free the slots for the prefetched rows, then store
        constexpr int CPP = C::OUT_PIXB / 16;  // 16-byte chunks per pixel
        constexpr int OUT_CPL = (C::SEG * CPP + 63) / 64;
        u32x4 outv[OUT_CPL];
#pragma unroll
        for (int i = 0; i < OUT_CPL; ++i) {
            const int id = lane + i * 64;
            const int ql = id / CPP, cc = id - ql * CPP;
            outv[i] = (active && id < C::SEG * CPP) ? *(const u32x4 *)(stage + ql * C::OUT_PIXB + cc * 16) : zero;
        }
        __syncthreads();  // staged outputs are read back; the slots are free
        if (more) {
            commit((g + 1) * C::GROUP_ROWS + C::HALO_R);
            __syncthreads();
        }
        if (active) {
            const int p = p_start + pr;
            elem *drow = (elem *)a.dst + ((size_t)img * a.P + p) * a.Q * a.ngemm;
#pragma unroll
            for (int i = 0; i < OUT_CPL; ++i) {
                const int id = lane + i * 64;
                const int ql = id / CPP, cc = id - ql * CPP;
                const int q = q0 + ql, ch = n0 + cc * 8;
                if (id < C::SEG * CPP && q < a.Q && ch < a.ngemm)
                    *(u32x4 *)(drow + (size_t)q * a.ngemm + ch) = outv[i];
            }
        }
    }
}

bool band_supported(int R, int S, int cin, int dil)
{
    return R == 3 && S == 3 && cin == 64 && dil == 1;
}

hipError_t launch_band(int dtype, int R, int S, int cin, int dil, const BandArgs &a, int grid_n, int grid_q,
                       hipStream_t st)
{
    if (!band_supported(R, S, cin, dil)) return hipErrorInvalidValue;
    dim3 grid((unsigned)(a.N * a.chunks_per_img), (unsigned)grid_n, (unsigned)grid_q);
    switch (dtype) {
    case CONV2D_DTYPE_F16: band_kernel<EF16, 3, 3, 64, 1><<<grid, 512, 0, st>>>(a); break;
    case CONV2D_DTYPE_BF16: band_kernel<EBF16, 3, 3, 64, 1><<<grid, 512, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cnv

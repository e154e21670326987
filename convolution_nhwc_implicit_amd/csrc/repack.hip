// repack.hip -- row re-layout for channel counts that do not fill whole
// 16-byte vectors.  The implicit-GEMM kernels load channels 16 bytes at a
// time, so a problem whose C or K is not a multiple of 8 (16 for int8) runs
// on copies padded with zero channels (zeros add nothing to any sum), and
// results come back through the same copy with the padding dropped.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace cnv {

// dst[r][c] = (r < src_rows && c < src_cols) ? src[r][c] : 0 for r < dst_rows,
// c < dst_cols.  A thread writes 8 consecutive elements of a dst row.
template <typename T>
__global__ __launch_bounds__(256) void repack_kernel(const RepackArgs a)
{
    const T *src = (const T *)a.src;
    T *dst = (T *)a.dst;
    const long long chunks_per_row = (a.dst_cols + 7) / 8;
    const long long total = a.dst_rows * chunks_per_row;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
        const long long r = i / chunks_per_row;
        const int c0 = (int)(i - r * chunks_per_row) * 8;
        const bool row_ok = r < a.src_rows;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = c0 + j;
            if (c >= a.dst_cols) break;
            dst[r * a.dst_ld + c] = (row_ok && c < a.src_cols) ? src[r * a.src_ld + c] : (T)0;
        }
    }
}

hipError_t launch_repack(int esz, const RepackArgs &a, hipStream_t st)
{
    const long long total = a.dst_rows * ((a.dst_cols + 7) / 8);
    if (total <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<long long>((total + 255) / 256, 8192);
    switch (esz) {
    case 1: repack_kernel<uint8_t><<<blocks, 256, 0, st>>>(a); break;
    case 2: repack_kernel<uint16_t><<<blocks, 256, 0, st>>>(a); break;
    case 4: repack_kernel<uint32_t><<<blocks, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace cnv

// Optional zero fill of the receive rows that no entry maps to.
//
// Dynamic routing meets static shapes either by dropping tokens or by padding
// each expert's segment with zeros (search-results page, the snippet on the
// limits of dynamic routing).  The layout pads segments but dispatch never
// writes the padding rows (they would dominate a decode call's bytes); a
// consumer that needs them zero -- a grouped GEMM over whole segments, say --
// calls this after dispatch.  Rows whose src is -1 (padding inside segments
// and the unused tail) become zero bytes, and with FP8 their scales 0.0f;
// rows that hold an entry are not touched.
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int kPadWaves = 4;  // rows per workgroup, one wave each

// Wave w of workgroup b owns row b*kPadWaves + w: if no entry maps to it, the
// wave clears the row in 16-byte non-temporal stores, then its scale row.
__global__ __launch_bounds__(kPadWaves * kWave) void k_zero_padding(const int32_t *__restrict__ src, int rows,
                                                                   int vec_per_row, u32x4 *recv, float *scales,
                                                                   int nsc) {
    const int r = blockIdx.x * kPadWaves + threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    if (r >= rows || src[r] >= 0) return;  // the same for the whole wave
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 *row = recv + static_cast<size_t>(r) * vec_per_row;
    for (int v = lane; v < vec_per_row; v += kWave) __builtin_nontemporal_store(zero, row + v);
    if (scales != nullptr)
        for (int j = lane; j < nsc; j += kWave) scales[static_cast<size_t>(r) * nsc + j] = 0.0f;
}

}  // namespace

hipError_t launch_zero_padding(const int32_t *src, int rows, int row_bytes, void *recv, float *scales, int nsc,
                               hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const int grid = (rows + kPadWaves - 1) / kPadWaves;
    hipLaunchKernelGGL(k_zero_padding, dim3(grid), dim3(kPadWaves * kWave), 0, s, src, rows, row_bytes / 16,
                       static_cast<u32x4 *>(recv), scales, nsc);
    return hipGetLastError();
}

}  // namespace moe

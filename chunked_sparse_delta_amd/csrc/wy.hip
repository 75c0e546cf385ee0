// The per-chunk solve of the chunked SDM forward on gfx950 (wy_solve.py docstring,
// sparse-delta-memory 2.0.0 wheel, diffend page 23):
//     X  = (I + Lm)^-1,  Lm = tril(diag(beta) A, -1)   (unit lower triangular)
//     QX = QK X          (QK lower triangular with its diagonal)
// Both are written dense [C, C] with +0 above the diagonal.
//
// One workgroup per chunk. The matrices are cut into 16 x 16 tiles (nb = ceil(C / 16) tile
// rows; rows and columns >= C act as identity rows of I + Lm, so any C is exact: the
// leading block of a lower-triangular inverse is the inverse of the leading block). X is
// held in LDS as its nb (nb + 1) / 2 lower tiles.
//   1. Diagonal tiles: 16 lanes per tile, lane j solves (I + Lm_bb) x = e_j by forward
//      substitution, fully unrolled (x_r = -sum_{k<r} Lm[r][k] x_k, k ascending).
//   2. Recursive doubling: for block sizes s = 16, 32, 64, 128, each pair of neighbouring
//      diagonal blocks [[X11, 0], [N21, X22]] gets X21 = -X22 (N21 X11), N21 = beta A21.
//   3. QX_IJ = sum_{K=J}^{I} QK_IK X_KJ.
// Tile products run on v_mfma_f32_16x16x4f32, k blocks of 16 ascending: a fixed order for
// every launch.
#include "wy_impl.h"

namespace sdm {

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void wy_kernel(WyArgs a) {
    extern __shared__ float lds[];
    wy_chunk<BLOCK>(a, blockIdx.x, lds);
}

hipError_t wy_prepare() {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&wy_kernel<1024>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(wy_lds_bytes(kMaxChunk)));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&wy_kernel<256>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(wy_lds_bytes(64)));
}

hipError_t launch_wy(const float *A, const float *beta, const float *QK, float *X, float *QX, int C, int64_t n,
                     int64_t stride, int64_t bstride, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    WyArgs a{A, beta, QK, X, QX, C, stride, bstride};
    if (C <= 64)
        hipLaunchKernelGGL(wy_kernel<256>, dim3(unsigned(n)), dim3(256), wy_lds_bytes(C), st, a);
    else
        hipLaunchKernelGGL(wy_kernel<1024>, dim3(unsigned(n)), dim3(1024), wy_lds_bytes(C), st, a);
    return hipGetLastError();
}

}  // namespace sdm

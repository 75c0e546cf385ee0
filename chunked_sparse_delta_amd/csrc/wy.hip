// The per-chunk solve of the chunked SDM forward on gfx950 (wy_solve.py docstring,
// sparse-delta-memory 2.0.0 wheel, diffend page 23):
//     X  = (I + Lm)^-1,  Lm = tril(diag(beta) A, -1)   (unit lower triangular)
//     QX = QK X          (QK lower triangular with its diagonal)
// Both are written dense [C, C] with +0 above the diagonal.
//
// One workgroup of 256 threads per chunk, 64 x 64 blocks (nb = ceil(C / 64) <= 4 block
// rows; rows and columns >= C act as identity rows of I + Lm, so any C is exact: the
// leading block of a lower-triangular inverse is the inverse of the leading block).
//   1. Diagonal blocks: thread (b, j) solves (I + Lm_bb) x = e_j by forward substitution
//      with the column kept in LDS; all nb diagonal blocks at once.
//   2. Blocks below the diagonal, one column block j at a time, going down:
//      X_ij = -X_ii (sum_{k=j}^{i-1} Lm_ik X_kj).
//   3. QX_ij = sum_{k=j}^{i} QK_ik X_kj for i >= j.
// Block products stage 64 x 64 tiles in LDS; each thread owns a 4 x 4 output tile and
// accumulates in float32 FMAs over k in ascending order, a fixed order for every launch.
#include "common.h"

namespace sdm {

constexpr int kB = 64;        // block edge
constexpr int kP = kB + 1;    // LDS row pitch

struct WyArgs {
    const float *A, *beta, *QK;
    float *X, *QX;
    int32_t C;
    int64_t stride;   // floats between consecutive chunks' matrices
    int64_t bstride;  // floats between consecutive chunks' beta
};

// tile <- rows r0.., cols c0.. of M (C x C, row-major); zero outside [C, C], and above
// the diagonal when `lower` (so that part of M is never read). rowscale (if given)
// multiplies row r by rowscale[r].
__device__ __forceinline__ void wy_load_tile(float *tile, const float *M, const float *rowscale, int C, int r0, int c0,
                                             bool lower = false) {
    for (int idx = threadIdx.x; idx < kB * kB; idx += blockDim.x) {
        const int r = idx >> 6, c = idx & 63;
        const int gr = r0 + r, gc = c0 + c;
        float v = 0.0f;
        if (gr < C && gc < C && (!lower || gc <= gr)) {
            v = M[int64_t(gr) * C + gc];
            if (rowscale) v *= rowscale[gr];
        }
        tile[r * kP + c] = v;
    }
}

__device__ __forceinline__ void wy_mma(float (&acc)[4][4], const float *Ta, const float *Tb) {
    const int rr = (threadIdx.x >> 4) * 4, cc = (threadIdx.x & 15) * 4;
#pragma unroll 8
    for (int k = 0; k < kB; ++k) {
        float a[4], b[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) a[x] = Ta[(rr + x) * kP + k];
#pragma unroll
        for (int y = 0; y < 4; ++y) b[y] = Tb[k * kP + cc + y];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(a[x], b[y], acc[x][y]);
    }
}

__device__ __forceinline__ void wy_store_tile(float *M, const float (&acc)[4][4], float sign, int C, int r0, int c0) {
    const int rr = (threadIdx.x >> 4) * 4, cc = (threadIdx.x & 15) * 4;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            const int gr = r0 + rr + x, gc = c0 + cc + y;
            if (gr < C && gc < C) M[int64_t(gr) * C + gc] = sign * acc[x][y];
        }
}

__device__ __forceinline__ void wy_acc_to_tile(float *tile, const float (&acc)[4][4]) {
    const int rr = (threadIdx.x >> 4) * 4, cc = (threadIdx.x & 15) * 4;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) tile[(rr + x) * kP + cc + y] = acc[x][y];
}

__global__ __launch_bounds__(256) void wy_kernel(WyArgs a) {
    extern __shared__ float lds[];
    const int64_t n = blockIdx.x;
    const int C = a.C;
    const float *A = a.A + n * a.stride;
    const float *QK = a.QK + n * a.stride;
    const float *beta = a.beta + n * a.bstride;
    float *X = a.X + n * a.stride;
    float *QX = a.QX + n * a.stride;
    const int nb = (C + kB - 1) / kB;
    const int tid = threadIdx.x;
    float *xs_all = lds + nb * kB * kP;   // [nb][64][64] column solutions

    // 1. diagonal blocks: stage Lm_bb (strict lower, beta-scaled) for every block b < nb.
    for (int idx = tid; idx < nb * kB * kB; idx += 256) {
        const int b = idx >> 12, r = (idx >> 6) & 63, c = idx & 63;
        const int gr = b * kB + r, gc = b * kB + c;
        float v = 0.0f;
        if (c < r && gr < C) v = beta[gr] * A[int64_t(gr) * C + gc];
        lds[b * kB * kP + r * kP + c] = v;
    }
    __syncthreads();
    {
        // Thread (b, j) solves column j of block b: x_r = -sum_{k=j}^{r-1} Lm[r][k] x_k.
        const int b = tid >> 6, j = tid & 63;
        if (b < nb) {
            const float *Lb = lds + b * kB * kP;
            float *xs = xs_all + b * kB * kB;
            const int gc = b * kB + j;
            for (int r = 0; r < kB; ++r) {
                float xr;
                if (r < j) {
                    xr = 0.0f;
                } else if (r == j) {
                    xr = 1.0f;
                } else {
                    float s = 0.0f;
                    for (int k = j; k < r; ++k) s = fmaf(Lb[r * kP + k], xs[k * kB + j], s);
                    xr = -s;
                }
                xs[r * kB + j] = xr;
                const int gr = b * kB + r;
                if (gr < C && gc < C) X[int64_t(gr) * C + gc] = xr;
            }
        }
    }
    // +0 above the diagonal blocks.
    for (int64_t idx = tid; idx < int64_t(C) * C; idx += 256) {
        const int r = int(idx / C), c = int(idx - int64_t(r) * C);
        if (c / kB > r / kB) {
            X[idx] = 0.0f;
            QX[idx] = 0.0f;
        }
    }
    __syncthreads();

    float *T0 = lds, *T1 = lds + kB * kP, *T2 = lds + 2 * kB * kP;
    // 2. blocks below the diagonal
    for (int j = 0; j < nb; ++j) {
        for (int i = j + 1; i < nb; ++i) {
            float acc[4][4] = {};
            for (int k = j; k < i; ++k) {
                wy_load_tile(T0, A, beta, C, i * kB, k * kB);   // Lm_ik = beta_i A_ik (k < i: whole block)
                wy_load_tile(T1, X, nullptr, C, k * kB, j * kB);
                __syncthreads();
                wy_mma(acc, T0, T1);
                __syncthreads();
            }
            wy_acc_to_tile(T2, acc);
            wy_load_tile(T0, X, nullptr, C, i * kB, i * kB);
            __syncthreads();
            float acc2[4][4] = {};
            wy_mma(acc2, T0, T2);
            wy_store_tile(X, acc2, -1.0f, C, i * kB, j * kB);
            __syncthreads();
        }
    }
    // 3. QX on and below the diagonal
    for (int j = 0; j < nb; ++j) {
        for (int i = j; i < nb; ++i) {
            float acc[4][4] = {};
            for (int k = j; k <= i; ++k) {
                wy_load_tile(T0, QK, nullptr, C, i * kB, k * kB, k == i);
                wy_load_tile(T1, X, nullptr, C, k * kB, j * kB);
                __syncthreads();
                wy_mma(acc, T0, T1);
                __syncthreads();
            }
            if (i == j) {
                // QK_ii X_ii is lower triangular: keep +0 above the diagonal exactly.
                const int rr = (tid >> 4) * 4, cc = (tid & 15) * 4;
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int y = 0; y < 4; ++y)
                        if (cc + y > rr + x) acc[x][y] = 0.0f;
            }
            wy_store_tile(QX, acc, 1.0f, C, i * kB, j * kB);
        }
    }
}

size_t wy_lds_bytes(int C) {
    const int nb = (C + kB - 1) / kB;
    const size_t need = size_t(nb) * kB * (kP + kB) * sizeof(float);
    const size_t tiles = size_t(3) * kB * kP * sizeof(float);
    return need > tiles ? need : tiles;
}

hipError_t wy_prepare() {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&wy_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               int(wy_lds_bytes(kMaxChunk)));
}

hipError_t launch_wy(const float *A, const float *beta, const float *QK, float *X, float *QX, int C, int64_t n,
                     int64_t stride, int64_t bstride, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    WyArgs a{A, beta, QK, X, QX, C, stride, bstride};
    hipLaunchKernelGGL(wy_kernel, dim3(unsigned(n)), dim3(256), wy_lds_bytes(C), st, a);
    return hipGetLastError();
}

}  // namespace sdm

// Device code of the per-chunk solve, shared by the solve kernel and the fused Phase-1
// kernel (see wy.hip for the method).
#pragma once

#include "common.h"

namespace sdm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct WyArgs {
    const float *A, *beta, *QK;
    float *X, *QX;
    int32_t C;
    int64_t stride;   // floats between consecutive chunks' matrices
    int64_t bstride;  // floats between consecutive chunks' beta
};

constexpr int kTile = 256;   // floats of a 16 x 16 tile (row-major, pitch 16)

__device__ __forceinline__ int tri_index(int I, int J) { return I * (I + 1) / 2 + J; }

// A-operand of a 16 x 16 x 16 block from global memory: lane l holds
// rs[r] * M[r][k0 + 4 (l >> 4) + kk], r = r0 + (l & 15), kk = 0..3, zero outside [C, C]
// and, with `lower`, above the diagonal (k > r).
__device__ __forceinline__ void wy_gop(const float *M, const float *rs, int C, int r0, int k0, bool lower, int lane,
                                       float (&o)[4]) {
    const int r = r0 + (lane & 15), k = k0 + 4 * (lane >> 4);
    const float sc = (rs && r < C) ? rs[r] : 1.0f;
    if (r < C && k + 3 < C && (C & 3) == 0) {
        const float4 x = *reinterpret_cast<const float4 *>(M + int64_t(r) * C + k);
        o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) o[kk] = (r < C && k + kk < C) ? M[int64_t(r) * C + k + kk] : 0.0f;
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        o[kk] *= sc;
        if (lower && k + kk > r) o[kk] = 0.0f;
    }
}

// A-operand from an LDS tile (row l & 15, columns 4 (l >> 4) .. + 3).
__device__ __forceinline__ void wy_lop_a(const float *T, int lane, float (&o)[4]) {
    const float4 x = *reinterpret_cast<const float4 *>(T + (lane & 15) * 16 + 4 * (lane >> 4));
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
}

// B-operand from an LDS tile: lane l holds T[4 (l >> 4) + kk][l & 15].
__device__ __forceinline__ void wy_lop_b(const float *T, int lane, float (&o)[4]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) o[kk] = T[(4 * (lane >> 4) + kk) * 16 + (lane & 15)];
}

__device__ __forceinline__ f32x4 mfma4(const float (&a)[4], const float (&b)[4], f32x4 acc) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk], b[kk], acc, 0, 0, 0);
    return acc;
}

// Accumulator tile (lane l holds rows 4 (l >> 4) + v, column l & 15) to an LDS tile.
__device__ __forceinline__ void wy_store_tile(float *T, const f32x4 &d, float sign, int lane) {
#pragma unroll
    for (int v = 0; v < 4; ++v) T[(4 * (lane >> 4) + v) * 16 + (lane & 15)] = sign * d[v];
}

// The solve of chunk n by one workgroup of BLOCK threads; lds: wy_lds_bytes(C).
template <int BLOCK>
__device__ __forceinline__ void wy_chunk(const WyArgs &a, int64_t n, float *lds) {
    constexpr int NW = BLOCK / kWave;
    constexpr int kMaxNb = BLOCK == 1024 ? 16 : 4;           // tile rows this block size serves
    constexpr int kMaxPer = (kMaxNb / 2) * (kMaxNb / 2) / NW > 0 ? (kMaxNb / 2) * (kMaxNb / 2) / NW : 1;
    const int C = a.C;
    const float *A = a.A + n * a.stride;
    const float *QK = a.QK + n * a.stride;
    const float *beta = a.beta + n * a.bstride;
    float *X = a.X + n * a.stride;
    float *QX = a.QX + n * a.stride;
    const int nb = (C + 15) >> 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float *Xt = lds;   // lower tiles of X

    // 1. diagonal tiles: stage Lm_bb (strict lower, beta-scaled), then invert in place.
    for (int idx = tid; idx < nb * kTile; idx += BLOCK) {
        const int b = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
        const int gr = 16 * b + r, gc = 16 * b + c;
        float v = 0.0f;
        if (c < r && gr < C) v = beta[gr] * A[int64_t(gr) * C + gc];
        Xt[tri_index(b, b) * kTile + r * 16 + c] = v;
    }
    __syncthreads();
    {
        const int b = wave * 4 + (lane >> 4), j = lane & 15;
        float x[16];
        if (b < nb) {
            const float *L = Xt + tri_index(b, b) * kTile;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = 0.0f;
#pragma unroll
                for (int k = 0; k < r; ++k) s = fmaf(L[r * 16 + k], x[k], s);   // x_k = 0 for k < j
                x[r] = r < j ? 0.0f : (r == j ? 1.0f : -s);
            }
        }
        __syncthreads();
        if (b < nb) {
            float *T = Xt + tri_index(b, b) * kTile;
#pragma unroll
            for (int r = 0; r < 16; ++r) T[r * 16 + j] = x[r];
        }
    }
    __syncthreads();

    // 2. doubling: blocks of h tiles, pairs starting at tile row P0 = 2 h p.
    for (int h = 1; h < nb; h <<= 1) {
        const int npairs = (nb + 2 * h - 1) / (2 * h);
        // items of the level: (pair, I, J) with I in [P0 + h, min(P0 + 2h, nb)), J in [P0, P0 + h)
        const int per = h * h, items = npairs * per;
        // 2a. T_IJ = sum_{K=J}^{P0+h-1} N_IK X_KJ -> slot (I, J)
        for (int it = wave; it < items; it += NW) {
            const int pr = it / per, q = it - pr * per, P0 = 2 * h * pr;
            const int I = P0 + h + q / h, J = P0 + q % h;
            if (I >= nb) continue;
            f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            for (int K = J; K < P0 + h; ++K) {
                float ao[4], bo[4];
                wy_gop(A, beta, C, 16 * I, 16 * K, false, lane, ao);
                wy_lop_b(Xt + tri_index(K, J) * kTile, lane, bo);
                acc = mfma4(ao, bo, acc);
            }
            wy_store_tile(Xt + tri_index(I, J) * kTile, acc, 1.0f, lane);
        }
        __syncthreads();
        // 2b. X21_IJ = -sum_{K=P0+h}^{I} X_IK T_KJ (into registers, then over T)
        f32x4 res[kMaxPer];
#pragma unroll
        for (int m = 0; m < kMaxPer; ++m) {
            res[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const int it = wave + m * NW;
            if (it >= items) continue;
            const int pr = it / per, q = it - pr * per, P0 = 2 * h * pr;
            const int I = P0 + h + q / h, J = P0 + q % h;
            if (I >= nb) continue;
            for (int K = P0 + h; K <= I; ++K) {
                float ao[4], bo[4];
                wy_lop_a(Xt + tri_index(I, K) * kTile, lane, ao);
                wy_lop_b(Xt + tri_index(K, J) * kTile, lane, bo);
                res[m] = mfma4(ao, bo, res[m]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < kMaxPer; ++m) {
            const int it = wave + m * NW;
            if (it >= items) continue;
            const int pr = it / per, q = it - pr * per, P0 = 2 * h * pr;
            const int I = P0 + h + q / h, J = P0 + q % h;
            if (I >= nb) continue;
            wy_store_tile(Xt + tri_index(I, J) * kTile, res[m], -1.0f, lane);
        }
        __syncthreads();
    }

    // X out: lower tiles from LDS, +0 above the diagonal.
    for (int64_t idx = tid; idx < int64_t(C) * C; idx += BLOCK) {
        const int r = int(idx / C), c = int(idx - int64_t(r) * C);
        X[idx] = c <= r ? Xt[tri_index(r >> 4, c >> 4) * kTile + (r & 15) * 16 + (c & 15)] : 0.0f;
    }

    // 3. QX_IJ = sum_{K=J}^{I} QK_IK X_KJ for I >= J; +0 above the diagonal.
    const int ntiles = nb * (nb + 1) / 2;
    for (int t = wave; t < ntiles; t += NW) {
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= t) ++I;
        const int J = t - I * (I + 1) / 2;
        f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int K = J; K <= I; ++K) {
            float ao[4], bo[4];
            wy_gop(QK, nullptr, C, 16 * I, 16 * K, K == I, lane, ao);
            wy_lop_b(Xt + tri_index(K, J) * kTile, lane, bo);
            acc = mfma4(ao, bo, acc);
        }
        const int c = 16 * J + (lane & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * I + 4 * (lane >> 4) + v;
            if (r < C && c < C) QX[int64_t(r) * C + c] = c <= r ? acc[v] : 0.0f;
        }
    }
    for (int64_t idx = tid; idx < int64_t(C) * C; idx += BLOCK) {
        const int r = int(idx / C), c = int(idx - int64_t(r) * C);
        if ((c >> 4) > (r >> 4)) QX[idx] = 0.0f;
    }
}

inline size_t wy_lds_bytes(int C) {
    const int nb = (C + 15) / 16;
    return size_t(nb) * (nb + 1) / 2 * kTile * sizeof(float);
}

}  // namespace sdm

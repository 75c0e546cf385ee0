// Arguments and launchers of the SDM backward (backward.hip).
#pragma once
#include "common.h"

namespace sdm {

constexpr int kBwdBlock = 256;

struct BwdArgs {
    int32_t P, T, W, R, G, hd, S, NS;   // S columns per slice (power of two, 4..64), NS slices
    int64_t M;
    const void *k_idx, *q_idx;
    int32_t k_id8, q_id8;
    const float *k_val, *q_val, *beta, *g, *v, *go;
    const int32_t *valid;
    float *bank;     // [P, M, hd], replayed and restored
    float *gbank;    // [P, M, hd], in: gradient of the final bank; out: of the initial bank
    float *gv;       // [P, T, hd]
    float *gk, *gq, *gbeta, *gg;   // [P, T, W], [P, T, R], [P, T], [P, T, G]
    float *snap;     // [P, T, W, hd]  old_w of every live write entry
    float2 *lead;    // [P, T, R]      (summed weight, 1) for a slot's first read entry, else (0, 0)
    float *part;     // [P, NS, T, J]  per-slice dots, J = 2W + R + 1
};

__host__ __device__ inline int bwd_parts(int W, int R) { return 2 * W + R + 1; }

size_t bwd_lds_bytes(int W, int S);
int bwd_slice_cols(int P, int hd);
hipError_t bwd_prepare();
hipError_t launch_bwd(const BwdArgs &a, hipStream_t st);

}  // namespace sdm

// Arguments and launchers of the SDM backward (backward.hip).
#pragma once
#include "common.h"

namespace sdm {

constexpr int kBwdBlock = 256;
constexpr int kBwdMaxLds = 160 * 1024 - 256;   // LDS a workgroup of the resident sweep may take
constexpr int kResRed = kWave;                 // words of the resident sweep's partial-sum array
constexpr int kPairMax = 8;                    // write and read slots per token, at most, for token pairs
constexpr int kWaveMaxSlots = 128;             // slots per token, at most, for the one-wavefront sweeps

struct BwdArgs {
    int32_t P, T, W, R, G, hd, S, NS;   // S columns per slice (power of two, 4..64), NS slices
    int32_t res;                        // 1, 2, 4: the one-wavefront sweep, rows in LDS, with that
                                        // many entries of each kind per lane; -1, -2, -4, -8: the
                                        // same with rows in memory; 0: the 256-thread sweep
    int32_t pair;                       // 1: the paired resident sweep (res == 1)
    int32_t bf16;                       // 1: bank, weights, v and grad_out are bfloat16, else float32
    int64_t M;
    int64_t bstride;                    // elements from one stream's bank to the next (M * hd, or 0 shared)
    const void *k_idx, *q_idx;
    int32_t k_id8, q_id8;
    const void *k_val, *q_val, *v, *go;   // in the bank dtype
    const float *beta, *g;
    const int32_t *valid;
    const void *bank;  // the bank the forward started from (never written)
    float *work;     // float32 rows the sweep in memory replays and restores: the bank itself
                     // (float32) or a copy of it in the workspace (bfloat16)
    float *gbank;    // [P, M, hd] (or [M, hd] shared), in: gradient of the final bank; out: of the initial bank
    float *gv;       // [P, T, hd]
    float *gk, *gq, *gbeta, *gg;   // [P, T, W], [P, T, R], [P, T], [P, T, G]
    void *snap;      // [P, NS, T, W, S]  old_w of every live write entry, slice by slice: float32,
                     // or bfloat16 (snap_bf16: rounded to nearest even, widened back where used)
    int32_t snap_bf16;
    float2 *lead;    // [P, T, R]      (summed weight, 1) for a slot's first read entry, else (0, 0)
    float *part;     // [P, NS, T, J]  per-slice dots, J = 2W + R + 1
    int32_t *pairs;  // [P, ceil(T / 2)]  1: tokens 2j, 2j + 1 live and selecting disjoint rows
};

__host__ __device__ inline int bwd_parts(int W, int R) { return 2 * W + R + 1; }

// Element index of the first saved row of slice sl of stream p, and one saved element in
// and out: the snapshot's element type is float32 or bfloat16 (snap_bf16).
__device__ __forceinline__ int64_t snap_slice(const BwdArgs &a, int p, int sl) {
    return (int64_t(p) * a.NS + sl) * a.T * a.W * a.S;
}
__device__ __forceinline__ float snap_ld(const BwdArgs &a, int64_t i) {
    if (a.snap_bf16) return __uint_as_float(uint32_t(static_cast<const uint16_t *>(a.snap)[i]) << 16);
    return static_cast<const float *>(a.snap)[i];
}
__device__ __forceinline__ void snap_st(const BwdArgs &a, int64_t i, float x) {
    if (a.snap_bf16) static_cast<uint16_t *>(a.snap)[i] = f32_to_bf16(x).bits;
    else static_cast<float *>(a.snap)[i] = x;
}

size_t bwd_lds_bytes(int W, int S, int64_t M, bool res);
int bwd_slice_cols(int P, int hd, int W, int R);
int bwd_res_entries(int W, int R, int S, int kj_max);
hipError_t bwd_prepare();
hipError_t launch_bwd(const BwdArgs &a, hipStream_t st, hipEvent_t *ev);

}  // namespace sdm

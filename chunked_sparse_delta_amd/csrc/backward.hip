// The backward of the SDM write/read forward: gradients of a scalar objective
//     J = <grad_out, readings> + <grad_bank_final, final bank>
// with respect to the bank the forward started from, the write and read slot weights, v,
// beta and the log-decays. The pages make sdm_write_read differentiable in all of these
// (SDMWriteRead, memory_ops.py, diffend page 21) and name their backward's stages without
// listing them; what it computes is the derivative of the per-token loop of the
// SDMWriteRead docstring, so this file differentiates that loop.
//
// Per token (live tokens only), forward:
//     old_w = bank[s_w];  dec_w = exp(g_w) old_w;  ret = sum_w k_w dec_w;
//     delta = beta (v - ret);  bank[s_w] = dec_w + k_w delta;  out = sum_r q_r bank[s_r]
// and in reverse, gb being the gradient with respect to the bank after the token:
//     grad_q_r = <grad_out, bank[s_r]>;  gb[s_r] += q_r grad_out
//     gdelta = sum_w k_w gb[s_w];  grad_k_w = <gb[s_w], delta>
//     grad_beta = <gdelta, v - ret>;  grad_v = beta gdelta;  gret = -beta gdelta
//     grad_k_w += <gret, dec_w>;  gdec_w = gb[s_w] + k_w gret;  grad_g_w = <gdec_w, dec_w>
//     gb[s_w] = exp(g_w) gdec_w;  bank[s_w] = old_w
//
// Every bank column evolves on its own, so one workgroup owns one (stream, column slice)
// for the whole call: it replays the forward token by token on its slice, saving old_w
// of every write entry in the workspace, then walks the tokens backwards, updating the
// bank gradient in place and restoring each written row from the saved value (so the
// bank ends exactly as it started, with no division by a decay). The dot products over
// columns (grad_q, grad_k, grad_g, grad_beta) are reduced over the slice's lanes and
// stored per slice; a second kernel sums the slices in ascending order. Read slots that
// repeat within a token are folded first (one lead entry per distinct slot carrying the
// sum of the repeats' weights, in slot order), so each bank row has one writer per pass.
// Every sum runs in a fixed order: the results are bitwise reproducible.
#include <stdlib.h>

#include "backward.h"

namespace sdm {

__device__ __forceinline__ int32_t live_tokens(const BwdArgs &a, int p) {
    int32_t n = a.valid ? a.valid[p] : a.T;
    return n < 0 ? 0 : (n > a.T ? a.T : n);
}

__device__ __forceinline__ int32_t clamp_row(int32_t s, int64_t M) {
    return s < 0 ? 0 : (s >= M ? int32_t(M - 1) : s);
}

// Sum over the S consecutive lanes of a group (butterfly: every lane gets the same bits).
__device__ __forceinline__ float group_sum(float x, int S) {
    for (int m = S >> 1; m > 0; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

// One workgroup per token: fold its read slots (first occurrence carries the sum of the
// weights of every entry with that slot, in entry order).
__global__ void __launch_bounds__(kBwdBlock) bwd_lead_kernel(BwdArgs a) {
    __shared__ int32_t ids[kMaxWidth];
    const int64_t tok = blockIdx.x;
    const int p = int(tok / a.T), t = int(tok % a.T);
    const int r = threadIdx.x;
    if (r < a.R) ids[r] = load_id(a.q_idx, tok * a.R + r, a.q_id8);
    __syncthreads();
    if (r >= a.R) return;
    float2 out = make_float2(0.0f, 0.0f);
    if (t < live_tokens(a, p)) {
        const int32_t s = ids[r];
        bool first = true;
        for (int j = 0; j < r; ++j) first = first && ids[j] != s;
        if (first) {
            float q = 0.0f;
            for (int j = r; j < a.R; ++j)
                if (ids[j] == s) q += a.q_val[tok * a.R + j];
            out = make_float2(q, 1.0f);
        }
    }
    a.lead[tok * a.R + r] = out;
}

struct BwdSmem {
    int32_t kid[kMaxWidth], qid[kMaxWidth];
    float kv[kMaxWidth], gam[kMaxWidth], lka[kMaxWidth];
    float2 qlead[kMaxWidth];
    float red[kBwdBlock];
    float lv[kWave], lgo[kWave], ldelta[kWave], lvr[kWave], lgret[kWave];
    float beta;
    // followed by old[W * S] and gbw[W * S] (dynamic)
};

size_t bwd_lds_bytes(int W, int S) { return sizeof(BwdSmem) + size_t(2) * W * S * sizeof(float); }

// Lanes are (entry e, column c): c = tid % S, entries e, e + E, ... with E = 256 / S.
// Loads of the token's parameters into LDS (the caller synchronizes afterwards).
__device__ __forceinline__ void load_token(const BwdArgs &a, BwdSmem &sm, int64_t tok, int col, bool colok,
                                           bool reads) {
    const int tid = threadIdx.x;
    if (tid < a.W) {
        const int32_t s = clamp_row(load_id(a.k_idx, tok * a.W + tid, a.k_id8), a.M);
        sm.kid[tid] = s;
        sm.kv[tid] = a.k_val[tok * a.W + tid];
        sm.gam[tid] = __expf(a.g[tok * a.G + (a.G == 1 ? 0 : tid)]);
    }
    if (reads && tid < a.R) {
        sm.qid[tid] = clamp_row(load_id(a.q_idx, tok * a.R + tid, a.q_id8), a.M);
        sm.qlead[tid] = a.lead[tok * a.R + tid];
    }
    if (tid < a.S) {
        const int64_t o = tok * a.hd + (colok ? col : 0);
        sm.lv[tid] = colok ? a.v[o] : 0.0f;
        if (reads) sm.lgo[tid] = colok ? a.go[o] : 0.0f;
    }
    if (tid == 0) sm.beta = a.beta[tok];
}

// old_w into LDS and the partial retrieval sums of this lane into sm.red. From the bank
// (forward replay, saving old_w) or from the saved rows (reverse): the same arithmetic, so
// both passes see the same delta.
template <bool kReplay>
__device__ __forceinline__ void retrieve(const BwdArgs &a, BwdSmem &sm, float *old, float *bank, int64_t tok,
                                         int e, int c, int E, int col, bool colok) {
    float acc = 0.0f;
    const int cc = colok ? col : 0;
    for (int w0 = 0; w0 < a.W; w0 += E) {
        const int w = w0 + e;
        if (w < a.W) {
            float o;
            float *sp = a.snap + (tok * a.W + w) * a.hd + cc;
            if (kReplay) {
                o = colok ? bank[int64_t(sm.kid[w]) * a.hd + cc] : 0.0f;
                if (colok) *sp = o;
            } else {
                o = colok ? *sp : 0.0f;
            }
            old[w * a.S + c] = o;
            acc = __builtin_fmaf(sm.kv[w], sm.gam[w] * o, acc);
        }
    }
    sm.red[threadIdx.x] = acc;
}

// ret = sum over entry groups in ascending order; delta = beta (v - ret). Lanes tid < S.
__device__ __forceinline__ void finish_delta(const BwdArgs &a, BwdSmem &sm, int E) {
    const int c = threadIdx.x;
    float ret = 0.0f;
    for (int e = 0; e < E; ++e) ret += sm.red[e * a.S + c];
    const float vr = sm.lv[c] - ret;
    sm.lvr[c] = vr;
    sm.ldelta[c] = sm.beta * vr;
}

__global__ void __launch_bounds__(kBwdBlock) bwd_sweep_kernel(BwdArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    BwdSmem &sm = *reinterpret_cast<BwdSmem *>(smem_raw);
    float *old = reinterpret_cast<float *>(smem_raw + sizeof(BwdSmem));
    float *gbw = old + a.W * a.S;
    const int sl = blockIdx.x % a.NS, p = blockIdx.x / a.NS;
    const int tid = threadIdx.x, S = a.S, E = kBwdBlock / S;
    const int c = tid % S, e = tid / S;
    const int col = sl * S + c;
    const bool colok = col < a.hd;
    const int cc = colok ? col : 0;
    float *bank = a.bank + int64_t(p) * a.M * a.hd;
    float *gb = a.gbank + int64_t(p) * a.M * a.hd;
    const int J = bwd_parts(a.W, a.R);
    const int32_t n = live_tokens(a, p);

    // forward replay
    for (int t = 0; t < n; ++t) {
        const int64_t tok = int64_t(p) * a.T + t;
        load_token(a, sm, tok, col, colok, false);
        __syncthreads();
        retrieve<true>(a, sm, old, bank, tok, e, c, E, col, colok);
        __syncthreads();
        if (tid < S) finish_delta(a, sm, E);
        __syncthreads();
        for (int w0 = 0; w0 < a.W; w0 += E) {
            const int w = w0 + e;
            if (w < a.W && colok)
                bank[int64_t(sm.kid[w]) * a.hd + cc] =
                    __builtin_fmaf(sm.kv[w], sm.ldelta[c], sm.gam[w] * old[w * S + c]);
        }
        __syncthreads();
    }

    // reverse
    for (int t = n - 1; t >= 0; --t) {
        const int64_t tok = int64_t(p) * a.T + t;
        float *pt = a.part + ((int64_t(p) * a.NS + sl) * a.T + t) * J;
        load_token(a, sm, tok, col, colok, true);
        __syncthreads();
        // reading: grad_q_r = <go, bank[s_r]> (bank after the token); gb[s_r] += q_r go
        for (int r0 = 0; r0 < a.R; r0 += E) {
            const int r = r0 + e;
            const int rr = r < a.R ? r : a.R - 1;
            const int64_t o = int64_t(sm.qid[rr]) * a.hd + cc;
            const float row = colok ? bank[o] : 0.0f;
            const float d = group_sum(sm.lgo[c] * row, S);
            const float2 ld = sm.qlead[rr];
            if (r < a.R) {
                if (c == 0) pt[2 * a.W + r] = d;
                if (colok && ld.y != 0.0f) gb[o] = __builtin_fmaf(ld.x, sm.lgo[c], gb[o]);
            }
        }
        retrieve<false>(a, sm, old, bank, tok, e, c, E, col, colok);
        __syncthreads();
        if (tid < S) finish_delta(a, sm, E);
        __syncthreads();
        // write: gdelta = sum_w k_w gb[s_w]; grad_k_w = <gb[s_w], delta>
        {
            float acc = 0.0f;
            for (int w0 = 0; w0 < a.W; w0 += E) {
                const int w = w0 + e;
                const int ww = w < a.W ? w : a.W - 1;
                const float x = colok ? gb[int64_t(sm.kid[ww]) * a.hd + cc] : 0.0f;
                const float d = group_sum(x * sm.ldelta[c], S);
                if (w < a.W) {
                    gbw[w * S + c] = x;
                    acc = __builtin_fmaf(sm.kv[w], x, acc);
                    if (c == 0) sm.lka[w] = d;
                }
            }
            sm.red[tid] = acc;
        }
        __syncthreads();
        if (tid < S) {
            float gd = 0.0f;
            for (int q = 0; q < E; ++q) gd += sm.red[q * S + tid];
            if (colok) a.gv[tok * a.hd + col] = sm.beta * gd;
            sm.lgret[tid] = -sm.beta * gd;
            const float gbeta = group_sum(gd * sm.lvr[tid], S);
            if (tid == 0) pt[2 * a.W + a.R] = gbeta;
        }
        __syncthreads();
        // retrieval and decay: grad_k_w += <gret, dec_w>; gdec = gb + k gret;
        // grad_g_w = <gdec, dec_w>; gb[s_w] = gamma gdec; bank[s_w] = old_w
        for (int w0 = 0; w0 < a.W; w0 += E) {
            const int w = w0 + e;
            const int ww = w < a.W ? w : a.W - 1;
            const float o = old[ww * S + c];
            const float dec = sm.gam[ww] * o;
            const float gret = sm.lgret[c];
            const float gdec = __builtin_fmaf(sm.kv[ww], gret, gbw[ww * S + c]);
            const float dk = group_sum(gret * dec, S);
            const float dg = group_sum(gdec * dec, S);
            if (w < a.W) {
                if (colok) {
                    const int64_t ro = int64_t(sm.kid[w]) * a.hd + cc;
                    gb[ro] = sm.gam[w] * gdec;
                    bank[ro] = o;
                }
                if (c == 0) {
                    pt[w] = sm.lka[w] + dk;
                    pt[a.W + w] = dg;
                }
            }
        }
        __syncthreads();
    }
}

// One workgroup per token: the slices' dots summed in ascending slice order; padding
// tokens get zeros (grad_v too).
__global__ void __launch_bounds__(kBwdBlock) bwd_reduce_kernel(BwdArgs a) {
    __shared__ float gsum[kMaxWidth];
    const int64_t tok = blockIdx.x;
    const int p = int(tok / a.T), t = int(tok % a.T);
    const int J = bwd_parts(a.W, a.R);
    const bool live = t < live_tokens(a, p);
    for (int j = threadIdx.x; j < J; j += kBwdBlock) {
        float s = 0.0f;
        if (live)
            for (int sl = 0; sl < a.NS; ++sl) s += a.part[((int64_t(p) * a.NS + sl) * a.T + t) * J + j];
        if (j < a.W) {
            a.gk[tok * a.W + j] = s;
        } else if (j < 2 * a.W) {
            if (a.G == 1) gsum[j - a.W] = s;
            else a.gg[tok * a.W + (j - a.W)] = s;
        } else if (j < 2 * a.W + a.R) {
            a.gq[tok * a.R + (j - 2 * a.W)] = s;
        } else {
            a.gbeta[tok] = s;
        }
    }
    if (!live)
        for (int x = threadIdx.x; x < a.hd; x += kBwdBlock) a.gv[tok * a.hd + x] = 0.0f;
    if (a.G == 1) {
        __syncthreads();
        if (threadIdx.x == 0) {
            float s = 0.0f;
            for (int w = 0; w < a.W; ++w) s += gsum[w];
            a.gg[tok] = s;
        }
    }
}

hipError_t bwd_prepare() {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(bwd_sweep_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(bwd_lds_bytes(kMaxWidth, kWave)));
}

// Columns per slice: the widest power of two up to 64 (and up to the head) that still
// gives 256 workgroups, else 4. SDM_BWD_SLICE (4, 8, 16, 32 or 64) overrides it, for tests
// and tuning sweeps (the results depend on it only through the order of the column sums).
int bwd_slice_cols(int P, int hd) {
    if (const char *env = getenv("SDM_BWD_SLICE")) {
        const int s = atoi(env);
        if (s == 4 || s == 8 || s == 16 || s == 32 || s == 64) return s;
    }
    int S = 4;
    while (S < 64 && S < hd) S <<= 1;
    while (S > 4 && int64_t(P) * ((hd + S - 1) / S) < 256) S >>= 1;
    return S;
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t st) {
    const int64_t toks = int64_t(a.P) * a.T;
    bwd_lead_kernel<<<dim3(unsigned(toks)), dim3(kBwdBlock), 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bwd_sweep_kernel<<<dim3(unsigned(a.P * a.NS)), dim3(kBwdBlock), bwd_lds_bytes(a.W, a.S), st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_reduce_kernel<<<dim3(unsigned(toks)), dim3(kBwdBlock), 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace sdm

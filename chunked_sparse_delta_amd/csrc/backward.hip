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

#include <type_traits>

#include "backward.h"

namespace sdm {

__device__ __forceinline__ int32_t live_tokens(const BwdArgs &a, int p) {
    int32_t n = a.valid ? a.valid[p] : a.T;
    return n < 0 ? 0 : (n > a.T ? a.T : n);
}

// Element i of an array in the bank dtype T, widened to float32.
template <typename T>
__device__ __forceinline__ float ldf(const void *p, int64_t i) {
    return to_f32(static_cast<const T *>(p)[i]);
}

__device__ __forceinline__ int32_t clamp_row(int32_t s, int64_t M) {
    return s < 0 ? 0 : (s >= M ? int32_t(M - 1) : s);
}

// (stream, slice) of a sweep workgroup. Workgroups are dealt to the 8 XCDs round-robin;
// when their count divides by 8, consecutive slices of one stream go to one XCD, so the
// stream's token values (read by every slice, twice) are fetched into one L2 only.
__device__ __forceinline__ void sweep_owner(const BwdArgs &a, int &p, int &sl) {
    const int nwg = a.P * a.NS, b = blockIdx.x;
    const int lin = nwg % kXcds == 0 ? (b % kXcds) * (nwg / kXcds) + b / kXcds : b;
    p = lin / a.NS;
    sl = lin % a.NS;
}

// Sum over the S consecutive lanes of a group (butterfly: every lane gets the same bits).
__device__ __forceinline__ float group_sum(float x, int S) {
    for (int m = S >> 1; m > 0; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

// One workgroup per token: fold its read slots (first occurrence carries the sum of the
// weights of every entry with that slot, in entry order).
template <typename T>
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
                if (ids[j] == s) q += ldf<T>(a.q_val, tok * a.R + j);
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

size_t bwd_lds_bytes(int W, int S, int64_t M, bool res) {
    return res ? kResRed * sizeof(float) + size_t(2) * M * S * sizeof(float)
               : sizeof(BwdSmem) + size_t(2) * W * S * sizeof(float);
}

// Lanes are (entry e, column c): c = tid % S, entries e, e + E, ... with E = 256 / S.
// Loads of the token's parameters into LDS (the caller synchronizes afterwards).
template <int NT, typename T>
__device__ __forceinline__ void load_token(const BwdArgs &a, BwdSmem &sm, int64_t tok, int col, bool colok,
                                           bool reads) {
    const int tid = threadIdx.x;
    for (int w = tid; w < a.W; w += NT) {
        const int32_t s = clamp_row(load_id(a.k_idx, tok * a.W + w, a.k_id8), a.M);
        sm.kid[w] = s;
        sm.kv[w] = ldf<T>(a.k_val, tok * a.W + w);
        sm.gam[w] = __expf(a.g[tok * a.G + (a.G == 1 ? 0 : w)]);
    }
    if (reads)
        for (int r = tid; r < a.R; r += NT) {
            sm.qid[r] = clamp_row(load_id(a.q_idx, tok * a.R + r, a.q_id8), a.M);
            sm.qlead[r] = a.lead[tok * a.R + r];
        }
    if (tid < a.S) {
        const int64_t o = tok * a.hd + (colok ? col : 0);
        sm.lv[tid] = colok ? ldf<T>(a.v, o) : 0.0f;
        if (reads) sm.lgo[tid] = colok ? ldf<T>(a.go, o) : 0.0f;
    }
    if (tid == 0) sm.beta = a.beta[tok];
}

// old_w into LDS and the partial retrieval sums of this lane into sm.red. From the bank
// (forward replay, saving old_w) or from the saved rows (reverse): the same arithmetic, so
// both passes see the same delta. Rows are addressed as bk[row * rs]: bk already points at
// the lane's column (of the bank in memory, or of the workgroup's slice held in LDS).
template <bool kReplay, int NT>
__device__ __forceinline__ void retrieve(const BwdArgs &a, BwdSmem &sm, float *old, float *bk, int64_t rs,
                                         int64_t snapt, int e, int c, bool colok) {
    const int E = NT / a.S;
    float acc = 0.0f;
    for (int w0 = 0; w0 < a.W; w0 += E) {
        const int w = w0 + e;
        if (w < a.W) {
            float o;
            const int64_t sp = snapt + w * a.S + c;
            if (kReplay) {
                o = colok ? bk[int64_t(sm.kid[w]) * rs] : 0.0f;
                if (colok) snap_st(a, sp, o);
            } else {
                o = colok ? snap_ld(a, sp) : 0.0f;
            }
            old[w * a.S + c] = o;
            acc = __builtin_fmaf(sm.kv[w], sm.gam[w] * o, acc);
        }
    }
    sm.red[threadIdx.x] = acc;
}

// ret = sum over entry groups in ascending order (groups past the last entry hold 0 and are
// skipped); delta = beta (v - ret). Lanes tid < S.
__device__ __forceinline__ void finish_delta(const BwdArgs &a, BwdSmem &sm, int E) {
    const int c = threadIdx.x;
    const int ne = a.W < E ? a.W : E;
    float ret = 0.0f;
    for (int e = 0; e < ne; ++e) ret += sm.red[e * a.S + c];
    const float vr = sm.lv[c] - ret;
    sm.lvr[c] = vr;
    sm.ldelta[c] = sm.beta * vr;
}

// The sweep in memory: NT threads per (stream, column slice), rows read and written in the
// bank and the bank gradient themselves, token values staged through LDS.
template <int NT, typename T>
__global__ void __launch_bounds__(NT) bwd_sweep_kernel(BwdArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    BwdSmem &sm = *reinterpret_cast<BwdSmem *>(smem_raw);
    float *old = reinterpret_cast<float *>(smem_raw + sizeof(BwdSmem));
    float *gbw = old + a.W * a.S;
    int p, sl;
    sweep_owner(a, p, sl);
    const int tid = threadIdx.x, S = a.S, E = NT / S;
    const int c = tid % S, e = tid / S;
    const int col = sl * S + c;
    const bool colok = col < a.hd;
    const int cc = colok ? col : 0;
    float *bk = a.work + int64_t(p) * a.bstride + cc;
    float *gk = a.gbank + int64_t(p) * a.bstride + cc;
    const int64_t rs = a.hd;
    const int64_t snapw = snap_slice(a, p, sl);   // this slice's saved rows [T][W][S]
    const int J = bwd_parts(a.W, a.R);
    const int32_t n = live_tokens(a, p);

    // forward replay
    for (int t = 0; t < n; ++t) {
        const int64_t tok = int64_t(p) * a.T + t;
        load_token<NT, T>(a, sm, tok, col, colok, false);
        __syncthreads();
        retrieve<true, NT>(a, sm, old, bk, rs, snapw + int64_t(t) * a.W * S, e, c, colok);
        __syncthreads();
        if (tid < S) finish_delta(a, sm, E);
        __syncthreads();
        for (int w0 = 0; w0 < a.W; w0 += E) {
            const int w = w0 + e;
            if (w < a.W && colok)
                bk[int64_t(sm.kid[w]) * rs] = __builtin_fmaf(sm.kv[w], sm.ldelta[c], sm.gam[w] * old[w * S + c]);
        }
        __syncthreads();
    }

    // reverse
    for (int t = n - 1; t >= 0; --t) {
        const int64_t tok = int64_t(p) * a.T + t;
        float *pt = a.part + ((int64_t(p) * a.NS + sl) * a.T + t) * J;
        load_token<NT, T>(a, sm, tok, col, colok, true);
        __syncthreads();
        // reading: grad_q_r = <go, bank[s_r]> (bank after the token); gb[s_r] += q_r go
        for (int r0 = 0; r0 < a.R; r0 += E) {
            const int r = r0 + e;
            const int rr = r < a.R ? r : a.R - 1;
            const int64_t o = int64_t(sm.qid[rr]) * rs;
            const float row = colok ? bk[o] : 0.0f;
            const float d = group_sum(sm.lgo[c] * row, S);
            const float2 ld = sm.qlead[rr];
            if (r < a.R) {
                if (c == 0) pt[2 * a.W + r] = d;
                if (colok && ld.y != 0.0f) gk[o] = __builtin_fmaf(ld.x, sm.lgo[c], gk[o]);
            }
        }
        retrieve<false, NT>(a, sm, old, bk, rs, snapw + int64_t(t) * a.W * S, e, c, colok);
        __syncthreads();
        if (tid < S) finish_delta(a, sm, E);
        __syncthreads();
        // write: gdelta = sum_w k_w gb[s_w]; grad_k_w = <gb[s_w], delta>
        {
            float acc = 0.0f;
            for (int w0 = 0; w0 < a.W; w0 += E) {
                const int w = w0 + e;
                const int ww = w < a.W ? w : a.W - 1;
                const float x = colok ? gk[int64_t(sm.kid[ww]) * rs] : 0.0f;
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
            const int ne = a.W < E ? a.W : E;
            float gd = 0.0f;
            for (int q = 0; q < ne; ++q) gd += sm.red[q * S + tid];
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
                    const int64_t ro = int64_t(sm.kid[w]) * rs;
                    gk[ro] = sm.gam[w] * gdec;
                    bk[ro] = o;
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

// ---------------------------------------------------------------------------------------
// Resident sweep: one wavefront per (stream, column slice) whose slices of the bank and of
// the bank gradient fit in LDS together. Lane (e, c) owns column c of entries e, e + E, ..
// (E = 64 / S, at most KJ entries of each kind per lane). A token's slot ids, weights and
// gates, v, grad_out and saved rows are loaded straight into the lanes that use them, D
// tokens ahead, so the only memory a token waits on is LDS; sums over the entries of a
// column go through a small LDS array read back by every lane of the column, sums over
// the columns of an entry through DPP / lane shuffles. A wavefront's LDS operations take
// effect in program order, so no workgroup barrier is needed.
// ---------------------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the S consecutive lanes of a group (S a power of two, 4..64); every lane of the
// group ends with the same bits (each step adds two equal-shaped partial sums).
__device__ __forceinline__ float lane_group_sum(float x, int S) {
    x = dpp_add<0xB1>(x);                 // quad_perm [1, 0, 3, 2]
    x = dpp_add<0x4E>(x);                 // quad_perm [2, 3, 0, 1]
    if (S >= 8) x = dpp_add<0x141>(x);    // lane i of 8 reads lane 7 - i
    if (S >= 16) x = dpp_add<0x140>(x);   // lane i of 16 reads lane 15 - i
    if (S >= 32) x += __shfl_xor(x, 16, kWave);
    if (S >= 64) x += __shfl_xor(x, 32, kWave);
    return x;
}

// Slot id i of an int32 or int64 id array without a branch: ids lie in [0, 2^31), so the
// low (first, little-endian) word of an int64 id is the id.
__device__ __forceinline__ int32_t id_word(const void *base, int64_t i, int32_t id8) {
    return static_cast<const int32_t *>(base)[i << id8];
}

template <int KJ>
struct ResTok {
    int32_t kid[KJ], qid[KJ];
    float kv[KJ], gam[KJ], ql[KJ], qf[KJ], snap[KJ];
    float v, go, beta;
};

// Token tok's values for lane (e, c); every load is issued (indices clamped into range),
// so the loads never wait on a branch.
// Token t of the stream whose first token is tok0; snapw: the slice's saved rows [T][W][S].
template <int KJ, bool kRev, typename T>
__device__ __forceinline__ void res_load(const BwdArgs &a, ResTok<KJ> &x, int64_t tok0, int t, int64_t snapw,
                                         int e, int E, int c, int cc) {
    const int64_t tok = tok0 + t;
    const int64_t snapt = snapw + int64_t(t) * a.W * a.S;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
        const int w = min(e + j * E, a.W - 1);
        x.kid[j] = clamp_row(id_word(a.k_idx, tok * a.W + w, a.k_id8), a.M);
        x.kv[j] = ldf<T>(a.k_val, tok * a.W + w);
        x.gam[j] = __expf(a.g[tok * a.G + (a.G == 1 ? 0 : w)]);
        if (kRev) {
            const int r = min(e + j * E, a.R - 1);
            x.qid[j] = clamp_row(id_word(a.q_idx, tok * a.R + r, a.q_id8), a.M);
            const float2 ld = a.lead[tok * a.R + r];
            x.ql[j] = ld.x;
            x.qf[j] = ld.y;
            x.snap[j] = snap_ld(a, snapt + w * a.S + c);
        }
    }
    x.v = ldf<T>(a.v, tok * a.hd + cc);
    if (kRev) x.go = ldf<T>(a.go, tok * a.hd + cc);
    x.beta = a.beta[tok];
}

// RES: rows in LDS as above; else the same wavefront works on rows in memory (the bank's
// float32 working rows and the bank gradient, row stride head_dim): a wavefront's memory
// operations take effect in program order for all its lanes, so it needs no barrier either.
template <int KJ, int D, typename T, bool RES>
__global__ void __launch_bounds__(kWave) bwd_res_kernel(BwdArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    float *red = reinterpret_cast<float *>(smem_raw);   // [S][E] entry-group partial sums
    float *lres = red + kResRed;                         // bank slice [M][S], then gradient slice [M][S]
    int p, sl;
    sweep_owner(a, p, sl);
    const int lane = threadIdx.x, S = a.S, E = kWave / S;
    const int c = lane % S, e = lane / S;
    const int col = sl * S + c;
    const bool colok = col < a.hd;
    const int cc = colok ? col : 0;
    const int ne = a.W < E ? a.W : E;   // entry groups holding a write entry
    const T *bank_g = static_cast<const T *>(a.bank) + int64_t(p) * a.bstride;
    float *gb_g = a.gbank + int64_t(p) * a.bstride;
    const int64_t MS = a.M * S;
    if (RES) {
        constexpr int kB = 16;
        for (int64_t i0 = lane; i0 < MS; i0 += int64_t(kB) * kWave) {
            float xb[kB], xg[kB];
#pragma unroll
            for (int k = 0; k < kB; ++k) {
                const int64_t i = i0 + int64_t(k) * kWave;
                const int cg = sl * S + int(i % S);
                const bool ok = i < MS && cg < a.hd;
                const int64_t o = ok ? (i / S) * a.hd + cg : 0;
                xb[k] = to_f32(bank_g[o]);
                xg[k] = gb_g[o];
                xb[k] = ok ? xb[k] : 0.0f;
                xg[k] = ok ? xg[k] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < kB; ++k) {
                const int64_t i = i0 + int64_t(k) * kWave;
                if (i < MS) {
                    lres[i] = xb[k];
                    lres[MS + i] = xg[k];
                }
            }
        }
    }
    __syncthreads();
    float *bk = RES ? lres + c : a.work + int64_t(p) * a.bstride + cc;
    float *gk = RES ? lres + MS + c : gb_g + cc;
    const int64_t rs = RES ? S : a.hd;   // row stride of bk and gk
    const int J = bwd_parts(a.W, a.R);
    const int32_t n = live_tokens(a, p);
    const int64_t tok0 = int64_t(p) * a.T;
    const int64_t snapw = snap_slice(a, p, sl);   // this slice's saved rows [T][W][S]

    // ret over the column's entry groups, in ascending group order (every lane of the
    // column reads the same partials, so all get the same bits)
    auto column_sum = [&](float part) {
        red[c * E + e] = part;
        __builtin_amdgcn_wave_barrier();
        float s = 0.0f;
        for (int q = 0; q < ne; ++q) s += red[c * E + q];
        __builtin_amdgcn_wave_barrier();
        return s;
    };

    // forward replay of token t from its prefetched values
    auto fwd_token = [&](ResTok<KJ> &cur, int t) {
        float old[KJ];
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const int w = e + j * E;
            old[j] = colok ? bk[int64_t(cur.kid[j]) * rs] : 0.0f;
            if (w < a.W) {
                if (colok) snap_st(a, snapw + (int64_t(t) * a.W + w) * S + c, old[j]);
                acc = __builtin_fmaf(cur.kv[j], cur.gam[j] * old[j], acc);
            }
        }
        const float ret = column_sum(acc);
        const float delta = cur.beta * ((colok ? cur.v : 0.0f) - ret);
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const int w = e + j * E;
            if (w < a.W && colok)
                bk[int64_t(cur.kid[j]) * rs] = __builtin_fmaf(cur.kv[j], delta, cur.gam[j] * old[j]);
        }
        __builtin_amdgcn_wave_barrier();
    };

    // the reverse of token t, from its prefetched values and saved rows
    auto rev_token = [&](ResTok<KJ> &cur, int t) {
        const int64_t tok = tok0 + t;
        float *pt = a.part + ((int64_t(p) * a.NS + sl) * a.T + t) * J;
        const float go = colok ? cur.go : 0.0f;
        // reading: grad_q_r = <go, bank[s_r]>; gb[s_r] += (summed q) go at a slot's first entry
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const int r = e + j * E;
            const int64_t o = int64_t(cur.qid[j]) * rs;
            const float d = lane_group_sum(go * (colok ? bk[o] : 0.0f), S);
            if (r < a.R) {
                if (c == 0) pt[2 * a.W + r] = d;
                if (colok && cur.qf[j] != 0.0f) gk[o] = __builtin_fmaf(cur.ql[j], go, gk[o]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        // the token's retrieval and delta, recomputed from the saved rows
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const int w = e + j * E;
            const float o = colok ? cur.snap[j] : 0.0f;
            cur.snap[j] = o;
            if (w < a.W) acc = __builtin_fmaf(cur.kv[j], cur.gam[j] * o, acc);
        }
        const float ret = column_sum(acc);
        const float vr = (colok ? cur.v : 0.0f) - ret;
        const float delta = cur.beta * vr;
        // write: gdelta = sum_w k_w gb[s_w]; grad_k_w = <gb[s_w], delta>
        float gbw[KJ], lka[KJ];
        float acc2 = 0.0f;
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const int w = e + j * E;
            gbw[j] = colok ? gk[int64_t(cur.kid[j]) * rs] : 0.0f;
            lka[j] = lane_group_sum(gbw[j] * delta, S);
            if (w < a.W) acc2 = __builtin_fmaf(cur.kv[j], gbw[j], acc2);
        }
        const float gd = column_sum(acc2);
        const float gret = -cur.beta * gd;
        const float gbeta = lane_group_sum(gd * vr, S);
        if (e == 0) {
            if (colok) a.gv[tok * a.hd + col] = cur.beta * gd;
            if (c == 0) pt[2 * a.W + a.R] = gbeta;
        }
        // retrieval and decay, then the bank row as it was before the token
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const int w = e + j * E;
            const float dec = cur.gam[j] * cur.snap[j];
            const float gdec = __builtin_fmaf(cur.kv[j], gret, gbw[j]);
            const float dk = lane_group_sum(gret * dec, S);
            const float dg = lane_group_sum(gdec * dec, S);
            if (w < a.W) {
                if (colok) {
                    const int64_t ro = int64_t(cur.kid[j]) * rs;
                    gk[ro] = cur.gam[j] * gdec;
                    bk[ro] = cur.snap[j];
                }
                if (c == 0) {
                    pt[w] = lka[j] + dk;
                    pt[a.W + w] = dg;
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    };

    // Token values are prefetched D tokens ahead into a ring of registers: the loop runs
    // whole rounds of D tokens, unrolled, so each slot is a fixed set of registers and every
    // round issues the same loads (refills past the end reload the last token); slot d of a
    // round holds the token of the round's d-th step and is refilled with the one D tokens
    // further on. The last n % D tokens load their values as they go.
    ResTok<KJ> ring[D];
    const int last = n > 0 ? n - 1 : 0;
    const int nfull = n - n % D;
#pragma unroll
    for (int d = 0; d < D; ++d) res_load<KJ, false, T>(a, ring[d], tok0, min(d, last), snapw, e, E, c, cc);
    for (int t0 = 0; t0 < nfull; t0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            fwd_token(ring[d], t0 + d);
            res_load<KJ, false, T>(a, ring[d], tok0, min(t0 + d + D, last), snapw, e, E, c, cc);
        }
    }
    for (int t = nfull; t < n; ++t) {
        ResTok<KJ> x;
        res_load<KJ, false, T>(a, x, tok0, t, snapw, e, E, c, cc);
        fwd_token(x, t);
    }
    // reverse: the first n % D tokens from the end go one by one, then whole rounds
    for (int t = n - 1; t >= nfull; --t) {
        ResTok<KJ> x;
        res_load<KJ, true, T>(a, x, tok0, t, snapw, e, E, c, cc);
        rev_token(x, t);
    }
    const int top = nfull - 1;
#pragma unroll
    for (int d = 0; d < D; ++d) res_load<KJ, true, T>(a, ring[d], tok0, max(top - d, 0), snapw, e, E, c, cc);
    for (int t0 = top; t0 >= 0; t0 -= D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            rev_token(ring[d], t0 - d);
            res_load<KJ, true, T>(a, ring[d], tok0, max(t0 - d - D, 0), snapw, e, E, c, cc);
        }
    }
    if (RES) {
        __syncthreads();
        // with bfloat16 snapshot rows (float32 banks only) the restored rows differ from the
        // bank's entry rows: the slice goes back to the bank with the gradient
        float *wk = a.snap_bf16 ? a.work + int64_t(p) * a.bstride : nullptr;
        for (int64_t i = lane; i < MS; i += kWave) {
            const int cg = sl * S + int(i % S);
            if (cg < a.hd) {
                gb_g[(i / S) * a.hd + cg] = lres[MS + i];
                if (wk) wk[(i / S) * a.hd + cg] = lres[i];
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Paired resident sweep: as the resident sweep with one entry of each kind per lane, for
// shapes where a token's entries fill at most half of the 64 / S entry groups. Tokens go
// in pairs (2j, 2j + 1), the first half of the entry groups taking token 2j and the second
// token 2j + 1; a pair whose tokens select disjoint rows (written or read: bwd_pairs_kernel)
// runs as one step, since neither token then sees a row the other changes; any other pair
// runs as two steps, one half at a time, in token order (reverse order going back).
// The sums are those of the resident sweep, term for term, so both give the same bits.
// ---------------------------------------------------------------------------------------

// pairs[p][j] = 1 if tokens 2j and 2j + 1 of stream p are both live and select disjoint rows.
// Pairs are taken only when W, R <= kPairMax (a token's entries fill at most half of at most
// 16 entry groups), so both tokens' ids sit in registers.

__global__ void __launch_bounds__(kBwdBlock) bwd_pairs_kernel(BwdArgs a) {
    const int npm = (a.T + 1) / 2;
    const int64_t idx = int64_t(blockIdx.x) * kBwdBlock + threadIdx.x;
    if (idx >= int64_t(a.P) * npm) return;
    const int p = int(idx / npm), j = int(idx % npm);
    const int64_t t0 = int64_t(p) * a.T + 2 * j;
    int32_t flag = 0;
    if (2 * j + 1 < live_tokens(a, p)) {
        int32_t x0[2 * kPairMax], x1[2 * kPairMax];
#pragma unroll
        for (int x = 0; x < 2 * kPairMax; ++x) {
            const bool wr = x < kPairMax;
            const int k = wr ? x : x - kPairMax;
            const int kk = min(k, (wr ? a.W : a.R) - 1);   // past the token's entries: repeat its last
            x0[x] = wr ? clamp_row(id_word(a.k_idx, t0 * a.W + kk, a.k_id8), a.M)
                       : clamp_row(id_word(a.q_idx, t0 * a.R + kk, a.q_id8), a.M);
            x1[x] = wr ? clamp_row(id_word(a.k_idx, (t0 + 1) * a.W + kk, a.k_id8), a.M)
                       : clamp_row(id_word(a.q_idx, (t0 + 1) * a.R + kk, a.q_id8), a.M);
        }
        bool disjoint = true;
#pragma unroll
        for (int x = 0; x < 2 * kPairMax; ++x)
#pragma unroll
            for (int y = 0; y < 2 * kPairMax; ++y) disjoint = disjoint && x0[x] != x1[y];
        flag = disjoint ? 1 : 0;
    }
    a.pairs[idx] = flag;
}

template <int D, typename T>
__global__ void __launch_bounds__(kWave) bwd_res_pair_kernel(BwdArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    float *red = reinterpret_cast<float *>(smem_raw);   // [S][E] entry-group partial sums
    float *lres = red + kResRed;                         // bank slice [M][S], then gradient slice [M][S]
    int p, sl;
    sweep_owner(a, p, sl);
    const int lane = threadIdx.x, S = a.S, E = kWave / S, EH = E / 2;
    const int c = lane % S, e = lane / S, h = e / EH, eh = e % EH;   // h: which token of the pair
    const int col = sl * S + c;
    const bool colok = col < a.hd;
    const int cc = colok ? col : 0;
    const int ne = a.W < EH ? a.W : EH;
    const T *bank_g = static_cast<const T *>(a.bank) + int64_t(p) * a.bstride;
    float *gb_g = a.gbank + int64_t(p) * a.bstride;
    const int64_t MS = a.M * S;
    {
        constexpr int kB = 16;
        for (int64_t i0 = lane; i0 < MS; i0 += int64_t(kB) * kWave) {
            float xb[kB], xg[kB];
#pragma unroll
            for (int k = 0; k < kB; ++k) {
                const int64_t i = i0 + int64_t(k) * kWave;
                const int cg = sl * S + int(i % S);
                const bool ok = i < MS && cg < a.hd;
                const int64_t o = ok ? (i / S) * a.hd + cg : 0;
                xb[k] = to_f32(bank_g[o]);
                xg[k] = gb_g[o];
                xb[k] = ok ? xb[k] : 0.0f;
                xg[k] = ok ? xg[k] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < kB; ++k) {
                const int64_t i = i0 + int64_t(k) * kWave;
                if (i < MS) {
                    lres[i] = xb[k];
                    lres[MS + i] = xg[k];
                }
            }
        }
    }
    __syncthreads();
    float *bk = lres + c, *gk = lres + MS + c;
    const int J = bwd_parts(a.W, a.R);
    const int32_t n = live_tokens(a, p);
    const int64_t tok0 = int64_t(p) * a.T;
    const int64_t snapw = snap_slice(a, p, sl);   // this slice's saved rows [T][W][S]
    const int32_t *pairs = a.pairs + int64_t(p) * ((a.T + 1) / 2);

    // sum over the entry groups of the lane's half, in ascending group order
    auto column_sum = [&](float part) {
        red[c * E + e] = part;
        __builtin_amdgcn_wave_barrier();
        float s = 0.0f;
        const int base = c * E + h * EH;
        for (int q = 0; q < ne; ++q) s += red[base + q];
        __builtin_amdgcn_wave_barrier();
        return s;
    };

    // forward replay of the lane's token t (act: the lane's half takes part in this step)
    auto fwd_token = [&](ResTok<1> &cur, int t, bool act) {
        const int w = eh;
        const bool on = act && w < a.W;
        const float old = colok ? bk[int64_t(cur.kid[0]) * S] : 0.0f;
        float acc = 0.0f;
        if (on) {
            if (colok) snap_st(a, snapw + (int64_t(t) * a.W + w) * S + c, old);
            acc = __builtin_fmaf(cur.kv[0], cur.gam[0] * old, acc);
        }
        const float ret = column_sum(acc);
        const float delta = cur.beta * ((colok ? cur.v : 0.0f) - ret);
        if (on && colok) bk[int64_t(cur.kid[0]) * S] = __builtin_fmaf(cur.kv[0], delta, cur.gam[0] * old);
        __builtin_amdgcn_wave_barrier();
    };

    // the reverse of the lane's token t
    auto rev_token = [&](ResTok<1> &cur, int t, bool act) {
        const int64_t tok = tok0 + t;
        float *pt = a.part + ((int64_t(p) * a.NS + sl) * a.T + t) * J;
        const float go = colok ? cur.go : 0.0f;
        const int w = eh, r = eh;
        const bool won = act && w < a.W, ron = act && r < a.R;
        {
            const int64_t o = int64_t(cur.qid[0]) * S;
            const float d = lane_group_sum(go * (colok ? bk[o] : 0.0f), S);
            if (ron) {
                if (c == 0) pt[2 * a.W + r] = d;
                if (colok && cur.qf[0] != 0.0f) gk[o] = __builtin_fmaf(cur.ql[0], go, gk[o]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        const float o = colok ? cur.snap[0] : 0.0f;
        const float ret = column_sum(won ? __builtin_fmaf(cur.kv[0], cur.gam[0] * o, 0.0f) : 0.0f);
        const float vr = (colok ? cur.v : 0.0f) - ret;
        const float delta = cur.beta * vr;
        const float gbw = colok ? gk[int64_t(cur.kid[0]) * S] : 0.0f;
        const float lka = lane_group_sum(gbw * delta, S);
        const float gd = column_sum(won ? __builtin_fmaf(cur.kv[0], gbw, 0.0f) : 0.0f);
        const float gret = -cur.beta * gd;
        const float gbeta = lane_group_sum(gd * vr, S);
        if (act && eh == 0) {
            if (colok) a.gv[tok * a.hd + col] = cur.beta * gd;
            if (c == 0) pt[2 * a.W + a.R] = gbeta;
        }
        const float dec = cur.gam[0] * o;
        const float gdec = __builtin_fmaf(cur.kv[0], gret, gbw);
        const float dk = lane_group_sum(gret * dec, S);
        const float dg = lane_group_sum(gdec * dec, S);
        if (won) {
            if (colok) {
                const int64_t ro = int64_t(cur.kid[0]) * S;
                gk[ro] = cur.gam[0] * gdec;
                bk[ro] = o;
            }
            if (c == 0) {
                pt[w] = lka + dk;
                pt[a.W + w] = dg;
            }
        }
        __builtin_amdgcn_wave_barrier();
    };

    // Pair j's values (the lane's token 2j + h, clamped to the last live one) are prefetched
    // D pairs ahead into a ring of registers, in whole unrolled rounds as in the resident
    // sweep; the remaining np % D pairs load as they go.
    const int last = n > 0 ? n - 1 : 0;
    const int np = (n + 1) / 2, lastp = np > 0 ? np - 1 : 0, npfull = np - np % D;
    auto tok_of = [&](int j) { return min(2 * j + h, last); };
    auto fwd_pair = [&](ResTok<1> &x, int fl, int j) {
        const int t = 2 * j + h;
        if (__builtin_amdgcn_readfirstlane(fl)) {
            fwd_token(x, t, t < n);
        } else {
            fwd_token(x, t, h == 0);
            fwd_token(x, t, h == 1 && t < n);
        }
    };
    auto rev_pair = [&](ResTok<1> &x, int fl, int j) {
        const int t = 2 * j + h;
        if (__builtin_amdgcn_readfirstlane(fl)) {
            rev_token(x, t, t < n);
        } else {
            rev_token(x, t, h == 1 && t < n);
            rev_token(x, t, h == 0);
        }
    };
    ResTok<1> ring[D];
    int fl[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        res_load<1, false, T>(a, ring[d], tok0, tok_of(min(d, lastp)), snapw, eh, EH, c, cc);
        fl[d] = pairs[min(d, lastp)];
    }
    for (int j0 = 0; j0 < npfull; j0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            fwd_pair(ring[d], fl[d], j0 + d);
            res_load<1, false, T>(a, ring[d], tok0, tok_of(min(j0 + d + D, lastp)), snapw, eh, EH, c, cc);
            fl[d] = pairs[min(j0 + d + D, lastp)];
        }
    }
    for (int j = npfull; j < np; ++j) {
        ResTok<1> x;
        res_load<1, false, T>(a, x, tok0, tok_of(j), snapw, eh, EH, c, cc);
        fwd_pair(x, pairs[j], j);
    }
    for (int j = np - 1; j >= npfull; --j) {
        ResTok<1> x;
        res_load<1, true, T>(a, x, tok0, tok_of(j), snapw, eh, EH, c, cc);
        rev_pair(x, pairs[j], j);
    }
    const int top = npfull - 1;
#pragma unroll
    for (int d = 0; d < D; ++d) {
        res_load<1, true, T>(a, ring[d], tok0, tok_of(max(top - d, 0)), snapw, eh, EH, c, cc);
        fl[d] = pairs[max(top - d, 0)];
    }
    for (int j0 = top; j0 >= 0; j0 -= D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            rev_pair(ring[d], fl[d], j0 - d);
            res_load<1, true, T>(a, ring[d], tok0, tok_of(max(j0 - d - D, 0)), snapw, eh, EH, c, cc);
            fl[d] = pairs[max(j0 - d - D, 0)];
        }
    }
    __syncthreads();
    float *wk = a.snap_bf16 ? a.work + int64_t(p) * a.bstride : nullptr;   // as in the unpaired sweep
    for (int64_t i = lane; i < MS; i += kWave) {
        const int cg = sl * S + int(i % S);
        if (cg < a.hd) {
            gb_g[(i / S) * a.hd + cg] = lres[MS + i];
            if (wk) wk[(i / S) * a.hd + cg] = lres[i];
        }
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

// The float32 working rows of a bfloat16 bank for the sweep in memory.
__global__ void __launch_bounds__(kBwdBlock) bwd_widen_kernel(const bf16 *bank, float *work, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * kBwdBlock + threadIdx.x; i < n; i += int64_t(gridDim.x) * kBwdBlock)
        work[i] = to_f32(bank[i]);
}

template <typename T>
hipError_t set_bwd_attrs() {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(bwd_sweep_kernel<kBwdBlock, T>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       int(bwd_lds_bytes(kMaxWidth, kWave, 0, false)));
    const void *res[] = {reinterpret_cast<const void *>(bwd_res_kernel<1, 4, T, true>),
                         reinterpret_cast<const void *>(bwd_res_kernel<2, 2, T, true>),
                         reinterpret_cast<const void *>(bwd_res_kernel<4, 1, T, true>)};
    for (const void *f : res)
        if (e == hipSuccess) e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kBwdMaxLds);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(bwd_res_pair_kernel<4, T>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kBwdMaxLds);
    return e;
}

hipError_t bwd_prepare() {
    hipError_t e = set_bwd_attrs<float>();
    return e == hipSuccess ? set_bwd_attrs<bf16>() : e;
}

// Entries of each kind per lane of the one-wavefront sweep: the smallest power of two up to
// kj_max that covers max(W, R) with 64 / S entry groups, or 0 where none does.
int bwd_res_entries(int W, int R, int S, int kj_max) {
    const int E = kWave / S, m = W > R ? W : R;
    for (int kj = 1; kj <= kj_max; kj <<= 1)
        if (kj * E >= m) return kj;
    return 0;
}

// Columns per slice, from shapes only: 4 where a token has at most kWaveMaxSlots slots of
// each kind (the one-wavefront sweeps: 16 entry groups per wavefront, and many workgroups
// whose chains hide each other's latency); otherwise the widest power of two up to 64 (and
// up to the head) that still gives 256 workgroups, else 4. SDM_BWD_SLICE (4, 8, 16, 32 or 64)
// overrides it, for tests and tuning sweeps (the results depend on it only through the
// order of the column sums).
int bwd_slice_cols(int P, int hd, int W, int R) {
    if (const char *env = getenv("SDM_BWD_SLICE")) {
        const int s = atoi(env);
        if (s == 4 || s == 8 || s == 16 || s == 32 || s == 64) return s;
    }
    if ((W > R ? W : R) <= kWaveMaxSlots) return 4;
    int S = 4;
    while (S < 64 && S < hd) S <<= 1;
    while (S > 4 && int64_t(P) * ((hd + S - 1) / S) < 256) S >>= 1;
    return S;
}

template <typename T>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t st, hipEvent_t *ev) {
    const int64_t toks = int64_t(a.P) * a.T;
    hipError_t e;
    if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
    bwd_lead_kernel<T><<<dim3(unsigned(toks)), dim3(kBwdBlock), 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (std::is_same<T, bf16>::value && a.res <= 0) {   // rows in memory: widen the bank first
        const int64_t n = (a.bstride ? int64_t(a.P) : 1) * a.M * a.hd;
        const int64_t blocks = (n + kBwdBlock - 1) / kBwdBlock;
        bwd_widen_kernel<<<dim3(unsigned(blocks < 4096 ? blocks : 4096)), dim3(kBwdBlock), 0, st>>>(
            static_cast<const bf16 *>(a.bank), a.work, n);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.pair) {
        const int64_t npairs = int64_t(a.P) * ((a.T + 1) / 2);
        bwd_pairs_kernel<<<dim3(unsigned((npairs + kBwdBlock - 1) / kBwdBlock)), dim3(kBwdBlock), 0, st>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
    const dim3 grid(unsigned(a.P * a.NS));
    const size_t lds = a.res > 0 ? bwd_lds_bytes(a.W, a.S, a.M, true)
                     : a.res < 0 ? size_t(kResRed) * sizeof(float) : bwd_lds_bytes(a.W, a.S, a.M, false);
    if (a.pair) bwd_res_pair_kernel<4, T><<<grid, dim3(kWave), lds, st>>>(a);
    else switch (a.res) {
        case 1: bwd_res_kernel<1, 4, T, true><<<grid, dim3(kWave), lds, st>>>(a); break;
        case 2: bwd_res_kernel<2, 2, T, true><<<grid, dim3(kWave), lds, st>>>(a); break;
        case 4: bwd_res_kernel<4, 1, T, true><<<grid, dim3(kWave), lds, st>>>(a); break;
        case -1: bwd_res_kernel<1, 4, T, false><<<grid, dim3(kWave), lds, st>>>(a); break;
        case -2: bwd_res_kernel<2, 4, T, false><<<grid, dim3(kWave), lds, st>>>(a); break;
        case -4: bwd_res_kernel<4, 2, T, false><<<grid, dim3(kWave), lds, st>>>(a); break;
        case -8: bwd_res_kernel<8, 2, T, false><<<grid, dim3(kWave), lds, st>>>(a); break;
        default: bwd_sweep_kernel<kBwdBlock, T><<<grid, dim3(kBwdBlock), lds, st>>>(a); break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
    bwd_reduce_kernel<<<dim3(unsigned(toks)), dim3(kBwdBlock), 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
    return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t st, hipEvent_t *ev) {
    return a.bf16 ? launch_bwd_t<bf16>(a, st, ev) : launch_bwd_t<float>(a, st, ev);
}

}  // namespace sdm

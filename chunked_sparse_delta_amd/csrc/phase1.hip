// Phase 1 of the chunked SDM forward on gfx950: the bank-independent quantities of every
// chunk of a slab (module docstring of memory_ops.py, sparse-delta-memory 2.0.0 wheel,
// diffend page 21: per-slot log-decays, dedup flags, gather weights, Gram matrices A
// and QK). Each chunk is handled by its own workgroup(s), so chunks never interact and
// every result depends only on its chunk's inputs.
//
//   p1_sort    stable LSD radix sort of the chunk's write entries by slot id
//              (entries enter in token order, so equal slots end in token order:
//              each run of one slot is that slot's write group)
//   p1_groups  group table, per-entry cumulative log-decay L as a sequential scan over
//              each group in token order, gather weights k exp(L), and the DW records:
//              per group {slot, first position, members, exp(L_last)}, per member
//              {token, k exp(L_last - L)}
//              and the split of the groups into hot (many members: their pair terms go
//              to the matrix cores) and cold (their pair terms are summed directly)
//   p1_reads   for each read entry, the latest write of its slot at or before its token
//              (binary search), its L and gather weight q exp(L)
//   p1_gram_sparse  the cold pair terms of A (strict lower) and QK (lower with diagonal)
//              by row ownership: the thread of row i adds its entries' pair terms in a
//              fixed order into an LDS window of columns
//   p1_gram_hot     the hot pair terms as dense products on the matrix cores
// No float atomics anywhere: every element has one writer and a fixed summation order.
#include "common.h"

namespace sdm {

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (uint64_t(1) << lane) - 1; }

// Exclusive scan of hist[0..255] in place by the first four wavefronts; block-wide barrier
// semantics are the caller's.
__device__ __forceinline__ void scan256_exclusive(int32_t *hist, int32_t *wtot) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int32_t x = 0, incl = 0;
    if (tid < 256) {
        x = hist[tid];
        incl = x;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            int32_t y = __shfl_up(incl, d, 64);
            if (lane >= d) incl += y;
        }
        if (lane == 63) wtot[wv] = incl;
    }
    __syncthreads();
    if (tid < 256) {
        int32_t off = 0;
        for (int w = 0; w < wv; ++w) off += wtot[w];
        hist[tid] = off + incl - x;
    }
    __syncthreads();
}

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void p1_sort_kernel(Problem pb, Slab sl) {
    constexpr int NW = BLOCK / kWave;
    __shared__ int32_t hist[256];
    __shared__ int32_t wtot[4];
    __shared__ int32_t wcnt[NW][256];
    const int64_t n = blockIdx.x;
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int nl = n_live_tokens(pb, p, ti);
    const int64_t El = int64_t(nl) * pb.W;
    uint32_t *cb = sl.chunk(n);
    uint32_t *key[2] = {cb + sl.lay.off_key0, cb + sl.lay.off_key1};
    uint32_t *val[2] = {cb + sl.lay.off_val0, cb + sl.lay.off_val1};
    const int32_t *kin = pb.k_idx + (int64_t(p) * pb.T + int64_t(ti) * pb.C) * pb.W;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint64_t lt = lanemask_lt(lane);

    for (int q = 0; q < pb.sort_passes; ++q) {
        const int shift = 8 * q;
        const uint32_t *sk = key[(q + 1) & 1];
        const uint32_t *sv = val[(q + 1) & 1];
        uint32_t *dk = key[q & 1];
        uint32_t *dv = val[q & 1];
        for (int d = tid; d < 256; d += BLOCK) hist[d] = 0;
        __syncthreads();
        for (int64_t e = tid; e < El; e += BLOCK) {
            uint32_t k = q == 0 ? uint32_t(kin[e]) : sk[e];
            atomicAdd(&hist[(k >> shift) & 255u], 1);
        }
        __syncthreads();
        scan256_exclusive(hist, wtot);
        for (int64_t t0 = 0; t0 < El; t0 += BLOCK) {
            const int64_t e = t0 + tid;
            const bool ok = e < El;
            uint32_t k = 0, vv = 0;
            if (ok) {
                k = q == 0 ? uint32_t(kin[e]) : sk[e];
                vv = q == 0 ? uint32_t(e) : sv[e];
            }
            const uint32_t d = (k >> shift) & 255u;
            uint64_t peers = __ballot(ok);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const bool bit = (d >> b) & 1u;
                const uint64_t bb = __ballot(bit);
                peers &= bit ? bb : ~bb;
            }
            const int rank = __popcll(peers & lt);
            for (int i = tid; i < NW * 256; i += BLOCK) (&wcnt[0][0])[i] = 0;
            __syncthreads();
            if (ok && rank == 0) wcnt[wv][d] = __popcll(peers);
            __syncthreads();
            if (tid < 256) {
                int32_t run = hist[tid];
                for (int w = 0; w < NW; ++w) {
                    const int32_t c = wcnt[w][tid];
                    wcnt[w][tid] = run;
                    run += c;
                }
                hist[tid] = run;
            }
            __syncthreads();
            if (ok) {
                const int32_t dst = wcnt[wv][d] + rank;
                dk[dst] = k;
                dv[dst] = vv;
            }
            __syncthreads();
        }
    }
}

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void p1_groups_kernel(Problem pb, Slab sl) {
    constexpr int NW = BLOCK / kWave;
    __shared__ int32_t wsum[NW];
    __shared__ int32_t woff[NW];
    __shared__ int32_t gcount, hcount;
    const int64_t n = blockIdx.x;
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int nl = n_live_tokens(pb, p, ti);
    const int W = pb.W, C = pb.C;
    const int64_t El = int64_t(nl) * W;
    const ChunkLayout &L = sl.lay;
    uint32_t *cb = sl.chunk(n);
    const int fin = (pb.sort_passes - 1) & 1;
    const uint32_t *skey = cb + (fin ? L.off_key1 : L.off_key0);
    const uint32_t *sval = cb + (fin ? L.off_val1 : L.off_val0);
    int32_t *spos = reinterpret_cast<int32_t *>(cb + L.off_spos);
    int32_t *stok = reinterpret_cast<int32_t *>(cb + L.off_stok);
    float *sL = reinterpret_cast<float *>(cb + L.off_sL);
    int32_t *shead = reinterpret_cast<int32_t *>(cb + L.off_shead);
    int2 *mrec = reinterpret_cast<int2 *>(cb + L.off_mrec);
    float *sk = reinterpret_cast<float *>(cb + L.off_sk);
    float *gw = reinterpret_cast<float *>(cb + L.off_gw);
    int32_t *gpos = reinterpret_cast<int32_t *>(cb + L.off_gpos);
    int4 *grec = reinterpret_cast<int4 *>(cb + L.off_grec);
    int32_t *sgrp = reinterpret_cast<int32_t *>(cb + L.off_sgrp);
    int32_t *ghot = reinterpret_cast<int32_t *>(cb + L.off_ghot);
    int32_t *whot = reinterpret_cast<int32_t *>(cb + L.off_whot);
    float *ka = reinterpret_cast<float *>(cb + L.off_ka);
    float *kb = reinterpret_cast<float *>(cb + L.off_kb);
    int2 *crange = reinterpret_cast<int2 *>(cb + L.off_crange);
    int32_t *meta = reinterpret_cast<int32_t *>(cb + L.off_meta);
    float *beta_c = reinterpret_cast<float *>(cb + L.off_beta);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint64_t lt = lanemask_lt(lane);
    const int64_t tok0 = int64_t(p) * pb.T + int64_t(ti) * C;

    if (tid == 0) {
        gcount = 0;
        hcount = 0;
    }
    for (int i = tid; i < C; i += BLOCK) beta_c[i] = i < nl ? pb.beta[tok0 + i] : 0.0f;
    __syncthreads();
    // Group starts: positions whose slot differs from the previous position's.
    for (int64_t t0 = 0; t0 < El; t0 += BLOCK) {
        const int64_t pos = t0 + tid;
        const bool head = pos < El && (pos == 0 || skey[pos] != skey[pos - 1]);
        const uint64_t b = __ballot(head);
        if (lane == 0) wsum[wv] = __popcll(b);
        __syncthreads();
        if (tid == 0) {
            int32_t run = gcount;
            for (int w = 0; w < NW; ++w) {
                woff[w] = run;
                run += wsum[w];
            }
            gcount = run;
        }
        __syncthreads();
        if (head) gpos[woff[wv] + __popcll(b & lt)] = int32_t(pos);
        __syncthreads();
    }
    const int32_t ng = gcount;
    if (tid == 0) {
        gpos[ng] = int32_t(El);
        meta[0] = nl;
        meta[1] = int32_t(El);
        meta[2] = ng;
    }
    __syncthreads();
    // Walk 1, one thread per group in token order: cumulative log-decay L, gather weights,
    // DW records, and whether the group is hot (many members, bounded decay span).
    for (int32_t g = tid; g < ng; g += BLOCK) {
        const int32_t a = gpos[g], e_end = gpos[g + 1];
        float Lc = 0.0f, Lref = 0.0f, dev = 0.0f;
        for (int32_t m = a; m < e_end; ++m) {
            const int32_t e = int32_t(sval[m]);
            const int32_t i = e / W, w = e - i * W;
            const int64_t tg = tok0 + i;
            Lc += pb.g[tg * pb.G + (pb.G == 1 ? 0 : w)];
            if (m == a) Lref = Lc;
            dev = fmaxf(dev, fabsf(Lc - Lref));
            sL[m] = Lc;
            stok[m] = i;
            sk[m] = load_weight(pb.k_val, tg * W + w, pb.dtype);
            spos[e] = m;
            shead[m] = a;
            sgrp[m] = g;
        }
        grec[g] = make_int4(int32_t(skey[a]), a, e_end - a, __float_as_int(expf(Lc)));
        for (int32_t m = a; m < e_end; ++m) {
            const int32_t e = int32_t(sval[m]);
            const float Lm = sL[m], kv = sk[m];
            mrec[m] = make_int2(stok[m], __float_as_int(kv * expf(Lc - Lm)));
            gw[e] = kv * expf(Lm);
        }
        ghot[g] = (e_end - a >= kHotMin && dev <= kHotSpan) ? 1 : 0;
    }
    __syncthreads();
    // Hot indices in group order.
    for (int32_t t0 = 0; t0 < ng; t0 += BLOCK) {
        const int32_t g = t0 + tid;
        const bool hot = g < ng && ghot[g] != 0;
        const uint64_t b = __ballot(hot);
        if (lane == 0) wsum[wv] = __popcll(b);
        __syncthreads();
        if (tid == 0) {
            int32_t run = hcount;
            for (int w = 0; w < NW; ++w) {
                woff[w] = run;
                run += wsum[w];
            }
            hcount = run;
        }
        __syncthreads();
        if (g < ng) ghot[g] = hot ? woff[wv] + __popcll(b & lt) : -1;
        __syncthreads();
    }
    if (tid == 0) meta[3] = hcount;
    // Walk 2: per write entry, its hot index and factored decays, or its cold predecessors.
    for (int32_t g = tid; g < ng; g += BLOCK) {
        const int32_t a = gpos[g], e_end = gpos[g + 1];
        const int32_t h = ghot[g];
        const float Lref = sL[a];
        for (int32_t m = a; m < e_end; ++m) {
            const int32_t e = int32_t(sval[m]);
            whot[e] = h;
            if (h >= 0) {
                const float d = sL[m] - Lref;
                ka[e] = sk[m] * expf(d);
                kb[e] = sk[m] * expf(-d);
                crange[e] = make_int2(0, 0);
            } else {
                crange[e] = make_int2(a, m);
            }
        }
    }
    for (int64_t e = El + tid; e < L.E; e += BLOCK) gw[e] = 0.0f;
}

__global__ __launch_bounds__(256) void p1_reads_kernel(Problem pb, Slab sl) {
    const int64_t n = blockIdx.y;
    const int64_t er = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const ChunkLayout &L = sl.lay;
    if (er >= L.F) return;
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int nl = n_live_tokens(pb, p, ti);
    const int R = pb.R;
    const int64_t El = int64_t(nl) * pb.W;
    uint32_t *cb = sl.chunk(n);
    const int fin = (pb.sort_passes - 1) & 1;
    const uint32_t *skey = cb + (fin ? L.off_key1 : L.off_key0);
    const int32_t *stok = reinterpret_cast<const int32_t *>(cb + L.off_stok);
    const float *sL = reinterpret_cast<const float *>(cb + L.off_sL);
    const int32_t *shead = reinterpret_cast<const int32_t *>(cb + L.off_shead);
    const int32_t *sgrp = reinterpret_cast<const int32_t *>(cb + L.off_sgrp);
    const int32_t *ghot = reinterpret_cast<const int32_t *>(cb + L.off_ghot);
    float *gr = reinterpret_cast<float *>(cb + L.off_gr);
    int32_t *rpos = reinterpret_cast<int32_t *>(cb + L.off_rpos);
    float *rL = reinterpret_cast<float *>(cb + L.off_rL);
    int32_t *rhot = reinterpret_cast<int32_t *>(cb + L.off_rhot);
    float *rval = reinterpret_cast<float *>(cb + L.off_rval);
    int2 *rcrange = reinterpret_cast<int2 *>(cb + L.off_rcrange);
    const int32_t i = int32_t(er / R), r = int32_t(er - int64_t(i) * R);
    if (i >= nl) {
        gr[er] = 0.0f;
        rpos[er] = -1;
        rL[er] = 0.0f;
        rhot[er] = -1;
        rcrange[er] = make_int2(0, 0);
        return;
    }
    const int64_t tg = int64_t(p) * pb.T + int64_t(ti) * pb.C + i;
    const uint32_t q = uint32_t(pb.q_idx[tg * R + r]);
    // First sorted position whose (slot, token) exceeds (q, i).
    int64_t lo = 0, hi = El;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        const uint32_t km = skey[mid];
        if (km < q || (km == q && stok[mid] <= i)) lo = mid + 1;
        else hi = mid;
    }
    const int64_t pos = lo - 1;
    const float qv = load_weight(pb.q_val, tg * R + r, pb.dtype);
    float l = 0.0f;
    int32_t rp = -1, h = -1;
    int2 cr = make_int2(0, 0);
    float rv = 0.0f;
    if (pos >= 0 && skey[pos] == q) {
        rp = int32_t(pos);
        l = sL[pos];
        const int32_t a = shead[pos];
        h = ghot[sgrp[pos]];
        if (h >= 0) rv = qv * expf(l - sL[a]);
        else cr = make_int2(a, rp + 1);
    }
    gr[er] = qv * expf(l);
    rpos[er] = rp;
    rL[er] = l;
    rhot[er] = h;
    rval[er] = rv;
    rcrange[er] = cr;
}

// The cold part of A and QK (pairs of write groups that are not hot). Thread i owns row
// i. Columns are covered in windows of WIN held in LDS (row pitch WIN + 1); each window
// is written out whole, zeros included, so A and QK are fully defined here (+0 outside
// their triangles) and the hot part is added afterwards. Row i sums its pair terms in
// entry order: writes w = 0..W-1, then reads r = 0..R-1.
template <int WIN>
__global__ __launch_bounds__(256) void p1_gram_sparse_kernel(Problem pb, Slab sl) {
    extern __shared__ float lds[];
    const int C = pb.C, W = pb.W, R = pb.R;
    float *accA = lds;
    float *accQ = lds + C * (WIN + 1);
    const int64_t n = blockIdx.x;
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int nl = n_live_tokens(pb, p, ti);
    const ChunkLayout &L = sl.lay;
    uint32_t *cb = sl.chunk(n);
    const int32_t *stok = reinterpret_cast<const int32_t *>(cb + L.off_stok);
    const float *sL = reinterpret_cast<const float *>(cb + L.off_sL);
    const float *sk = reinterpret_cast<const float *>(cb + L.off_sk);
    const int2 *crange = reinterpret_cast<const int2 *>(cb + L.off_crange);
    const int2 *rcrange = reinterpret_cast<const int2 *>(cb + L.off_rcrange);
    float *A = reinterpret_cast<float *>(cb + L.off_A);
    float *QK = reinterpret_cast<float *>(cb + L.off_QK);
    const int tid = threadIdx.x;
    const int i = tid;
    const int64_t tg = int64_t(p) * pb.T + int64_t(ti) * C + i;

    for (int c0 = 0; c0 < C; c0 += WIN) {
        const int cw = C - c0 < WIN ? C - c0 : WIN;
        const int c1 = c0 + cw;
        if (i < C) {
            float *ra = accA + i * (WIN + 1);
            float *rq = accQ + i * (WIN + 1);
            for (int j = 0; j < WIN; ++j) {
                ra[j] = 0.0f;
                rq[j] = 0.0f;
            }
            if (i < nl && c0 <= i) {
                for (int w = 0; w < W; ++w) {
                    const int2 cr = crange[int64_t(i) * W + w];
                    if (cr.y <= cr.x) continue;
                    const float ki = sk[cr.y], Li = sL[cr.y];
                    for (int32_t mm = cr.x; mm < cr.y; ++mm) {
                        const int32_t tj = stok[mm];
                        if (tj < c0) continue;
                        if (tj >= c1) break;
                        ra[tj - c0] += (ki * sk[mm]) * expf(Li - sL[mm]);
                    }
                }
                for (int r = 0; r < R; ++r) {
                    const int2 cr = rcrange[int64_t(i) * R + r];
                    if (cr.y <= cr.x) continue;
                    const float qv = load_weight(pb.q_val, tg * R + r, pb.dtype), Lr = sL[cr.y - 1];
                    for (int32_t mm = cr.x; mm < cr.y; ++mm) {
                        const int32_t tj = stok[mm];
                        if (tj < c0) continue;
                        if (tj >= c1) break;
                        rq[tj - c0] += (qv * sk[mm]) * expf(Lr - sL[mm]);
                    }
                }
            }
        }
        __syncthreads();
        for (int idx = tid; idx < C * cw; idx += blockDim.x) {
            const int r = idx / cw, c = idx - r * cw;
            A[int64_t(r) * C + c0 + c] = accA[r * (WIN + 1) + c];
            QK[int64_t(r) * C + c0 + c] = accQ[r * (WIN + 1) + c];
        }
        __syncthreads();
    }
}

// The hot part of A and QK on the matrix cores. For hot write group h with reference
// log-decay L_ref (its first member's), token t writing it carries Ka[t][h] = k e^(L-L_ref)
// and Kb[t][h] = k e^(L_ref-L); a token reading it after a write carries
// Qa[t][h] = q e^(Lr-L_ref). Then A += tril(Ka Kb^T, -1) and QK += tril(Qa Kb^T), the
// factored exponents multiplying back to the pair decays e^(L_t - L_t'). One workgroup per
// chunk; the hot slots are taken HS at a time into LDS; every wave owns a fixed set of
// 16 x 16 lower output tiles and accumulates them with v_mfma_f32_16x16x4_f32 over the
// slots in ascending order (a fixed order), then adds them to the cold part in memory.
constexpr int kHS = 16;            // hot slots per LDS slice
constexpr int kHP = kHS + 1;       // LDS row pitch
constexpr int kHotBlock = 512;
constexpr int kHotMaxTiles = 34;   // per wave: 2 * 136 lower 16x16 tiles of C = 256 over 8 waves

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kHotBlock) void p1_gram_hot_kernel(Problem pb, Slab sl) {
    extern __shared__ float lds[];
    const int64_t n = blockIdx.x;
    const ChunkLayout &L = sl.lay;
    uint32_t *cb = sl.chunk(n);
    const int32_t *meta = reinterpret_cast<const int32_t *>(cb + L.off_meta);
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int nl = n_live_tokens(pb, p, ti);
    if (nl == 0) return;
    const int nhot = meta[3];
    if (nhot == 0) return;
    const int C = pb.C, W = pb.W, R = pb.R;
    const int nt = (C + 15) / 16, rows = nt * 16;
    const int T1 = nt * (nt + 1) / 2, T2 = 2 * T1;
    float *Ka = lds, *Kb = lds + rows * kHP, *Qa = lds + 2 * rows * kHP;
    const int32_t *whot = reinterpret_cast<const int32_t *>(cb + L.off_whot);
    const float *ka = reinterpret_cast<const float *>(cb + L.off_ka);
    const float *kbv = reinterpret_cast<const float *>(cb + L.off_kb);
    const int32_t *rhot = reinterpret_cast<const int32_t *>(cb + L.off_rhot);
    const float *rval = reinterpret_cast<const float *>(cb + L.off_rval);
    float *A = reinterpret_cast<float *>(cb + L.off_A);
    float *QK = reinterpret_cast<float *>(cb + L.off_QK);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    constexpr int NWAVE = kHotBlock / kWave;

    // This wave's tiles: t = wv + NWAVE q; t < T1 is A tile t, else QK tile t - T1;
    // lower tile index tt maps to (I, J), J <= I, row-major over the lower triangle
    // (tile_ij[tt] = 16 I + J, rows and columns in units of 16).
    __shared__ int32_t tile_ij[136];
    for (int tt = tid; tt < T1; tt += kHotBlock) {
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= tt) ++I;
        tile_ij[tt] = 16 * I + (tt - I * (I + 1) / 2);
    }
    f32x4 acc[kHotMaxTiles];
#pragma unroll
    for (int q = 0; q < kHotMaxTiles; ++q) acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int h0 = 0; h0 < nhot; h0 += kHS) {
        for (int idx = tid; idx < 3 * rows * kHP; idx += kHotBlock) lds[idx] = 0.0f;
        __syncthreads();
        if (tid < nl) {
            const int i = tid;
            for (int w = 0; w < W; ++w) {
                const int64_t e = int64_t(i) * W + w;
                const int h = whot[e] - h0;
                if (h >= 0 && h < kHS) {
                    Ka[i * kHP + h] = ka[e];
                    Kb[i * kHP + h] = kbv[e];
                }
            }
            for (int r = 0; r < R; ++r) {
                const int64_t er = int64_t(i) * R + r;
                const int h = rhot[er] - h0;
                if (h >= 0 && h < kHS) Qa[i * kHP + h] += rval[er];
            }
        }
        __syncthreads();
#pragma unroll
        for (int k0 = 0; k0 < kHS; k0 += 4) {
            const int kk = k0 + (lane >> 4), rr = lane & 15;
#pragma unroll
            for (int q = 0; q < kHotMaxTiles; ++q) {
                const int t = wv + NWAVE * q;
                if (t < T2) {
                    const float *Aop = t < T1 ? Ka : Qa;
                    const int ij = tile_ij[t < T1 ? t : t - T1];
                    const float a = Aop[((ij >> 4) * 16 + rr) * kHP + kk];
                    const float b = Kb[((ij & 15) * 16 + rr) * kHP + kk];
                    acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[q], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }
    // Add the hot part to the cold part, inside the triangles only.
#pragma unroll
    for (int q = 0; q < kHotMaxTiles; ++q) {
        const int t = wv + NWAVE * q;
        if (t >= T2) continue;
        float *M = t < T1 ? A : QK;
        const bool strict = t < T1;
        const int ij = tile_ij[t < T1 ? t : t - T1];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = (ij >> 4) * 16 + 4 * (lane >> 4) + v, c = (ij & 15) * 16 + (lane & 15);
            if (r < C && c < C && (strict ? c < r : c <= r)) M[int64_t(r) * C + c] += acc[q][v];
        }
    }
}

// ---------------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------------
constexpr int kSortBlock = 1024;
constexpr int kGroupBlock = 1024;

static int gram_win(int C) { return C > 128 ? 32 : 64; }

size_t gram_lds_bytes(int C) { return size_t(2) * C * (gram_win(C) + 1) * sizeof(float); }

static size_t hot_lds_bytes(int C) { return size_t(3) * ((C + 15) / 16 * 16) * kHP * sizeof(float); }

hipError_t phase1_prepare() {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&p1_gram_sparse_kernel<64>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(gram_lds_bytes(128)));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&p1_gram_sparse_kernel<32>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(gram_lds_bytes(kMaxChunk)));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&p1_gram_hot_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(hot_lds_bytes(kMaxChunk)));
}

// ev: nullptr, or 5 events recorded before each of the five kernels.
hipError_t launch_phase1(const Problem &pb, const Slab &sl, hipStream_t st, hipEvent_t *ev) {
    const unsigned nch = unsigned(int64_t(pb.P) * sl.steps);
    hipError_t e;
    if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
    hipLaunchKernelGGL(p1_sort_kernel<kSortBlock>, dim3(nch), dim3(kSortBlock), 0, st, pb, sl);
    if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
    hipLaunchKernelGGL(p1_groups_kernel<kGroupBlock>, dim3(nch), dim3(kGroupBlock), 0, st, pb, sl);
    if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
    const unsigned fx = unsigned((sl.lay.F + 255) / 256);
    hipLaunchKernelGGL(p1_reads_kernel, dim3(fx, nch), dim3(256), 0, st, pb, sl);
    if (ev && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
    const int gb = pb.C <= 64 ? 64 : (pb.C <= 128 ? 128 : 256);
    if (gram_win(pb.C) == 64)
        hipLaunchKernelGGL(p1_gram_sparse_kernel<64>, dim3(nch), dim3(gb), gram_lds_bytes(pb.C), st, pb, sl);
    else
        hipLaunchKernelGGL(p1_gram_sparse_kernel<32>, dim3(nch), dim3(gb), gram_lds_bytes(pb.C), st, pb, sl);
    if (ev && (e = hipEventRecord(ev[4], st)) != hipSuccess) return e;
    hipLaunchKernelGGL(p1_gram_hot_kernel, dim3(nch), dim3(kHotBlock), hot_lds_bytes(pb.C), st, pb, sl);
    return hipGetLastError();
}

}  // namespace sdm

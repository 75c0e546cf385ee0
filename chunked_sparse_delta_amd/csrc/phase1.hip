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
//   p1_reads   for each read entry, the latest write of its slot at or before its token
//              (binary search), its L and gather weight q exp(L)
//   p1_gram    A (strict lower) and QK (lower with diagonal) by row ownership: the
//              thread of row i adds its entries' pair terms in a fixed order into an LDS
//              window of columns; no float atomics, no two writers per element.
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
    __shared__ int32_t gcount;
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
    int32_t *meta = reinterpret_cast<int32_t *>(cb + L.off_meta);
    float *beta_c = reinterpret_cast<float *>(cb + L.off_beta);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint64_t lt = lanemask_lt(lane);
    const int64_t tok0 = int64_t(p) * pb.T + int64_t(ti) * C;

    if (tid == 0) gcount = 0;
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
        if (head) {
            const int32_t g = woff[wv] + __popcll(b & lt);
            gpos[g] = int32_t(pos);
        }
        __syncthreads();
    }
    const int32_t ng = gcount;
    if (tid == 0) {
        gpos[ng] = int32_t(El);
        meta[0] = nl;
        meta[1] = int32_t(El);
        meta[2] = ng;
        meta[3] = 0;
    }
    __syncthreads();
    // One thread walks each group in token order.
    for (int32_t g = tid; g < ng; g += BLOCK) {
        const int32_t a = gpos[g], e_end = gpos[g + 1];
        float Lc = 0.0f;
        for (int32_t m = a; m < e_end; ++m) {
            const int32_t e = int32_t(sval[m]);
            const int32_t i = e / W, w = e - i * W;
            const int64_t tg = tok0 + i;
            const float gate = pb.g[tg * pb.G + (pb.G == 1 ? 0 : w)];
            Lc += gate;
            sL[m] = Lc;
            stok[m] = i;
            sk[m] = load_weight(pb.k_val, tg * W + w, pb.dtype);
            spos[e] = m;
            shead[m] = a;
        }
        grec[g] = make_int4(int32_t(skey[a]), a, e_end - a, __float_as_int(expf(Lc)));
        for (int32_t m = a; m < e_end; ++m) {
            const int32_t e = int32_t(sval[m]);
            const float Lm = sL[m], kv = sk[m];
            mrec[m] = make_int2(stok[m], __float_as_int(kv * expf(Lc - Lm)));
            gw[e] = kv * expf(Lm);
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
    float *gr = reinterpret_cast<float *>(cb + L.off_gr);
    int32_t *rpos = reinterpret_cast<int32_t *>(cb + L.off_rpos);
    float *rL = reinterpret_cast<float *>(cb + L.off_rL);
    const int32_t i = int32_t(er / R), r = int32_t(er - int64_t(i) * R);
    if (i >= nl) {
        gr[er] = 0.0f;
        rpos[er] = -1;
        rL[er] = 0.0f;
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
    float l = 0.0f;
    int32_t rp = -1;
    if (pos >= 0 && skey[pos] == q) {
        rp = int32_t(pos);
        l = sL[pos];
    }
    gr[er] = load_weight(pb.q_val, tg * R + r, pb.dtype) * expf(l);
    rpos[er] = rp;
    rL[er] = l;
}

// First position in [a, b) whose token is >= c (tokens ascend within a group).
__device__ __forceinline__ int32_t first_token_at_least(const int32_t *stok, int32_t a, int32_t b, int32_t c) {
    while (a < b) {
        const int32_t mid = (a + b) >> 1;
        if (stok[mid] < c) a = mid + 1;
        else b = mid;
    }
    return a;
}

// A and QK of one chunk. Thread i owns row i. Columns are covered in windows of WIN
// held in LDS (row pitch WIN + 1 to spread banks); each window is written out whole,
// zeros included, so A, QK are fully defined (+0 outside their triangles).
template <int WIN>
__global__ __launch_bounds__(256) void p1_gram_kernel(Problem pb, Slab sl) {
    extern __shared__ float lds[];
    const int C = pb.C, W = pb.W, R = pb.R;
    float *accA = lds;
    float *accQ = lds + C * (WIN + 1);
    const int64_t n = blockIdx.x;
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int nl = n_live_tokens(pb, p, ti);
    const ChunkLayout &L = sl.lay;
    uint32_t *cb = sl.chunk(n);
    const int32_t *spos = reinterpret_cast<const int32_t *>(cb + L.off_spos);
    const int32_t *stok = reinterpret_cast<const int32_t *>(cb + L.off_stok);
    const float *sL = reinterpret_cast<const float *>(cb + L.off_sL);
    const int32_t *shead = reinterpret_cast<const int32_t *>(cb + L.off_shead);
    const float *sk = reinterpret_cast<const float *>(cb + L.off_sk);
    const int32_t *rpos = reinterpret_cast<const int32_t *>(cb + L.off_rpos);
    const float *rL = reinterpret_cast<const float *>(cb + L.off_rL);
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
                    const int32_t m = spos[int64_t(i) * W + w];
                    const int32_t a = shead[m];
                    if (a == m) continue;
                    const float ki = sk[m], Li = sL[m];
                    for (int32_t mm = first_token_at_least(stok, a, m, c0); mm < m; ++mm) {
                        const int32_t tj = stok[mm];
                        if (tj >= c1) break;
                        ra[tj - c0] += (ki * sk[mm]) * expf(Li - sL[mm]);
                    }
                }
                for (int r = 0; r < R; ++r) {
                    const int64_t er = int64_t(i) * R + r;
                    const int32_t m = rpos[er];
                    if (m < 0) continue;
                    const int32_t a = shead[m];
                    const float qv = load_weight(pb.q_val, tg * R + r, pb.dtype), Lr = rL[er];
                    for (int32_t mm = first_token_at_least(stok, a, m + 1, c0); mm <= m; ++mm) {
                        const int32_t tj = stok[mm];
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

// ---------------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------------
constexpr int kSortBlock = 1024;
constexpr int kGroupBlock = 1024;
constexpr int kGramWin = 64;

size_t gram_lds_bytes(int C) { return size_t(2) * C * (kGramWin + 1) * sizeof(float); }

hipError_t phase1_prepare() {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&p1_gram_kernel<kGramWin>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(gram_lds_bytes(kMaxChunk)));
}

// ev: nullptr, or 4 events recorded before each of the four kernels.
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
    hipLaunchKernelGGL(p1_gram_kernel<kGramWin>, dim3(nch), dim3(gb), gram_lds_bytes(pb.C), st, pb, sl);
    return hipGetLastError();
}

}  // namespace sdm

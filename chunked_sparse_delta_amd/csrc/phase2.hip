// Phase 2 of the chunked SDM forward on gfx950: the sequential steps that carry the bank
// across chunks (phase2_kernels.py docstring and _sdm_dual_matmul, sparse-delta-memory
// 2.0.0 wheel, diffend page 23). Per step, for the chunk of each stream:
//     gather       retrieved[i] = sum_w gw[i,w] B[s_iw],  inter[i] = sum_r gr[i,r] B[q_ir]
//     dual matmul  u = beta (v - retrieved);  delta_v = X u;  readings = QX u + inter
//     DW           each written slot s: B[s] = exp(L_last) B[s] + sum_members cw delta_v[t]
//
// Every column of the bank evolves on its own (all Phase-1 quantities are column-free),
// so the work of a stream splits by column slices with no exchange at all: one
// persistent workgroup per (stream, slice) runs every step of a slab. A slice is NV
// vectors of V elements (V * NV * sizeof(T) <= 128 bytes, one cache line of a row).
// Workgroups of one stream are placed on one XCD (blocks are dealt round-robin to the
// 8 XCDs) so that its slices share one L2 for the chunk's ids, weights and matrices.
//
// Per step, with 16 wavefronts of up to 128 VGPRs each:
//   gather   a wavefront takes whole tokens; each load instruction fetches one slice of
//            64 / NV rows (8 entry classes x 8 / NV tokens), several instructions in
//            flight, the next batch's ids and weights loaded under the current batch's rows
//   u        u = beta (v - retrieved) in LDS
//   matmul   D^T = u^T QX^T and u^T X^T on v_mfma_f32_16x16x4f32: 16 x 16 output tiles
//            (16 columns x 16 tokens), lower-triangular tiles only; readings (+ inter)
//            go straight to memory, delta_v to LDS
//   DW       64 / NV groups per load instruction, four in flight per lane; the first
//            member rides in the group record, the second comes with the bank row (and,
//            records in memory, the next NV too, one per lane of the group), the rest four
//            at a time; the next batch's records load under the current one; groups of 16
//            or more members by whole wavefronts, the next one's loads under this one's sums;
//            a bank in memory has its DW rows loaded and stored with the non-temporal hint
//
// Determinism: each output element has exactly one writer, and every sum runs in an order
// fixed by the shapes W, R and C only (never by the slicing or the launch):
//   gather  token t's entries are split into eight classes of consecutive entries (class r:
//           entries r ceil(W/8) ..), each summed in ascending order (one fmaf chain),
//           and the classes combine as ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7));
//   matmul  16-wide k blocks ascending, each one MFMA chain of four k-steps;
//   DW      decay term first, then the group's members in token order.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "common.h"

namespace sdm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Per block size: wavefronts, gather row loads in flight per lane, DW groups in flight per
// lane, 16 x 16 matmul tiles per wavefront (C <= 256, slices of <= 64 columns), k blocks of
// matrix operands loaded at once. 1024 threads leave 128 VGPRs per lane, 512 threads 256.
template <int BLOCK, int V> struct P2Cfg {
    static constexpr int NW = BLOCK / kWave;
    static constexpr int kBatch = BLOCK == 1024 ? (V == 1 ? 8 : 6) : (V == 1 ? 16 : 12);
    static constexpr int kDwBatch = BLOCK == 1024 ? 4 : 8;
    static constexpr int kMaxTiles = (kMaxChunk / 16) * 4 / NW;
    static constexpr int kMmDepth = BLOCK == 1024 ? 2 : 3;
    static constexpr int kUItems = (kMaxChunk * 8 + BLOCK - 1) / BLOCK;
};

struct P2Args {
    const void *v;                  // [P, T, hd]
    void *bank;                     // [P, M, hd]
    void *out;                      // [P, T, hd]
    const int32_t *valid;           // [P] or nullptr
    const uint32_t *ws;             // slab base: chunk n at ws + n * words
    int64_t M, words;
    int64_t bstride;                // elements between the streams' banks (0: one shared bank)
    int32_t T, C, W, R, hd, P;
    int32_t S, hv;                  // slices per row, vectors per row (hd / V)
    int32_t ti0, steps;             // the slab
    int32_t off_gw, off_gr, off_beta, off_X, off_QX, off_meta, off_grec, off_mrec, off_brec;   // words within a chunk
    int32_t off_kid, off_qid, off_stage0, off_stage1;
    int32_t off_xu;                 // teams: the exchange area of a chunk
    uint32_t steal_ticks;           // teams: wait before claiming another workgroup's piece (100 MHz ticks)
    int32_t nt_gather;              // rows of ids marked kIdOnce load with the non-temporal hint
};

// Live tokens of stream p (valid_tokens clamped to [0, T]), and of its chunk ti.
__device__ __forceinline__ int32_t stream_tokens(const P2Args &a, int p) {
    const int32_t vt = a.valid ? a.valid[p] : a.T;
    return vt < 0 ? 0 : (vt > a.T ? a.T : vt);
}
__device__ __forceinline__ int32_t chunk_tokens(const P2Args &a, int32_t vt, int ti) {
    const int32_t n = vt - ti * a.C;
    return n < 0 ? 0 : (n > a.C ? a.C : n);
}

// Element pointer + 32-bit element offset (the host bounds every offset below 2^31 bytes).
template <typename T>
__device__ __forceinline__ const T *at(const T *base, uint32_t off) {
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + uint64_t(off) * sizeof(T));
}
template <typename T>
__device__ __forceinline__ T *at(T *base, uint32_t off) {
    return reinterpret_cast<T *>(reinterpret_cast<char *>(base) + uint64_t(off) * sizeof(T));
}

// LDS row pitch (floats) of a slice of cw columns: 16-byte aligned rows, 4 mod 8 words.
__host__ __device__ inline int p2_pitch(int cw) { return ((cw + 3) & ~3) + 4; }
__host__ __device__ inline int p2_rows(int C) { return (C + 15) & ~15; }

// s_waitcnt immediate of gfx9-family targets for vmcnt(0), expcnt and lgkmcnt left at their
// maxima (vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int kWaitVmcnt0 = 0x0F70;

// Workgroup barrier for data exchanged through LDS only: unlike __syncthreads() it does
// not wait for this wave's outstanding global stores (the readings, the bank rows).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// End of a Phase-2 step: a bank held in LDS needs an LDS barrier only; a bank in memory
// needs the DW's global stores visible to the whole workgroup.
template <bool RB>
__device__ __forceinline__ void step_end_barrier() {
    if constexpr (RB) lds_barrier();
    else __syncthreads();
}

// x + x of lane (lane ^ k) for k = 1, 2 (quad permutations), and x + x of lane
// (lane ^ 7) within each group of 8 lanes (the row half-mirror), all on the VALU.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // lane i of a group of 8 reads lane 7 - i

// Combine the eight entry classes of a lane's sum (classes are lane bits NV, 2NV, 4NV)
// as ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)). With NV = 1 the classes are lanes 0..7 of a
// group: after the xor-1 and xor-2 rounds the four lanes of a quad hold the same value
// (each sum is formed from the same two operands), so the half-mirror lane of the other
// quad is as good a partner as lane ^ 4. Every lane of the wavefront must be active.
template <int V, int NV>
__device__ __forceinline__ void combine_classes(float (&acc)[V]) {
    if constexpr (NV == 1) {
#pragma unroll
        for (int c = 0; c < V; ++c) acc[c] = add_dpp<kDppXor1>(acc[c]);
#pragma unroll
        for (int c = 0; c < V; ++c) acc[c] = add_dpp<kDppXor2>(acc[c]);
#pragma unroll
        for (int c = 0; c < V; ++c) acc[c] = add_dpp<kDppHalfMirror>(acc[c]);
        return;
    }
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] += __shfl_xor(acc[c], NV, 64);
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] += __shfl_xor(acc[c], 2 * NV, 64);
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] += __shfl_xor(acc[c], 4 * NV, 64);
}

template <int V>
__device__ __forceinline__ void lds_store_vec(float *p, const float (&x)[V]) {
    if constexpr (V % 4 == 0) {
#pragma unroll
        for (int c = 0; c < V; c += 4) *reinterpret_cast<float4 *>(p + c) = make_float4(x[c], x[c + 1], x[c + 2], x[c + 3]);
    } else {
#pragma unroll
        for (int c = 0; c < V; ++c) p[c] = x[c];
    }
}

template <int V>
__device__ __forceinline__ void lds_load_vec(const float *p, float (&x)[V]) {
    if constexpr (V % 4 == 0) {
#pragma unroll
        for (int c = 0; c < V; c += 4) {
            const float4 y = *reinterpret_cast<const float4 *>(p + c);
            x[c] = y.x; x[c + 1] = y.y; x[c + 2] = y.z; x[c + 3] = y.w;
        }
    } else {
#pragma unroll
        for (int c = 0; c < V; ++c) x[c] = p[c];
    }
}

// Bank row loads and stores that may take the non-temporal hint (NT): the line is streamed,
// not kept for reuse. The DW of a bank in memory (it exceeds every cache) uses it for its
// second read of each written row and for the row's store, neither used again within the
// step, whose kept lines would displace the rows the gather reuses; the gather uses it, on
// large workloads, for rows that one entry of the chunk alone reads. 16-byte vectors only;
// narrower ones load and store plainly.
template <typename T, int V>
constexpr bool kHasNt = (std::is_same<T, bf16>::value && V == 8) || (std::is_same<T, float>::value && V == 4);

template <typename T, int V, bool NT>
__device__ __forceinline__ typename Vec<T, V>::raw_t bank_load(const T *p) {
    if constexpr (NT && kHasNt<T, V>) return Vec<T, V>::load_raw_nt(p);
    else return Vec<T, V>::load_raw(p);
}
template <typename T, int V, bool NT>
__device__ __forceinline__ void bank_store(T *p, const float (&o)[V]) {
    if constexpr (NT && kHasNt<T, V>) Vec<T, V>::store_nt(p, o);
    else Vec<T, V>::store(p, o);
}

// Weighted row sums of one region (the write entries or the read entries) for the live
// tokens of the chunk, into dst[t * pitch + vq * V + c]. Lane layout: vq = lane % NV (the
// vector of the slice), class r = (lane / NV) % 8, ts = lane / (8 NV) (the token within a
// group of TPI = 8 / NV tokens). Class r owns the run of entries r NI .. r NI + NI - 1 of
// its token (NI = ceil(width / 8); entries past width are empty) and sums them in
// ascending order. A slot is Q consecutive entries of a class run, one id / weight load
// of Q elements (Q = 4 needs width % 32 == 0, so that every run is a whole number of
// 16-byte aligned quads); a token group takes NI / Q slots. The wave walks its token
// groups (wave, wave + nw, ...) as one flat list of slots, kBatch at a time (the next
// batch's ids and weights load under the current batch's rows). The calling waves are
// wave = 0 .. nw - 1 of the region.
// UFT && uf: the sums are the write entries' retrieved rows, and u = beta (v - retrieved)
// is stored in their place (v from vsrc[t * NV + vq], beta from beta[t]). Ids carry the
// kIdOnce bit; with ntg, the rows of ids that have it load with the non-temporal hint.
template <typename T, int V, int NV, int kBatch, int Q, bool UFT>
__device__ __forceinline__ void gather_region(const T *bank, int hd, const int32_t *ids, const float *wts, int width,
                                              int nl, int col0, int nvs, float *dst, int pitch, int wave, int nw,
                                              int lane, bool uf, const typename Vec<T, V>::raw_t *vsrc,
                                              const float *beta, bool ntg) {
    static_assert(Q == 1 || Q == 4, "one or four entries per id load");
    constexpr int TPI = 8 / NV;
    const int vq = lane % NV, r = (lane / NV) & 7, ts = lane / (8 * NV);
    const int NI = (width + 7) >> 3;
    const int NS = Q == 1 ? NI : NI >> 2;     // slots per token group
    const int NG = (nl + TPI - 1) / TPI;
    const int ngw = NG > wave ? (NG - wave + nw - 1) / nw : 0;
    const int total = ngw * NS;
    if (total == 0) return;
    const bool vok = vq < nvs;
    const uint32_t col = uint32_t(col0 + vq * V);

    // (k, j) of the first slot of the next batch whose pairs are to be loaded
    int pk = 0, pj = 0;
    int32_t id[kBatch][Q], nid[kBatch][Q] = {};
    float wt[kBatch][Q], nwt[kBatch][Q] = {};
    // Every load below is issued unconditionally (an unused slot reads entry 0, row 0 or the
    // slice's first vector, all in bounds), so that the compiler can count the loads in
    // flight exactly; a load under a branch makes it wait for all of them.
    auto load_pairs = [&](int32_t (&di)[kBatch][Q], float (&dw)[kBatch][Q]) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int t = (wave + pk * nw) * TPI + ts, e = r * NI + Q * pj;
            if constexpr (Q == 1) {
                const bool ok = pk < ngw && t < nl && e < width;
                const uint32_t x = ok ? uint32_t(t * width + e) : 0u;
                const int32_t iv = *at(ids, x);
                const float wv = *at(wts, x);
                di[u][0] = ok ? iv : -1;
                dw[u][0] = ok ? wv : 0.0f;
            } else {
                const bool ok = pk < ngw && t < nl;
                const uint32_t x = ok ? uint32_t(t * width + e) : 0u;
                const int4 iv = *reinterpret_cast<const int4 *>(at(ids, x));
                const float4 wv = *reinterpret_cast<const float4 *>(at(wts, x));
                di[u][0] = ok ? iv.x : -1; di[u][1] = ok ? iv.y : -1;
                di[u][2] = ok ? iv.z : -1; di[u][3] = ok ? iv.w : -1;
                dw[u][0] = wv.x; dw[u][1] = wv.y; dw[u][2] = wv.z; dw[u][3] = wv.w;
            }
            if (++pj == NS) { pj = 0; ++pk; }
        }
    };
    load_pairs(id, wt);

    float acc[V];
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] = 0.0f;
    int ck = 0, cj = 0;   // (k, j) of the slot being consumed
    for (int i0 = 0; i0 < total; i0 += kBatch) {
        typename Vec<T, V>::raw_t raw[kBatch][Q];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const bool ok = id[u][q] >= 0 && vok;
                const T *rp = at(bank, uint32_t(ok ? id[u][q] & kIdMask : 0) * uint32_t(hd) + (vok ? col : uint32_t(col0)));
                raw[u][q] = ntg && (id[u][q] & kIdOnce) ? bank_load<T, V, true>(rp) : Vec<T, V>::load_raw(rp);
            }
        // staged, ids and weights come from LDS: a wave-uniform branch skips the loads past
        // the last batch without making any memory load wait
        if (!UFT || i0 + kBatch < total) load_pairs(nid, nwt);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (i0 + u >= total) continue;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                if (id[u][q] >= 0 && vok) {
                    float row[V];
                    Vec<T, V>::unpack(raw[u][q], row);
#pragma unroll
                    for (int c = 0; c < V; ++c) acc[c] = fmaf(wt[u][q], row[c], acc[c]);
                }
            }
            if (cj == NS - 1) {
                combine_classes<V, NV>(acc);
                const int t = (wave + ck * nw) * TPI + ts;
                if (r == 0 && t < nl && vok) {
                    if constexpr (UFT) {
                        if (uf) {   // u = beta (v - retrieved), as the separate u pass computes it
                            float vv[V];
                            Vec<T, V>::unpack(vsrc[t * NV + vq], vv);
                            const float b = beta[t];
#pragma unroll
                            for (int c = 0; c < V; ++c) acc[c] = b * (vv[c] - acc[c]);
                        }
                    }
                    lds_store_vec<V>(dst + t * pitch + vq * V, acc);
                }
#pragma unroll
                for (int c = 0; c < V; ++c) acc[c] = 0.0f;
                cj = 0;
                ++ck;
            } else {
                ++cj;
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                id[u][q] = nid[u][q];
                wt[u][q] = nwt[u][q];
            }
    }
}

template <typename T>
__device__ __forceinline__ void store_out4(T *p, const f32x4 &y, int n) {
    // n (1..4) consecutive elements; n == 4 takes one vector store
    if constexpr (sizeof(T) == 4) {
        if (n == 4) {
            *reinterpret_cast<float4 *>(p) = make_float4(y[0], y[1], y[2], y[3]);
            return;
        }
    } else {
        if (n == 4) {
            uint2 w;
            w.x = f32x2_to_bf16x2(y[0], y[1]);
            w.y = f32x2_to_bf16x2(y[2], y[3]);
            *reinterpret_cast<uint2 *>(p) = w;
            return;
        }
    }
    for (int v = 0; v < n; ++v) p[v] = from_f32<T>(y[v]);
}

// The B operand of one 16 x 16 x 16 block: lane l holds M[i0 + (l & 15)][k0 + 4 (l >> 4) + kk]
// for kk = 0..3 (0 outside the C x C matrix). FULL: C is a multiple of 16, so every lane's
// four elements are inside the matrix and 16-byte aligned.
template <bool FULL>
__device__ __forceinline__ void load_bop(const float *M, int C, int i, int k, bool vec4, float (&b)[4]) {
    if constexpr (FULL) {
        const float4 x = *reinterpret_cast<const float4 *>(M + i * C + k);
        b[0] = x.x; b[1] = x.y; b[2] = x.z; b[3] = x.w;
    } else if (i < C && k + 3 < C && vec4) {
        const float4 x = *reinterpret_cast<const float4 *>(M + int64_t(i) * C + k);
        b[0] = x.x; b[1] = x.y; b[2] = x.z; b[3] = x.w;
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b[kk] = (i < C && k + kk < C) ? M[int64_t(i) * C + k + kk] : 0.0f;
    }
}

// The A operand of one 16 x 16 x 16 block: lane l holds u[k0 + 4 (l >> 4) + kk][c0 + (l & 15)]
// for kk = 0..3, or 0 for a column outside the slice (ok false). The four loads are
// unconditional, so that they issue together: a column past the slice reads inside the
// next row, or for the last row a few words into the LDS region after u.
__device__ __forceinline__ void load_aop(const float *p, int pitch, bool ok, float (&a)[4]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) a[kk] = p[kk * pitch];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) a[kk] = ok ? a[kk] : 0.0f;
}

// DW of one group with many members (>= kHotMin) by a whole wavefront: lane (r, p) =
// (lane / 8, lane % 8) sums the members m = r, r + 8, ... of the group in token order for
// vector p of the slice; the eight classes combine as in the gather, and the decay term
// comes first: B[s] = exp(L_last) B[s] + ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)). The member
// records (at most 256) are loaded once, four per lane, and broadcast by lane shuffles.
// big_issue loads a group's row and member records; big_finish sums and stores them, so
// that the next group's loads can be in flight while this one is summed.
template <typename T, int V>
struct BigLoads {
    typename Vec<T, V>::raw_t raw;
    int32_t rt[4], rc[4];
};

template <typename T, int V, bool NT>
__device__ __forceinline__ void big_issue(const T *bank, int hd, const int4 &rec, const int2 *mrec, int col0, int nvs,
                                          int lane, BigLoads<T, V> &L) {
    const int p = lane & 7;
    const bool pok = p < nvs;
    const int32_t m0 = rec.y & 0xFFFF, n = ((rec.y >> 16) & 0xFF) + 1;
    const uint32_t col = uint32_t(col0 + p * V);
    // loads unconditional (in-bounds fallbacks), as in the gather
    L.raw = bank_load<T, V, NT>(at(bank, uint32_t(rec.x) * uint32_t(hd) + (pok ? col : uint32_t(col0))));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int m = lane + 64 * q;
        const int2 x = *at(mrec, uint32_t(m0 + (m < n ? m : 0)));
        L.rt[q] = m < n ? x.x : 0;
        L.rc[q] = m < n ? x.y : 0;
    }
}

template <typename T, int V, bool NT>
__device__ __forceinline__ void big_finish(T *bank, int hd, const int4 &rec, const BigLoads<T, V> &L, const float *dl,
                                           int pitch, int col0, int nvs, int lane) {
    const int r = lane >> 3, p = lane & 7;
    const bool pok = p < nvs;
    const int32_t n = ((rec.y >> 16) & 0xFF) + 1;
    const uint32_t col = uint32_t(col0 + p * V);
    float acc[V];
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] = 0.0f;
    // member j of class r is m = r + 8 j: lane m % 64 = r + 8 (j % 8), register j / 8
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (64 * q >= n) break;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int src = r + 8 * jj;
            const int32_t t = __shfl(L.rt[q], src, 64);
            const float cw = __int_as_float(__shfl(L.rc[q], src, 64));
            if (64 * q + src < n && pok) {
                float dv[V];
                lds_load_vec<V>(dl + t * pitch + p * V, dv);
#pragma unroll
                for (int c = 0; c < V; ++c) acc[c] = fmaf(cw, dv[c], acc[c]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] += __shfl_xor(acc[c], 8, 64);
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] += __shfl_xor(acc[c], 16, 64);
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] += __shfl_xor(acc[c], 32, 64);
    if (r == 0 && pok) {
        float b[V];
        Vec<T, V>::unpack(L.raw, b);
        const float dec = __int_as_float(rec.z);
#pragma unroll
        for (int c = 0; c < V; ++c) b[c] = b[c] * dec + acc[c];
        bank_store<T, V, NT>(at(bank, uint32_t(rec.x) * uint32_t(hd) + col), b);
    }
}

// DW of the groups grec[0, ng) and of the groups with >= kHotMin members brec[0, nbig): one
// writer per written row. The many-member groups go to whole wavefronts (big_issue /
// big_finish: the records two groups ahead, the rows and member records one group ahead);
// the others are summed in token order by the NV lanes of their slice: lane (gs, vq) of
// slot u takes group gb + u * NW * GPI + gs of each batch, the first member rides in the
// group record, the second loads with the bank row, and (records in memory) the next NV
// with it too, one per lane of the group (broadcast by lane shuffles), so that most groups
// need no load while they are summed; any further members come four at a time. kB groups
// per lane are in flight; SM: the records are in LDS (the loads past the last batch are
// skipped, and every member beyond the second is read from LDS where it is summed).
template <typename T, int V, int NV, int NW, int kB, bool SM>
__device__ __forceinline__ void dw_groups(T *bank, int bst, const int4 *grec, int32_t ng, const int4 *brec,
                                          int32_t nbig, const int2 *mrec, const float *db, int pitch, int nvs,
                                          int wave) {
    int dlane = threadIdx.x & 63;                        // opaque: nothing of the DW moves up
    asm volatile("" : "+v"(dlane));
    if (wave < nbig) {
        // unconditional (clamped) loads: a big group past the end reloads the last one
        auto brec_at = [&](int32_t bi) { return *at(brec, uint32_t(bi < nbig ? bi : nbig - 1)); };
        int4 rc0 = brec_at(wave), rc1 = brec_at(wave + NW);
        BigLoads<T, V> cur;
        big_issue<T, V, !SM>(bank, bst, rc0, mrec, 0, nvs, dlane, cur);
        for (int32_t bi = wave; bi < nbig; bi += NW) {
            BigLoads<T, V> nxt;
            big_issue<T, V, !SM>(bank, bst, rc1, mrec, 0, nvs, dlane, nxt);
            const int4 rc2 = brec_at(bi + 2 * NW);
            big_finish<T, V, !SM>(bank, bst, rc0, cur, db, pitch, 0, nvs, dlane);
            cur = nxt;
            rc0 = rc1;
            rc1 = rc2;
        }
    }
    constexpr int GPI = kWave / NV;                       // groups per load instruction
    constexpr int kStride = NW * GPI * kB;                 // groups per workgroup batch
    const int gs = dlane / NV, vq = dlane % NV;
    const bool vok = vq < nvs;
    const uint32_t col = uint32_t(vq * V);
    // a record of a group with fewer than kHotMin members (slot -1: no group)
    auto small = [](const int4 &r) { return r.x >= 0 && ((r.y >> 16) & 0xFF) < kHotMin - 1; };
    // slot u of a batch takes groups gb + u * NW * GPI + gs: the instructions of a batch
    // are dealt to all waves first, so that a few groups still keep every wave busy
    // loads unconditional (in-bounds fallbacks), as in the gather
    auto load_rec = [&](int32_t g) {
        const int4 x = *at(grec, uint32_t(g < ng ? g : 0));
        return g < ng ? x : make_int4(-1, 0, 0, 0);
    };
    int4 rec[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) rec[u] = load_rec(wave * GPI + u * NW * GPI + gs);
    for (int32_t gb = wave * GPI; gb < ng; gb += kStride) {
        typename Vec<T, V>::raw_t raw[kB];
        int2 mr[kB];
        [[maybe_unused]] int2 mw[kB];   // records in memory: member 2 + vq of the group
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const bool sm = small(rec[u]);
            raw[u] = bank_load<T, V, !SM>(at(bank, uint32_t(sm ? rec[u].x : 0) * uint32_t(bst) + (vok ? col : 0u)));
            const int32_t m0 = rec[u].y & 0xFFFF, n1 = (rec[u].y >> 16) & 0xFF;
            const bool two = sm && n1 > 0;
            const int2 x = *at(mrec, uint32_t(two ? m0 + 1 : 0));
            mr[u] = two ? x : make_int2(0, 0);
            if constexpr (!SM) {
                const bool inw = sm && n1 >= 2 + vq;
                mw[u] = *at(mrec, uint32_t(inw ? m0 + 2 + vq : 0));
            }
        }
        int4 nrec[kB];
        // records in LDS (staged): the loads past the last batch are skipped
        if (!SM || gb + kStride < ng) {
#pragma unroll
            for (int u = 0; u < kB; ++u) nrec[u] = load_rec(gb + kStride + u * NW * GPI + gs);
        } else {
#pragma unroll
            for (int u = 0; u < kB; ++u) nrec[u] = make_int4(-1, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const bool sm = small(rec[u]);
            const int32_t m0 = rec[u].y & 0xFFFF, n1 = sm ? (rec[u].y >> 16) & 0xFF : 0, t0 = (rec[u].y >> 24) & 0xFF;
            float acc[V];
            if (vok && sm) {
                Vec<T, V>::unpack(raw[u], acc);
            } else {
#pragma unroll
                for (int c = 0; c < V; ++c) acc[c] = 0.0f;
            }
            const float dec = __int_as_float(rec[u].z);
#pragma unroll
            for (int c = 0; c < V; ++c) acc[c] *= dec;
            if (sm) {
                const float cwv = __int_as_float(rec[u].w);
                float dv[V];
                lds_load_vec<V>(db + t0 * pitch + vq * V, dv);
#pragma unroll
                for (int c = 0; c < V; ++c) acc[c] = fmaf(cwv, dv[c], acc[c]);
            }
            if (n1 > 0) {
                const float cwv = __int_as_float(mr[u].y);
                float dv[V];
                lds_load_vec<V>(db + mr[u].x * pitch + vq * V, dv);
#pragma unroll
                for (int c = 0; c < V; ++c) acc[c] = fmaf(cwv, dv[c], acc[c]);
            }
            int32_t mfirst = m0 + 2;   // the first member still to be summed from the records
            if constexpr (!SM) {
                // members 2 .. NV + 1 from the window, lane gs * NV + j holding member 2 + j;
                // the shuffles run with every lane active (wave-uniform trip count)
#pragma unroll
                for (int j = 0; j < NV; ++j) {
                    if (__ballot(n1 >= 2 + j) == 0) break;
                    const int src = gs * NV + j;
                    const int32_t t = __shfl(mw[u].x, src, 64);
                    const float cwv = __int_as_float(__shfl(mw[u].y, src, 64));
                    if (n1 >= 2 + j) {
                        float dv[V];
                        lds_load_vec<V>(db + t * pitch + vq * V, dv);
#pragma unroll
                        for (int c = 0; c < V; ++c) acc[c] = fmaf(cwv, dv[c], acc[c]);
                    }
                }
                mfirst = m0 + 2 + NV;
            }
            // the members past those, four records at a time
            for (int32_t m = mfirst; m <= m0 + n1; m += 4) {
                int2 mb[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) mb[q] = *at(mrec, uint32_t(min(m + q, m0 + n1)));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (m + q > m0 + n1) break;
                    const float cwv = __int_as_float(mb[q].y);
                    float dv[V];
                    lds_load_vec<V>(db + mb[q].x * pitch + vq * V, dv);
#pragma unroll
                    for (int c = 0; c < V; ++c) acc[c] = fmaf(cwv, dv[c], acc[c]);
                }
            }
            if (vok && sm) bank_store<T, V, !SM>(at(bank, uint32_t(rec[u].x) * uint32_t(bst) + col), acc);
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) rec[u] = nrec[u];
    }
}

// Modes:
//   kP2Global    every array is read from the workspace, every bank row from memory.
//   kP2Staged    the chunk's whole Phase-2 block of the workspace (records, weights, ids,
//                meta, beta, X, QX) fits in LDS next to the two row regions; it is copied
//                there at the start of every step with one sweep of 16-byte loads (and this
//                slice of v with it), so that a step waits on memory only for its gather
//                and its DW bank rows.
//   kP2Resident  staged, and this workgroup's column slice of the stream's bank (M rows x
//                NV vectors, in the bank dtype) also fits: it is loaded into LDS once per
//                slab and written back at its end, and the gather and the DW run on it.
//                Rows are held in the bank dtype, so every value is rounded exactly where
//                the other modes round it on the way to memory: the bits are the same.
constexpr int kP2Block = 1024;
constexpr int kStageUnits = 8;   // 16-byte units of the staged block per thread per round
constexpr int kP2Global = 0, kP2Staged = 1, kP2Resident = 2;

// Bytes of the staged copy of C x NV vectors of v, rounded up to 16 bytes.
__host__ __device__ inline int p2_vst_bytes(int C, int nv, int V, int es) { return (C * nv * V * es + 15) & ~15; }

template <typename T, int V, int NV, int MODE>
__global__ __launch_bounds__(kP2Block) void phase2_kernel(P2Args a) {
    constexpr int BLOCK = kP2Block;
    constexpr bool SM = MODE >= kP2Staged, RB = MODE == kP2Resident;
    using Cfg = P2Cfg<BLOCK, V>;
    constexpr int NW = Cfg::NW;
    extern __shared__ float lds[];
    const int C = a.C, hd = a.hd, S = a.S;
    constexpr int CW = V * NV;                // columns of a full slice
    const int pitch = p2_pitch(CW);
    const int CP = p2_rows(C);

    // Decode (stream, slice); a stream's slices stay on one XCD when P % 8 == 0.
    const int bid = blockIdx.x;
    int p, slice;
    if (a.P % kXcds == 0) {
        const int xcd = bid % kXcds, m = bid / kXcds;
        p = xcd + kXcds * (m / S);
        slice = m % S;
    } else {
        p = bid / S;
        slice = bid % S;
    }
    const int vq0 = slice * NV;
    const int nvs = min(NV, a.hv - vq0);      // vectors of this slice
    const int cwv = nvs * V;                  // valid columns of this slice
    const int col0 = vq0 * V;
    using raw_t = typename Vec<T, V>::raw_t;
    T *gbank = static_cast<T *>(a.bank) + int64_t(p) * a.bstride + col0;   // this slice, row stride hd
    const bool vec4 = (C & 3) == 0, full = (C & 15) == 0;

    float *ub = lds;                  // [CP][pitch]: u (retrieved first, without staging)
    float *ib = lds + CP * pitch;     // [CP][pitch]: inter (without staging, then delta_v)
    float *db = SM ? ib + CP * pitch : ib;   // [CP][pitch]: delta_v
    float *stg = ib + (SM ? 2 : 1) * CP * pitch;   // SM: the staged block, then [C][NV] vectors of v
    const int nstage = a.off_stage1 - a.off_stage0;           // words (a multiple of 64)
    const int nu = nstage >> 2;                               // 16-byte units of the staged block
    // the block starts with the DW's records (group, member and big-group records), read
    // only by the DW; the gather and matmul inputs follow
    const int nudw = (a.off_gw - a.off_stage0) >> 2;
    raw_t *vst = reinterpret_cast<raw_t *>(stg + nstage);
    // Prefetch (SM, a staged block of at most one round of kStageUnits units per thread):
    // the next step's block and vector of v are loaded into registers at the start of this
    // step, and stored to LDS after its final barrier.
    // Prefetch units per thread: 8 staged; 4 resident, whose blocks that fit beside the bank
    // slice need no more (the loads of unused units would cost the step their issue time).
    constexpr int PFU = RB ? 4 : kStageUnits;
    const bool pf = SM && nu <= BLOCK * PFU;
    // RB: [M][CW] elements of the bank slice, after v's vectors
    T *lbank = reinterpret_cast<T *>(reinterpret_cast<char *>(vst) + p2_vst_bytes(C, NV, V, int(sizeof(T))));
    // the bank the gather and the DW work on: the slice in LDS (row stride CW) or in memory
    T *bank = RB ? lbank : gbank;
    const int bst = RB ? CW : hd;
    const int32_t Mr = int32_t(a.M);
    if constexpr (RB) {
        for (int i = threadIdx.x; i < Mr * NV; i += BLOCK) {
            const int row = i / NV, vq = i % NV;
            if (vq < nvs) *reinterpret_cast<raw_t *>(lbank + row * CW + vq * V) =
                Vec<T, V>::load_raw(at(gbank, uint32_t(row) * uint32_t(hd) + uint32_t(vq * V)));
        }
        // the first step's staging barrier orders these stores before any gather
    }

    // MFMA tiles of this wave: (it, ct) dealt in a snake order over tiles sorted by it,
    // so that every wave gets a similar share of the triangular work.
    const int NIT = CP / 16, NCT = (cwv + 15) / 16, NT = NIT * NCT;

    // the stream's live tokens, read once (the compiler cannot prove that the kernel's own
    // stores leave valid_tokens unchanged, and would reload it every step)
    const int32_t vtp = stream_tokens(a, p);

    for (int s = 0; s < a.steps; ++s) {
        // Thread ids are re-read opaquely every step, so that the per-lane address
        // arithmetic of all phases is not hoisted out of the step loop (it would be held
        // in registers across the whole loop and spill).
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        asm volatile("" : "+s"(wave));
        int lane = tid & 63;
        const int ti = a.ti0 + s;
        const uint32_t *cbg = a.ws + (int64_t(p) * a.steps + s) * a.words;
        // Phase-2 arrays of the chunk: in LDS (SM) or in the workspace
        auto arr = [&](int32_t off) -> const uint32_t * {
            if constexpr (SM) return reinterpret_cast<const uint32_t *>(stg) + (off - a.off_stage0);
            else return cbg + off;
        };
        const int nl = chunk_tokens(a, vtp, ti);
        const int rows = min(C, a.T - ti * C);
        const int64_t tok0 = int64_t(p) * a.T + int64_t(ti) * C;
        const T *vin = static_cast<const T *>(a.v) + tok0 * hd;     // this chunk's rows of v and out
        T *out = static_cast<T *>(a.out) + tok0 * hd;
        if constexpr (SM) {
          uint4 *dst = reinterpret_cast<uint4 *>(stg);
          // otherwise the previous step has stored this one's block: the gather and matmul
          // inputs during its DW, the DW records after its final barrier
          if (s == 0 || !pf) {
            const uint4 *src = reinterpret_cast<const uint4 *>(cbg + a.off_stage0);
            const int vt = tid / NV, vv = tid % NV;
            const bool vok = tid < C * NV && vt < rows && vv < nvs;
            // unconditional loads (clamped in-bounds indices), as in the gather
            const typename Vec<T, V>::raw_t vr =
                Vec<T, V>::load_raw(at(vin, vok ? uint32_t(vt * hd + col0 + vv * V) : uint32_t(col0)));
            // rounds of kStageUnits 16-byte loads in flight per thread, then their stores
            for (int u0 = tid; u0 < nu; u0 += BLOCK * kStageUnits) {
                static_assert(kStageUnits == 8, "unrolled by hand");
                const uint4 t0 = src[min(u0 + 0 * BLOCK, nu - 1)];
                const uint4 t1 = src[min(u0 + 1 * BLOCK, nu - 1)];
                const uint4 t2 = src[min(u0 + 2 * BLOCK, nu - 1)];
                const uint4 t3 = src[min(u0 + 3 * BLOCK, nu - 1)];
                const uint4 t4 = src[min(u0 + 4 * BLOCK, nu - 1)];
                const uint4 t5 = src[min(u0 + 5 * BLOCK, nu - 1)];
                const uint4 t6 = src[min(u0 + 6 * BLOCK, nu - 1)];
                const uint4 t7 = src[min(u0 + 7 * BLOCK, nu - 1)];
                if (u0 + 0 * BLOCK < nu) dst[u0 + 0 * BLOCK] = t0;
                if (u0 + 1 * BLOCK < nu) dst[u0 + 1 * BLOCK] = t1;
                if (u0 + 2 * BLOCK < nu) dst[u0 + 2 * BLOCK] = t2;
                if (u0 + 3 * BLOCK < nu) dst[u0 + 3 * BLOCK] = t3;
                if (u0 + 4 * BLOCK < nu) dst[u0 + 4 * BLOCK] = t4;
                if (u0 + 5 * BLOCK < nu) dst[u0 + 5 * BLOCK] = t5;
                if (u0 + 6 * BLOCK < nu) dst[u0 + 6 * BLOCK] = t6;
                if (u0 + 7 * BLOCK < nu) dst[u0 + 7 * BLOCK] = t7;
            }
            if (vok) vst[tid] = vr;
            lds_barrier();
          }
            // u rows of padding tokens and rows C..CP-1: +0 (the gather writes rows < nl)
            for (int i = tid; i < (CP - nl) * NV; i += BLOCK) {
                float z[V];
#pragma unroll
                for (int c = 0; c < V; ++c) z[c] = 0.0f;
                lds_store_vec<V>(ub + (nl + i / NV) * pitch + (i % NV) * V, z);
            }
        }

        // the next step's staged block and vector of v, loaded now and held in registers
        // through the gather, the matmul and the DW (the loads' latency stays off the step)
        const bool pfn = pf && s + 1 < a.steps;
        uint4 pf0, pf1, pf2, pf3, pf4, pf5, pf6, pf7;
        raw_t pfv;
        bool pfvok = false;
        if constexpr (SM) {
            // Nothing loaded before this point is still needed. An explicit wait on every
            // path retires it, so that the compiler's wait tracking (which merges the paths
            // of predicated loads and stores) cannot make a later instruction of this step
            // wait for the loads below as well.
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            if (pfn) {
                // unconditional loads (clamped in-bounds indices), as in the gather
                const uint4 *src = reinterpret_cast<const uint4 *>(cbg + a.words + a.off_stage0);
                pf0 = src[min(tid + 0 * BLOCK, nu - 1)];
                pf1 = src[min(tid + 1 * BLOCK, nu - 1)];
                pf2 = src[min(tid + 2 * BLOCK, nu - 1)];
                pf3 = src[min(tid + 3 * BLOCK, nu - 1)];
                if constexpr (PFU > 4) pf4 = src[min(tid + 4 * BLOCK, nu - 1)];
                if constexpr (PFU > 4) pf5 = src[min(tid + 5 * BLOCK, nu - 1)];
                if constexpr (PFU > 4) pf6 = src[min(tid + 6 * BLOCK, nu - 1)];
                if constexpr (PFU > 4) pf7 = src[min(tid + 7 * BLOCK, nu - 1)];
                const int rows_n = min(C, a.T - (ti + 1) * C), vt = tid / NV, vv = tid % NV;
                pfvok = tid < C * NV && vt < rows_n && vv < nvs;
                pfv = Vec<T, V>::load_raw(at(vin, pfvok ? uint32_t((C + vt) * hd + col0 + vv * V) : uint32_t(C * hd + col0)));
            }
        }


        // From memory, this step's vectors of v, its beta and the DW's group counts are loaded
        // before the gather, so that their round trip overlaps it (the asm keeps the compiler
        // from moving the loads down to their uses).
        [[maybe_unused]] float mv[Cfg::kUItems][V];
        [[maybe_unused]] float mb[Cfg::kUItems];
        [[maybe_unused]] int32_t mng = 0, mnbig = 0;
        if constexpr (!SM) {
            const float *beta_c = reinterpret_cast<const float *>(arr(a.off_beta));
#pragma unroll
            for (int x = 0; x < Cfg::kUItems; ++x) {
                const int item = tid + BLOCK * x, t = item / NV, vq = item % NV;
                const bool live = t < CP && t < nl && vq < nvs;
                Vec<T, V>::load(at(vin, live ? uint32_t(t * hd + col0 + vq * V) : uint32_t(col0)), mv[x]);
                mb[x] = beta_c[live ? t : 0];
            }
            const int32_t *meta = reinterpret_cast<const int32_t *>(arr(a.off_meta));
            mng = meta[2];
            mnbig = meta[4];
            asm volatile("" ::: "memory");
        }

        // ---- gather: u (staged; retrieved otherwise) -> ub, inter -> ib (live tokens)
        {
            const float *beta_c = reinterpret_cast<const float *>(arr(a.off_beta));
            const float *gw = reinterpret_cast<const float *>(arr(a.off_gw));
            const float *gr = reinterpret_cast<const float *>(arr(a.off_gr));
            const int32_t *kid = reinterpret_cast<const int32_t *>(arr(a.off_kid));
            const int32_t *qid = reinterpret_cast<const int32_t *>(arr(a.off_qid));
            // the write entries on the first nww waves, the read entries on the others
            // (waves in proportion to W : R)
            int nww = (NW * a.W + (a.W + a.R) / 2) / (a.W + a.R);
            nww = nww < 1 ? 1 : (nww > NW - 1 ? NW - 1 : nww);
            const bool wr = wave < nww;   // wave-uniform: one inlined copy of the gather
            // rows from memory: kBatch loads in flight per lane; from LDS one at a time (the
            // predicated slots of a deep batch cost more than LDS latency when a wave has
            // one or two instructions of work). Widths that are multiples of 32 load ids
            // and weights four at a time.
            const int32_t *rid = wr ? kid : qid;
            const float *rwt = wr ? gw : gr;
            const int rwidth = wr ? a.W : a.R, rwave = wr ? wave : wave - nww, rnw = wr ? nww : NW - nww;
            float *rdst = wr ? ub : ib;
            const bool ntg = !SM && a.nt_gather;   // a bank in memory only
            if (((a.W | a.R) & 31) == 0)
                gather_region<T, V, NV, RB ? 1 : 2, 4, SM>(bank, bst, rid, rwt, rwidth, nl, 0, nvs, rdst, pitch,
                                                          rwave, rnw, lane, wr, vst, beta_c, ntg);
            else
                gather_region<T, V, NV, RB ? 1 : Cfg::kBatch, 1, SM>(bank, bst, rid, rwt, rwidth, nl, 0, nvs, rdst,
                                                                    pitch, rwave, rnw, lane, wr, vst, beta_c, ntg);
        }
        lds_barrier();

        // ---- u = beta (v - retrieved); +0 for padding tokens and rows C..CP-1 (without
        //      staging; staged, the gather has done it)
        if constexpr (!SM) {
#pragma unroll
        for (int x = 0; x < Cfg::kUItems; ++x) {
            const int item = tid + BLOCK * x, t = item / NV, vq = item % NV;
            if (t >= CP) continue;
            float *ur = ub + t * pitch + vq * V;
            float uu[V];
            const bool live = t < nl && vq < nvs;
            if (live) {
                float rr[V];
                lds_load_vec<V>(ur, rr);
#pragma unroll
                for (int c = 0; c < V; ++c) uu[c] = mb[x] * (mv[x][c] - rr[c]);
            } else {
#pragma unroll
                for (int c = 0; c < V; ++c) uu[c] = 0.0f;
            }
            lds_store_vec<V>(ur, uu);
        }
        lds_barrier();
        }

        // Staged, the DW's group counts are read now: the next step's block overwrites the
        // chunk's meta words during the DW.
        int32_t dw_ng = 0, dw_nbig = 0;
        if constexpr (SM) {
            const int32_t *meta = reinterpret_cast<const int32_t *>(arr(a.off_meta));
            if (nl > 0) {
                dw_ng = meta[2];
                dw_nbig = meta[4];
            }
            asm volatile("" : "+v"(dw_ng), "+v"(dw_nbig));
        }

        // ---- dual matmul on the matrix cores: readings to memory, delta_v to db
        asm volatile("" : "+v"(lane));
        const float *QX = reinterpret_cast<const float *>(arr(a.off_QX));
        const float *X = reinterpret_cast<const float *>(arr(a.off_X));
        [[maybe_unused]] f32x4 dacc[SM ? 1 : Cfg::kMaxTiles];   // memory mode: delta_v until inter is read
        // FULL (C a multiple of 16) is decided once per step, for straight-line operand loads
        auto matmul = [&](auto fullc) {
        constexpr bool FULL = decltype(fullc)::value;
        if constexpr (SM) {
            // Staged: each tile's two products are separate items, y0 .. y(NT-1) then
            // d(NT-1) .. d0, dealt to waves in turn, so that a heavy readings tile shares a
            // SIMD with a light delta tile. Each item runs the same MFMA chain as below.
            const int NI2 = 2 * NT;
            for (int iota = wave; iota < NI2; iota += NW) {
                const bool isy = iota < NT;
                const int tau = isy ? iota : NI2 - 1 - iota;
                const int it = tau / NCT, ct = tau - it * NCT;
                const int ti_row = 16 * it + (lane & 15);
                const int cu = 16 * ct + (lane & 15);
                const int co = 16 * ct + 4 * (lane >> 4);
                const int ko = 4 * (lane >> 4);
                const float *Bm = isy ? QX : X;
                f32x4 y = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                if (isy && co < cwv) {
                    const float4 iv = *reinterpret_cast<const float4 *>(ib + ti_row * pitch + co);
                    y = f32x4{iv.x, iv.y, iv.z, iv.w};
                }
                for (int kb = 0; kb <= it; kb += Cfg::kMmDepth) {
                    float bm[Cfg::kMmDepth][4], av[Cfg::kMmDepth][4];
#pragma unroll
                    for (int j = 0; j < Cfg::kMmDepth; ++j) {
                        if (kb + j > it) continue;
                        load_bop<FULL>(Bm, C, ti_row, 16 * (kb + j) + ko, vec4, bm[j]);
                        load_aop(ub + (16 * (kb + j) + ko) * pitch + cu, pitch, cu < cwv, av[j]);
                    }
#pragma unroll
                    for (int j = 0; j < Cfg::kMmDepth; ++j) {
                        if (kb + j > it) continue;
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            y = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j][kk], bm[j][kk], y, 0, 0, 0);
                    }
                }
                if (isy) {
                    if (ti_row < rows && co < cwv) {
                        if (ti_row >= nl) y = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                        store_out4<T>(at(out, uint32_t(ti_row * hd + col0 + co)), y, min(4, cwv - co));
                    }
                } else if (ti_row < C && co < cwv) {
                    *reinterpret_cast<float4 *>(db + ti_row * pitch + co) = make_float4(y[0], y[1], y[2], y[3]);
                }
            }
        } else {
#pragma unroll
        for (int q = 0; q < Cfg::kMaxTiles; ++q) {
            const int tau = q * NW + ((q & 1) ? NW - 1 - wave : wave);
            if (tau >= NT) continue;
            const int it = tau / NCT, ct = tau - it * NCT;
            const int ti_row = 16 * it + (lane & 15);          // token of the B operand / output
            const int cu = 16 * ct + (lane & 15);              // column of the A operand
            const int co = 16 * ct + 4 * (lane >> 4);          // first output column of this lane
            const int ko = 4 * (lane >> 4);
            f32x4 y = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (co < cwv) {
                const float4 iv = *reinterpret_cast<const float4 *>(ib + ti_row * pitch + co);
                y = f32x4{iv.x, iv.y, iv.z, iv.w};
            }
            f32x4 d = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            // k blocks kMmDepth at a time: the operands of those blocks are loaded together
            for (int kb = 0; kb <= it; kb += Cfg::kMmDepth) {
                float bq[Cfg::kMmDepth][4], bx[Cfg::kMmDepth][4], av[Cfg::kMmDepth][4];
#pragma unroll
                for (int j = 0; j < Cfg::kMmDepth; ++j) {
                    if (kb + j > it) continue;
                    load_bop<FULL>(QX, C, ti_row, 16 * (kb + j) + ko, vec4, bq[j]);
                    load_bop<FULL>(X, C, ti_row, 16 * (kb + j) + ko, vec4, bx[j]);
                    load_aop(ub + (16 * (kb + j) + ko) * pitch + cu, pitch, cu < cwv, av[j]);
                }
#pragma unroll
                for (int j = 0; j < Cfg::kMmDepth; ++j) {
                    if (kb + j > it) continue;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        y = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j][kk], bq[j][kk], y, 0, 0, 0);
                        d = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j][kk], bx[j][kk], d, 0, 0, 0);
                    }
                }
            }
            dacc[q] = d;
            if (ti_row < rows && co < cwv) {
                if (ti_row >= nl) y = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                store_out4<T>(at(out, uint32_t(ti_row * hd + col0 + co)), y, min(4, cwv - co));
            }
        }
        }
        };
        if (full) matmul(std::true_type{});
        else matmul(std::false_type{});
        lds_barrier();
        if constexpr (SM) {
            // Every gather and matmul input of this step has been read: the next step's
            // (units from nudw on, and its vectors of v) take their place during the DW.
            if (pfn) {
                uint4 *dst = reinterpret_cast<uint4 *>(stg);
                if (tid + 0 * BLOCK >= nudw && tid + 0 * BLOCK < nu) dst[tid + 0 * BLOCK] = pf0;
                if (tid + 1 * BLOCK >= nudw && tid + 1 * BLOCK < nu) dst[tid + 1 * BLOCK] = pf1;
                if (tid + 2 * BLOCK >= nudw && tid + 2 * BLOCK < nu) dst[tid + 2 * BLOCK] = pf2;
                if (tid + 3 * BLOCK >= nudw && tid + 3 * BLOCK < nu) dst[tid + 3 * BLOCK] = pf3;
                if constexpr (PFU > 4) if (tid + 4 * BLOCK >= nudw && tid + 4 * BLOCK < nu) dst[tid + 4 * BLOCK] = pf4;
                if constexpr (PFU > 4) if (tid + 5 * BLOCK >= nudw && tid + 5 * BLOCK < nu) dst[tid + 5 * BLOCK] = pf5;
                if constexpr (PFU > 4) if (tid + 6 * BLOCK >= nudw && tid + 6 * BLOCK < nu) dst[tid + 6 * BLOCK] = pf6;
                if constexpr (PFU > 4) if (tid + 7 * BLOCK >= nudw && tid + 7 * BLOCK < nu) dst[tid + 7 * BLOCK] = pf7;
                if (pfvok) vst[tid] = pfv;
            }
        }
        if constexpr (!SM) {   // delta_v over inter, now that every tile has read it
#pragma unroll
            for (int q = 0; q < Cfg::kMaxTiles; ++q) {
                const int tau = q * NW + ((q & 1) ? NW - 1 - wave : wave);
                if (tau >= NT) continue;
                const int it = tau / NCT, ct = tau - it * NCT;
                const int ti_row = 16 * it + (lane & 15), co = 16 * ct + 4 * (lane >> 4);
                if (ti_row < C && co < cwv)
                    *reinterpret_cast<float4 *>(db + ti_row * pitch + co) = make_float4(dacc[q][0], dacc[q][1], dacc[q][2], dacc[q][3]);
            }
            lds_barrier();
        }

        // ---- DW: one writer per written row
        {
            if constexpr (!SM) {
                if (nl > 0) {
                    dw_ng = mng;
                    dw_nbig = mnbig;
                }
            }
            // groups per lane in flight: the bank in LDS needs no batching; staged, two leave
            // room for the prefetch registers
            constexpr int kB = RB ? 1 : (SM ? 2 : Cfg::kDwBatch);
            dw_groups<T, V, NV, NW, kB, SM>(bank, bst, reinterpret_cast<const int4 *>(arr(a.off_grec)), dw_ng,
                                            reinterpret_cast<const int4 *>(arr(a.off_brec)), dw_nbig,
                                            reinterpret_cast<const int2 *>(arr(a.off_mrec)), db, pitch, nvs, wave);
        }
        step_end_barrier<RB>();   // the DW's bank stores are visible to the next step's gather
        if constexpr (SM) {
            if (pfn) {   // the DW has read its records: the next step's take their place
                uint4 *dst = reinterpret_cast<uint4 *>(stg);
                if (tid + 0 * BLOCK < nudw) dst[tid + 0 * BLOCK] = pf0;
                if (tid + 1 * BLOCK < nudw) dst[tid + 1 * BLOCK] = pf1;
                if (tid + 2 * BLOCK < nudw) dst[tid + 2 * BLOCK] = pf2;
                if (tid + 3 * BLOCK < nudw) dst[tid + 3 * BLOCK] = pf3;
                if constexpr (PFU > 4) if (tid + 4 * BLOCK < nudw) dst[tid + 4 * BLOCK] = pf4;
                if constexpr (PFU > 4) if (tid + 5 * BLOCK < nudw) dst[tid + 5 * BLOCK] = pf5;
                if constexpr (PFU > 4) if (tid + 6 * BLOCK < nudw) dst[tid + 6 * BLOCK] = pf6;
                if constexpr (PFU > 4) if (tid + 7 * BLOCK < nudw) dst[tid + 7 * BLOCK] = pf7;
            }
        }
    }
    if constexpr (RB) {
        for (int i = threadIdx.x; i < Mr * NV; i += BLOCK) {
            const int row = i / NV, vq = i % NV;
            if (vq < nvs) *reinterpret_cast<raw_t *>(at(gbank, uint32_t(row) * uint32_t(hd) + uint32_t(vq * V))) =
                *reinterpret_cast<const raw_t *>(lbank + row * CW + vq * V);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Teams (memory mode). When slices of one 128-byte line per row leave most CUs idle (few
// streams), TEAM workgroups share one (stream, slice) instead of narrowing the slices: the
// chunk's tokens are cut into TEAM pieces of CT = C / TEAM tokens (whole 16-token tiles)
// and its DW groups into TEAM shares of consecutive records. A step has two phases of
// TEAM pieces each:
//   G(k)  gather of piece k's tokens, whole lines per row; u = beta (v - retrieved) and
//         inter of those tokens go to the chunk's exchange area
//   D(k)  after every G piece: delta_v = X u over all tokens, the readings of piece k's
//         tokens (QX u + inter), the DW of share k
// Every piece runs the same arithmetic as the one-workgroup kernel on the same operands,
// so the bits do not depend on the team size or on which workgroup runs which piece.
//
// Pieces are claimed with an atomic OR on the team's word for the phase (bit k claims
// piece k, bit 8 + k marks it done). A workgroup claims its own piece first and then waits
// for the others; a piece nobody has claimed after kTeamStealTicks is claimed and run by
// the waiting workgroup. A wait is therefore only ever on a piece that a running
// workgroup holds: a team does not need all of its workgroups on CUs at once (another
// kernel may hold some CUs), and every wait ends.
//
// Memory ordering. A team's workgroups sit on one XCD (blocks are dealt to the XCDs
// round-robin and a team's block ids are congruent mod 8; the library checks that
// placement on each device before it plans teams), so they share one L2, and the L1 is
// write-through: a piece's stores are complete in that L2 once every wave has waited for
// them (s_waitcnt vmcnt(0)), before its done bit is set. The words are only touched by
// atomics and agent-scope loads. A workgroup that has seen every done bit of a phase
// invalidates its L1 (the agent-scope acquire, buffer_inv sc1) before it reads what the
// others wrote. The agent-scope release (an L2 write-back, for readers on other XCDs) is
// not needed between workgroups of one L2, and would cost a quarter of the step.
constexpr uint32_t kTeamStealTicks = 2000;         // 20 us of the 100 MHz real-time counter
constexpr uint64_t kTeamGiveUpTicks = 200000000;   // 2 s: the bound of a workgroup's team waits
constexpr uint32_t kTeamGaveUp = 1u << 31;         // set in a word whose wait gave up


// Thread 0: the piece this workgroup runs next (claimed for it), or -1 once every piece of
// the phase is done. `first`: try the workgroup's own piece before waiting. A wait ends at
// the latest when the workgroup's waits have taken kTeamGiveUpTicks in all (`waited`);
// that cannot happen while every claimed piece completes, and it is then marked in the
// word (kTeamGaveUp) and every later wait of the workgroup returns at once.
template <int TEAM>
__device__ int team_next(uint32_t *word, int own, bool first, uint32_t steal_ticks, uint64_t &waited) {
    constexpr uint32_t kAllDone = ((1u << TEAM) - 1u) << 8;
    if (first) {
        const uint32_t old = __hip_atomic_fetch_or(word, 1u << own, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!(old & (1u << own))) return own;
    }
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        const uint32_t v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((v & kAllDone) == kAllDone) break;
        const uint64_t dt = __builtin_amdgcn_s_memrealtime() - t0;
        if (dt >= steal_ticks) {
            for (int k = 0; k < TEAM; ++k) {
                if (v & (1u << k)) continue;
                const uint32_t old = __hip_atomic_fetch_or(word, 1u << k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (!(old & (1u << k))) {
                    waited += dt;
                    return k;
                }
            }
        }
        if (waited + dt > kTeamGiveUpTicks) {
            __hip_atomic_fetch_or(word, kTeamGaveUp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            waited = kTeamGiveUpTicks + 1;
            return -1;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    waited += __builtin_amdgcn_s_memrealtime() - t0;
    return -1;
}

template <typename T, int V>
__device__ __forceinline__ void store_zero(T *p) {
    float z[V];
#pragma unroll
    for (int c = 0; c < V; ++c) z[c] = 0.0f;
    Vec<T, V>::store(p, z);
}

template <int V>
__device__ __forceinline__ void gmem_store_f32(float *p, const float (&x)[V]) {
#pragma unroll
    for (int c = 0; c < V; c += 4) *reinterpret_cast<float4 *>(p + c) = make_float4(x[c], x[c + 1], x[c + 2], x[c + 3]);
}

template <int V>
__device__ __forceinline__ void gmem_load_f32(const float *p, float (&x)[V]) {
#pragma unroll
    for (int c = 0; c < V; c += 4) {
        const float4 y = *reinterpret_cast<const float4 *>(p + c);
        x[c] = y.x; x[c + 1] = y.y; x[c + 2] = y.z; x[c + 3] = y.w;
    }
}

template <typename T, int V, int TEAM>
__global__ __launch_bounds__(kP2Block) void phase2_team_kernel(P2Args a) {
    constexpr int BLOCK = kP2Block, NV = 8, CW = V * NV;
    static_assert(V % 4 == 0, "slices of whole 16-byte float groups");
    using Cfg = P2Cfg<BLOCK, V>;
    constexpr int NW = Cfg::NW;
    extern __shared__ float lds[];
    // the piece thread 0 has claimed for the workgroup (-1: the phase is done), one word per
    // phase: thread 0 may claim the next step's first G piece while a wave still reads the
    // end of this step's D phase
    __shared__ int sel[2];
    const int C = a.C, hd = a.hd, S = a.S;
    const int CT = C / TEAM;                  // tokens per piece: whole 16-token tiles
    const int pitch = p2_pitch(CW);

    // Decode (stream, slice, member): block ids of one team are congruent mod 8 (one XCD).
    const int bid = blockIdx.x;
    const int xcd = bid % kXcds, m = bid / kXcds, unit = m / TEAM, me = m % TEAM;
    const int p = xcd + kXcds * (unit / S), slice = unit % S;
    const int vq0 = slice * NV;
    const int nvs = min(NV, a.hv - vq0);
    const int cwv = nvs * V;
    const int col0 = vq0 * V;
    T *gbank = static_cast<T *>(a.bank) + int64_t(p) * a.bstride + col0;

    float *ub = lds;                  // [C][pitch]: retrieved of a G piece's tokens, then u of every token
    float *db = lds + C * pitch;      // [C][pitch]: delta_v
    float *ib = db + C * pitch;       // [CT][pitch]: inter of one piece's tokens
    const int NIT = C / 16, NCT = (cwv + 15) / 16, NT = NIT * NCT;
    const int32_t vtp = stream_tokens(a, p);
    uint64_t waited = 0;   // thread 0: time spent in team waits

    for (int s = 0; s < a.steps; ++s) {
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        asm volatile("" : "+s"(wave));
        int lane = tid & 63;
        const int ti = a.ti0 + s;
        uint32_t *cb = const_cast<uint32_t *>(a.ws) + (int64_t(p) * a.steps + s) * a.words;
        const int nl = chunk_tokens(a, vtp, ti);
        const int rows = min(C, a.T - ti * C);
        const int64_t tok0 = int64_t(p) * a.T + int64_t(ti) * C;
        const T *vin = static_cast<const T *>(a.v) + tok0 * hd;
        T *out = static_cast<T *>(a.out) + tok0 * hd;
        if (nl == 0) {
            // past the stream's live tokens: no row changes; the readings of this member's
            // piece are zeros (each member's own piece: every member runs every step)
            for (int i = tid; i < CT * NV; i += BLOCK) {
                const int t = me * CT + i / NV, vq = i % NV;
                if (t < rows && vq < nvs) store_zero<T, V>(at(out, uint32_t(t * hd + col0 + vq * V)));
            }
            continue;
        }
        uint32_t *words = cb + a.off_meta + 8 + 2 * slice;     // [0]: G pieces, [1]: D pieces
        float *xus = reinterpret_cast<float *>(cb + a.off_xu) + int64_t(slice) * 2 * C * CW;   // [C][CW] u
        float *xis = xus + C * CW;                                                             // [C][CW] inter
        const float *beta_c = reinterpret_cast<const float *>(cb + a.off_beta);

        // ---- phase G
        for (bool first = true;; first = false) {
            if (tid == 0) {
                const int k = team_next<TEAM>(words, me, first, a.steal_ticks, waited);
                if (k < 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                sel[0] = k;
            }
            __syncthreads();
            const int k = sel[0];
            if (k < 0) break;
            const int t0 = k * CT, nlk = min(max(nl - t0, 0), CT);
            // v and beta of the piece's tokens, loaded before the gather (their round trip
            // overlaps it; the asm keeps the compiler from moving them down to their use)
            const int it_t = t0 + tid / NV, it_v = tid % NV;
            const bool mine = tid < CT * NV;
            const bool live = mine && it_t < t0 + nlk && it_v < nvs;
            float mv[V];
            Vec<T, V>::load(at(vin, live ? uint32_t(it_t * hd + col0 + it_v * V) : uint32_t(col0)), mv);
            const float mb = beta_c[live ? it_t : 0];
            asm volatile("" ::: "memory");
            {
                const float *gw = reinterpret_cast<const float *>(cb + a.off_gw);
                const float *gr = reinterpret_cast<const float *>(cb + a.off_gr);
                const int32_t *kid = reinterpret_cast<const int32_t *>(cb + a.off_kid);
                const int32_t *qid = reinterpret_cast<const int32_t *>(cb + a.off_qid);
                int nww = (NW * a.W + (a.W + a.R) / 2) / (a.W + a.R);
                nww = nww < 1 ? 1 : (nww > NW - 1 ? NW - 1 : nww);
                const bool wr = wave < nww;
                const int32_t *rid = wr ? kid + t0 * a.W : qid + t0 * a.R;
                const float *rwt = wr ? gw + t0 * a.W : gr + t0 * a.R;
                const int rwidth = wr ? a.W : a.R, rwave = wr ? wave : wave - nww, rnw = wr ? nww : NW - nww;
                float *rdst = wr ? ub + t0 * pitch : ib;
                if (((a.W | a.R) & 31) == 0)
                    gather_region<T, V, NV, 2, 4, false>(gbank, hd, rid, rwt, rwidth, nlk, 0, nvs, rdst, pitch, rwave,
                                                         rnw, lane, false, nullptr, nullptr, a.nt_gather != 0);
                else
                    gather_region<T, V, NV, Cfg::kBatch, 1, false>(gbank, hd, rid, rwt, rwidth, nlk, 0, nvs, rdst,
                                                                   pitch, rwave, rnw, lane, false, nullptr, nullptr,
                                                                   a.nt_gather != 0);
            }
            lds_barrier();
            if (mine) {   // u and inter of the piece's rows (zeros for padding tokens) to the exchange
                float uu[V], ii[V];
                if (live) {
                    float rr[V];
                    lds_load_vec<V>(ub + it_t * pitch + it_v * V, rr);
                    lds_load_vec<V>(ib + (it_t - t0) * pitch + it_v * V, ii);
#pragma unroll
                    for (int c = 0; c < V; ++c) uu[c] = mb * (mv[c] - rr[c]);
                } else {
#pragma unroll
                    for (int c = 0; c < V; ++c) uu[c] = ii[c] = 0.0f;
                }
                gmem_store_f32<V>(xus + it_t * CW + it_v * V, uu);
                gmem_store_f32<V>(xis + it_t * CW + it_v * V, ii);
            }
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            if (tid == 0) __hip_atomic_fetch_or(words, 1u << (8 + k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- u of every token
        for (int i = tid; i < C * NV; i += BLOCK) {
            float x[V];
            gmem_load_f32<V>(xus + (i / NV) * CW + (i % NV) * V, x);
            lds_store_vec<V>(ub + (i / NV) * pitch + (i % NV) * V, x);
        }
        __syncthreads();

        // ---- phase D
        const float *QX = reinterpret_cast<const float *>(cb + a.off_QX);
        const float *X = reinterpret_cast<const float *>(cb + a.off_X);
        bool have_d = false;
        for (bool first = true;; first = false) {
            if (tid == 0) {
                const int k = team_next<TEAM>(words + 1, me, first, a.steal_ticks, waited);
                if (k < 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                sel[1] = k;
            }
            __syncthreads();
            const int k = sel[1];
            if (k < 0) break;
            const int t0 = k * CT;
            for (int i = tid; i < CT * NV; i += BLOCK) {
                float x[V];
                gmem_load_f32<V>(xis + (t0 + i / NV) * CW + (i % NV) * V, x);
                lds_store_vec<V>(ib + (i / NV) * pitch + (i % NV) * V, x);
            }
            lds_barrier();
            // delta_v of every token (first piece only) and the readings of piece k, on the
            // matrix cores: the same tiles, k blocks and MFMA chains as the one-workgroup kernel
            asm volatile("" : "+v"(lane));
            const bool dod = !have_d;
            const int iy0 = t0 / 16, iy1 = (t0 + CT) / 16;
#pragma unroll
            for (int q = 0; q < Cfg::kMaxTiles; ++q) {
                const int tau = q * NW + ((q & 1) ? NW - 1 - wave : wave);
                if (tau >= NT) continue;
                const int it = tau / NCT, ct = tau - it * NCT;
                const bool cy = it >= iy0 && it < iy1;
                if (!cy && !dod) continue;
                const int ti_row = 16 * it + (lane & 15);
                const int cu = 16 * ct + (lane & 15);
                const int co = 16 * ct + 4 * (lane >> 4);
                const int ko = 4 * (lane >> 4);
                f32x4 y = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                if (cy && co < cwv) {
                    const float4 iv = *reinterpret_cast<const float4 *>(ib + (ti_row - t0) * pitch + co);
                    y = f32x4{iv.x, iv.y, iv.z, iv.w};
                }
                f32x4 d = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                for (int kb = 0; kb <= it; kb += Cfg::kMmDepth) {
                    // zero-initialized: operands loaded under a condition would otherwise stay
                    // live across the step loop (and spill)
                    float bq[Cfg::kMmDepth][4] = {}, bx[Cfg::kMmDepth][4] = {}, av[Cfg::kMmDepth][4] = {};
#pragma unroll
                    for (int j = 0; j < Cfg::kMmDepth; ++j) {
                        if (kb + j > it) continue;
                        if (cy) load_bop<true>(QX, C, ti_row, 16 * (kb + j) + ko, true, bq[j]);
                        if (dod) load_bop<true>(X, C, ti_row, 16 * (kb + j) + ko, true, bx[j]);
                        load_aop(ub + (16 * (kb + j) + ko) * pitch + cu, pitch, cu < cwv, av[j]);
                    }
#pragma unroll
                    for (int j = 0; j < Cfg::kMmDepth; ++j) {
                        if (kb + j > it) continue;
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) {
                            if (cy) y = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j][kk], bq[j][kk], y, 0, 0, 0);
                            if (dod) d = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j][kk], bx[j][kk], d, 0, 0, 0);
                        }
                    }
                }
                if (dod && co < cwv)
                    *reinterpret_cast<float4 *>(db + ti_row * pitch + co) = make_float4(d[0], d[1], d[2], d[3]);
                if (cy && ti_row < rows && co < cwv) {
                    if (ti_row >= nl) y = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    store_out4<T>(at(out, uint32_t(ti_row * hd + col0 + co)), y, min(4, cwv - co));
                }
            }
            have_d = true;
            lds_barrier();
            // DW of share k: group records [g0, g1) and many-member records [b0, b1)
            {
                const int32_t *meta = reinterpret_cast<const int32_t *>(cb + a.off_meta);
                const int32_t ng = meta[2], nbig = meta[4];
                const int32_t g0 = int32_t(int64_t(ng) * k / TEAM), g1 = int32_t(int64_t(ng) * (k + 1) / TEAM);
                const int32_t b0 = int32_t(int64_t(nbig) * k / TEAM), b1 = int32_t(int64_t(nbig) * (k + 1) / TEAM);
                dw_groups<T, V, NV, NW, Cfg::kDwBatch, false>(
                    gbank, hd, reinterpret_cast<const int4 *>(cb + a.off_grec) + g0, g1 - g0,
                    reinterpret_cast<const int4 *>(cb + a.off_brec) + b0, b1 - b0,
                    reinterpret_cast<const int2 *>(cb + a.off_mrec), db, pitch, nvs, wave);
            }
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            if (tid == 0) __hip_atomic_fetch_or(words + 1, 1u << (8 + k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------
template <typename T, int V, int MODE>
static const void *p2_fn_nv(int nv) {
    switch (nv) {
        case 1: return reinterpret_cast<const void *>(&phase2_kernel<T, V, 1, MODE>);
        case 2: return reinterpret_cast<const void *>(&phase2_kernel<T, V, 2, MODE>);
        case 4: return reinterpret_cast<const void *>(&phase2_kernel<T, V, 4, MODE>);
        default: return reinterpret_cast<const void *>(&phase2_kernel<T, V, 8, MODE>);
    }
}

template <int MODE>
static const void *phase2_fn_m(int dtype, int V, int nv) {
    if (dtype == 0) return V == 4 ? p2_fn_nv<float, 4, MODE>(nv) : p2_fn_nv<float, 1, MODE>(nv);
    if (V == 8) return p2_fn_nv<bf16, 8, MODE>(nv);
    // 8-byte vectors only for one-vector slices of a resident bank (the narrow slices the
    // planner picks for few streams); any other geometry has no kernel
    if (V == 4)
        return nv == 1 && MODE == kP2Resident ? reinterpret_cast<const void *>(&phase2_kernel<bf16, 4, 1, kP2Resident>)
                                               : nullptr;
    return p2_fn_nv<bf16, 1, MODE>(nv);
}

static const void *phase2_fn(int dtype, int V, int nv, int mode) {
    switch (mode) {
        case kP2Global: return phase2_fn_m<kP2Global>(dtype, V, nv);
        case kP2Staged: return phase2_fn_m<kP2Staged>(dtype, V, nv);
        default: return phase2_fn_m<kP2Resident>(dtype, V, nv);
    }
}

template <typename T, int V>
static const void *p2_team_fn_t(int team) {
    return team == 2 ? reinterpret_cast<const void *>(&phase2_team_kernel<T, V, 2>)
                     : reinterpret_cast<const void *>(&phase2_team_kernel<T, V, 4>);
}

// Team kernels: float banks in 16-byte vectors of 4, bfloat16 banks in vectors of 8.
static const void *phase2_team_fn(int dtype, int team) {
    return dtype == 0 ? p2_team_fn_t<float, 4>(team) : p2_team_fn_t<bf16, 8>(team);
}

// LDS of a team workgroup: u and delta_v of every token, inter of one piece's tokens.
size_t phase2_team_lds_bytes(int C, int V, int team) {
    return size_t(2 * C + C / team) * p2_pitch(8 * V) * sizeof(float);
}

// One workgroup of 64 threads per block id: the XCD it runs on.
__global__ __launch_bounds__(64) void xcd_probe_kernel(int32_t *xcc) {
    uint32_t x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    if (threadIdx.x == 0) xcc[blockIdx.x] = int32_t(x);
}

// Whether blocks whose ids are congruent mod 8 run on one XCD (teams share an L2 only
// then): one launch of 4096 blocks on a private stream, its XCD ids compared. `buf`:
// 4096 int32 of device memory. Any failure answers false.
bool phase2_teams_share_l2(int32_t *buf) {
    constexpr int kBlocks = 4096;
    hipStream_t st = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    static int32_t host[kBlocks];
    hipLaunchKernelGGL(xcd_probe_kernel, dim3(kBlocks), dim3(64), 0, st, buf);
    const bool ok = hipGetLastError() == hipSuccess && hipMemcpyAsync(host, buf, sizeof(host), hipMemcpyDeviceToHost, st) == hipSuccess &&
         hipStreamSynchronize(st) == hipSuccess;
    (void)hipStreamDestroy(st);
    if (!ok) {
        (void)hipGetLastError();
        return false;
    }
    for (int b = kXcds; b < kBlocks; ++b)
        if (host[b] != host[b % kXcds]) return false;
    return true;
}

hipError_t phase2_prepare() {
    for (int dt = 0; dt < 2; ++dt)
        for (int V : {1, dt == 0 ? 4 : 8})
            for (int nv : {1, 2, 4, 8})
                for (int mode : {kP2Global, kP2Staged, kP2Resident}) {
                    hipError_t e = hipFuncSetAttribute(phase2_fn(dt, V, nv, mode),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
                    if (e != hipSuccess) return e;
                }
    for (int dt = 0; dt < 2; ++dt)
        for (int team : {2, 4}) {
            hipError_t e = hipFuncSetAttribute(phase2_team_fn(dt, team), hipFuncAttributeMaxDynamicSharedMemorySize,
                                               160 * 1024 - 256);
            if (e != hipSuccess) return e;
        }
    return hipFuncSetAttribute(phase2_fn(1, 4, 1, kP2Resident), hipFuncAttributeMaxDynamicSharedMemorySize,
                               160 * 1024 - 256);
}

// LDS of a Phase-2 workgroup: the row regions (u, inter; staged, delta_v too); staged, the chunk's Phase-2 block and
// C x NV vectors of v; resident, the M x NV vectors of the bank slice besides.
size_t phase2_lds_bytes(const ChunkLayout &L, int C, int nv, int V, int es, int mode, int64_t M) {
    size_t b = size_t(mode >= kP2Staged ? 3 : 2) * p2_rows(C) * p2_pitch(nv * V) * sizeof(float);
    if (mode >= kP2Staged) b += size_t(L.off_stage1 - L.off_stage0) * 4 + size_t(p2_vst_bytes(C, nv, V, es));
    if (mode == kP2Resident) b += size_t(M) * nv * V * es;
    return b;
}

// The largest mode whose LDS fits the device (v's C x NV vectors staged one per thread).
int phase2_mode(const ChunkLayout &L, int C, int nv, int V, int es, int64_t M, int lds_limit) {
    if (int64_t(C) * nv > kP2Block) return kP2Global;
    if (M <= int64_t(lds_limit) && phase2_lds_bytes(L, C, nv, V, es, kP2Resident, M) + 256 <= size_t(lds_limit))
        return kP2Resident;
    if (phase2_lds_bytes(L, C, nv, V, es, kP2Staged, M) + 256 <= size_t(lds_limit)) return kP2Staged;
    return kP2Global;
}

hipError_t launch_phase2(const Problem &pb, const Slab &sl, int V, const P2Geom &g, hipStream_t st) {
    const ChunkLayout &L = sl.lay;
    // The staged modes replace the block's leading DW records and the rest at different
    // points of a step: the DW reads nothing at or past off_gw, the gather and matmul nothing
    // before it.
    const int64_t dw_end = std::max({L.off_grec + 4 * L.E, L.off_mrec + 2 * L.E, L.off_brec + 4 * L.HMAX});
    if (L.off_grec != L.off_stage0 || dw_end > L.off_gw || L.off_gr < L.off_gw || L.off_kid < L.off_gw ||
        L.off_qid < L.off_gw || L.off_meta < L.off_gw || L.off_beta < L.off_gw || L.off_X < L.off_gw ||
        L.off_QX < L.off_gw)
        return hipErrorInvalidValue;
    P2Args a{};
    a.v = pb.v; a.bank = pb.bank; a.out = pb.out; a.valid = pb.valid;
    a.ws = sl.ws; a.M = pb.M; a.words = L.words; a.bstride = pb.bank_stride;
    a.T = pb.T; a.C = pb.C; a.W = pb.W; a.R = pb.R; a.hd = pb.hd; a.P = pb.P;
    a.S = g.S; a.hv = pb.hd / V; a.ti0 = sl.ti0; a.steps = sl.steps;
    a.off_gw = int32_t(L.off_gw); a.off_gr = int32_t(L.off_gr); a.off_beta = int32_t(L.off_beta);
    a.off_X = int32_t(L.off_X); a.off_QX = int32_t(L.off_QX); a.off_meta = int32_t(L.off_meta);
    a.off_grec = int32_t(L.off_grec); a.off_mrec = int32_t(L.off_mrec); a.off_brec = int32_t(L.off_brec);
    a.off_kid = int32_t(L.off_kid); a.off_qid = int32_t(L.off_qid);
    a.off_stage0 = int32_t(L.off_stage0); a.off_stage1 = int32_t(L.off_stage1);
    a.off_xu = int32_t(L.off_xu);
    const int es = pb.dtype == 0 ? 4 : 2;
    a.nt_gather = once_rows_streamed(pb) ? 1 : 0;
    void *args[] = {&a};
    if (g.team > 1) {
        // the planner's conditions, checked again where the kernel's indexing depends on them
        if (g.mode != kP2Global || g.nv != 8 || V * es != 16 || pb.P % kXcds != 0 || pb.C % (16 * g.team) != 0 ||
            pb.C / g.team * 8 > kP2Block || g.S > kTeamMaxSlices || int64_t(g.S) * 8 * V > ((pb.hd + 63) & ~63))
            return hipErrorInvalidValue;
        // SDM_P2_TEAM_STEAL: the steal wait in ticks (0: claim any unclaimed piece at once)
        const char *se = getenv("SDM_P2_TEAM_STEAL");
        a.steal_ticks = se ? uint32_t(strtoul(se, nullptr, 10)) : kTeamStealTicks;
        const void *fn = phase2_team_fn(pb.dtype, g.team);
        return hipLaunchKernel(fn, dim3(unsigned(int64_t(pb.P) * g.S * g.team)), dim3(kP2Block), args,
                               phase2_team_lds_bytes(pb.C, V, g.team), st);
    }
    const dim3 grid(unsigned(int64_t(pb.P) * g.S)), block(kP2Block);
    const void *fn = phase2_fn(pb.dtype, V, g.nv, g.mode);
    if (!fn) return hipErrorInvalidValue;
    return hipLaunchKernel(fn, grid, block, args,
                           phase2_lds_bytes(L, pb.C, g.nv, V, es, g.mode, pb.M), st);
}

}  // namespace sdm

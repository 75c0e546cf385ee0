// Phase 2 of the chunked SDM forward on gfx950: the sequential steps that carry the bank
// across chunks (phase2_kernels.py docstring and _sdm_dual_matmul, sparse-delta-memory
// 2.0.0 wheel, diffend page 23). Per step, for the chunk of each stream:
//     gather       retrieved[i] = sum_w gw[i,w] B[s_iw],  inter[i] = sum_r gr[i,r] B[q_ir]
//     dual matmul  u = beta (v - retrieved);  delta_v = X u;  readings = QX u + inter
//     DW           each written slot s: B[s] = exp(L_last) B[s] + sum_members cw delta_v[t]
//
// Every column of the bank evolves on its own (all Phase-1 quantities are column-free),
// so the work of a stream splits by column slices with no exchange at all. A slice is a
// 128-byte segment of each row (one cache line), or the whole row if shorter: narrower
// slices would make every workgroup re-read the chunk's ids, weights, X and QX.
//
// Where slices alone leave too few workgroups to cover the chip, a TEAM of K workgroups
// shares one (stream, slice): member k gathers and multiplies the tokens of its share of
// the chunk and writes the bank rows of its share of the groups. The u and delta_v rows
// pass between members through L2 (the team's exchange rows), and three team barriers
// per step order gather -> matmul -> DW -> next gather. Teams run as a cooperative
// launch (all workgroups resident); a barrier gives up after a bounded spin and raises a
// flag word, so every wave always terminates. With K = 1 the barriers are plain
// workgroup barriers.
//
// Workgroups of one stream are placed on one XCD (blocks are dealt round-robin to the
// 8 XCDs) so that its slices and team members share one L2.
//
// Determinism: each output element has exactly one writer, and every sum runs in a fixed
// order (gather: entry order; matmul: column index ascending; DW: decay term first, then
// the group's members in token order), so the bits do not depend on the slicing, the team
// size or the launch size.
#include "common.h"

namespace sdm {

constexpr int kSpinLimit = 1 << 22;   // about 0.2 s of polling before a barrier gives up

struct P2Args {
    Problem pb;
    Slab sl;
    int32_t nv;        // vectors per column slice
    int32_t S;         // slices per row
    int32_t K;         // workgroups per (stream, slice) team
    int32_t hv;        // vectors per row (hd / V)
    float *xchg;       // team exchange rows: [teams][2][C][nv * V]
    int32_t *ctr;      // [teams] barrier counters, zero at launch
    int32_t *err;      // set to 1 by a barrier that timed out
};

// Team barrier: every global write of the workgroup before it is visible to the team
// after it.
__device__ __forceinline__ void team_barrier(int32_t *ctr, int32_t target, int32_t *err, int *broken) {
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0 && !*broken) {
        __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        int spins = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++spins > kSpinLimit) {
                __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                *broken = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
    __threadfence();
}

// acc[c] = sum_w wts[w] * bank[ids[w]][col + c], w ascending; eight rows in flight.
template <typename T, int V>
__device__ __forceinline__ void gather_row(const T *bank, int hd, const int32_t *ids, const float *wts, int width,
                                           int64_t col, float (&acc)[V]) {
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] = 0.0f;
    int w = 0;
    for (; w + 8 <= width; w += 8) {
        int32_t s[8];
        float wt[8];
        typename Vec<T, V>::raw_t raw[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            s[u] = ids[w + u];
            wt[u] = wts[w + u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) raw[u] = Vec<T, V>::load_raw(bank + int64_t(s[u]) * hd + col);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            float row[V];
            Vec<T, V>::unpack(raw[u], row);
#pragma unroll
            for (int c = 0; c < V; ++c) acc[c] = fmaf(wt[u], row[c], acc[c]);
        }
    }
    for (; w < width; ++w) {
        float row[V];
        Vec<T, V>::load(bank + int64_t(ids[w]) * hd + col, row);
        const float wt = wts[w];
#pragma unroll
        for (int c = 0; c < V; ++c) acc[c] = fmaf(wt, row[c], acc[c]);
    }
}

// acc[c] += sum_{j < n} xrow[j] * u[j * pitch + c], j ascending.
template <int V>
__device__ __forceinline__ void dot_row(const float *xrow, int n, const float *u, int pitch, bool vec4,
                                        float (&acc)[V]) {
    int j = 0;
    if (vec4) {
#pragma unroll 4
        for (; j + 4 <= n; j += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(xrow + j);
            const float *u0 = u + j * pitch;
#pragma unroll
            for (int c = 0; c < V; ++c) acc[c] = fmaf(x.x, u0[c], acc[c]);
#pragma unroll
            for (int c = 0; c < V; ++c) acc[c] = fmaf(x.y, u0[pitch + c], acc[c]);
#pragma unroll
            for (int c = 0; c < V; ++c) acc[c] = fmaf(x.z, u0[2 * pitch + c], acc[c]);
#pragma unroll
            for (int c = 0; c < V; ++c) acc[c] = fmaf(x.w, u0[3 * pitch + c], acc[c]);
        }
    }
    for (; j < n; ++j) {
        const float x = xrow[j];
#pragma unroll
        for (int c = 0; c < V; ++c) acc[c] = fmaf(x, u[j * pitch + c], acc[c]);
    }
}

// Reductions are cut into a shape-only number of contiguous parts (never the launch
// geometry): each part is summed in order by one lane, and the parts of one output are
// combined by a fixed xor butterfly, ((p0 + p1) + (p2 + p3)); every lane of the group ends
// with the same bits (additions only, no fused products). Items come in wavefront-sized
// chunks of 64: lane l of a chunk holds part l / (64 / parts) of output
// chunk * (64 / parts) + l % (64 / parts), so the lanes of one part read neighbouring
// outputs (broadcast / consecutive LDS words) and the partners sit 16 or 32 lanes apart.
__host__ __device__ __forceinline__ int split_parts(int n) { return n >= 32 ? 4 : (n >= 16 ? 2 : 1); }
// Gather: entries of one token; no split once a chunk has plenty of entries (C * width).
__host__ __device__ __forceinline__ int gather_parts(int C, int width) {
    return int64_t(C) * width >= 16384 ? 1 : split_parts(width);
}
// Matmul: columns of one row; no split for the largest chunks.
__host__ __device__ __forceinline__ int matmul_parts(int C) { return C >= 256 ? 1 : split_parts(C); }

__device__ __forceinline__ void split_item(int it, int parts, int &out, int &part) {
    const int G = kWave / parts, ch = it >> 6, l = it & 63;
    part = l / G;
    out = ch * G + (l - part * G);
}

__host__ __device__ __forceinline__ int split_items(int outputs, int parts) {
    const int G = kWave / parts;
    return (outputs + G - 1) / G * kWave;
}

template <int V>
__device__ __forceinline__ void combine_parts(float (&acc)[V], int parts) {
    if (parts >= 4) {
#pragma unroll
        for (int c = 0; c < V; ++c) acc[c] += __shfl_xor(acc[c], 16, 64);
    }
    if (parts >= 2) {
#pragma unroll
        for (int c = 0; c < V; ++c) acc[c] += __shfl_xor(acc[c], 32, 64);
    }
}

__device__ __forceinline__ void copy_rows(float *dst, const float *src, int rows, int nvs, int pitch, int V, int BLOCK) {
    // rows x (nvs * V) floats, both with row pitch `pitch`
    const int per = nvs * V;
    for (int it = threadIdx.x; it < rows * per; it += BLOCK) {
        const int r = it / per, c = it - r * per;
        dst[r * pitch + c] = src[r * pitch + c];
    }
}

template <typename T, int V, int BLOCK>
__global__ __launch_bounds__(BLOCK) void phase2_kernel(P2Args a) {
    extern __shared__ float lds[];
    __shared__ int broken;
    const Problem &pb = a.pb;
    const Slab &sl = a.sl;
    const int C = pb.C, W = pb.W, R = pb.R, hd = pb.hd;
    const int nv = a.nv, S = a.S, K = a.K;
    const int cw = nv * V;                  // LDS / exchange row pitch in floats
    const int tpw = (C + K - 1) / K;        // tokens per team member

    // Decode (stream, slice, member); streams stay on one XCD when P % 8 == 0.
    const int bid = blockIdx.x, per_stream = S * K;
    int p, r;
    if (pb.P % kXcds == 0) {
        const int xcd = bid % kXcds, m = bid / kXcds;
        p = xcd + kXcds * (m / per_stream);
        r = m % per_stream;
    } else {
        p = bid / per_stream;
        r = bid % per_stream;
    }
    const int slice = r / K, k = r % K;
    const int team = p * S + slice;
    const int vq0 = slice * nv;
    const int nvs = min(nv, a.hv - vq0);
    const int i0 = min(C, k * tpw), i1 = min(C, i0 + tpw);
    const int tid = threadIdx.x;
    T *bank = static_cast<T *>(pb.bank) + int64_t(p) * pb.M * hd;
    const T *vin = static_cast<const T *>(pb.v);
    T *out = static_cast<T *>(pb.out);
    const ChunkLayout &L = sl.lay;
    const bool vec4 = (C & 3) == 0;

    float *ub = lds;                        // [C][cw]: u of every token (K = 1: own), then delta (K > 1)
    float *ib = lds + C * cw;               // [K == 1 ? C : tpw][cw]: inter of own tokens (K = 1: then delta)
    float *xu = a.xchg + int64_t(team) * 2 * C * cw;
    float *xd = xu + int64_t(C) * cw;
    int32_t *ctr = a.ctr + team;
    int32_t bar = 0;
    if (tid == 0) broken = 0;
    __syncthreads();

    for (int s = 0; s < sl.steps; ++s) {
        const int ti = sl.ti0 + s;
        const int64_t n = int64_t(p) * sl.steps + s;
        const uint32_t *cb = sl.chunk(n);
        const int nl = n_live_tokens(pb, p, ti);
        const int rows = min(C, pb.T - ti * C);
        const int64_t tok0 = int64_t(p) * pb.T + int64_t(ti) * C;
        const int own_live = max(0, min(i1, nl) - i0);

        // ---- gather of own live tokens: retrieved -> ub[i], inter -> ib[i - i0]. Outputs
        //      (token, vector) of the writes, then of the reads, each region in whole
        //      wavefront chunks (split_item).
        const float *gw = reinterpret_cast<const float *>(cb + L.off_gw);
        const float *gr = reinterpret_cast<const float *>(cb + L.off_gr);
        const int sfw = gather_parts(C, W), sfr = gather_parts(C, R);
        const int nout = own_live * nvs;
        const int nwp = split_items(nout, sfw), nrp = split_items(nout, sfr);
        for (int it = tid; it < nwp + nrp; it += BLOCK) {
            const bool rd = it >= nwp;
            const int sf = rd ? sfr : sfw;
            int o, blk;
            split_item(rd ? it - nwp : it, sf, o, blk);
            const bool live = o < nout;
            const int li = live ? o / nvs : 0, vq = live ? o - li * nvs : 0;
            const int i = i0 + li;
            const int width = rd ? R : W;
            const int per = (width + sf - 1) / sf;
            const int w0 = min(width, blk * per), w1 = live ? min(width, w0 + per) : w0;
            const int32_t *ids = (rd ? pb.q_idx : pb.k_idx) + (tok0 + i) * width + w0;
            const float *wts = (rd ? gr : gw) + int64_t(i) * width + w0;
            float acc[V];
            gather_row<T, V>(bank, hd, ids, wts, w1 - w0, int64_t(vq0 + vq) * V, acc);
            combine_parts<V>(acc, sf);
            if (live && blk == 0) {
                float *dst = rd ? ib + li * cw + vq * V : ub + i * cw + vq * V;
#pragma unroll
                for (int c = 0; c < V; ++c) dst[c] = acc[c];
            }
        }
        __syncthreads();

        // ---- u = beta (v - retrieved) on own rows; 0 for padding rows
        const float *beta_c = reinterpret_cast<const float *>(cb + L.off_beta);
        for (int it = tid; it < (i1 - i0) * nvs; it += BLOCK) {
            const int li = it / nvs, vq = it - li * nvs;
            const int i = i0 + li;
            float *ur = ub + i * cw + vq * V;
            float uu[V];
            if (i < nl) {
                float vv[V];
                Vec<T, V>::load(vin + (tok0 + i) * hd + int64_t(vq0 + vq) * V, vv);
                const float b = beta_c[i];
#pragma unroll
                for (int c = 0; c < V; ++c) uu[c] = b * (vv[c] - ur[c]);
            } else {
#pragma unroll
                for (int c = 0; c < V; ++c) uu[c] = 0.0f;
            }
#pragma unroll
            for (int c = 0; c < V; ++c) ur[c] = uu[c];
            if (K > 1) {
#pragma unroll
                for (int c = 0; c < V; ++c) xu[i * cw + vq * V + c] = uu[c];
            }
        }
        if (K > 1) {
            team_barrier(ctr, ++bar * K, a.err, &broken);
            copy_rows(ub, xu, nl, nvs, cw, V, BLOCK);   // rows >= nl are never read
        }
        __syncthreads();

        // ---- readings = QX u + inter on own rows that exist (padding rows +0);
        //      K > 1: delta_v = X u of own live rows into the exchange rows
        const float *QX = reinterpret_cast<const float *>(cb + L.off_QX);
        const float *X = reinterpret_cast<const float *>(cb + L.off_X);
        const int own_rows = max(0, min(i1, rows) - i0);
        // Output (row, vector); part p sums columns [p * cq, (p + 1) * cq) of the row.
        const int sfm = matmul_parts(C), cq = (((C + sfm - 1) / sfm) + 3) & ~3;
        const int nmo = own_rows * nvs;
        for (int it = tid; it < split_items(nmo, sfm); it += BLOCK) {
            int k3, blk;
            split_item(it, sfm, k3, blk);
            const bool exists = k3 < nmo;
            const int li = exists ? k3 / nvs : 0, vq = exists ? k3 - li * nvs : 0;
            const int i = i0 + li;
            const bool live = exists && i < nl;
            const int j0 = min(i + 1, blk * cq), j1 = live ? min(i + 1, j0 + cq) : j0;
            float o[V];
#pragma unroll
            for (int c = 0; c < V; ++c) o[c] = 0.0f;
            dot_row<V>(QX + int64_t(i) * C + j0, j1 - j0, ub + j0 * cw + vq * V, cw, vec4, o);
            combine_parts<V>(o, sfm);
            float d[V];
            if (K > 1) {
#pragma unroll
                for (int c = 0; c < V; ++c) d[c] = 0.0f;
                dot_row<V>(X + int64_t(i) * C + j0, j1 - j0, ub + j0 * cw + vq * V, cw, vec4, d);
                combine_parts<V>(d, sfm);
            }
            if (exists && blk == 0) {
                if (live) {
                    const float *ir = ib + li * cw + vq * V;
#pragma unroll
                    for (int c = 0; c < V; ++c) o[c] += ir[c];
                    if (K > 1) {
#pragma unroll
                        for (int c = 0; c < V; ++c) xd[i * cw + vq * V + c] = d[c];
                    }
                }
                Vec<T, V>::store(out + (tok0 + i) * hd + int64_t(vq0 + vq) * V, o);
            }
        }
        const float *D;
        if (K > 1) {
            team_barrier(ctr, ++bar * K, a.err, &broken);
            copy_rows(ub, xd, nl, nvs, cw, V, BLOCK);
            D = ub;
        } else {
            __syncthreads();
            // delta_v = X u into ib (inter is no longer needed)
            const int ndo = nl * nvs;
            for (int it = tid; it < split_items(ndo, sfm); it += BLOCK) {
                int k3, blk;
                split_item(it, sfm, k3, blk);
                const bool exists = k3 < ndo;
                const int i = exists ? k3 / nvs : 0, vq = exists ? k3 - i * nvs : 0;
                const int j0 = min(i + 1, blk * cq), j1 = exists ? min(i + 1, j0 + cq) : j0;
                float d[V];
#pragma unroll
                for (int c = 0; c < V; ++c) d[c] = 0.0f;
                dot_row<V>(X + int64_t(i) * C + j0, j1 - j0, ub + j0 * cw + vq * V, cw, vec4, d);
                combine_parts<V>(d, sfm);
                if (exists && blk == 0) {
                    float *dr = ib + i * cw + vq * V;
#pragma unroll
                    for (int c = 0; c < V; ++c) dr[c] = d[c];
                }
            }
            D = ib;
        }
        __syncthreads();

        // ---- DW on own groups: one writer per written row, members in token order
        const int32_t *meta = reinterpret_cast<const int32_t *>(cb + L.off_meta);
        const int32_t ng = nl > 0 ? meta[2] : 0;
        const int32_t g0 = int32_t(int64_t(ng) * k / K), g1 = int32_t(int64_t(ng) * (k + 1) / K);
        const int4 *grec = reinterpret_cast<const int4 *>(cb + L.off_grec);
        const int2 *mrec = reinterpret_cast<const int2 *>(cb + L.off_mrec);
        const int64_t nit = int64_t(g1 - g0) * nvs;
        for (int64_t base = tid; base < nit; base += 4 * BLOCK) {
            int4 rec[4];
            int vq[4];
            bool ok[4];
            typename Vec<T, V>::raw_t raw[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t it = base + int64_t(u) * BLOCK;
                ok[u] = it < nit;
                const int32_t g = ok[u] ? g0 + int32_t(it / nvs) : g0;
                vq[u] = ok[u] ? int(it % nvs) : 0;
                rec[u] = ok[u] ? grec[g] : make_int4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (ok[u]) raw[u] = Vec<T, V>::load_raw(bank + int64_t(rec[u].x) * hd + int64_t(vq0 + vq[u]) * V);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (!ok[u]) continue;
                float acc[V];
                Vec<T, V>::unpack(raw[u], acc);
                const float dec = __int_as_float(rec[u].w);
#pragma unroll
                for (int c = 0; c < V; ++c) acc[c] *= dec;
                const int32_t m1 = rec[u].y + rec[u].z;
                for (int32_t m = rec[u].y; m < m1; ++m) {
                    const int2 mr = mrec[m];
                    const float cwv = __int_as_float(mr.y);
                    const float *dr = D + mr.x * cw + vq[u] * V;
#pragma unroll
                    for (int c = 0; c < V; ++c) acc[c] = fmaf(cwv, dr[c], acc[c]);
                }
                Vec<T, V>::store(bank + int64_t(rec[u].x) * hd + int64_t(vq0 + vq[u]) * V, acc);
            }
        }
        if (K > 1) team_barrier(ctr, ++bar * K, a.err, &broken);
        else __syncthreads();
    }
}

__global__ void zero_words_kernel(int32_t *p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
        p[i] = 0;
}

// ---------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------
template <typename T, int V, int B>
static const void *p2_fn() {
    return reinterpret_cast<const void *>(&phase2_kernel<T, V, B>);
}

static const void *phase2_fn(int dtype, int V, int block) {
    if (dtype == 0) {
        if (V == 4) return block == 256 ? p2_fn<float, 4, 256>() : block == 512 ? p2_fn<float, 4, 512>() : p2_fn<float, 4, 1024>();
        return block == 256 ? p2_fn<float, 1, 256>() : block == 512 ? p2_fn<float, 1, 512>() : p2_fn<float, 1, 1024>();
    }
    if (V == 8) return block == 256 ? p2_fn<bf16, 8, 256>() : block == 512 ? p2_fn<bf16, 8, 512>() : p2_fn<bf16, 8, 1024>();
    return block == 256 ? p2_fn<bf16, 1, 256>() : block == 512 ? p2_fn<bf16, 1, 512>() : p2_fn<bf16, 1, 1024>();
}

hipError_t phase2_prepare() {
    for (int dt = 0; dt < 2; ++dt)
        for (int V : {1, dt == 0 ? 4 : 8})
            for (int b : {256, 512, 1024}) {
                hipError_t e = hipFuncSetAttribute(phase2_fn(dt, V, b), hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   160 * 1024 - 256);
                if (e != hipSuccess) return e;
            }
    return hipSuccess;
}

size_t phase2_lds_bytes(int C, int nv, int V, int K) {
    const int tpw = (C + K - 1) / K;
    return size_t(C + (K == 1 ? C : tpw)) * nv * V * sizeof(float);
}

// Words of the workspace's Phase-2 control area: flag word, barrier counters and
// exchange rows, bounded for any slicing of a head of hd columns.
int64_t phase2_control_words(int P, int C, int hd) {
    const int64_t ctr = align_words(int64_t(P) * (hd + 1));
    const int64_t xch = align_words(int64_t(2) * C * P * (int64_t(hd) + 256));
    return 64 + ctr + xch;
}


hipError_t launch_phase2(const Problem &pb, const Slab &sl, int V, const P2Geom &g, uint32_t *control,
                         hipStream_t st) {
    P2Args a{pb, sl, g.nv, g.S, g.K, pb.hd / V, nullptr, nullptr, nullptr};
    a.err = reinterpret_cast<int32_t *>(control);
    a.ctr = reinterpret_cast<int32_t *>(control + 64);
    a.xchg = reinterpret_cast<float *>(control + 64 + align_words(int64_t(pb.P) * (pb.hd + 1)));
    const int64_t teams = int64_t(pb.P) * g.S;
    const dim3 grid(unsigned(teams * g.K)), block(unsigned(g.block));
    const size_t lds = phase2_lds_bytes(pb.C, g.nv, V, g.K);
    const void *fn = phase2_fn(pb.dtype, V, g.block);
    if (g.K > 1) {
        hipLaunchKernelGGL(zero_words_kernel, dim3(unsigned((teams + 255) / 256)), dim3(256), 0, st, a.ctr, teams);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        void *args[] = {&a};
        return hipLaunchCooperativeKernel(fn, grid, block, args, unsigned(lds), st);
    }
    void *args[] = {&a};
    return hipLaunchKernel(fn, grid, block, args, lds, st);
}

// Occupancy of a geometry: workgroups that fit on the device at once.
hipError_t phase2_max_resident(int dtype, int V, const P2Geom &g, int C, int cus, int64_t *out) {
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, phase2_fn(dtype, V, g.block), g.block,
                                                                phase2_lds_bytes(C, g.nv, V, g.K));
    *out = int64_t(per_cu) * cus;
    return e;
}

}  // namespace sdm

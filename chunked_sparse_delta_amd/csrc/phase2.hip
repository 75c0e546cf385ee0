// Phase 2 of the chunked SDM forward on gfx950: the sequential steps that carry the bank
// across chunks (phase2_kernels.py docstring and _sdm_dual_matmul, sparse-delta-memory
// 2.0.0 wheel, diffend page 23). Per step, for the chunk of each stream:
//     gather       retrieved[i] = sum_w gw[i,w] B[s_iw],  inter[i] = sum_r gr[i,r] B[q_ir]
//     dual matmul  u = beta (v - retrieved);  delta_v = X u;  readings = QX u + inter
//     DW           each written slot s: B[s] = exp(L_last) B[s] + sum_members cw delta_v[t]
//
// Every column of the bank evolves on its own (all Phase-1 quantities are column-free),
// so one workgroup owns one (stream, column slice) and runs all steps of the slab with
// no synchronization beyond its own barriers: its gather, matmul and DW touch only its
// columns of its stream's rows. Workgroups of one stream are placed on one XCD (blocks
// are dealt round-robin to the 8 XCDs), so the slices of a bank row, and the stream's
// Phase-1 arrays, meet in one L2.
//
// Determinism: each output element has exactly one writer, and every sum runs in a fixed
// order (gather: entry order; matmul: column index ascending; DW: decay term first, then
// the group's members in token order), whatever the slicing or the launch size.
#include "common.h"

namespace sdm {

struct P2Args {
    Problem pb;
    Slab sl;
    int32_t nv;        // vectors per column slice
    int32_t nslices;   // slices per row
    int32_t hv;        // vectors per row (hd / V)
};

template <typename T, int V, int BLOCK>
__global__ __launch_bounds__(BLOCK) void phase2_kernel(P2Args a) {
    extern __shared__ float lds[];
    const Problem &pb = a.pb;
    const Slab &sl = a.sl;
    const int C = pb.C, W = pb.W, R = pb.R, hd = pb.hd;
    const int nv = a.nv;
    const int cwid = nv * V;                // floats per LDS row
    float *us = lds;                        // [C][cwid]  retrieved, then u
    float *xs = lds + C * cwid;             // [C][cwid]  inter, then delta_v

    // (stream, slice) of this workgroup; all slices of a stream share an XCD when P % 8 == 0.
    int p, slice;
    const int bid = blockIdx.x;
    if (pb.P % kXcds == 0) {
        const int xcd = bid % kXcds, m = bid / kXcds;
        p = xcd + kXcds * (m / a.nslices);
        slice = m % a.nslices;
    } else {
        p = bid / a.nslices;
        slice = bid % a.nslices;
    }
    const int vq0 = slice * nv;                        // first vector of the slice
    const int nvs = min(nv, a.hv - vq0);               // vectors in this slice
    const int tid = threadIdx.x;
    T *bank = static_cast<T *>(pb.bank) + int64_t(p) * pb.M * hd;
    const T *vin = static_cast<const T *>(pb.v);
    T *out = static_cast<T *>(pb.out);
    const ChunkLayout &L = sl.lay;

    for (int s = 0; s < sl.steps; ++s) {
        const int ti = sl.ti0 + s;
        const int64_t n = int64_t(p) * sl.steps + s;
        const uint32_t *cb = sl.chunk(n);
        const int nl = n_live_tokens(pb, p, ti);
        const int rows = min(C, pb.T - ti * C);       // token rows of this chunk in `out`
        const int64_t tok0 = int64_t(p) * pb.T + int64_t(ti) * C;
        const int nitem = nl * nvs;

        // ---- gather (retrieved into us, inter into xs)
        const float *gw = reinterpret_cast<const float *>(cb + L.off_gw);
        const float *gr = reinterpret_cast<const float *>(cb + L.off_gr);
        for (int it = tid; it < 2 * nitem; it += BLOCK) {
            const bool rd = it >= nitem;
            const int k = rd ? it - nitem : it;
            const int i = k / nvs, vq = k - i * nvs;
            const int width = rd ? R : W;
            const int32_t *ids = (rd ? pb.q_idx : pb.k_idx) + (tok0 + i) * width;
            const float *wts = (rd ? gr : gw) + int64_t(i) * width;
            const int64_t col = int64_t(vq0 + vq) * V;
            float acc[V];
#pragma unroll
            for (int c = 0; c < V; ++c) acc[c] = 0.0f;
            int w = 0;
            for (; w + 4 <= width; w += 4) {
                int32_t sid[4];
                float wt[4], row[4][V];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    sid[u] = ids[w + u];
                    wt[u] = wts[w + u];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) Vec<T, V>::load(bank + int64_t(sid[u]) * hd + col, row[u]);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int c = 0; c < V; ++c) acc[c] = fmaf(wt[u], row[u][c], acc[c]);
            }
            for (; w < width; ++w) {
                float row[V];
                Vec<T, V>::load(bank + int64_t(ids[w]) * hd + col, row);
                const float wt = wts[w];
#pragma unroll
                for (int c = 0; c < V; ++c) acc[c] = fmaf(wt, row[c], acc[c]);
            }
            float *dst = (rd ? xs : us) + i * cwid + vq * V;
#pragma unroll
            for (int c = 0; c < V; ++c) dst[c] = acc[c];
        }
        __syncthreads();

        // ---- u = beta (v - retrieved); 0 for padding rows
        const float *beta_c = reinterpret_cast<const float *>(cb + L.off_beta);
        for (int it = tid; it < C * nvs; it += BLOCK) {
            const int i = it / nvs, vq = it - i * nvs;
            float *ur = us + i * cwid + vq * V;
            if (i < nl) {
                float vv[V];
                Vec<T, V>::load(vin + (tok0 + i) * hd + int64_t(vq0 + vq) * V, vv);
                const float b = beta_c[i];
#pragma unroll
                for (int c = 0; c < V; ++c) ur[c] = b * (vv[c] - ur[c]);
            } else {
#pragma unroll
                for (int c = 0; c < V; ++c) ur[c] = 0.0f;
            }
        }
        __syncthreads();

        // ---- readings = QX u + inter (rows that exist; padding rows +0)
        const float *QX = reinterpret_cast<const float *>(cb + L.off_QX);
        const float *X = reinterpret_cast<const float *>(cb + L.off_X);
        for (int it = tid; it < rows * nvs; it += BLOCK) {
            const int i = it / nvs, vq = it - i * nvs;
            float o[V];
#pragma unroll
            for (int c = 0; c < V; ++c) o[c] = 0.0f;
            if (i < nl) {
                const float *qrow = QX + int64_t(i) * C;
                const float *ucol = us + vq * V;
                for (int j = 0; j <= i; ++j) {
                    const float x = qrow[j];
#pragma unroll
                    for (int c = 0; c < V; ++c) o[c] = fmaf(x, ucol[j * cwid + c], o[c]);
                }
                const float *ir = xs + i * cwid + vq * V;
#pragma unroll
                for (int c = 0; c < V; ++c) o[c] += ir[c];
            }
            Vec<T, V>::store(out + (tok0 + i) * hd + int64_t(vq0 + vq) * V, o);
        }
        __syncthreads();

        // ---- delta_v = X u (into xs)
        for (int it = tid; it < nl * nvs; it += BLOCK) {
            const int i = it / nvs, vq = it - i * nvs;
            float d[V];
#pragma unroll
            for (int c = 0; c < V; ++c) d[c] = 0.0f;
            const float *xrow = X + int64_t(i) * C;
            const float *ucol = us + vq * V;
            for (int j = 0; j <= i; ++j) {
                const float x = xrow[j];
#pragma unroll
                for (int c = 0; c < V; ++c) d[c] = fmaf(x, ucol[j * cwid + c], d[c]);
            }
            float *dr = xs + i * cwid + vq * V;
#pragma unroll
            for (int c = 0; c < V; ++c) dr[c] = d[c];
        }
        __syncthreads();

        // ---- DW: one writer per written row (the group), members in token order
        const int32_t *meta = reinterpret_cast<const int32_t *>(cb + L.off_meta);
        const int32_t ng = nl > 0 ? meta[2] : 0;
        const int32_t *gpos = reinterpret_cast<const int32_t *>(cb + L.off_gpos);
        const int32_t *gslot = reinterpret_cast<const int32_t *>(cb + L.off_gslot);
        const float *gdecay = reinterpret_cast<const float *>(cb + L.off_gdecay);
        const int32_t *stok = reinterpret_cast<const int32_t *>(cb + L.off_stok);
        const float *scw = reinterpret_cast<const float *>(cb + L.off_scw);
        for (int64_t it = tid; it < int64_t(ng) * nvs; it += BLOCK) {
            const int32_t g = int32_t(it / nvs);
            const int vq = int(it - int64_t(g) * nvs);
            T *row = bank + int64_t(gslot[g]) * hd + int64_t(vq0 + vq) * V;
            const float dec = gdecay[g];
            float acc[V];
            Vec<T, V>::load(row, acc);
#pragma unroll
            for (int c = 0; c < V; ++c) acc[c] *= dec;
            const int32_t m1 = gpos[g + 1];
            for (int32_t m = gpos[g]; m < m1; ++m) {
                const float cw = scw[m];
                const float *dr = xs + stok[m] * cwid + vq * V;
#pragma unroll
                for (int c = 0; c < V; ++c) acc[c] = fmaf(cw, dr[c], acc[c]);
            }
            Vec<T, V>::store(row, acc);
        }
        __syncthreads();
    }
}

constexpr int kP2Block = 256;

template <typename T, int V>
static hipError_t p2_prepare_one() {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&phase2_kernel<T, V, kP2Block>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

hipError_t phase2_prepare() {
    hipError_t e;
    if ((e = p2_prepare_one<float, 4>()) != hipSuccess) return e;
    if ((e = p2_prepare_one<float, 1>()) != hipSuccess) return e;
    if ((e = p2_prepare_one<bf16, 8>()) != hipSuccess) return e;
    return p2_prepare_one<bf16, 1>();
}

size_t phase2_lds_bytes(int C, int nv, int V) { return size_t(2) * C * nv * V * sizeof(float); }

hipError_t launch_phase2(const Problem &pb, const Slab &sl, int V, int nv, hipStream_t st) {
    P2Args a{pb, sl, nv, 0, pb.hd / V};
    a.nslices = (a.hv + nv - 1) / nv;
    const dim3 grid(unsigned(int64_t(pb.P) * a.nslices)), block(kP2Block);
    const size_t lds = phase2_lds_bytes(pb.C, nv, V);
    if (pb.dtype == 0) {
        if (V == 4) hipLaunchKernelGGL((phase2_kernel<float, 4, kP2Block>), grid, block, lds, st, a);
        else hipLaunchKernelGGL((phase2_kernel<float, 1, kP2Block>), grid, block, lds, st, a);
    } else {
        if (V == 8) hipLaunchKernelGGL((phase2_kernel<bf16, 8, kP2Block>), grid, block, lds, st, a);
        else hipLaunchKernelGGL((phase2_kernel<bf16, 1, kP2Block>), grid, block, lds, st, a);
    }
    return hipGetLastError();
}

}  // namespace sdm

// Exact top-k over all sums of product-key factor values, forward (product_key_topk, page
// 23, product_key_topk.py, the function's docstring): the selection that turns a layer's
// factor scores into slot ids for the memory op.
//
// Rule, as numbered conditions: (1) a slot chooses one column per factor and its score is
// the float32 total of the chosen values in factor order (bfloat16 input with F > 2: the
// running total is brought to bfloat16 before each further factor joins it); (2) scores
// compare as float32, negative zero beneath positive zero, NaN as negative infinity;
// (3) within a factor, columns go by value, highest first, the higher column index first
// among equal values, and stage 0 keeps n = min(k, f_0) of factor 0's; (4) stage f pairs a
// surviving rank i < n with a rank j < m = min(k, f_f) of factor f where (i + 1)(j + 1) <= c
// = min(k, n m) and keeps the c best, an exact tie going to the greater i + j and then the
// greater i; (5) survivors leave by ascending linear index with scores rounded to the input
// dtype.
//
// General rows: one workgroup of 256 threads per row; every ordering is a bitonic sort in LDS of 64-bit
// keys whose high word is the float32 order and whose low word encodes the tie rule, so
// each comparison is one unsigned compare and the result is unique:
//   factor ranks   key = order(value) << 32 | column               (descending)
//   stage pairs    key = order(score) << 32 | (i + j) << 8 | i      (descending)
//   output         key = lin << 8 | position in the last stage      (ascending)
#include <stdlib.h>

#include <type_traits>

#include "common.h"

namespace sdm {

// Limits (the host entry point checks them before any launch).
constexpr int kTopkBlock = 256;
constexpr int kTopkMaxK = 256;
constexpr int kTopkMaxFactor = 4096;      // columns of a factor ranked by one sort in LDS (wider
                                          // factors, up to the host's limit of 65535, in pieces)
constexpr int kTopkMaxFactors = 8;
constexpr int kTopkPairs = 2048;          // >= sum over i < 256 of min(256, 256 / (i + 1)) = 1567

// The float32 order of the rule as an unsigned key: NaN as -inf, -0 below +0.
__device__ __forceinline__ uint32_t topk_order(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) u = 0xFF800000u;   // NaN -> -inf
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float bf16_round(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7F800000u) == 0x7F800000u) return x;   // inf, NaN
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    return __uint_as_float(r);
}

// Bitonic sort of n (a power of two) keys in LDS by the whole workgroup; descending when
// desc. Ends with a barrier.
__device__ void topk_bitonic(uint64_t *key, int n, bool desc) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < (n >> 1); t += kTopkBlock) {
                // t-th pair of this step: i has bit `stride` clear, partner i + stride
                const int i = ((t / stride) * (stride << 1)) + (t % stride);
                const int jx = i + stride;
                const bool up = ((i & size) == 0) != desc;   // ascending block unless desc
                const uint64_t a = key[i], b = key[jx];
                if ((a > b) == up) {
                    key[i] = b;
                    key[jx] = a;
                }
            }
            __syncthreads();
        }
    }
}

struct TopkArgs {
    const void *raw;          // [rows, D]
    void *val;                // [rows, kk] in the input dtype
    int64_t *lin;             // [rows, kk]
    int64_t rows;
    int32_t D, F, k, kk, bf16;
    int32_t fw[kTopkMaxFactors];   // factor widths
    int32_t f0[kTopkMaxFactors];   // first column of each factor
};

__global__ __launch_bounds__(kTopkBlock) void topk_kernel(TopkArgs a) {
    __shared__ uint64_t key[kTopkMaxFactor > kTopkPairs ? kTopkMaxFactor : kTopkPairs];
    static_assert((kTopkMaxFactor & (kTopkMaxFactor - 1)) == 0 && kTopkMaxFactor > kTopkMaxK, "sort buffer");
    __shared__ float rval[kTopkMaxFactors][kTopkMaxK];   // factor f's rank r: value
    __shared__ int32_t rcol[kTopkMaxFactors][kTopkMaxK];  //                    column
    __shared__ float cs[2][kTopkMaxK];                    // current / next stage: scores
    __shared__ int64_t cl[2][kTopkMaxK];                  //                       linear indices
    __shared__ int32_t off[kTopkMaxK + 1];                // pair offsets per rank i
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const char *rowp = static_cast<const char *>(a.raw) + row * int64_t(a.D) * (a.bf16 ? 2 : 4);
    auto value = [&](int c) -> float {
        return a.bf16 ? __uint_as_float(uint32_t(reinterpret_cast<const uint16_t *>(rowp)[c]) << 16)
                      : reinterpret_cast<const float *>(rowp)[c];
    };

    // Rank every factor: the first min(k, f) entries of (value desc, column desc). A factor
    // wider than the sort buffer is ranked in pieces: the running first kTopkMaxK keys and
    // the next kTopkMaxFactor - kTopkMaxK columns are sorted together, so the leading
    // kTopkMaxK keys stay those of every column seen (keys are unique; 0 pads below all).
    for (int f = 0; f < a.F; ++f) {
        const int w = a.fw[f];
        if (w <= kTopkMaxFactor) {
            const int n2 = w <= 1 ? 1 : 1 << (32 - __clz(w - 1));
            for (int c = tid; c < n2; c += kTopkBlock)
                key[c] = c < w ? (uint64_t(topk_order(value(a.f0[f] + c))) << 32) | uint32_t(c) : 0ull;
            __syncthreads();
            topk_bitonic(key, n2, true);
        } else {
            constexpr int CH = kTopkMaxFactor - kTopkMaxK;
            for (int c = tid; c < kTopkMaxK; c += kTopkBlock) key[c] = 0ull;
            for (int c0 = 0; c0 < w; c0 += CH) {
                for (int c = tid; c < CH; c += kTopkBlock)
                    key[kTopkMaxK + c] =
                        c0 + c < w ? (uint64_t(topk_order(value(a.f0[f] + c0 + c))) << 32) | uint32_t(c0 + c) : 0ull;
                __syncthreads();
                topk_bitonic(key, kTopkMaxFactor, true);
            }
        }
        const int m = min(a.k, w);
        for (int r = tid; r < m; r += kTopkBlock) {
            const int c = int(uint32_t(key[r]));
            rcol[f][r] = c;
            rval[f][r] = value(a.f0[f] + c);
        }
        __syncthreads();
    }
    // Stage 0
    int n = min(a.k, a.fw[0]);
    for (int r = tid; r < n; r += kTopkBlock) {
        cs[0][r] = rval[0][r];
        cl[0][r] = rcol[0][r];
    }
    __syncthreads();
    int cur = 0;
    for (int f = 1; f < a.F; ++f) {
        const int m = min(a.k, a.fw[f]);
        const int c = int(min(int64_t(a.k), int64_t(n) * m));
        const bool rnd = a.bf16 && a.F > 2 && f < a.F - 1;
        // pairs of rank i: j < min(m, c / (i + 1)); offsets by a serial scan (n <= 256)
        if (tid == 0) {
            int s = 0;
            for (int i = 0; i < n; ++i) {
                off[i] = s;
                s += min(m, c / (i + 1));
            }
            off[n] = s;
        }
        __syncthreads();
        const int np = off[n];
        const int n2 = np <= 1 ? 1 : 1 << (32 - __clz(np - 1));
        for (int q = tid; q < n2; q += kTopkBlock) {
            uint64_t kv = 0ull;
            if (q < np) {
                int lo = 0, hi = n - 1;   // the rank i whose pairs hold q
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (off[mid] <= q) lo = mid;
                    else hi = mid - 1;
                }
                const int i = lo, j = q - off[i];
                float s = cs[cur][i] + rval[f][j];
                if (rnd) s = bf16_round(s);
                kv = (uint64_t(topk_order(s)) << 32) | uint32_t(((i + j) << 8) | i);
            }
            key[q] = kv;
        }
        __syncthreads();
        topk_bitonic(key, n2, true);
        for (int r = tid; r < c; r += kTopkBlock) {
            const uint32_t lo32 = uint32_t(key[r]);
            const int i = int(lo32 & 0xFFu), j = int((lo32 >> 8) & 0x1FFu) - i;
            float s = cs[cur][i] + rval[f][j];
            if (rnd) s = bf16_round(s);
            cs[cur ^ 1][r] = s;
            cl[cur ^ 1][r] = cl[cur][i] * a.fw[f] + rcol[f][j];
        }
        __syncthreads();
        cur ^= 1;
        n = c;
    }
    // Output by ascending linear index (unique, < 2^55)
    const int n2 = n <= 1 ? 1 : 1 << (32 - __clz(n - 1));
    for (int r = tid; r < n2; r += kTopkBlock) key[r] = r < n ? (uint64_t(cl[cur][r]) << 8) | uint32_t(r) : ~0ull;
    __syncthreads();
    topk_bitonic(key, n2, false);
    for (int r = tid; r < n; r += kTopkBlock) {
        const int src = int(key[r] & 0xFFu);
        const float s = cs[cur][src];
        a.lin[row * a.kk + r] = cl[cur][src];
        if (a.bf16) reinterpret_cast<uint16_t *>(a.val)[row * a.kk + r] = uint16_t(__float_as_uint(bf16_round(s)) >> 16);
        else reinterpret_cast<float *>(a.val)[row * a.kk + r] = s;
    }
}

// ---------------------------------------------------------------------------------------
// Small rows (every factor <= 256 columns, k <= 64): one row per wavefront, four rows per
// workgroup. The same keys, sorted in registers: element e = r * 64 + lane of a wave's
// R registers; partners at distance >= 64 are the lane's own registers, nearer ones come
// by lane shuffles. Only the per-wave LDS tables (factor ranks, stage lists, pair offsets)
// are shared between lanes, with nothing but the wave's own in-order LDS accesses.
constexpr int kTopkWaveFactor = 256, kTopkWaveK = 64;

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t x, int m) {
    const uint32_t lo = uint32_t(__shfl_xor(int(uint32_t(x)), m, 64));
    const uint32_t hi = uint32_t(__shfl_xor(int(uint32_t(x >> 32)), m, 64));
    return (uint64_t(hi) << 32) | lo;
}

// Bitonic sort of the 64 R keys held by the wave (element r * 64 + lane in k[r]).
template <int R>
__device__ __forceinline__ void wave_bitonic(uint64_t (&k)[R], bool desc, int lane) {
    constexpr int N = 64 * R;
#pragma unroll
    for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= 64) {
                const int rs = stride >> 6;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int r2 = r ^ rs;
                    if (r2 < r) continue;
                    const int e = r * 64 + lane;
                    const bool up = ((e & size) == 0) != desc;
                    const uint64_t a = k[r], b = k[r2];
                    if ((a > b) == up) {
                        k[r] = b;
                        k[r2] = a;
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint64_t o = shfl_xor64(k[r], stride);
                    const int e = r * 64 + lane;
                    const bool up = ((e & size) == 0) != desc, lower = (lane & stride) == 0;
                    // the lower element of the pair keeps the smaller key in an ascending block
                    k[r] = (lower == up) ? (k[r] < o ? k[r] : o) : (k[r] > o ? k[r] : o);
                }
            }
        }
    }
}

struct TopkWaveLds {
    float rval[kTopkMaxFactors][kTopkWaveK];
    int32_t rcol[kTopkMaxFactors][kTopkWaveK];
    float cs[2][kTopkWaveK];
    int64_t cl[2][kTopkWaveK];
    int32_t off[kTopkWaveK + 1];
};

__global__ __launch_bounds__(kTopkBlock) void topk_wave_kernel(TopkArgs a) {
    constexpr int kWaves = kTopkBlock / 64;
    __shared__ TopkWaveLds lds_all[kWaves];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t row = int64_t(blockIdx.x) * kWaves + wv;
    if (row >= a.rows) return;
    TopkWaveLds &L = lds_all[wv];
    const char *rowp = static_cast<const char *>(a.raw) + row * int64_t(a.D) * (a.bf16 ? 2 : 4);
    auto value = [&](int c) -> float {
        return a.bf16 ? __uint_as_float(uint32_t(reinterpret_cast<const uint16_t *>(rowp)[c]) << 16)
                      : reinterpret_cast<const float *>(rowp)[c];
    };
    // factor ranks: sort (order(value) << 32 | column) descending, keep the first min(k, w);
    // the sort spans the fewest registers that hold the factor
    for (int f = 0; f < a.F; ++f) {
        const int w = a.fw[f];
        auto rank = [&](auto rc) {
            constexpr int R = decltype(rc)::value;
            uint64_t k[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int c = r * 64 + lane;
                k[r] = c < w ? (uint64_t(topk_order(value(a.f0[f] + c))) << 32) | uint32_t(c) : 0ull;
            }
            wave_bitonic<R>(k, true, lane);
            if (lane < min(a.k, w)) {
                const int c = int(uint32_t(k[0]));
                L.rcol[f][lane] = c;
                L.rval[f][lane] = value(a.f0[f] + c);
            }
        };
        if (w <= 64) rank(std::integral_constant<int, 1>{});
        else if (w <= 128) rank(std::integral_constant<int, 2>{});
        else rank(std::integral_constant<int, 4>{});
    }
    __builtin_amdgcn_wave_barrier();
    int n = min(a.k, a.fw[0]);
    if (lane < n) {
        L.cs[0][lane] = L.rval[0][lane];
        L.cl[0][lane] = L.rcol[0][lane];
    }
    __builtin_amdgcn_wave_barrier();
    int cur = 0;
    for (int f = 1; f < a.F; ++f) {
        const int m = min(a.k, a.fw[f]);
        const int c = min(a.k, n * m);
        const bool rnd = a.bf16 && a.F > 2 && f < a.F - 1;
        // pairs of rank i (one lane each): j < min(m, c / (i + 1)); exclusive offsets by a scan
        const int cnt = lane < n ? min(m, c / (lane + 1)) : 0;
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d, 64);
            if (lane >= d) incl += y;
        }
        L.off[lane] = incl - cnt;
        if (lane == 63) L.off[64] = incl;
        __builtin_amdgcn_wave_barrier();
        const int np = L.off[64];
        // the stage's pairs, sorted over the fewest registers that hold them; leaves the
        // best pair keys in registers 0 of lanes 0 .. c - 1
        uint64_t best = 0ull;
        auto pairs = [&](auto rc) {
            constexpr int R = decltype(rc)::value;
            uint64_t k[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int q = r * 64 + lane;
                k[r] = 0ull;
                if (q < np) {
                    int lo = 0, hi = n - 1;   // the rank i whose pairs hold q
                    while (lo < hi) {
                        const int mid = (lo + hi + 1) >> 1;
                        if (L.off[mid] <= q) lo = mid;
                        else hi = mid - 1;
                    }
                    const int i = lo, j = q - L.off[i];
                    float s = L.cs[cur][i] + L.rval[f][j];
                    if (rnd) s = bf16_round(s);
                    k[r] = (uint64_t(topk_order(s)) << 32) | uint32_t(((i + j) << 8) | i);
                }
            }
            wave_bitonic<R>(k, true, lane);
            best = k[0];
        };
        if (np <= 64) pairs(std::integral_constant<int, 1>{});
        else if (np <= 128) pairs(std::integral_constant<int, 2>{});
        else if (np <= 256) pairs(std::integral_constant<int, 4>{});
        else pairs(std::integral_constant<int, 8>{});
        if (lane < c) {
            const uint32_t lo32 = uint32_t(best);
            const int i = int(lo32 & 0xFFu), j = int((lo32 >> 8) & 0x1FFu) - i;
            float s = L.cs[cur][i] + L.rval[f][j];
            if (rnd) s = bf16_round(s);
            L.cs[cur ^ 1][lane] = s;
            L.cl[cur ^ 1][lane] = L.cl[cur][i] * a.fw[f] + L.rcol[f][j];
        }
        __builtin_amdgcn_wave_barrier();
        cur ^= 1;
        n = c;
    }
    // output by ascending linear index
    uint64_t k1[1];
    k1[0] = lane < n ? (uint64_t(L.cl[cur][lane]) << 8) | uint32_t(lane) : ~0ull;
    wave_bitonic<1>(k1, false, lane);
    if (lane < n) {
        const int src = int(k1[0] & 0xFFu);
        const float s = L.cs[cur][src];
        a.lin[row * a.kk + lane] = L.cl[cur][src];
        if (a.bf16) reinterpret_cast<uint16_t *>(a.val)[row * a.kk + lane] = uint16_t(__float_as_uint(bf16_round(s)) >> 16);
        else reinterpret_cast<float *>(a.val)[row * a.kk + lane] = s;
    }
}

// ---------------------------------------------------------------------------------------
// Backward: d(val)/d(raw) is 1 at each factor column of a selected slot (the roundings of a
// score pass the gradient through), so the gradient of a raw column is the sum of the
// output gradients of the selected slots that use it. One row per wavefront: the slots'
// factor columns are decoded once into LDS, then each lane owns columns and adds, slot by
// slot in output (ascending index) order, the gradients of the slots that use them, so
// every sum runs in one fixed order with no atomics. The sums are float32, rounded once.
struct TopkBwdArgs {
    const int64_t *lin;       // [rows, kk]
    const void *gval;         // [rows, kk] in the dtype
    void *graw;               // [rows, D] in the dtype
    int64_t rows;
    int32_t D, F, kk, bf16;
    int32_t fw[kTopkMaxFactors];
    int32_t f0[kTopkMaxFactors];
};

__global__ __launch_bounds__(kTopkBlock) void topk_bwd_kernel(TopkBwdArgs a) {
    constexpr int kWaves = kTopkBlock / 64;
    __shared__ int32_t cols[kWaves][kTopkMaxK][kTopkMaxFactors];
    __shared__ float gsh[kWaves][kTopkMaxK];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t row = int64_t(blockIdx.x) * kWaves + wv;
    if (row >= a.rows) return;
    for (int sidx = lane; sidx < a.kk; sidx += 64) {
        int64_t l = a.lin[row * a.kk + sidx];
        for (int f = a.F - 1; f >= 0; --f) {   // lin = (..(c_0 f_1 + c_1) ..) f_{F-1} + c_{F-1}
            cols[wv][sidx][f] = int32_t(l % a.fw[f]);
            l /= a.fw[f];
        }
        gsh[wv][sidx] = a.bf16 ? __uint_as_float(uint32_t(static_cast<const uint16_t *>(a.gval)[row * a.kk + sidx]) << 16)
                               : static_cast<const float *>(a.gval)[row * a.kk + sidx];
    }
    __builtin_amdgcn_wave_barrier();
    for (int c0 = 0; c0 < a.D; c0 += 64) {
        const int col = c0 + lane;
        int f = 0;
        while (f + 1 < a.F && col >= a.f0[f + 1]) ++f;
        const int c = col - a.f0[f];
        float acc = 0.0f;
        for (int sidx = 0; sidx < a.kk; ++sidx)
            if (cols[wv][sidx][f] == c) acc += gsh[wv][sidx];
        if (col < a.D) {
            if (a.bf16) static_cast<uint16_t *>(a.graw)[row * a.D + col] = uint16_t(__float_as_uint(bf16_round(acc)) >> 16);
            else static_cast<float *>(a.graw)[row * a.D + col] = acc;
        }
    }
}

hipError_t launch_topk_bwd(const int64_t *lin, const void *gval, void *graw, int64_t rows, int32_t D, int32_t F,
                           int32_t kk, bool bf16, const int32_t *fw, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    TopkBwdArgs a{};
    a.lin = lin;
    a.gval = gval;
    a.graw = graw;
    a.rows = rows;
    a.D = D;
    a.F = F;
    a.kk = kk;
    a.bf16 = bf16 ? 1 : 0;
    int32_t c0 = 0;
    for (int f = 0; f < F; ++f) {
        a.fw[f] = fw[f];
        a.f0[f] = c0;
        c0 += fw[f];
    }
    hipLaunchKernelGGL(topk_bwd_kernel, dim3(unsigned((rows + 3) / 4)), dim3(kTopkBlock), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_topk(const void *raw, void *val, int64_t *lin, int64_t rows, int32_t D, int32_t F, int32_t k,
                       int32_t kk, bool bf16, const int32_t *fw, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    TopkArgs a{};
    a.raw = raw;
    a.val = val;
    a.lin = lin;
    a.rows = rows;
    a.D = D;
    a.F = F;
    a.k = k;
    a.kk = kk;
    a.bf16 = bf16 ? 1 : 0;
    int32_t c0 = 0;
    for (int f = 0; f < F; ++f) {
        a.fw[f] = fw[f];
        a.f0[f] = c0;
        c0 += fw[f];
    }
    bool small = k <= kTopkWaveK;
    for (int f = 0; f < F; ++f) small = small && fw[f] <= kTopkWaveFactor;
    const char *env = getenv("SDM_TOPK_PATH");   // "block" forces the general kernel (tests)
    if (env && env[0] == 'b') small = false;
    if (small)
        hipLaunchKernelGGL(topk_wave_kernel, dim3(unsigned((rows + 3) / 4)), dim3(kTopkBlock), 0, st, a);
    else
        hipLaunchKernelGGL(topk_kernel, dim3(unsigned(rows)), dim3(kTopkBlock), 0, st, a);
    return hipGetLastError();
}

}  // namespace sdm

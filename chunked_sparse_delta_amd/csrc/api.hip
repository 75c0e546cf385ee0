// C ABI of the SDM forward (include/sdm.h): argument checks on the host, slab planning
// from shapes only, and the launch sequence per slab:
//     Phase 1 (sort, groups, reads, Gram) -> solve -> Phase 2 (all steps of the slab).
// Everything is enqueued on the caller's stream; nothing is allocated, nothing synchronizes.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <stdlib.h>

#include <mutex>

#include "sdm.h"
#include "common.h"
#include "wy_impl.h"
#include "backward.h"

namespace sdm {
hipError_t phase1_prepare();
hipError_t phase2_prepare();
hipError_t wy_prepare();
hipError_t launch_phase1(const Problem &pb, const Slab &sl, hipStream_t st, hipEvent_t *ev, bool fused,
                         const WyArgs &wa, int lognp);
bool phase1_fused(const ChunkLayout &L, int C, int lds_limit);
hipError_t part_prepare();
int part_lognp(int64_t E, int64_t F, int key_bits);
hipError_t launch_wy(const float *A, const float *beta, const float *QK, float *X, float *QX, int C, int64_t n,
                     int64_t stride, int64_t bstride, hipStream_t st);
hipError_t launch_phase2(const Problem &pb, const Slab &sl, int V, const P2Geom &g, hipStream_t st);
size_t gram_lds_bytes(int C);
hipError_t launch_topk(const void *raw, void *val, int64_t *lin, int64_t rows, int32_t D, int32_t F, int32_t k,
                       int32_t kk, bool bf16, const int32_t *fw, hipStream_t st);
hipError_t launch_topk_bwd(const int64_t *lin, const void *gval, void *graw, int64_t rows, int32_t D, int32_t F,
                           int32_t kk, bool bf16, const int32_t *fw, hipStream_t st);
constexpr int kTopkMaxK = 256, kTopkMaxWidth = 65535, kTopkMaxFactors = 8;
size_t phase2_lds_bytes(const ChunkLayout &L, int C, int nv, int V, int es, int mode, int64_t M);
size_t phase2_team_lds_bytes(int C, int V, int team);
bool phase2_teams_share_l2(int32_t *buf);
int phase2_mode(const ChunkLayout &L, int C, int nv, int V, int es, int64_t M, int lds_limit);
}  // namespace sdm

using namespace sdm;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(SDM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The scratch of sdm_fwd_noalloc: a file-scope device array, one copy per GPU the library
// runs on, held until the process ends. In host code its name is a host-side stand-in, not
// a device address: the setup below takes each device's own address of it once
// (hipGetSymbolAddress, with that device current) and every use goes through that pointer.
__device__ __align__(256) unsigned char scratch[SDM_NOALLOC_SCRATCH_BYTES];

// Per-device one-time setup: the large-LDS kernel attributes, the LDS limit, and the
// device address of the static scratch.
struct DeviceInfo {
    bool ready = false;
    int lds_per_block = 0;   // the limit the plans use
    int lds_default = 0;     // the device's default per-block limit (reported by sdm_fwd_plan)
    int cus = 0;
    void *scratch = nullptr; // this device's copy of `scratch`
    bool teams = false;      // blocks congruent mod 8 share an XCD (Phase-2 teams allowed)
};
// The kernels' opt-in LDS attribute is set to at most this many bytes.
constexpr int kMaxLdsPerBlock = 160 * 1024 - 256;
DeviceInfo g_dev[64];
std::mutex g_dev_mu;

int device_info(DeviceInfo **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(SDM_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DeviceInfo &d = g_dev[dev];
    if (!d.ready) {
        // LDS per workgroup: the default per-block limit, or the larger limit a kernel may opt
        // into with hipFuncAttributeMaxDynamicSharedMemorySize (every kernel here does)
        int optin = 0;
        if ((e = hipDeviceGetAttribute(&d.lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev)) != hipSuccess)
            return hip_fail(e, "hipDeviceGetAttribute(MaxSharedMemoryPerBlock)");
        if ((e = hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev)) != hipSuccess)
            return hip_fail(e, "hipDeviceGetAttribute(SharedMemPerBlockOptin)");
        d.lds_default = d.lds_per_block;
        if (optin > d.lds_per_block) d.lds_per_block = optin;
        if (d.lds_per_block > kMaxLdsPerBlock) d.lds_per_block = kMaxLdsPerBlock;
        if ((e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
            return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
        if ((e = phase1_prepare()) != hipSuccess) return hip_fail(e, "hipFuncSetAttribute (phase 1)");
        if ((e = phase2_prepare()) != hipSuccess) return hip_fail(e, "hipFuncSetAttribute (phase 2)");
        if ((e = wy_prepare()) != hipSuccess) return hip_fail(e, "hipFuncSetAttribute (solve)");
        if ((e = part_prepare()) != hipSuccess) return hip_fail(e, "hipFuncSetAttribute (phase 1, partitioned)");
        if ((e = bwd_prepare()) != hipSuccess) return hip_fail(e, "hipFuncSetAttribute (backward)");
        void *sp = nullptr;
        if ((e = hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch))) != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress (static scratch)");
        d.scratch = sp;
        // nothing else uses the scratch before this setup returns
        d.teams = phase2_teams_share_l2(static_cast<int32_t *>(sp));
        d.ready = true;
    }
    *out = &d;
    return SDM_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int key_bits(int64_t M) {
    int bits = 0;
    for (int64_t m = M - 1; m > 0; m >>= 1) ++bits;
    return bits;
}

// Radix passes of at most 9 bits over the slot id, as even as possible.
int sort_passes(int64_t M) {
    const int passes = (key_bits(M) + 8) / 9;
    return passes < 1 ? 1 : passes;
}

int sort_digit(int64_t M) {
    const int p = sort_passes(M), d = (key_bits(M) + p - 1) / p;
    return d < 1 ? 1 : d;
}

// Phase 1 of chunks that do not run fused: the partitioned kernel (LDS-resident slot
// partitions) first, unless SDM_P1_PART=0; returns log2 of its partition count (shapes
// only; SDM_P1_NP_LOG overrides it, for sweeps), or -1 with pb.part_on cleared.
int plan_part(Problem &pb, const ChunkLayout &L, bool fused) {
    pb.part_on = 0;
    if (fused) return -1;
    const char *env = getenv("SDM_P1_PART");
    if (env && env[0] == '0') return -1;
    int lg = part_lognp(L.E, L.F, pb.key_bits);
    const char *ov = getenv("SDM_P1_NP_LOG");
    if (ov && ov[0] >= '0' && ov[0] <= '7') lg = ov[0] - '0';
    pb.part_on = 1;
    return lg;
}

struct Checked {
    Problem pb;
    ChunkLayout lay;
    int V;       // elements per vector move (16 B, or 1)
    int es;      // bank element bytes
};

// Shape checks shared by sdm_fwd, sdm_chunk_mats and the workspace query.
int check_shape(int32_t P, int32_t T, int32_t C, int32_t W, int32_t R, int32_t hd) {
    if (P < 1 || T < 1) return fail(SDM_ERR_SHAPE, "need streams >= 1 and tokens >= 1, got %d and %d", P, T);
    if (C < 16 || C > kMaxChunk) return fail(SDM_ERR_RANGE, "chunk must be in 16..256, got %d", C);
    if (W < 1 || W > kMaxWidth || R < 1 || R > kMaxWidth)
        return fail(SDM_ERR_SHAPE, "need 1..256 write and read slots per token, got W=%d R=%d", W, R);
    if (hd < 1) return fail(SDM_ERR_SHAPE, "head_dim must be >= 1, got %d", hd);
    if (hd > (1 << 20)) return fail(SDM_ERR_RANGE, "head_dim %d is above 2^20", hd);
    const int64_t Nt = (int64_t(T) + C - 1) / C;
    if (int64_t(P) * Nt * C >= (int64_t(1) << 31))
        return fail(SDM_ERR_RANGE, "%d streams of %d tokens padded to chunks of %d exceed 2^31 - 1 token rows", P, T, C);
    return SDM_OK;
}

int check_call(int32_t P, int32_t T, int32_t C, const sdm_slots *slots, const sdm_weights *weights, const float *beta,
               const float *g, int32_t G, const void *v, int64_t M, int32_t hd, int32_t dtype, void *bank_data,
               bool shared, const int32_t *valid, void *out, bool need_bank, Checked *ck) {
    if (!slots || !weights) return fail(SDM_ERR_NULL, "slots and weights must not be NULL");
    int rc = check_shape(P, T, C, slots->W, slots->R, hd);
    if (rc) return rc;
    if (dtype != SDM_F32 && dtype != SDM_BF16) return fail(SDM_ERR_DTYPE, "bank dtype must be SDM_F32 or SDM_BF16, got %d", dtype);
    const int kb = slots->write_id_bytes ? slots->write_id_bytes : 4, qb = slots->read_id_bytes ? slots->read_id_bytes : 4;
    if ((kb != 4 && kb != 8) || (qb != 4 && qb != 8))
        return fail(SDM_ERR_DTYPE, "slot ids must be int32 or int64 (4 or 8 bytes), got %d and %d", kb, qb);
    const int W = slots->W, R = slots->R;
    if (G != 1 && G != W) return fail(SDM_ERR_SHAPE, "log_decay must hold 1 or W=%d gates per token, got %d", W, G);
    if (M < 1) return fail(SDM_ERR_SHAPE, "the bank needs at least one row per stream, got %lld", (long long)M);
    if ((shared ? 1 : int64_t(P)) * M >= (int64_t(1) << 31))
        return fail(SDM_ERR_RANGE, "a bank of %lld rows (x %d streams) has 2^31 or more slots", (long long)M,
                    shared ? 1 : P);
    if (M * hd * (dtype == SDM_F32 ? 4 : 2) >= (int64_t(1) << 31))
        return fail(SDM_ERR_RANGE, "a stream's bank of %lld rows x %d columns is 2 GiB or more", (long long)M, hd);
    if (!slots->write || !slots->read || !weights->write || !weights->read || !beta || !g)
        return fail(SDM_ERR_NULL, "slot ids, weights, beta and log_decay must not be NULL");
    if (need_bank && (!v || !bank_data || !out)) return fail(SDM_ERR_NULL, "v, bank and out must not be NULL");
    const int es = dtype == SDM_F32 ? 4 : 2;
    const void *ptr4[] = {beta, g, valid};
    for (const void *q : ptr4)
        if (q && !aligned(q, 4)) return fail(SDM_ERR_ALIGN, "int32/float32 arrays must be 4-byte aligned");
    if (!aligned(slots->write, size_t(kb)) || !aligned(slots->read, size_t(qb)))
        return fail(SDM_ERR_ALIGN, "slot id arrays must be aligned to their element size");
    const void *ptre[] = {weights->write, weights->read, v, bank_data, out};
    for (const void *q : ptre)
        if (q && !aligned(q, size_t(es))) return fail(SDM_ERR_ALIGN, "bank-dtype arrays must be %d-byte aligned", es);
    if (need_bank) {
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(bank_data), b1 = b0 + uintptr_t(shared ? 1 : P) * M * hd * es;
        const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), o1 = o0 + uintptr_t(P) * T * hd * es;
        if (o0 < b1 && b0 < o1) return fail(SDM_ERR_SHAPE, "out overlaps the bank");
    }
    const int vec = 16 / es;
    int V = 1;
    if (hd % vec == 0 && (!need_bank || (aligned(v, 16) && aligned(bank_data, 16) && aligned(out, 16)))) V = vec;
    Problem pb{};
    pb.P = P; pb.T = T; pb.C = C; pb.Nt = int32_t((int64_t(T) + C - 1) / C); pb.W = W; pb.R = R; pb.G = G; pb.hd = hd;
    pb.M = M; pb.dtype = dtype; pb.sort_passes = sort_passes(M); pb.sort_digit = sort_digit(M); pb.key_bits = key_bits(M);
    pb.k_idx = slots->write; pb.q_idx = slots->read; pb.k_id8 = kb == 8; pb.q_id8 = qb == 8;
    pb.k_val = weights->write; pb.q_val = weights->read;
    pb.beta = beta; pb.g = g; pb.v = v; pb.valid = valid; pb.bank = bank_data; pb.out = out;
    pb.bank_stride = shared ? 0 : M * hd;
    pb.repeats = nullptr;
    ck->pb = pb;
    ck->lay = make_layout(C, W, R, hd);
    ck->V = V;
    ck->es = es;
    return SDM_OK;
}

// Phase-2 geometry from shapes only (the bits never depend on it): slices of NV vectors,
// NV the largest power of two with NV * V * es <= 128 bytes (one cache line of a row),
// halved while that leaves fewer than one workgroup per CU; one workgroup per
// (stream, slice); the chunk's Phase-2 block staged in LDS when it fits, and the slice of
// the bank resident in LDS when that fits too.
// SDM_P2_GEOM="nv[,mode]" overrides NV (1, 2, 4 or 8) and caps the mode (0 from memory,
// 1 staged, 2 resident; the largest that fits is taken below the cap), for tuning sweeps.
P2Geom plan_phase2(const Problem &pb, const ChunkLayout &L, int V, int es, int cus, int lds_limit) {
    const int hv = pb.hd / V;
    P2Geom g{};
    g.nv = 8;
    while (g.nv > 1 && (g.nv * V * es > 128 || g.nv > hv)) g.nv >>= 1;
    const char *env = getenv("SDM_P2_GEOM");
    int enk = 0, est = -1;
    const int got = env ? sscanf(env, "%d,%d", &enk, &est) : 0;
    if (got >= 1 && (enk == 1 || enk == 2 || enk == 4 || enk == 8)) {
        g.nv = enk;
    } else {
        g.S = (hv + g.nv - 1) / g.nv;
        while (g.nv > 1 && int64_t(pb.P) * g.S < cus) {
            g.nv >>= 1;
            g.S = (hv + g.nv - 1) / g.nv;
        }
    }
    g.S = (hv + g.nv - 1) / g.nv;
    g.team = 1;
    g.mode = phase2_mode(L, pb.C, g.nv, V, es, pb.M, lds_limit);
    // A shared bank is never held resident: each workgroup writes its whole slice back at
    // the end of a slab, which would overwrite the rows of the other streams.
    if (pb.bank_stride == 0 && g.mode > 1) g.mode = 1;
    if (got == 2 && est >= 0 && est < g.mode) g.mode = est;
    return g;
}

// The geometry actually launched, and the vector width V it uses. For a bfloat16 bank whose
// slice is resident in LDS, when slices of one 16-byte vector (8 columns) still leave more
// than half of the CUs without a workgroup, 8-byte vectors (4 columns) are taken instead:
// twice the workgroups, each with half the per-entry vector work (the step is bound by
// instruction issue), and still room beside them for another batch's Phase 1. Slices never
// change the bits. (Narrower still, 2 columns, measured no faster and fills every CU.)
// Teams: when slices of one 128-byte line per row (8 vectors of 16 bytes) leave CUs idle and
// the narrower slices planned instead read the bank from memory, 4 (else 2) workgroups
// share each (stream, slice) (whole lines per request: a quarter of the requests of 32-byte
// slices for the same bytes). Needs streams in whole groups of 8 (a team on one XCD),
// pieces of whole 16-token tiles, and room for the team's LDS. SDM_P2_TEAM=0 turns teams
// off, =2 or =4 asks for that size only; SDM_P2_GEOM alone turns them off (geometry sweeps).
bool plan_team(const Problem &pb, const ChunkLayout &L, int V, int es, int cus, int lds_limit, P2Geom &g) {
    DeviceInfo *dev = nullptr;
    if (device_info(&dev) != SDM_OK || !dev->teams) return false;
    const char *env = getenv("SDM_P2_TEAM");
    const int want = env ? atoi(env) : -1;
    if (want == 0 || (want < 0 && getenv("SDM_P2_GEOM"))) return false;
    if (V * es != 16 || pb.P % kXcds != 0) return false;
    const int hv = pb.hd / V, S8 = (hv + 7) / 8;
    if (S8 > kTeamMaxSlices) return false;
    // unasked, teams only replace narrow slices that read the bank from memory (narrow
    // slices that stage the chunk's arrays or hold the bank in LDS are faster); asked for
    // by size, any shape the kernel takes (for tests and sweeps)
    if (want < 0 && (int64_t(pb.P) * S8 >= cus || g.mode != 0)) return false;
    for (int t = 4; t >= 2; t /= 2) {
        if (want > 0 && want != t) continue;
        if ((want < 0 && int64_t(pb.P) * S8 * t > cus) || pb.C % (16 * t) != 0 || pb.C / t * 8 > 1024) continue;
        if (phase2_team_lds_bytes(pb.C, V, t) + 256 > size_t(lds_limit)) continue;
        g.nv = 8;
        g.S = S8;
        g.mode = 0;
        g.team = t;
        return true;
    }
    return false;
}

P2Geom plan_phase2_v(const Problem &pb, const ChunkLayout &L, int &V, int es, int cus, int lds_limit) {
    P2Geom g = plan_phase2(pb, L, V, es, cus, lds_limit);
    if (plan_team(pb, L, V, es, cus, lds_limit, g)) return g;
    if (es == 2 && V == 8 && g.nv == 1 && g.mode == 2 && int64_t(pb.P) * g.S * 2 <= cus && !getenv("SDM_P2_GEOM")) {
        const P2Geom g4 = plan_phase2(pb, L, 4, es, cus, lds_limit);
        if (g4.nv == 1 && g4.mode == 2) {
            V = 4;
            return g4;
        }
    }
    return g;
}

}  // namespace

extern "C" {

const char *sdm_error_string(int code) {
    switch (code) {
        case SDM_OK: return "success";
        case SDM_ERR_DTYPE: return "unsupported dtype";
        case SDM_ERR_SHAPE: return "invalid shape";
        case SDM_ERR_RANGE: return "size out of range";
        case SDM_ERR_NULL: return "null pointer";
        case SDM_ERR_ALIGN: return "misaligned pointer";
        case SDM_ERR_WORKSPACE: return "workspace missing or too small";
        case SDM_ERR_UNSUPPORTED: return "unsupported configuration";
        case SDM_ERR_HIP: return "HIP runtime error";
        default: return "unknown error";
    }
}

const char *sdm_last_error(void) { return g_err; }

int sdm_fwd_plan(int32_t P, int32_t T, int32_t C, int32_t W, int32_t R, int32_t hd, int64_t M, int32_t dtype,
                 sdm_plan *plan) {
    g_err[0] = 0;
    if (!plan) return fail(SDM_ERR_NULL, "plan must not be NULL");
    int rc = check_shape(P, T, C, W, R, hd);
    if (rc) return rc;
    if (dtype != SDM_F32 && dtype != SDM_BF16) return fail(SDM_ERR_DTYPE, "bank dtype must be SDM_F32 or SDM_BF16, got %d", dtype);
    if (M < 1 || int64_t(P) * M >= (int64_t(1) << 31)) return fail(SDM_ERR_RANGE, "rows per stream out of range");
    DeviceInfo *dev = nullptr;
    if ((rc = device_info(&dev)) != SDM_OK) return rc;
    const int es = dtype == SDM_F32 ? 4 : 2, vec = 16 / es;
    int V = hd % vec == 0 ? vec : 1;
    Problem pb{};
    pb.P = P; pb.T = T; pb.C = C; pb.W = W; pb.R = R; pb.hd = hd; pb.M = M; pb.dtype = dtype;
    pb.bank_stride = M * hd;   // per-stream banks
    const ChunkLayout lay = make_layout(C, W, R, hd);
    const P2Geom g = plan_phase2_v(pb, lay, V, es, dev->cus, dev->lds_per_block);
    plan->vec = V;
    plan->slice_vectors = g.nv;
    plan->slices = g.S;
    plan->phase2_mode = g.mode;
    plan->phase2_team = g.team;
    plan->phase2_lds_bytes = int32_t(g.team > 1 ? phase2_team_lds_bytes(C, V, g.team)
                                                 : phase2_lds_bytes(lay, C, g.nv, V, es, g.mode, M));
    plan->phase1_fused = phase1_fused(lay, C, dev->lds_per_block) ? 1 : 0;
    pb.key_bits = key_bits(M);
    plan->phase1_partitions_log2 = plan_part(pb, lay, plan->phase1_fused != 0);
    plan->lds_limit = dev->lds_per_block;
    plan->lds_default = dev->lds_default;
    return SDM_OK;
}

int sdm_product_key_topk(int64_t rows, const void *raw, int32_t dtype, const int32_t *factors, int32_t num_factors,
                         int32_t k, void *val, int64_t *lin, const sdm_exec *exec) {
    g_err[0] = 0;
    if (!exec) return fail(SDM_ERR_NULL, "exec must not be NULL");
    if (!factors) return fail(SDM_ERR_NULL, "factors must not be NULL");
    if (dtype != SDM_F32 && dtype != SDM_BF16) return fail(SDM_ERR_DTYPE, "raw must be SDM_F32 or SDM_BF16, got %d", dtype);
    if (rows < 0) return fail(SDM_ERR_SHAPE, "rows must be >= 0, got %lld", (long long)rows);
    if (rows > int64_t(0x7FFFFFFF)) return fail(SDM_ERR_RANGE, "at most 2^31 - 1 rows, got %lld", (long long)rows);
    if (num_factors < 1 || num_factors > kTopkMaxFactors)
        return fail(SDM_ERR_SHAPE, "1 to %d factors, got %d", kTopkMaxFactors, num_factors);
    if (k < 1 || k > kTopkMaxK) return fail(SDM_ERR_SHAPE, "k must be in 1..%d, got %d", kTopkMaxK, k);
    int64_t D = 0, prod = 1;
    for (int f = 0; f < num_factors; ++f) {
        if (factors[f] < 1) return fail(SDM_ERR_SHAPE, "factor %d has %d columns", f, factors[f]);
        if (factors[f] > kTopkMaxWidth)
            return fail(SDM_ERR_UNSUPPORTED, "factor %d has %d columns; at most %d", f, factors[f], kTopkMaxWidth);
        D += factors[f];
        if (prod > (int64_t(1) << 55) / factors[f])
            return fail(SDM_ERR_UNSUPPORTED, "the factors address 2^55 or more slots");
        prod *= factors[f];
    }
    if (rows > 0 && (!raw || !val || !lin)) return fail(SDM_ERR_NULL, "raw, val and lin must not be NULL");
    const int es = dtype == SDM_F32 ? 4 : 2;
    if (!aligned(raw, size_t(es)) || !aligned(val, size_t(es)) || !aligned(lin, 8))
        return fail(SDM_ERR_ALIGN, "raw and val must be aligned to their element size, lin to 8 bytes");
    const int32_t kk = int32_t(prod < k ? prod : k);
    const hipError_t e = launch_topk(raw, val, lin, rows, int32_t(D), num_factors, k, kk, dtype == SDM_BF16, factors,
                                     static_cast<hipStream_t>(exec->stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "top-k launch");
}

int sdm_product_key_topk_backward(int64_t rows, const int64_t *lin, const void *grad_val, int32_t dtype,
                                  const int32_t *factors, int32_t num_factors, int32_t kk, void *grad_raw,
                                  const sdm_exec *exec) {
    g_err[0] = 0;
    if (!exec) return fail(SDM_ERR_NULL, "exec must not be NULL");
    if (!factors) return fail(SDM_ERR_NULL, "factors must not be NULL");
    if (dtype != SDM_F32 && dtype != SDM_BF16) return fail(SDM_ERR_DTYPE, "dtype must be SDM_F32 or SDM_BF16, got %d", dtype);
    if (rows < 0) return fail(SDM_ERR_SHAPE, "rows must be >= 0, got %lld", (long long)rows);
    if (rows > int64_t(0x7FFFFFFF)) return fail(SDM_ERR_RANGE, "at most 2^31 - 1 rows, got %lld", (long long)rows);
    if (num_factors < 1 || num_factors > kTopkMaxFactors)
        return fail(SDM_ERR_SHAPE, "1 to %d factors, got %d", kTopkMaxFactors, num_factors);
    int64_t D = 0, prod = 1;
    for (int f = 0; f < num_factors; ++f) {
        if (factors[f] < 1) return fail(SDM_ERR_SHAPE, "factor %d has %d columns", f, factors[f]);
        if (factors[f] > kTopkMaxWidth)
            return fail(SDM_ERR_UNSUPPORTED, "factor %d has %d columns; at most %d", f, factors[f], kTopkMaxWidth);
        D += factors[f];
        if (prod > (int64_t(1) << 55) / factors[f])
            return fail(SDM_ERR_UNSUPPORTED, "the factors address 2^55 or more slots");
        prod *= factors[f];
    }
    if (kk < 1 || kk > kTopkMaxK || kk > prod)
        return fail(SDM_ERR_SHAPE, "kk must be in 1..min(256, slots), got %d", kk);
    if (rows > 0 && (!lin || !grad_val || !grad_raw)) return fail(SDM_ERR_NULL, "lin, grad_val and grad_raw must not be NULL");
    const int es = dtype == SDM_F32 ? 4 : 2;
    if (!aligned(lin, 8) || !aligned(grad_val, size_t(es)) || !aligned(grad_raw, size_t(es)))
        return fail(SDM_ERR_ALIGN, "lin must be 8-byte aligned, grad_val and grad_raw aligned to their element size");
    const hipError_t e = launch_topk_bwd(lin, grad_val, grad_raw, rows, int32_t(D), num_factors, kk, dtype == SDM_BF16,
                                         factors, static_cast<hipStream_t>(exec->stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "top-k backward launch");
}

size_t sdm_fwd_workspace_bytes(int32_t P, int32_t T, int32_t C, int32_t W, int32_t R, int32_t hd, int32_t slab_steps) {
    if (check_shape(P, T, C, W, R, hd) != SDM_OK) return 0;
    const int32_t Nt = int32_t((int64_t(T) + C - 1) / C);
    if (slab_steps <= 0 || slab_steps > Nt) slab_steps = Nt;
    const ChunkLayout lay = make_layout(C, W, R, hd);
    return size_t(lay.words) * 4 * size_t(P) * size_t(slab_steps);
}

}  // extern "C"

namespace {

// The forward's launch sequence. parts: 1 Phase 1 and the solve, 2 Phase 2, 3 both (sdm_fwd).
// A call of one part needs the workspace to hold every step, so that Phase 1's outputs for
// all chunks stay there for the Phase-2 call that follows it.
// noalloc: the workspace is this device's static scratch (SDM_NOALLOC_SCRATCH_BYTES), not
// exec->workspace, which must then be NULL with workspace_bytes 0.
int fwd_run(int parts, int32_t P, int32_t T, int32_t C, const sdm_slots *slots, const sdm_weights *weights,
            const float *beta, const float *log_decay, int32_t gate_width, const void *v, const sdm_bank *bank,
            const int32_t *valid_tokens, void *out, const sdm_exec *exec_in, bool noalloc = false) {
    g_err[0] = 0;
    if (!bank || !exec_in) return fail(SDM_ERR_NULL, "bank and exec must not be NULL");
    sdm_exec exec_static;
    const sdm_exec *exec = exec_in;
    if (noalloc) {
        if (exec_in->workspace || exec_in->workspace_bytes)
            return fail(SDM_ERR_WORKSPACE, "sdm_fwd_noalloc runs on its static scratch: exec->workspace must be NULL "
                                           "and exec->workspace_bytes 0");
        exec_static = *exec_in;
        exec = &exec_static;
    }
    Checked ck;
    if (bank->shared != 0 && bank->shared != 1) return fail(SDM_ERR_SHAPE, "bank.shared must be 0 or 1, got %d", bank->shared);
    const bool p1 = parts & 1, p2 = parts & 2;
    int rc = check_call(P, T, C, slots, weights, beta, log_decay, gate_width, v, bank->rows, bank->head_dim, bank->dtype,
                        bank->data, bank->shared == 1, valid_tokens, out, p2, &ck);
    if (rc) return rc;
    if (exec->repeated_writes && !aligned(exec->repeated_writes, 8))
        return fail(SDM_ERR_ALIGN, "the repeated-writes counter must be 8-byte aligned");
    ck.pb.repeats = reinterpret_cast<unsigned long long *>(exec->repeated_writes);
    const size_t per_step = size_t(ck.lay.words) * 4 * size_t(P);
    if (noalloc) {
        if (per_step > size_t(SDM_NOALLOC_SCRATCH_BYTES))
            return fail(SDM_ERR_WORKSPACE, "one step of these shapes needs %zu bytes of workspace; the static scratch "
                                           "of sdm_fwd_noalloc holds %zu (use sdm_fwd with a caller workspace)",
                        per_step, size_t(SDM_NOALLOC_SCRATCH_BYTES));
        DeviceInfo *d0 = nullptr;
        if ((rc = device_info(&d0)) != SDM_OK) return rc;
        exec_static.workspace = d0->scratch;
        exec_static.workspace_bytes = SDM_NOALLOC_SCRATCH_BYTES;
    }
    if (!exec->workspace || exec->workspace_bytes < per_step)
        return fail(SDM_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes one step needs",
                    exec->workspace ? exec->workspace_bytes : size_t(0), per_step);
    if (!aligned(exec->workspace, 256)) return fail(SDM_ERR_ALIGN, "workspace must be 256-byte aligned");
    DeviceInfo *dev = nullptr;
    if ((rc = device_info(&dev)) != SDM_OK) return rc;
    if (gram_lds_bytes(C) > size_t(dev->lds_per_block))
        return fail(SDM_ERR_UNSUPPORTED, "chunk %d needs %zu bytes of LDS per workgroup, the device has %d", C,
                    gram_lds_bytes(C), dev->lds_per_block);
    if (exec->phase2_cus < 0) return fail(SDM_ERR_SHAPE, "phase2_cus must be >= 0, got %d", exec->phase2_cus);
    const int p2cus = exec->phase2_cus > 0 && exec->phase2_cus < dev->cus ? exec->phase2_cus : dev->cus;
    const P2Geom geom = plan_phase2_v(ck.pb, ck.lay, ck.V, ck.es, p2cus, dev->lds_per_block);
    const size_t p2lds = geom.team > 1 ? phase2_team_lds_bytes(C, ck.V, geom.team)
                                       : phase2_lds_bytes(ck.lay, C, geom.nv, ck.V, ck.es, geom.mode, ck.pb.M);
    if (p2lds + 256 > size_t(dev->lds_per_block))
        return fail(SDM_ERR_UNSUPPORTED, "chunk %d needs %zu bytes of LDS per workgroup in phase 2, the device has %d", C,
                    p2lds, dev->lds_per_block);
    const int32_t Nt = ck.pb.Nt;
    int64_t slab64 = int64_t(exec->workspace_bytes / per_step);
    int32_t slab = slab64 > Nt ? Nt : int32_t(slab64);
    if (parts != 3 && slab < Nt)
        return fail(SDM_ERR_WORKSPACE, "a split forward needs the workspace of all %d steps (%zu bytes), got %zu", Nt,
                    per_step * size_t(Nt), exec->workspace_bytes);
    hipStream_t st = static_cast<hipStream_t>(exec->stream);
    const bool fused = phase1_fused(ck.lay, C, dev->lds_per_block);
    const int lognp = plan_part(ck.pb, ck.lay, fused);
    hipEvent_t *ev = nullptr;
    if (parts == 3 && exec->events && exec->num_events >= SDM_TIMING_EVENTS)
        ev = reinterpret_cast<hipEvent_t *>(exec->events);
    for (int32_t ti0 = 0; ti0 < Nt; ti0 += slab) {
        Slab sl{};
        sl.ti0 = ti0;
        sl.steps = Nt - ti0 < slab ? Nt - ti0 : slab;
        sl.ws = static_cast<uint32_t *>(exec->workspace);
        sl.lay = ck.lay;
        hipEvent_t *sev = ti0 == 0 ? ev : nullptr;
        float *w = reinterpret_cast<float *>(sl.ws);
        const WyArgs wa{w + sl.lay.off_A, w + sl.lay.off_beta, w + sl.lay.off_QK, w + sl.lay.off_X,
                        w + sl.lay.off_QX, C, sl.lay.words, sl.lay.words};
        hipError_t e = hipSuccess;
        if (p1) {
            e = launch_phase1(ck.pb, sl, st, sev, fused, wa, lognp);
            if (e != hipSuccess) return hip_fail(e, "phase 1 launch");
            if (sev && (e = hipEventRecord(sev[5], st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
            if (!fused) {
                e = launch_wy(wa.A, wa.beta, wa.QK, wa.X, wa.QX, C, int64_t(P) * sl.steps, sl.lay.words, sl.lay.words,
                              st);
                if (e != hipSuccess) return hip_fail(e, "solve launch");
            }
        }
        if (sev && (e = hipEventRecord(sev[6], st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
        if (p2) {
            e = launch_phase2(ck.pb, sl, ck.V, geom, st);
            if (e != hipSuccess) return hip_fail(e, "phase 2 launch");
        }
        if (sev && (e = hipEventRecord(sev[7], st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    return SDM_OK;
}

}  // namespace

extern "C" {

int sdm_fwd(int32_t P, int32_t T, int32_t C, const sdm_slots *slots, const sdm_weights *weights, const float *beta,
            const float *log_decay, int32_t gate_width, const void *v, const sdm_bank *bank, const int32_t *valid_tokens,
            void *out, const sdm_exec *exec) {
    return fwd_run(3, P, T, C, slots, weights, beta, log_decay, gate_width, v, bank, valid_tokens, out, exec);
}

int sdm_fwd_noalloc(int32_t P, int32_t T, int32_t C, const sdm_slots *slots, const sdm_weights *weights,
                    const float *beta, const float *log_decay, int32_t gate_width, const void *v, const sdm_bank *bank,
                    const int32_t *valid_tokens, void *out, const sdm_exec *exec) {
    return fwd_run(3, P, T, C, slots, weights, beta, log_decay, gate_width, v, bank, valid_tokens, out, exec, true);
}

int sdm_fwd_phase1(int32_t P, int32_t T, int32_t C, const sdm_slots *slots, const sdm_weights *weights,
                   const float *beta, const float *log_decay, int32_t gate_width, const void *v, const sdm_bank *bank,
                   const int32_t *valid_tokens, void *out, const sdm_exec *exec) {
    return fwd_run(1, P, T, C, slots, weights, beta, log_decay, gate_width, v, bank, valid_tokens, out, exec);
}

int sdm_fwd_phase2(int32_t P, int32_t T, int32_t C, const sdm_slots *slots, const sdm_weights *weights,
                   const float *beta, const float *log_decay, int32_t gate_width, const void *v, const sdm_bank *bank,
                   const int32_t *valid_tokens, void *out, const sdm_exec *exec) {
    return fwd_run(2, P, T, C, slots, weights, beta, log_decay, gate_width, v, bank, valid_tokens, out, exec);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// Intermediates out (sdm_chunk_mats)
// ---------------------------------------------------------------------------------------
namespace sdm {
struct MatsOut {
    float *A, *QK, *X, *QX, *gw, *gr;
};

__global__ void copy_mats_kernel(Slab sl, int32_t P, int32_t Nt, MatsOut o) {
    const int64_t n = blockIdx.y;
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int64_t dst = int64_t(p) * Nt + ti;
    const ChunkLayout &L = sl.lay;
    const float *cb = reinterpret_cast<const float *>(sl.chunk(n));
    for (int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; k < L.C2; k += int64_t(gridDim.x) * blockDim.x) {
        o.A[dst * L.C2 + k] = cb[L.off_A + k];
        o.QK[dst * L.C2 + k] = cb[L.off_QK + k];
        o.X[dst * L.C2 + k] = cb[L.off_X + k];
        o.QX[dst * L.C2 + k] = cb[L.off_QX + k];
    }
    for (int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; k < L.E; k += int64_t(gridDim.x) * blockDim.x)
        o.gw[dst * L.E + k] = cb[L.off_gw + k];
    for (int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; k < L.F; k += int64_t(gridDim.x) * blockDim.x)
        o.gr[dst * L.F + k] = cb[L.off_gr + k];
}
struct RecsOut {
    int32_t *meta, *spk, *grec, *ecr, *rcr;
};

// Phase 1's integer records of every chunk of the slab, copied out verbatim.
__global__ void copy_recs_kernel(Slab sl, int32_t P, int32_t Nt, RecsOut o) {
    const int64_t n = blockIdx.y;
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int64_t dst = int64_t(p) * Nt + ti;
    const ChunkLayout &L = sl.lay;
    const int32_t *cb = reinterpret_cast<const int32_t *>(sl.chunk(n));
    const int64_t i0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x, step = int64_t(gridDim.x) * blockDim.x;
    for (int64_t k = i0; k < 8; k += step) o.meta[dst * 8 + k] = cb[L.off_meta + k];
    for (int64_t k = i0; k < 4 * L.E; k += step) {
        o.spk[dst * 4 * L.E + k] = cb[L.off_spk + k];
        o.grec[dst * 4 * L.E + k] = cb[L.off_grec + k];
        o.ecr[dst * 4 * L.E + k] = cb[L.off_ecr + k];
    }
    for (int64_t k = i0; k < 4 * L.F; k += step) o.rcr[dst * 4 * L.F + k] = cb[L.off_rcr + k];
}
}  // namespace sdm

namespace {

// Phase 1 and the solve over every slab of the chunk-intermediate queries, then copy(sl, st).
template <typename CopyF>
int run_phase1_slabs(const Checked &ck0, int32_t P, int32_t C, const sdm_exec *exec, CopyF copy) {
    Checked ck = ck0;
    const size_t per_step = size_t(ck.lay.words) * 4 * size_t(P);
    if (!exec->workspace || exec->workspace_bytes < per_step)
        return fail(SDM_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes one step needs",
                    exec->workspace ? exec->workspace_bytes : size_t(0), per_step);
    if (!aligned(exec->workspace, 256)) return fail(SDM_ERR_ALIGN, "workspace must be 256-byte aligned");
    DeviceInfo *dev = nullptr;
    int rc = device_info(&dev);
    if (rc != SDM_OK) return rc;
    const int32_t Nt = ck.pb.Nt;
    int32_t slab = int32_t(exec->workspace_bytes / per_step);
    if (slab > Nt) slab = Nt;
    hipStream_t st = static_cast<hipStream_t>(exec->stream);
    for (int32_t ti0 = 0; ti0 < Nt; ti0 += slab) {
        Slab sl{};
        sl.ti0 = ti0;
        sl.steps = Nt - ti0 < slab ? Nt - ti0 : slab;
        sl.ws = static_cast<uint32_t *>(exec->workspace);
        sl.lay = ck.lay;
        float *w = reinterpret_cast<float *>(sl.ws);
        const WyArgs wa{w + sl.lay.off_A, w + sl.lay.off_beta, w + sl.lay.off_QK, w + sl.lay.off_X,
                        w + sl.lay.off_QX, C, sl.lay.words, sl.lay.words};
        const bool fused = phase1_fused(ck.lay, C, dev->lds_per_block);
        const int lognp = plan_part(ck.pb, ck.lay, fused);
        hipError_t e = launch_phase1(ck.pb, sl, st, nullptr, fused, wa, lognp);
        if (e != hipSuccess) return hip_fail(e, "phase 1 launch");
        if (!fused) {
            e = launch_wy(wa.A, wa.beta, wa.QK, wa.X, wa.QX, C, int64_t(P) * sl.steps, sl.lay.words, sl.lay.words, st);
            if (e != hipSuccess) return hip_fail(e, "solve launch");
        }
        copy(sl, st);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "copy launch");
    }
    return SDM_OK;
}

}  // namespace

extern "C" {

int sdm_chunk_records(int32_t P, int32_t T, int32_t C, const sdm_slots *slots, const sdm_weights *weights,
                      const float *beta, const float *log_decay, int32_t gate_width, int64_t rows, int32_t head_dim,
                      int32_t dtype, const int32_t *valid_tokens, int32_t *meta, int32_t *spk, int32_t *grec,
                      int32_t *ecr, int32_t *rcr, const sdm_exec *exec) {
    g_err[0] = 0;
    if (!exec) return fail(SDM_ERR_NULL, "exec must not be NULL");
    if (!meta || !spk || !grec || !ecr || !rcr) return fail(SDM_ERR_NULL, "output arrays must not be NULL");
    Checked ck;
    int rc = check_call(P, T, C, slots, weights, beta, log_decay, gate_width, nullptr, rows, head_dim, dtype, nullptr,
                        false, valid_tokens, nullptr, false, &ck);
    if (rc) return rc;
    const RecsOut o{meta, spk, grec, ecr, rcr};
    const int32_t Nt = ck.pb.Nt;
    return run_phase1_slabs(ck, P, C, exec, [&](const Slab &sl, hipStream_t st) {
        hipLaunchKernelGGL(copy_recs_kernel, dim3(64, unsigned(int64_t(P) * sl.steps)), dim3(256), 0, st, sl, P, Nt, o);
    });
}

int sdm_chunk_mats(int32_t P, int32_t T, int32_t C, const sdm_slots *slots, const sdm_weights *weights, const float *beta,
                   const float *log_decay, int32_t gate_width, int64_t rows, int32_t head_dim, int32_t dtype,
                   const int32_t *valid_tokens, float *A, float *QK, float *X, float *QX, float *gw, float *gr,
                   const sdm_exec *exec) {
    g_err[0] = 0;
    if (!exec) return fail(SDM_ERR_NULL, "exec must not be NULL");
    if (!A || !QK || !X || !QX || !gw || !gr) return fail(SDM_ERR_NULL, "output arrays must not be NULL");
    Checked ck;
    int rc = check_call(P, T, C, slots, weights, beta, log_decay, gate_width, nullptr, rows, head_dim, dtype, nullptr,
                        false, valid_tokens, nullptr, false, &ck);
    if (rc) return rc;
    const size_t per_step = size_t(ck.lay.words) * 4 * size_t(P);
    if (!exec->workspace || exec->workspace_bytes < per_step)
        return fail(SDM_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes one step needs",
                    exec->workspace ? exec->workspace_bytes : size_t(0), per_step);
    if (!aligned(exec->workspace, 256)) return fail(SDM_ERR_ALIGN, "workspace must be 256-byte aligned");
    DeviceInfo *dev = nullptr;
    if ((rc = device_info(&dev)) != SDM_OK) return rc;
    const int32_t Nt = ck.pb.Nt;
    int32_t slab = int32_t(exec->workspace_bytes / per_step);
    if (slab > Nt) slab = Nt;
    hipStream_t st = static_cast<hipStream_t>(exec->stream);
    MatsOut o{A, QK, X, QX, gw, gr};
    for (int32_t ti0 = 0; ti0 < Nt; ti0 += slab) {
        Slab sl{};
        sl.ti0 = ti0;
        sl.steps = Nt - ti0 < slab ? Nt - ti0 : slab;
        sl.ws = static_cast<uint32_t *>(exec->workspace);
        sl.lay = ck.lay;
        float *w = reinterpret_cast<float *>(sl.ws);
        const WyArgs wa{w + sl.lay.off_A, w + sl.lay.off_beta, w + sl.lay.off_QK, w + sl.lay.off_X,
                        w + sl.lay.off_QX, C, sl.lay.words, sl.lay.words};
        const bool fused = phase1_fused(ck.lay, C, dev->lds_per_block);
        const int lognp = plan_part(ck.pb, ck.lay, fused);
        hipError_t e = launch_phase1(ck.pb, sl, st, nullptr, fused, wa, lognp);
        if (e != hipSuccess) return hip_fail(e, "phase 1 launch");
        if (!fused) {
            e = launch_wy(wa.A, wa.beta, wa.QK, wa.X, wa.QX, C, int64_t(P) * sl.steps, sl.lay.words, sl.lay.words, st);
            if (e != hipSuccess) return hip_fail(e, "solve launch");
        }
        hipLaunchKernelGGL(copy_mats_kernel, dim3(64, unsigned(int64_t(P) * sl.steps)), dim3(256), 0, st, sl, P, Nt, o);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "copy launch");
    }
    return SDM_OK;
}

int sdm_wy_solve(int64_t n, int32_t C, const float *A, const float *beta, const float *QK, float *X, float *QX,
                 const sdm_exec *exec) {
    g_err[0] = 0;
    if (!exec) return fail(SDM_ERR_NULL, "exec must not be NULL");
    if (n < 0) return fail(SDM_ERR_SHAPE, "chunk count must be >= 0, got %lld", (long long)n);
    if (C < 1 || C > kMaxChunk) return fail(SDM_ERR_RANGE, "chunk must be in 1..256, got %d", C);
    if (n == 0) return SDM_OK;
    if (!A || !beta || !QK || !X || !QX) return fail(SDM_ERR_NULL, "A, beta, QK, X and QX must not be NULL");
    const void *ps[] = {A, beta, QK, X, QX};
    for (const void *q : ps)
        if (!aligned(q, 4)) return fail(SDM_ERR_ALIGN, "float32 arrays must be 4-byte aligned");
    if (n > int64_t(0x7fffffff)) return fail(SDM_ERR_RANGE, "too many chunks (%lld)", (long long)n);
    DeviceInfo *dev = nullptr;
    int rc = device_info(&dev);
    if (rc != SDM_OK) return rc;
    const int64_t C2 = int64_t(C) * C;
    hipError_t e = launch_wy(A, beta, QK, X, QX, C, n, C2, C, static_cast<hipStream_t>(exec->stream));
    if (e != hipSuccess) return hip_fail(e, "solve launch");
    return SDM_OK;
}

// ---------------------------------------------------------------------------------------
// The backward (backward.hip): one workgroup per (stream, column slice) replays the forward
// and walks it back; the workspace holds the saved rows, the folded read slots and the
// per-slice dots.
// ---------------------------------------------------------------------------------------

namespace {

struct BwdSizes {
    size_t snap, lead, part, pairs, work, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// snap_es: bytes per saved element (4 float32, 2 bfloat16 snapshot rows)
BwdSizes bwd_sizes(int32_t P, int32_t T, int32_t W, int32_t R, int32_t hd, int64_t M, int32_t dtype, bool shared,
                   int snap_es) {
    const int S = sdm::bwd_slice_cols(P, hd, W, R);
    const int64_t NS = (hd + S - 1) / S;
    BwdSizes z{};
    z.snap = align256(size_t(P) * size_t(NS) * size_t(S) * size_t(T) * size_t(W) * size_t(snap_es));
    z.lead = align256(size_t(P) * size_t(T) * size_t(R) * 8);
    z.part = align256(size_t(P) * size_t(NS) * size_t(T) * size_t(sdm::bwd_parts(W, R)) * 4);
    z.pairs = align256(size_t(P) * size_t((T + 1) / 2) * 4);
    z.work = dtype == SDM_BF16 ? align256(size_t(shared ? 1 : P) * size_t(M) * size_t(hd) * 4) : 0;
    z.total = z.snap + z.lead + z.part + z.pairs + z.work;
    return z;
}

}  // namespace

// Bytes per saved snapshot element for a supported mode on a bank of dtype: bfloat16 rows
// on a float32 bank, float32 otherwise (a bfloat16 bank runs "bf16" as "none", the pages'
// effective_snapshot_quant, page 21); 0 for a mode that is refused.
static int snap_elem_bytes(int32_t mode, int32_t dtype) {
    if (mode == SDM_SNAP_NONE) return 4;
    if (mode == SDM_SNAP_BF16) return dtype == SDM_F32 ? 2 : 4;
    return 0;
}

size_t sdm_bwd_workspace_bytes(int32_t P, int32_t T, int32_t W, int32_t R, int32_t hd, int64_t rows, int32_t dtype,
                               int32_t shared, int32_t snapshot_quant) {
    if (check_shape(P, T, 16, W, R, hd) != SDM_OK || rows < 1 || (dtype != SDM_F32 && dtype != SDM_BF16) ||
        (shared != 0 && shared != 1) || snap_elem_bytes(snapshot_quant, dtype) == 0)
        return 0;
    return bwd_sizes(P, T, W, R, hd, rows, dtype, shared == 1, snap_elem_bytes(snapshot_quant, dtype)).total;
}

int sdm_bwd(int32_t P, int32_t T, const sdm_slots *slots, const sdm_weights *weights, const float *beta,
            const float *log_decay, int32_t gate_width, const void *v, const sdm_bank *bank, const int32_t *valid_tokens,
            const void *grad_out, const sdm_grads *grads, int32_t snapshot_quant, const sdm_exec *exec) {
    g_err[0] = 0;
    if (!bank || !exec || !grads) return fail(SDM_ERR_NULL, "bank, grads and exec must not be NULL");
    if (snapshot_quant < SDM_SNAP_NONE || snapshot_quant > SDM_SNAP_BF16)
        return fail(SDM_ERR_SHAPE, "snapshot_quant must be SDM_SNAP_NONE, _FP8, _INT4 or _BF16, got %d", snapshot_quant);
    if (snapshot_quant == SDM_SNAP_FP8 || snapshot_quant == SDM_SNAP_INT4)
        return fail(SDM_ERR_UNSUPPORTED, "snapshot_quant %s: the scaling of %s snapshot rows is not defined; "
                                         "SDM_SNAP_BF16 and SDM_SNAP_NONE are supported",
                    snapshot_quant == SDM_SNAP_FP8 ? "fp8" : "int4",
                    snapshot_quant == SDM_SNAP_FP8 ? "float8_e4m3fn" : "4-bit");
    if (bank->shared != 0 && bank->shared != 1) return fail(SDM_ERR_SHAPE, "bank.shared must be 0 or 1, got %d", bank->shared);
    const bool shared = bank->shared == 1;
    Checked ck;
    // chunk 16 only bounds the token count here: the backward has no chunks
    int rc = check_call(P, T, 16, slots, weights, beta, log_decay, gate_width, v, bank->rows, bank->head_dim,
                        bank->dtype, bank->data, shared, valid_tokens, const_cast<void *>(grad_out), true, &ck);
    if (rc) return rc;
    if (!grads->bank || !grads->v || !grads->beta || !grads->log_decay || !grads->write || !grads->read)
        return fail(SDM_ERR_NULL, "every gradient array must be given");
    const void *g4[] = {grads->bank, grads->v, grads->beta, grads->log_decay, grads->write, grads->read};
    for (const void *q : g4)
        if (!aligned(q, 4)) return fail(SDM_ERR_ALIGN, "gradient arrays must be 4-byte aligned");
    const int W = slots->W, R = slots->R, hd = bank->head_dim;
    const int64_t M = bank->rows, banks = shared ? 1 : P;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(bank->data), b1 = b0 + uintptr_t(banks) * M * hd * ck.es;
    const uintptr_t g0 = reinterpret_cast<uintptr_t>(grads->bank), g1 = g0 + uintptr_t(banks) * M * hd * 4;
    if (g0 < b1 && b0 < g1) return fail(SDM_ERR_SHAPE, "the bank gradient overlaps the bank");
    const int snap_es = snap_elem_bytes(snapshot_quant, bank->dtype);
    const BwdSizes z = bwd_sizes(P, T, W, R, hd, M, bank->dtype, shared, snap_es);
    if (!exec->workspace || exec->workspace_bytes < z.total)
        return fail(SDM_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes the backward needs",
                    exec->workspace ? exec->workspace_bytes : size_t(0), z.total);
    if (!aligned(exec->workspace, 256)) return fail(SDM_ERR_ALIGN, "workspace must be 256-byte aligned");
    DeviceInfo *dev = nullptr;
    if ((rc = device_info(&dev)) != SDM_OK) return rc;
    sdm::BwdArgs a{};
    a.P = P; a.T = T; a.W = W; a.R = R; a.G = gate_width; a.hd = hd; a.M = M;
    a.bf16 = bank->dtype == SDM_BF16;
    a.bstride = shared ? 0 : M * hd;
    a.S = sdm::bwd_slice_cols(P, hd, W, R);
    a.NS = (hd + a.S - 1) / a.S;
    // one wavefront per slice with the slices of the bank and of its gradient in LDS when they fit
    // and a lane covers its entries in at most 4 (SDM_BWD_RES=0 turns it off)
    const char *res_env = getenv("SDM_BWD_RES");
    const size_t res_lds = sdm::bwd_lds_bytes(W, a.S, M, true);
    // (never for a shared bank: a workgroup writes its whole gradient slice back at the end,
    // which would overwrite the rows of the other streams)
    const bool res_ok = !shared && (!res_env || atoi(res_env) != 0) && res_lds <= size_t(dev->lds_per_block) &&
                        res_lds <= size_t(sdm::kBwdMaxLds);
    a.res = res_ok ? sdm::bwd_res_entries(W, R, a.S, 4) : 0;
    // otherwise one wavefront per slice on rows in memory where a lane covers its entries in
    // at most 8 (SDM_BWD_WAVE=0 keeps the 256-thread sweep)
    const char *wave_env = getenv("SDM_BWD_WAVE");
    if (a.res == 0 && (!wave_env || atoi(wave_env) != 0)) a.res = -sdm::bwd_res_entries(W, R, a.S, 8);
    // tokens in pairs when a token's entries fill at most half the entry groups
    // (SDM_BWD_PAIR=0 turns it off)
    const char *pair_env = getenv("SDM_BWD_PAIR");
    a.pair = a.res == 1 && 2 * (W > R ? W : R) <= sdm::kWave / a.S && (W > R ? W : R) <= sdm::kPairMax &&
             (!pair_env || atoi(pair_env) != 0);
    if (!a.res && sdm::bwd_lds_bytes(W, a.S, M, false) > size_t(dev->lds_per_block))
        return fail(SDM_ERR_UNSUPPORTED, "the backward needs %zu bytes of LDS per workgroup, the device has %d",
                    sdm::bwd_lds_bytes(W, a.S, M, false), dev->lds_per_block);
    a.k_idx = ck.pb.k_idx; a.q_idx = ck.pb.q_idx; a.k_id8 = ck.pb.k_id8; a.q_id8 = ck.pb.q_id8;
    a.k_val = weights->write;
    a.q_val = weights->read;
    a.beta = beta; a.g = log_decay; a.v = v; a.go = grad_out; a.valid = valid_tokens;
    a.bank = bank->data;
    a.gbank = grads->bank; a.gv = grads->v; a.gk = grads->write; a.gq = grads->read;
    a.gbeta = grads->beta; a.gg = grads->log_decay;
    unsigned char *ws = static_cast<unsigned char *>(exec->workspace);
    a.snap = ws;
    a.snap_bf16 = snap_es == 2;
    a.lead = reinterpret_cast<float2 *>(ws + z.snap);
    a.part = reinterpret_cast<float *>(ws + z.snap + z.lead);
    a.pairs = reinterpret_cast<int32_t *>(ws + z.snap + z.lead + z.part);
    a.work = a.bf16 ? reinterpret_cast<float *>(ws + z.snap + z.lead + z.part + z.pairs)
                    : static_cast<float *>(bank->data);
    hipEvent_t *ev = nullptr;
    if (exec->events && exec->num_events >= SDM_BWD_TIMING_EVENTS) ev = reinterpret_cast<hipEvent_t *>(exec->events);
    const hipError_t e = sdm::launch_bwd(a, static_cast<hipStream_t>(exec->stream), ev);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "backward launch");
}

}  // extern "C"

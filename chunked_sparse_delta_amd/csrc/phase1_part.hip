// Phase 1 of large chunks in slot partitions held in LDS (gfx950). It computes what the
// sorting path of phase1.hip computes (module docstring of memory_ops.py, sparse-delta-
// memory 2.0.0 wheel, diffend page 21: per-slot log-decays, dedup flags, gather weights;
// the inputs of the Gram pair sums) for chunks of many entries, with every per-entry record
// read once and written once in order:
//
//   count      the chunk's write and read entries per slot partition (slot mod NP)
//   scatter    token tile by token tile, the entries in token order (a token's writes, then
//              its reads) are ranked by partition in LDS and written to the partition lists
//              as 16-byte records {slot, code, bits of k or q, bits of g}, each partition's
//              part of a tile in one contiguous run
//   partition  one partition at a time: its list is loaded into LDS, sorted by slot (stable
//              LSD radix on the slot bits above the partition bits, so that each slot's
//              entries stay in token order, a token's write before its reads), and three
//              block scans give every position its cumulative log-decay L (a sum of the
//              writes' log-decays restarted at each slot), its write rank and its count of
//              earlier writes of the slot; a read then takes the L of the latest write of
//              its slot at or before its token. Groups (the writes of one slot), their
//              records (in sorted order), the hot test, and each entry's output record (its
//              cold pair range or hot operand, its gather weight) are formed from these; the
//              entry records go back to the entry's own list slot, which the partition has
//              just read (so the lines are whole in L2 when they leave)
//   emit       token tile by token tile, each entry fetches its record through the slot map
//              the scatter wrote, and the entry-order arrays (gather weights, cold records)
//              and the rows of the dense hot operands are written whole, in order
//
// One workgroup per chunk; partitions run one after another so that positions, groups,
// big groups and hot groups are numbered across the chunk in partition order (partition,
// then slot), carried in LDS. A chunk with a partition larger than the LDS holds (kPartCap
// entries) is left to the sorting path (meta[7] = 1), which then handles it alone.
// Every sum has a fixed order given the chunk's data and the partition count, which is a
// function of the shapes only: the bits never depend on the launch, the slab or other
// streams. No float atomics; LDS integer atomics only count.
#include "common.h"

namespace sdm {

// Two sizes of the kernel: chunks of at least kPartBigEntries entries take 512-thread
// workgroups holding partitions of up to 3072 entries (at most 64 partitions, two workgroups
// per CU); smaller chunks take 256-thread workgroups with half of that LDS (up to 128
// partitions of 1536 entries, four workgroups per CU), whose barrier stalls overlap more.
// The configuration, like the partition count, is a function of the shapes only.
template <int BLOCK, int CAP, int MAXLOGNP>
struct PartCfg {
    static constexpr int kBlock = BLOCK;
    static constexpr int kNW = BLOCK / kWave;
    static constexpr int kCap = CAP;                          // entries of one partition held in LDS
    static constexpr int kIpt = (CAP + BLOCK - 1) / BLOCK;    // positions per thread
    static constexpr int kMaxLogNP = MAXLOGNP;
    static constexpr int kCand = CAP / kHotMin + 1;           // big groups of one partition, at most
};
using PartBig = PartCfg<512, 3072, 6>;
using PartSmall = PartCfg<256, 1536, 7>;
constexpr int64_t kPartBigEntries = 65536;
constexpr int kPartDigit = 7;                       // radix digit bits

// The constants of configuration Cfg under their short names, in a kernel or helper body.
#define PART_CFG_NAMES(Cfg)                                                                   \
    constexpr int kPartBlock = Cfg::kBlock, kPartNW = Cfg::kNW, kPartCap = Cfg::kCap,        \
                  kPartIpt = Cfg::kIpt, kPartMaxLogNP = Cfg::kMaxLogNP, kPartCand = Cfg::kCand; \
    (void)kPartBlock; (void)kPartNW; (void)kPartCap; (void)kPartIpt; (void)kPartMaxLogNP; (void)kPartCand

template <class Cfg>
struct PartSmem {
    static constexpr int kPartCap = Cfg::kCap, kPartNW = Cfg::kNW, kPartMaxLogNP = Cfg::kMaxLogNP,
                         kPartCand = Cfg::kCand;
    uint32_t slot[kPartCap];
    uint32_t code[kPartCap];     // read << 31 | group id << 16 (writes, once known) | token << 8 | entry in token
    uint32_t v1[kPartCap];       // bits of k (write) or q (read), float32
    uint32_t v2[kPartCap];       // bits of g (write); then of L
    uint16_t perm[2][kPartCap];  // sort permutations; then sorted order and write positions
    union {
        int32_t cnt[kPartNW][1 << kPartDigit];        // digit counts of the stable scatter
        uint16_t gpos[kPartCap + 64];                 // group head write ranks
    };
    int16_t hotr[kPartCap];      // at a group head's write rank: its hot index, or -1
    int32_t cand[kPartCand];     // big groups of the partition, in group order
    uint8_t cand_ok[kPartCand];
    int32_t dstart[1 << kPartDigit];   // first sorted position of each digit (scatter)
    int32_t dsum[kPartNW];
    int32_t wi[3][kPartNW];
    float wf[kPartNW];
    int32_t pcnt[1 << kPartMaxLogNP];  // entries per partition
    int32_t poff[(1 << kPartMaxLogNP) + 1];
    int32_t pcur[1 << kPartMaxLogNP];
    int32_t nw, ng, nc, nh;      // of the current partition
    int32_t wo, go, co, ho;      // carried over the partitions: writes, groups, big groups, hot groups
    int32_t nrep, fallback;
};

constexpr int kPartBatch = 8;   // global loads in flight per thread in the streaming loops

// Count ids base + off .. + n - 1 (int32 or int64) in their partitions, pcnt[id & pmask], and
// with copy store them to dst in entry order (Phase 2 reads them); kPartBatch loads in flight
// per thread (the LDS atomics are unconditional, adding 0 past n: a branch would make each
// of them wait for every load).
template <class Cfg>
__device__ __forceinline__ void count_ids(const void *base, int32_t id8, int64_t off, int32_t n, bool copy,
                                          uint32_t *dst, int32_t *pcnt, uint32_t pmask) {
    PART_CFG_NAMES(Cfg);
    const int tid = threadIdx.x;
    for (int32_t x0 = 0; x0 < n; x0 += kPartBlock * kPartBatch) {
        int32_t v[kPartBatch];
#pragma unroll
        for (int u = 0; u < kPartBatch; ++u) {
            const int32_t x = x0 + u * kPartBlock + tid;
            v[u] = load_id(base, off + (x < n ? x : 0), id8);
        }
#pragma unroll
        for (int u = 0; u < kPartBatch; ++u) {
            const int32_t x = x0 + u * kPartBlock + tid;
            if (copy && x < n) dst[x] = uint32_t(v[u]);
            atomicAdd(&pcnt[uint32_t(v[u]) & pmask], x < n ? 1 : 0);
        }
    }
}

// Stable counting scatter of items 0..n-1 by a digit of db bits: item i (digit(i)) goes to
// sorted position pos, emitted as emit(i, pos); equal digits keep the item order. Wave w
// owns a contiguous segment of the items; per (wave, digit) counts, turned into first
// positions (digits ascending, waves in order), ranks within a wavefront by ballot match.
// Also fills s.dstart[d] (first position of digit d). Ends with a barrier.
template <class Cfg, typename DigitF, typename EmitF>
__device__ __forceinline__ void part_scatter(PartSmem<Cfg> &s, int n, int db, DigitF digit, EmitF emit) {
    PART_CFG_NAMES(Cfg);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nd = 1 << db;
    const uint64_t lt = lanemask_lt(lane);
    const int seg = ((n + kPartNW - 1) / kPartNW + 63) & ~63;
    const int s0 = min(n, wv * seg), s1 = min(n, s0 + seg);
    for (int d = lane; d < nd; d += kWave) s.cnt[wv][d] = 0;
    __builtin_amdgcn_wave_barrier();
    for (int b0 = s0; b0 < s1; b0 += kWave) {
        const int i = b0 + lane;
        const bool ok = i < s1;
        const uint32_t d = ok ? digit(i) : 0u;
        const uint64_t peers = match_digit(d, ok, db);
        if (ok && (peers & lt) == 0) s.cnt[wv][d] += __popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    int32_t tot = 0, incl = 0;
    if (tid < (1 << kPartDigit)) {
        if (tid < nd)
            for (int w = 0; w < kPartNW; ++w) tot += s.cnt[w][tid];
        incl = tot;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int32_t y = __shfl_up(incl, d, 64);
            if (lane >= d) incl += y;
        }
        if (lane == kWave - 1) s.dsum[wv] = incl;
    }
    __syncthreads();
    if (tid < nd) {
        int32_t run = incl - tot;
        for (int w = 0; w < wv; ++w) run += s.dsum[w];
        s.dstart[tid] = run;
        for (int w = 0; w < kPartNW; ++w) {
            const int32_t c = s.cnt[w][tid];
            s.cnt[w][tid] = run;
            run += c;
        }
    }
    __syncthreads();
    for (int b0 = s0; b0 < s1; b0 += kWave) {
        const int i = b0 + lane;
        const bool ok = i < s1;
        const uint32_t d = ok ? digit(i) : 0u;
        const uint64_t peers = match_digit(d, ok, db);
        const int32_t base = ok ? s.cnt[wv][d] : 0;
        __builtin_amdgcn_wave_barrier();
        if (ok) emit(i, base + int32_t(__popcll(peers & lt)));
        if (ok && (peers & lt) == 0) s.cnt[wv][d] = base + __popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
}

// Inclusive block scan of one int per thread (thread order); *total gets the sum.
// Two barriers; wi is one of the s.wi rows.
template <class Cfg>
__device__ __forceinline__ int32_t part_scan_int(int32_t x, int32_t *wi, int32_t *total) {
    PART_CFG_NAMES(Cfg);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int32_t incl = x;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == kWave - 1) wi[wv] = incl;
    __syncthreads();
    int32_t pre = 0, tot = 0;
    for (int k = 0; k < kPartNW; ++k) {
        const int32_t v = wi[k];
        if (k < wv) pre += v;
        tot += v;
    }
    __syncthreads();
    *total = tot;
    return pre + incl;
}

// A segment scan element: writes so far, whether a segment head was seen, the log-decay
// sum and the write count since the last head.
struct SegAcc {
    int32_t tot;
    int32_t hh;
    float seg;
    int32_t scnt;
};

__device__ __forceinline__ SegAcc seg_op(const SegAcc &a, const SegAcc &b) {
    SegAcc r;
    r.tot = a.tot + b.tot;
    r.hh = a.hh | b.hh;
    r.seg = b.hh ? b.seg : a.seg + b.seg;
    r.scnt = b.hh ? b.scnt : a.scnt + b.scnt;
    return r;
}

struct PartArgs {
    int32_t lognp;      // log2 of the partition count
    int32_t sort_bits;  // slot bits above the partition bits
    int32_t once;       // the emit stage writes the id copies, marking ids with kIdOnce (else the
                        // count stage copies them unmarked)
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::kBlock, 4) void p1_part_kernel(Problem pb, Slab sl, PartArgs pa) {
    PART_CFG_NAMES(Cfg);
    extern __shared__ __align__(16) char part_lds[];
    PartSmem<Cfg> &s = *reinterpret_cast<PartSmem<Cfg> *>(part_lds);
    const int64_t n = blockIdx.x;
    const ChunkLayout &L = sl.lay;
    uint32_t *cb = sl.chunk(n);
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int nl = n_live_tokens(pb, p, ti);
    const int W = pb.W, R = pb.R, C = pb.C, WR = W + R;
    const int32_t El = nl * W, Fl = nl * R;
    const int64_t tok0 = int64_t(p) * pb.T + int64_t(ti) * C;
    const int tid = threadIdx.x;
    const int NP = 1 << pa.lognp;
    const uint32_t pmask = uint32_t(NP - 1);
    int32_t *meta = reinterpret_cast<int32_t *>(cb + L.off_meta);

    // ---- count the entries of each partition (copying the ids in entry order unless the emit
    //      stage writes them marked); a partition past the LDS leaves the chunk to the sorting
    //      path (which writes the copies itself)
    uint32_t *kid = cb + L.off_kid;
    uint32_t *qid = cb + L.off_qid;
    const bool once = pa.once != 0;
    for (int d = tid; d < NP; d += kPartBlock) s.pcnt[d] = 0;
    __syncthreads();
    count_ids<Cfg>(pb.k_idx, pb.k_id8, tok0 * W, El, !once, kid, s.pcnt, pmask);
    count_ids<Cfg>(pb.q_idx, pb.q_id8, tok0 * R, Fl, !once, qid, s.pcnt, pmask);
    __syncthreads();
    if (tid == 0) {
        int32_t o = 0, fb = 0;
        for (int d = 0; d < NP; ++d) {
            s.poff[d] = o;
            s.pcur[d] = 0;
            o += s.pcnt[d];
            fb |= s.pcnt[d] > kPartCap;
        }
        s.poff[NP] = o;
        s.fallback = fb;
        s.wo = s.go = s.co = s.ho = 0;
        s.nrep = 0;
        meta[7] = fb;
    }
    __syncthreads();
    if (s.fallback) return;
    for (int x = 8 + tid; x < 64; x += kPartBlock) meta[x] = 0;   // Phase-2 team barrier counters

    // ---- chunk prologue: beta, padding weights and records
    float *beta_c = reinterpret_cast<float *>(cb + L.off_beta);
    float *gw = reinterpret_cast<float *>(cb + L.off_gw);
    float *gr = reinterpret_cast<float *>(cb + L.off_gr);
    int4 *rcr = reinterpret_cast<int4 *>(cb + L.off_rcr);
    for (int i = tid; i < C; i += kPartBlock) beta_c[i] = i < nl ? pb.beta[tok0 + i] : 0.0f;
    for (int64_t e = El + tid; e < L.E; e += kPartBlock) gw[e] = 0.0f;
    for (int64_t f = Fl + tid; f < L.F; f += kPartBlock) {
        gr[f] = 0.0f;
        rcr[f] = make_int4(0, 0, 0, 0);
    }

    // ---- scatter the entries to the partition lists, tile by tile of tokens; inv maps each
    //      entry (token-major, a token's writes then reads) to its list slot
    int4 *plist = reinterpret_cast<int4 *>(cb + L.off_plist);
    uint32_t *oval = cb + L.off_oval;
    int32_t *inv = reinterpret_cast<int32_t *>(cb + L.off_inv);
    const int TT = max(1, kPartCap / WR);
    for (int t0 = 0; t0 < nl; t0 += TT) {
        const int nt = min(TT, nl - t0) * WR;
        const int32_t xb = t0 * WR;
        {
            uint32_t sid[kPartIpt], c[kPartIpt], a[kPartIpt], b[kPartIpt];
#pragma unroll
            for (int u = 0; u < kPartIpt; ++u) {
                const int32_t i = u * kPartBlock + tid;
                const bool ok = i < nt;
                const int t = t0 + (ok ? i / WR : 0), o = ok ? i % WR : 0;
                const bool w = o < W;
                // one load per value from a selected address (no branch: the loads of all
                // items issue back to back)
                const int64_t x = w ? (tok0 + t) * W + o : (tok0 + t) * R + (o - W);
                const int32_t id = load_id(w ? pb.k_idx : pb.q_idx, x, w ? pb.k_id8 : pb.q_id8);
                const float kq = load_weight(w ? pb.k_val : pb.q_val, x, pb.dtype);
                const float gv = pb.g[(tok0 + t) * pb.G + (pb.G == 1 ? 0 : (w ? o : 0))];
                sid[u] = uint32_t(id);
                c[u] = w ? uint32_t(t << 8 | o) : 0x80000000u | uint32_t(t << 8 | (o - W));
                a[u] = __float_as_uint(kq);
                b[u] = w ? __float_as_uint(gv) : 0u;
            }
#pragma unroll
            for (int u = 0; u < kPartIpt; ++u) {
                const int32_t i = u * kPartBlock + tid;
                if (i < nt) {
                    s.slot[i] = sid[u];
                    s.code[i] = c[u];
                    s.v1[i] = a[u];
                    s.v2[i] = b[u];
                }
            }
        }
        __syncthreads();
        if (NP > 1) {
            part_scatter(s, nt, pa.lognp, [&](int i) { return s.slot[i] & pmask; },
                         [&](int i, int pos) { s.perm[0][pos] = uint16_t(i); });
        } else {
            for (int32_t i = tid; i < nt; i += kPartBlock) s.perm[0][i] = uint16_t(i);
            if (tid == 0) s.dstart[0] = 0;
            __syncthreads();
        }
        for (int32_t pos = tid; pos < nt; pos += kPartBlock) {
            const int i = s.perm[0][pos];
            const uint32_t d = s.slot[i] & pmask;
            const int32_t dst = s.poff[d] + s.pcur[d] + (pos - s.dstart[d]);
            plist[dst] = make_int4(int32_t(s.slot[i]), int32_t(s.code[i]), int32_t(s.v1[i]), int32_t(s.v2[i]));
            s.perm[1][i] = uint16_t(pos);   // this entry's place in the tile's partition order
        }
        __syncthreads();
        for (int32_t i = tid; i < nt; i += kPartBlock) {   // the slot map, in entry order
            const int pos = s.perm[1][i];
            const uint32_t d = s.slot[i] & pmask;
            inv[xb + i] = s.poff[d] + s.pcur[d] + (pos - s.dstart[d]);
        }
        __syncthreads();
        if (tid < NP) {   // this tile's count of partition tid
            const int32_t end = tid + 1 < NP ? s.dstart[tid + 1] : nt;
            s.pcur[tid] += end - s.dstart[tid];
        }
        __syncthreads();
    }

    // ---- the partitions, one after another
    int4 *spk = reinterpret_cast<int4 *>(cb + L.off_spk);
    int2 *mrec = reinterpret_cast<int2 *>(cb + L.off_mrec);
    int4 *grec = reinterpret_cast<int4 *>(cb + L.off_grec);
    int4 *brec = reinterpret_cast<int4 *>(cb + L.off_brec);
    float *Ka = reinterpret_cast<float *>(cb + L.off_ka);
    float *Kb = reinterpret_cast<float *>(cb + L.off_kb);
    float *Qa = reinterpret_cast<float *>(cb + L.off_qa);
    const int HC = int(L.HCAP);
    const int lane = tid & 63, wv = tid >> 6;
    int32_t nrep = 0;
    // each partition's list is loaded into registers while the partition before it is
    // processed (its records go back to its own list slots, never the next one's)
    auto next_part = [&](int q) {
        while (q < NP && s.pcnt[q] == 0) ++q;
        return q;
    };
    auto load_list = [&](int q, int4 (&dst)[kPartIpt]) {
        const int32_t base = s.poff[q], nq = s.pcnt[q];
#pragma unroll
        for (int u = 0; u < kPartIpt; ++u) {
            const int32_t i = u * kPartBlock + tid;
            dst[u] = plist[base + (i < nq ? i : 0)];
        }
    };
    int4 rr[kPartIpt];
    int pnext = next_part(0);
    if (pnext < NP) load_list(pnext, rr);
    for (int pp = pnext; pp < NP; pp = pnext) {
        const int nn = s.pcnt[pp];
        {
#pragma unroll
            for (int u = 0; u < kPartIpt; ++u) {
                const int32_t i = u * kPartBlock + tid;
                if (i < nn) {
                    s.slot[i] = uint32_t(rr[u].x);
                    s.code[i] = uint32_t(rr[u].y);
                    s.v1[i] = uint32_t(rr[u].z);
                    s.v2[i] = uint32_t(rr[u].w);
                    s.perm[0][i] = uint16_t(i);
                }
            }
        }
        __syncthreads();
        pnext = next_part(pp + 1);
        if (pnext < NP) load_list(pnext, rr);
        // stable LSD radix sort by the slot bits above the partition bits
        int cur = 0;
        {
            const int bits = pa.sort_bits;
            const int passes = (bits + kPartDigit - 1) / kPartDigit;
            const int db = passes ? (bits + passes - 1) / passes : 0;
            for (int q = 0; q < passes; ++q) {
                const int shift = pa.lognp + q * db;
                const int dq = min(db, bits - q * db);
                const uint32_t dm = (1u << dq) - 1u;
                const uint16_t *src = s.perm[cur];
                uint16_t *dst = s.perm[cur ^ 1];
                part_scatter(s, nn, dq, [&](int i) { return (s.slot[src[i]] >> shift) & dm; },
                             [&](int i, int pos) { dst[pos] = src[i]; });
                cur ^= 1;
            }
        }
        const uint16_t *ord = s.perm[cur];
        uint16_t *wpos = s.perm[cur ^ 1];   // write rank -> sorted position

        // Scan A over the sorted positions (thread tid owns [tid * ipt, tid * ipt + ipt)):
        // L (segmented log-decay sum, reads adding nothing), write counts global and per slot.
        const int ipt = (nn + kPartBlock - 1) / kPartBlock;
        const int j0 = tid * ipt;
        float Lj[kPartIpt];
        int32_t cwj[kPartIpt], swj[kPartIpt];
        SegAcc agg{0, 0, 0.0f, 0};
#pragma unroll
        for (int u = 0; u < kPartIpt; ++u) {
            const int j = j0 + u;
            if (u >= ipt || j >= nn) break;
            const int idx = ord[j];
            const uint32_t sj = s.slot[idx];
            const bool head = j == 0 || s.slot[ord[j - 1]] != sj;
            const bool isw = !(s.code[idx] >> 31);
            if (head) {
                agg.hh = 1;
                agg.seg = 0.0f;
                agg.scnt = 0;
            }
            if (isw) {
                agg.seg = agg.seg + __uint_as_float(s.v2[idx]);
                agg.scnt += 1;
                agg.tot += 1;
            }
        }
        SegAcc incl = agg;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            SegAcc y;
            y.tot = __shfl_up(incl.tot, d, 64);
            y.hh = __shfl_up(incl.hh, d, 64);
            y.seg = __shfl_up(incl.seg, d, 64);
            y.scnt = __shfl_up(incl.scnt, d, 64);
            if (lane >= d) incl = seg_op(y, incl);
        }
        if (lane == kWave - 1) {
            s.wi[0][wv] = incl.tot;
            s.wi[1][wv] = incl.hh;
            s.wf[wv] = incl.seg;
            s.wi[2][wv] = incl.scnt;
        }
        SegAcc ex;
        ex.tot = __shfl_up(incl.tot, 1, 64);
        ex.hh = __shfl_up(incl.hh, 1, 64);
        ex.seg = __shfl_up(incl.seg, 1, 64);
        ex.scnt = __shfl_up(incl.scnt, 1, 64);
        __syncthreads();
        SegAcc run{0, 0, 0.0f, 0};
        for (int k = 0; k < wv; ++k) run = seg_op(run, SegAcc{s.wi[0][k], s.wi[1][k], s.wf[k], s.wi[2][k]});
        if (lane > 0) run = seg_op(run, ex);
#pragma unroll
        for (int u = 0; u < kPartIpt; ++u) {
            const int j = j0 + u;
            if (u >= ipt || j >= nn) break;
            const int idx = ord[j];
            const uint32_t sj = s.slot[idx];
            const bool head = j == 0 || s.slot[ord[j - 1]] != sj;
            const bool isw = !(s.code[idx] >> 31);
            if (head) {
                run.seg = 0.0f;
                run.scnt = 0;
            }
            if (isw) {
                run.seg = run.seg + __uint_as_float(s.v2[idx]);
                run.scnt += 1;
                run.tot += 1;
            }
            Lj[u] = run.seg;
            cwj[u] = run.tot;
            swj[u] = run.scnt;
        }
        if (tid == kPartBlock - 1) s.nw = run.tot;
        __syncthreads();   // every thread has read v2's log-decays
#pragma unroll
        for (int u = 0; u < kPartIpt; ++u) {
            const int j = j0 + u;
            if (u >= ipt || j >= nn) break;
            const int idx = ord[j];
            if (!(s.code[idx] >> 31)) {
                s.v2[idx] = __float_as_uint(Lj[u]);
                wpos[cwj[u] - 1] = uint16_t(j);
                // a write repeating the slot of the previous write of its own token (the
                // sort keeps equal slots in entry order, so such writes are adjacent)
                if (pb.repeats && swj[u] > 1 && j > 0) {
                    const int ip = ord[j - 1];
                    if (!(s.code[ip] >> 31) && ((s.code[ip] >> 8) & 0xFF) == ((s.code[idx] >> 8) & 0xFF)) ++nrep;
                }
            }
        }
        __syncthreads();
        const int nw = s.nw;

        // Scan B over the write ranks: groups (the writes of one slot), their head ranks
        const int ipw = (nw + kPartBlock - 1) / kPartBlock;
        const int r0 = tid * ipw;
        int32_t nhd = 0;
        for (int u = 0; u < ipw; ++u) {
            const int r = r0 + u;
            if (r >= nw) break;
            nhd += r == 0 || s.slot[ord[wpos[r]]] != s.slot[ord[wpos[r - 1]]];
        }
        int32_t ngt = 0;
        int32_t gcur = part_scan_int<Cfg>(nhd, s.wi[0], &ngt) - nhd;   // groups before this thread's ranks
        for (int u = 0; u < ipw; ++u) {
            const int r = r0 + u;
            if (r >= nw) break;
            const int idx = ord[wpos[r]];
            if (r == 0 || s.slot[idx] != s.slot[ord[wpos[r - 1]]]) {
                s.gpos[gcur] = uint16_t(r);
                s.hotr[r] = -1;
                ++gcur;
            }
            s.code[idx] |= uint32_t(gcur - 1) << 16;
        }
        if (tid == 0) {
            s.gpos[ngt] = uint16_t(nw);
            s.ng = ngt;
        }
        __syncthreads();

        // Groups (thread per group): DW records; big groups (>= kHotMin members) listed
        const int ng = s.ng;
        const int ipg = (ng + kPartBlock - 1) / kPartBlock;
        const int g0 = tid * ipg;
        int32_t ncl = 0;
        for (int u = 0; u < ipg; ++u) {
            const int g = g0 + u;
            if (g >= ng) break;
            ncl += s.gpos[g + 1] - s.gpos[g] >= kHotMin;
        }
        int32_t nct = 0;
        int32_t ccur = part_scan_int<Cfg>(ncl, s.wi[1], &nct) - ncl;
        for (int u = 0; u < ipg; ++u) {
            const int g = g0 + u;
            if (g >= ng) break;
            const int a = s.gpos[g], b = s.gpos[g + 1];
            const int ih = ord[wpos[a]], il = ord[wpos[b - 1]];
            const float kh = __uint_as_float(s.v1[ih]), Lh = __uint_as_float(s.v2[ih]);
            const float Ll = __uint_as_float(s.v2[il]);
            const int th = (s.code[ih] >> 8) & 0xFF;
            // first member inline: position (< 2^16), members - 1 (< 2^8), token (< 2^8)
            const int4 rec = make_int4(int32_t(s.slot[ih]), (s.wo + a) | ((b - a - 1) << 16) | (th << 24),
                                       __float_as_int(expf(Ll)), __float_as_int(kh * expf(Ll - Lh)));
            grec[s.go + g] = rec;
            if (b - a >= kHotMin) {
                s.cand[ccur] = g;
                brec[s.co + ccur] = rec;
                ++ccur;
            }
        }
        if (tid == 0) s.nc = nct;
        __syncthreads();

        // Hot test of the big groups, a wavefront each: every member's L within kHotSpan of
        // the first member's
        const int nc = s.nc;
        for (int c = wv; c < nc; c += kPartNW) {
            const int g = s.cand[c], a = s.gpos[g], b = s.gpos[g + 1];
            const float Lref = __uint_as_float(s.v2[ord[wpos[a]]]);
            float dev = 0.0f;
            for (int r = a + lane; r < b; r += kWave)
                dev = fmaxf(dev, fabsf(__uint_as_float(s.v2[ord[wpos[r]]]) - Lref));
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) dev = fmaxf(dev, __shfl_xor(dev, d, 64));
            if (lane == 0) s.cand_ok[c] = dev <= kHotSpan ? 1 : 0;
        }
        __syncthreads();
        {
            const bool h = tid < nc && s.cand_ok[tid];
            int32_t nht = 0;
            const int32_t rk = part_scan_int<Cfg>(h ? 1 : 0, s.wi[2], &nht) - (h ? 1 : 0);
            if (h && s.ho + rk < HC) s.hotr[s.gpos[s.cand[tid]]] = int16_t(s.ho + rk);   // past the cap: cold
            if (tid == 0) s.nh = nht;
        }
        __syncthreads();

        // Records (thread per sorted position). Sorted-order arrays go out directly; each
        // entry's record goes to its own list slot (read by the emit stage):
        //   write  cold {first member's position, own position, bits k, bits L}, hot
        //          {-1 - hot index, own position, bits of k e^(L - L_ref), bits of k e^(L_ref - L)};
        //   read   after a cold write {first member's position, latest write's position + 1,
        //          bits q, bits Lr}, of a hot group {-1 - hot index, 1 for the first read of a
        //          run of this token's reads of the slot (which carries the run's sum of
        //          q e^(Lr - L_ref), in read order), bits of that sum, 0}, no write before: 0;
        //   oval   the gather weight, k e^L or q e^Lr.
        // Bit 30 of .y (free in every record: positions stay below 2^17) marks an entry whose
        // slot no other entry of the chunk has; the emit stage moves it to the id copy.
        const int32_t lbase = s.poff[pp];
#pragma unroll
        for (int u = 0; u < kPartIpt; ++u) {
            const int j = j0 + u;
            if (u >= ipt || j >= nn) break;
            const int idx = ord[j];
            const uint32_t c = s.code[idx];
            const int t = (c >> 8) & 0xFF;
            const float v1 = __uint_as_float(s.v1[idx]);
            int4 orec = make_int4(0, 0, 0, 0);
            float ov;
            if (!(c >> 31)) {
                const int r = cwj[u] - 1, m = s.wo + r;
                const int g = (c >> 16) & 0x7FFF;
                const int a = s.gpos[g], b = s.gpos[g + 1];
                const float Lm = Lj[u], Ll = __uint_as_float(s.v2[ord[wpos[b - 1]]]);
                spk[m] = make_int4(int32_t(s.slot[idx]), t, __float_as_int(v1), __float_as_int(Lm));
                mrec[m] = make_int2(t, __float_as_int(v1 * expf(Ll - Lm)));
                ov = v1 * expf(Lm);
                const int h = s.hotr[a];
                if (h >= 0) {
                    const float d = Lm - __uint_as_float(s.v2[ord[wpos[a]]]);
                    orec = make_int4(-1 - h, m, __float_as_int(v1 * expf(d)), __float_as_int(v1 * expf(-d)));
                } else {
                    orec = make_int4(s.wo + a, m, __float_as_int(v1), __float_as_int(Lm));
                }
            } else if (swj[u] > 0) {
                const int a = cwj[u] - swj[u], rs = cwj[u] - 1;
                const float Lr = __uint_as_float(s.v2[ord[wpos[rs]]]);   // the latest write's L
                ov = v1 * expf(Lr);
                const int h = s.hotr[a];
                if (h >= 0) {
                    // the first read of a run of this token's reads of the slot sums the run
                    const bool first = j == 0 || (s.code[ord[j - 1]] >> 31) == 0 ||
                                       ((s.code[ord[j - 1]] >> 8) & 0xFF) != uint32_t(t) ||
                                       s.slot[ord[j - 1]] != s.slot[idx];
                    float acc = 0.0f;
                    if (first) {
                        const float Lref = __uint_as_float(s.v2[ord[wpos[a]]]);
                        acc = v1 * expf(Lr - Lref);
                        for (int jj = j + 1; jj < nn; ++jj) {
                            const int i2 = ord[jj];
                            const uint32_t c2 = s.code[i2];
                            if (!(c2 >> 31) || ((c2 >> 8) & 0xFF) != uint32_t(t) || s.slot[i2] != s.slot[idx]) break;
                            acc += __uint_as_float(s.v1[i2]) * expf(Lr - Lref);
                        }
                    }
                    orec = make_int4(-1 - h, first ? 1 : 0, __float_as_int(acc), 0);
                } else {
                    orec = make_int4(s.wo + a, s.wo + rs + 1, __float_as_int(v1), __float_as_int(Lr));
                }
            } else {
                ov = v1 * expf(0.0f);
            }
            const bool once = (j == 0 || s.slot[ord[j - 1]] != s.slot[idx]) &&
                              (j + 1 == nn || s.slot[ord[j + 1]] != s.slot[idx]);
            orec.y |= once ? kIdOnce : 0;
            plist[lbase + idx] = orec;
            oval[lbase + idx] = __float_as_uint(ov);
        }
        __syncthreads();
        if (tid == 0) {
            s.wo += nw;
            s.go += ng;
            s.co += nc;
            s.ho += s.nh;
        }
        __syncthreads();
    }
    if (nrep) atomicAdd(&s.nrep, nrep);
    __syncthreads();

    // ---- emit, tile by tile of tokens: the entry-order arrays and the dense hot rows
    {
        int4 *ecr = reinterpret_cast<int4 *>(cb + L.off_ecr);
        const int nh = min(s.ho, HC), HP = (nh + 15) & ~15;
        float *hrow = reinterpret_cast<float *>(s.slot);   // [3][TE][HP] dense rows of the tile (LDS)
        const int TE = max(1, min(nl, int(sizeof(s.slot) * 4 / (3 * sizeof(float) * (HP ? HP : 1)))));
        const int TE2 = min(TE, TT);
        // each tile's list slots are loaded during the tile before it, so that a tile waits
        // for one round trip (its records) instead of two
        auto load_slots = [&](int t0_, int32_t (&dst)[kPartIpt]) {
            const int nt_ = min(TE2, nl - t0_) * WR;
#pragma unroll
            for (int u = 0; u < kPartIpt; ++u) {
                const int32_t i = u * kPartBlock + tid;
                dst[u] = inv[t0_ * WR + (i < nt_ ? i : 0)];
            }
        };
        int32_t sl_[kPartIpt];
        if (nl > 0) load_slots(0, sl_);
        for (int t0 = 0; t0 < nl; t0 += TE2) {
            const int ntok = min(TE2, nl - t0);
            const int nt = ntok * WR;
            int4 rec[kPartIpt];
            uint32_t ovv[kPartIpt];
            int32_t idv[kPartIpt] = {};
#pragma unroll
            for (int u = 0; u < kPartIpt; ++u) {
                rec[u] = plist[sl_[u]];
                ovv[u] = oval[sl_[u]];
                // this entry's slot id from the input (entry 0 of the tile past its end)
                const int32_t i = u * kPartBlock + tid;
                const int tt = i < nt ? i / WR : 0, o = i < nt ? i - tt * WR : 0;
                if (once)
                    idv[u] = o < W ? load_id(pb.k_idx, (tok0 + t0 + tt) * W + o, pb.k_id8)
                                   : load_id(pb.q_idx, (tok0 + t0 + tt) * R + (o - W), pb.q_id8);
            }
            if (t0 + TE2 < nl) load_slots(t0 + TE2, sl_);
            for (int x = tid; x < 3 * ntok * HP; x += kPartBlock) hrow[x] = 0.0f;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kPartIpt; ++u) {
                const int32_t i = u * kPartBlock + tid;
                if (i >= nt) break;
                const int tt = i / WR, o = i - tt * WR, t = t0 + tt;
                int4 r = rec[u];
                const int32_t single = r.y & kIdOnce;
                r.y &= ~kIdOnce;
                if (o < W) {
                    if (once) kid[t * W + o] = uint32_t(idv[u] | single);
                    gw[t * W + o] = __uint_as_float(ovv[u]);
                    if (r.x < 0) {
                        ecr[t * W + o] = make_int4(r.y, r.y, 0, 0);
                        const int h = -1 - r.x;
                        hrow[(0 * ntok + tt) * HP + h] = __int_as_float(r.z);
                        hrow[(1 * ntok + tt) * HP + h] = __int_as_float(r.w);
                    } else {
                        ecr[t * W + o] = r;
                    }
                } else {
                    if (once) qid[t * R + (o - W)] = uint32_t(idv[u] | single);
                    gr[t * R + (o - W)] = __uint_as_float(ovv[u]);
                    if (r.x < 0) {
                        rcr[t * R + (o - W)] = make_int4(0, 0, 0, 0);
                        if (r.y) hrow[(2 * ntok + tt) * HP + (-1 - r.x)] = __int_as_float(r.z);
                    } else {
                        rcr[t * R + (o - W)] = r;
                    }
                }
            }
            __syncthreads();
            for (int x = tid; x < 3 * ntok * HP; x += kPartBlock) {
                const int k = x / (ntok * HP), rem = x - k * ntok * HP, tt = rem / HP, h = rem - tt * HP;
                float *dst = k == 0 ? Ka : (k == 1 ? Kb : Qa);
                dst[(t0 + tt) * HC + h] = hrow[x];
            }
            __syncthreads();
        }
        // padding tokens' rows: +0 (the dense products cover every row of the chunk, and a
        // 0 x NaN of stale memory would reach the live rows through the solve's products)
        const int npad = C - nl;
        for (int x = tid; x < 3 * npad * HP; x += kPartBlock) {
            const int k = x / (npad * HP), rem = x - k * npad * HP, tt = rem / HP, h = rem - tt * HP;
            float *dst = k == 0 ? Ka : (k == 1 ? Kb : Qa);
            dst[(nl + tt) * HC + h] = 0.0f;
        }
    }

    __syncthreads();
    if (tid == 0) {
        const int32_t nh = min(s.ho, int32_t(L.HCAP));
        meta[0] = nl;
        meta[1] = El;
        meta[2] = s.go;
        meta[3] = nh;
        meta[4] = s.co;
        meta[5] = (nh + 15) & ~15;
        if (pb.repeats && s.nrep > 0) atomicAdd(pb.repeats, static_cast<unsigned long long>(s.nrep));
    }
}

hipError_t part_prepare() {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&p1_part_kernel<PartBig>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(sizeof(PartSmem<PartBig>)));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&p1_part_kernel<PartSmall>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(sizeof(PartSmem<PartSmall>)));
}

// log2 of the partition count for chunks of E write and F read entries: the smallest that
// leaves about two thirds of the configuration's partition capacity per partition on average,
// at most its partition limit, and no more partitions than slot values (key_bits).
template <class Cfg>
static int part_lognp_cfg(int64_t E, int64_t F, int key_bits) {
    int lg = 0;
    while (lg < Cfg::kMaxLogNP && lg < key_bits && (E + F) > (int64_t(Cfg::kCap) * 2 / 3) << lg) ++lg;
    return lg;
}

int part_lognp(int64_t E, int64_t F, int key_bits) {
    return E + F >= kPartBigEntries ? part_lognp_cfg<PartBig>(E, F, key_bits) : part_lognp_cfg<PartSmall>(E, F, key_bits);
}

hipError_t launch_phase1_part(const Problem &pb, const Slab &sl, int lognp, hipStream_t st) {
    PartArgs pa{lognp, pb.key_bits > lognp ? pb.key_bits - lognp : 0, once_rows_streamed(pb) ? 1 : 0};
    const unsigned nch = unsigned(int64_t(pb.P) * sl.steps);
    if (sl.lay.E + sl.lay.F >= kPartBigEntries) {
        if (lognp > PartBig::kMaxLogNP) return hipErrorInvalidValue;
        hipLaunchKernelGGL(p1_part_kernel<PartBig>, dim3(nch), dim3(PartBig::kBlock), sizeof(PartSmem<PartBig>), st,
                           pb, sl, pa);
    } else {
        if (lognp > PartSmall::kMaxLogNP) return hipErrorInvalidValue;
        hipLaunchKernelGGL(p1_part_kernel<PartSmall>, dim3(nch), dim3(PartSmall::kBlock), sizeof(PartSmem<PartSmall>),
                           st, pb, sl, pa);
    }
    return hipGetLastError();
}

}  // namespace sdm

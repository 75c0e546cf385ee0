// Phase 1 of the chunked SDM forward on gfx950: the bank-independent quantities of every
// chunk of a slab (module docstring of memory_ops.py, sparse-delta-memory 2.0.0 wheel,
// diffend page 21: per-slot log-decays, dedup flags, gather weights, Gram matrices A
// and QK). Each chunk is handled by its own workgroup(s), so chunks never interact and
// every result depends only on its chunk's inputs.
//
//   p1_sort    stable LSD radix sort of the chunk's write entries by slot id
//              (entries enter in token order, so equal slots end in token order:
//              each run of one slot is that slot's write group)
//   p1_groups  block-parallel passes over the sorted entries: group table, the
//              cumulative log-decay L of each member (a segmented scan over each group in
//              token order), gather weights k exp(L), the DW records (per group {slot,
//              first position, members, exp(L_last)}, per member {token, k exp(L_last -
//              L)}), a bucket index of the sorted slots for the read lookups, and the split
//              of the groups into hot (many members, bounded decay span: their pair terms
//              go to the matrix cores) and cold (their pair terms are summed directly)
//   p1_reads   for each read entry, the latest write of its slot at or before its token
//              (bucketed binary search), its L and gather weight q exp(L)
//   p1_gram_cold  the cold pair terms of A (strict lower) and QK (lower with diagonal) by
//              row ownership: the wavefront of row i lists its entries' pair terms in a
//              fixed order and replays them into the lanes that own their columns
//   p1_gram_hot   the hot pair terms as dense products on the matrix cores
// No float atomics anywhere: every element has one writer and a fixed summation order.
#include <stdlib.h>

#include <algorithm>

#include "common.h"
#include "wy_impl.h"

namespace sdm {


// Stable LSD radix sort of one chunk's write entries by slot id, in passes of at most
// kSortDigit bits. Wave w owns a fixed contiguous segment of the input of every pass: it
// counts the digits of its segment (wave-private LDS row), the block turns the counts into
// each wave's first output position per digit (digits ascending, waves in order), and the
// wave scatters its segment in order, ranking equal digits within a wavefront by lane
// (ballot match) and advancing its own per-digit positions. Two block barriers per pass.
constexpr int kSortDigit = 9;

template <int BLOCK>
constexpr size_t sort_smem_bytes() { return size_t(BLOCK / kWave) * (1 << kSortDigit) * 4 + (1 << kSortDigit) / kWave * 4; }

// The sort of chunk n by one workgroup of BLOCK threads; smem: sort_smem_bytes<BLOCK>().
template <int BLOCK>
__device__ __forceinline__ void sort_chunk(const Problem &pb, const Slab &sl, int64_t n, char *smem) {
    constexpr int NW = BLOCK / kWave;
    constexpr int NBK = 1 << kSortDigit;
    static_assert(BLOCK >= NBK, "one thread per digit");
    int32_t(*cnt)[NBK] = reinterpret_cast<int32_t(*)[NBK]>(smem);
    int32_t *dsum = reinterpret_cast<int32_t *>(smem + NW * NBK * 4);
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int nl = n_live_tokens(pb, p, ti);
    const int32_t El = nl * pb.W;
    uint32_t *cb = sl.chunk(n);
    uint32_t *key[2] = {cb + sl.lay.off_key0, cb + sl.lay.off_key1};
    uint32_t *val[2] = {cb + sl.lay.off_val0, cb + sl.lay.off_val1};
    const int64_t kin0 = (int64_t(p) * pb.T + int64_t(ti) * pb.C) * pb.W;   // the chunk's first write id
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint64_t lt = lanemask_lt(lane);
    const int32_t seg = ((El + NW - 1) / NW + 63) & ~63;
    const int32_t s0 = min(El, wv * seg), s1 = min(El, s0 + seg);
    uint32_t *kid = cb + sl.lay.off_kid;
    // ids in entry order (int32), for Phase 2 and as the first pass's keys
    for (int32_t e = threadIdx.x; e < El; e += BLOCK) kid[e] = uint32_t(load_id(pb.k_idx, kin0 + e, pb.k_id8));
    __syncthreads();

    for (int q = 0; q < pb.sort_passes; ++q) {
        const int shift = q * pb.sort_digit;
        const int db = max(1, min(pb.sort_digit, pb.key_bits - shift));
        const int nd = 1 << db;
        const uint32_t dmask = uint32_t(nd - 1);
        const uint32_t *sk = q == 0 ? kid : key[(q + 1) & 1];
        const uint32_t *sv = val[(q + 1) & 1];
        uint32_t *dk = key[q & 1];
        uint32_t *dv = val[q & 1];

        // Count the digits of this wave's segment.
        for (int d = lane; d < nd; d += kWave) cnt[wv][d] = 0;
        for (int32_t b0 = s0; b0 < s1; b0 += 4 * kWave) {
            uint32_t kk[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int32_t e = b0 + u * kWave + lane;
                kk[u] = e < s1 ? sk[e] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = b0 + u * kWave + lane < s1;
                const uint32_t d = (kk[u] >> shift) & dmask;
                const uint64_t peers = match_digit(d, ok, db);
                if (ok && (peers & lt) == 0) cnt[wv][d] += __popcll(peers);
            }
        }
        __syncthreads();
        // First output position of every (wave, digit): digits ascending, waves in order.
        int32_t tot = 0, incl = 0;
        if (tid < NBK) {
            if (tid < nd)
                for (int w = 0; w < NW; ++w) tot += cnt[w][tid];
            incl = tot;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int32_t y = __shfl_up(incl, d, 64);
                if (lane >= d) incl += y;
            }
            if (lane == kWave - 1) dsum[wv] = incl;
        }
        __syncthreads();
        if (tid < nd) {
            int32_t run = incl - tot;
            for (int w = 0; w < wv; ++w) run += dsum[w];
            for (int w = 0; w < NW; ++w) {
                const int32_t c = cnt[w][tid];
                cnt[w][tid] = run;
                run += c;
            }
        }
        __syncthreads();
        // Scatter this wave's segment in order.
        for (int32_t b0 = s0; b0 < s1; b0 += 4 * kWave) {
            uint32_t kk[4], vv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int32_t e = b0 + u * kWave + lane;
                const bool ok = e < s1;
                kk[u] = ok ? sk[e] : 0u;
                vv[u] = ok ? (q == 0 ? uint32_t(e) : sv[e]) : 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = b0 + u * kWave + lane < s1;
                const uint32_t d = (kk[u] >> shift) & dmask;
                const uint64_t peers = match_digit(d, ok, db);
                const int32_t rank = __popcll(peers & lt);
                const int32_t base = cnt[wv][d];
                if (ok && rank == 0) cnt[wv][d] = base + __popcll(peers);
                if (ok) {
                    dk[base + rank] = kk[u];
                    dv[base + rank] = vv[u];
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------
// Block scans over one tile of BLOCK elements (one per thread, thread order), continuing
// the previous tile's inclusive value. Wave scans by shuffles, then each wave adds the
// totals of the waves before it; every sum has a fixed shape, so the bits depend only on
// the data.
// ---------------------------------------------------------------------------------------
template <int NW>
struct TileScan {
    int32_t cnt[NW];
    int32_t mx[NW];
    float val[NW];
    int32_t flag[NW];
    int32_t carry_cnt, carry_mx;
    float carry_val;
};

// One tile of three inclusive scans: a count (head flags), a running maximum (head
// positions) and a sum of x restarted at every head (segmented). Updates the carries.
template <int NW>
__device__ __forceinline__ void tile_scan3(TileScan<NW> &ts, int32_t &cnt, int32_t &mx, float &x, int head) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int f = head;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t c = __shfl_up(cnt, d, 64);
        const int32_t m = __shfl_up(mx, d, 64);
        const float y = __shfl_up(x, d, 64);
        const int fy = __shfl_up(f, d, 64);
        if (lane >= d) {
            cnt += c;
            mx = max(mx, m);
            if (!f) x = y + x;
            f |= fy;
        }
    }
    if (lane == 63) {
        ts.cnt[wv] = cnt;
        ts.mx[wv] = mx;
        ts.val[wv] = x;
        ts.flag[wv] = f;
    }
    __syncthreads();
    int32_t pc = ts.carry_cnt, pm = ts.carry_mx;
    float pv = ts.carry_val;
    for (int k = 0; k < wv; ++k) {
        pc += ts.cnt[k];
        pm = max(pm, ts.mx[k]);
        pv = ts.flag[k] ? ts.val[k] : pv + ts.val[k];
    }
    cnt += pc;
    mx = max(mx, pm);
    if (!f) x = pv + x;
    __syncthreads();
    if (tid == NW * kWave - 1) {
        ts.carry_cnt = cnt;
        ts.carry_mx = mx;
        ts.carry_val = x;
    }
    __syncthreads();
}

// Exclusive ballot compaction of one tile: returns the rank of a set flag among the set
// flags of the tile (thread order) plus the running total, which it advances.
template <int NW>
__device__ __forceinline__ int32_t tile_compact(bool flag, int32_t *wsum, int32_t *total) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint64_t b = __ballot(flag);
    if (lane == 0) wsum[wv] = __popcll(b);
    __syncthreads();
    int32_t off = *total;
    for (int k = 0; k < wv; ++k) off += wsum[k];
    const int32_t rank = off + __popcll(b & lanemask_lt(lane));
    __syncthreads();
    if (tid == 0) {
        int32_t t = *total;
        for (int k = 0; k < NW; ++k) t += wsum[k];
        *total = t;
    }
    __syncthreads();
    return rank;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
    return v;
}

__device__ __forceinline__ int bucket_shift(const Problem &pb, int64_t E) {
    const int s = pb.key_bits - bucket_bits(E);
    return s > 0 ? s : 0;
}

constexpr int kMaxHot = kMaxChunk * kMaxWidth / kHotMin;   // hot groups of a chunk, at most

template <int NW> struct GroupsSmem {
    TileScan<NW> ts;
    int32_t wsum[NW];
    int32_t ncand, nhot;
    int32_t nrep;              // write entries repeating a slot of their own token
    int32_t cand[kMaxHot];
    uint8_t cand_hot[kMaxHot];
};

// The group scan of chunk n by one workgroup of BLOCK threads; smem: GroupsSmem.
template <int BLOCK>
__device__ __forceinline__ void groups_chunk(const Problem &pb, const Slab &sl, int64_t n, char *smem) {
    constexpr int NW = BLOCK / kWave;
    GroupsSmem<NW> &gs = *reinterpret_cast<GroupsSmem<NW> *>(smem);
    TileScan<NW> &ts = gs.ts;
    int32_t *wsum = gs.wsum;
    int32_t &ncand = gs.ncand, &nhot = gs.nhot;
    int32_t *cand = gs.cand;
    uint8_t *cand_hot = gs.cand_hot;
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int nl = n_live_tokens(pb, p, ti);
    const int W = pb.W, C = pb.C;
    const int32_t El = nl * W;
    const ChunkLayout &L = sl.lay;
    uint32_t *cb = sl.chunk(n);
    const int fin = (pb.sort_passes - 1) & 1;
    const uint32_t *skey = cb + (fin ? L.off_key1 : L.off_key0);
    const uint32_t *sval = cb + (fin ? L.off_val1 : L.off_val0);
    int4 *spk = reinterpret_cast<int4 *>(cb + L.off_spk);
    int32_t *shead = reinterpret_cast<int32_t *>(cb + L.off_shead);
    int32_t *sgrp = reinterpret_cast<int32_t *>(cb + L.off_sgrp);
    int32_t *gpos = reinterpret_cast<int32_t *>(cb + L.off_gpos);
    int4 *grec = reinterpret_cast<int4 *>(cb + L.off_grec);
    int2 *mrec = reinterpret_cast<int2 *>(cb + L.off_mrec);
    float *gw = reinterpret_cast<float *>(cb + L.off_gw);
    int4 *ecr = reinterpret_cast<int4 *>(cb + L.off_ecr);
    int4 *sgh = reinterpret_cast<int4 *>(cb + L.off_sgh);
    int32_t *ghot = reinterpret_cast<int32_t *>(cb + L.off_ghot);
    float *Ka = reinterpret_cast<float *>(cb + L.off_ka);
    float *Kb = reinterpret_cast<float *>(cb + L.off_kb);
    int32_t *hgrp = reinterpret_cast<int32_t *>(cb + L.off_hgrp);
    int4 *brec = reinterpret_cast<int4 *>(cb + L.off_brec);
    int32_t *bstart = reinterpret_cast<int32_t *>(cb + L.off_bstart);
    int32_t *meta = reinterpret_cast<int32_t *>(cb + L.off_meta);
    float *beta_c = reinterpret_cast<float *>(cb + L.off_beta);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t tok0 = int64_t(p) * pb.T + int64_t(ti) * C;
    const int bsh = bucket_shift(pb, L.E);
    const int32_t NB = int32_t(L.NB);

    if (tid == 0) {
        ts.carry_cnt = 0;
        ts.carry_mx = -1;
        ts.carry_val = 0.0f;
        ncand = 0;
        nhot = 0;
        gs.nrep = 0;
    }
    for (int i = tid; i < C; i += BLOCK) beta_c[i] = i < nl ? pb.beta[tok0 + i] : 0.0f;
    for (int64_t e = El + tid; e < L.E; e += BLOCK) gw[e] = 0.0f;
    __syncthreads();

    // Pass 1, tile by tile over the sorted positions: group starts, group index, last
    // group start, cumulative log-decay L, the per-position record, bucket starts; and,
    // when counted, the entries repeating a slot of their own token (the sort is stable,
    // so such entries sit right after an entry of the same slot and token).
    int32_t nrep = 0;
    for (int32_t t0 = 0; t0 < El; t0 += BLOCK) {
        const int32_t m = t0 + tid;
        const bool ok = m < El;
        uint32_t key = 0;
        int head = 0;
        int32_t i = 0;
        float gv = 0.0f, kv = 0.0f;
        if (ok) {
            key = skey[m];
            const uint32_t prev = m > 0 ? skey[m - 1] : ~key;
            head = prev != key;
            const int32_t e = int32_t(sval[m]);
            i = e / W;
            const int32_t w = e - i * W;
            const int64_t tg = tok0 + i;
            gv = pb.g[tg * pb.G + (pb.G == 1 ? 0 : w)];
            kv = load_weight(pb.k_val, tg * W + w, pb.dtype);
            const int32_t bp = m > 0 ? min(int32_t(prev >> bsh), NB - 1) : -1, bc = min(int32_t(key >> bsh), NB - 1);
            for (int32_t b = bp + 1; b <= bc; ++b) bstart[b] = m;
            if (pb.repeats && !head && int32_t(sval[m - 1]) / W == i) ++nrep;
        }
        int32_t cnt = head, mx = head ? m : -1;
        float Lc = gv;
        tile_scan3<NW>(ts, cnt, mx, Lc, head);
        if (ok) {
            spk[m] = make_int4(int32_t(key), i, __float_as_int(kv), __float_as_int(Lc));
            sgrp[m] = cnt - 1;
            shead[m] = mx;
            if (head) gpos[cnt - 1] = m;
        }
    }
    const int32_t ng = ts.carry_cnt;
    {
        const int32_t bl = El > 0 ? min(int32_t(skey[El - 1] >> bsh), NB - 1) : -1;
        for (int32_t b = bl + 1 + tid; b <= NB; b += BLOCK) bstart[b] = El;
    }
    for (int x = 8 + tid; x < 64; x += BLOCK) meta[x] = 0;   // Phase-2 team barrier counters
    if (tid == 0) {
        gpos[ng] = El;
        meta[0] = nl;
        meta[1] = El;
        meta[2] = ng;
    }
    for (int32_t g = tid; g < ng; g += BLOCK) ghot[g] = -1;
    if (nrep) atomicAdd(&gs.nrep, nrep);
    __syncthreads();
    if (tid == 0 && pb.repeats && gs.nrep > 0) atomicAdd(pb.repeats, static_cast<unsigned long long>(gs.nrep));

    // Pass 2, per sorted position: DW records and gather weights.
    for (int32_t m = tid; m < El; m += BLOCK) {
        const int4 pk = spk[m];
        const int32_t g = sgrp[m], a = shead[m], b = gpos[g + 1];
        const float Lm = __int_as_float(pk.w), kv = __int_as_float(pk.z);
        const float Llast = __int_as_float(spk[b - 1].w);
        const float cwm = kv * expf(Llast - Lm);
        mrec[m] = make_int2(pk.y, __float_as_int(cwm));
        gw[int32_t(sval[m])] = kv * expf(Lm);
        // first member inline: position (< 2^16), members - 1 (< 2^8) and token (< 2^8) in one word
        if (m == a) grec[g] = make_int4(pk.x, a | ((b - a - 1) << 16) | (pk.y << 24), __float_as_int(expf(Llast)),
                                        __float_as_int(cwm));
    }

    // Pass 3: hot groups. Candidates (at least kHotMin members) in group order; a wave
    // per candidate finds its largest |L - L_first|; hot ones are numbered in order.
    for (int32_t t0 = 0; t0 < ng; t0 += BLOCK) {
        const int32_t g = t0 + tid;
        const bool c = g < ng && gpos[g + 1] - gpos[g] >= kHotMin;
        const int32_t r = tile_compact<NW>(c, wsum, &ncand);
        if (c) cand[r] = g;
    }
    __syncthreads();
    const int32_t nc = ncand;
    for (int32_t c = wv; c < nc; c += NW) {
        const int32_t g = cand[c], a = gpos[g], b = gpos[g + 1];
        const float Lref = __int_as_float(spk[a].w);
        float dev = 0.0f;
        for (int32_t m = a + lane; m < b; m += kWave) dev = fmaxf(dev, fabsf(__int_as_float(spk[m].w) - Lref));
        dev = wave_max(dev);
        if (lane == 0) {
            cand_hot[c] = dev <= kHotSpan ? 1 : 0;
            brec[c] = grec[g];   // the big groups' DW records, in group order
        }
    }
    __syncthreads();
    for (int32_t t0 = 0; t0 < nc; t0 += BLOCK) {
        const int32_t c = t0 + tid;
        const bool h = c < nc && cand_hot[c];
        const int32_t r = tile_compact<NW>(h, wsum, &nhot);
        if (h && r < L.HCAP) {   // past the cap a group stays cold
            ghot[cand[c]] = r;
            hgrp[r] = cand[c];
        }
    }
    __syncthreads();
    const int32_t nh = min(nhot, int32_t(L.HCAP)), HP = (nh + 15) & ~15;
    if (tid == 0) {
        meta[3] = nh;
        meta[4] = nc;
        meta[5] = HP;
    }
    for (int32_t x = tid; x < C * HP; x += BLOCK) {   // rows [C][HCAP], columns < HP read
        const int32_t r = x / HP, c = x - r * HP;
        Ka[r * L.HCAP + c] = 0.0f;
        Kb[r * L.HCAP + c] = 0.0f;
    }
    __syncthreads();

    // Pass 4, per sorted position: factored decays of hot members into the dense
    // operands; the cold pair ranges (earlier members of the group) by entry (token-major);
    // the read lookup's record of the position: group head, hot index, the head's L (hot).
    for (int32_t m = tid; m < El; m += BLOCK) {
        const int4 pk = spk[m];
        const int32_t g = sgrp[m], a = shead[m];
        const int32_t e = int32_t(sval[m]), w = e - pk.y * W;
        int4 rec = make_int4(m, m, 0, 0);
        const int32_t h = ghot[g];
        const int32_t Lref = h >= 0 ? spk[a].w : 0;   // the read lookup needs it for hot groups only
        if (h >= 0) {
            const float d = __int_as_float(pk.w) - __int_as_float(Lref), kv = __int_as_float(pk.z);
            Ka[pk.y * L.HCAP + h] = kv * expf(d);
            Kb[pk.y * L.HCAP + h] = kv * expf(-d);
        } else {
            rec = make_int4(a, m, pk.z, pk.w);
        }
        ecr[int64_t(pk.y) * W + w] = rec;
        sgh[m] = make_int4(a, h, Lref, 0);
    }
}

// One wavefront per token i of the chunk, lanes over its reads r. The latest write of the
// read slot at or before the read's token is the last sorted position with
// (slot, token) <= (q, i), searched inside the slot's bucket. Reads of hot groups add
// q exp(Lr - L_ref) into the token's row of the dense operand Qa in read order (one lane
// at a time, lanes ascending), so duplicate reads of a slot sum in a fixed order.
constexpr int kReadWaves = 4;

// The reads of token i of chunk n by one wavefront; qr: kHotCap floats of LDS.
// lspk, lsgh, lbst, lqid, lqv: copies of the sorted member records, the lookup records, the
// bucket starts and the chunk's read ids and weights (in LDS for the fused kernel), or
// nullptr to read the workspace and the inputs.
// KR: reads per lane (ceil(R / 64), rounded up to 1, 2 or 4).
template <int KR>
__device__ __forceinline__ void reads_token_k(const Problem &pb, const Slab &sl, int64_t n, int i, float *qr,
                                              const int4 *lspk, const int4 *lsgh, const int32_t *lbst,
                                              const int32_t *lqid, const float *lqv) {
    const int lane = threadIdx.x & 63;
    const ChunkLayout &L = sl.lay;
    const int R = pb.R, C = pb.C;
    if (i >= C) return;
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int nl = n_live_tokens(pb, p, ti);
    uint32_t *cb = sl.chunk(n);
    const int4 *spk = lspk ? lspk : reinterpret_cast<const int4 *>(cb + L.off_spk);
    const int4 *sgh = lsgh ? lsgh : reinterpret_cast<const int4 *>(cb + L.off_sgh);
    const int32_t *bstart = lbst ? lbst : reinterpret_cast<const int32_t *>(cb + L.off_bstart);
    const int32_t *meta = reinterpret_cast<const int32_t *>(cb + L.off_meta);
    float *gr = reinterpret_cast<float *>(cb + L.off_gr);
    int4 *rcr = reinterpret_cast<int4 *>(cb + L.off_rcr);
    float *Qa = reinterpret_cast<float *>(cb + L.off_qa);
    int32_t *qid = reinterpret_cast<int32_t *>(cb + L.off_qid);
    const int HP = meta[5];
    for (int h = lane; h < HP; h += kWave) qr[h] = 0.0f;
    __builtin_amdgcn_wave_barrier();
    const int64_t tg = int64_t(p) * pb.T + int64_t(ti) * C + i;
    const int bsh = bucket_shift(pb, L.E);
    // A lane's reads (r = lane, lane + 64, ...) are looked up together: their loads are
    // issued side by side and their searches advance in lockstep, so one chain of
    // dependent round trips serves all of them. Every load reads an in-bounds element
    // (index 0 for a read without work).
    const int nr = (R + kWave - 1) / kWave;   // <= KR
    const bool live = i < nl;
    int32_t q[KR], lo[KR], hi[KR], b0[KR];
    float qv[KR];
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        const int r = k * kWave + lane;
        const bool ok = k < nr && r < R && live;
        const int64_t x = ok ? tg * R + r : 0;
        q[k] = lqid ? lqid[ok ? i * R + r : 0] : load_id(pb.q_idx, x, pb.q_id8);
        qv[k] = lqv ? lqv[ok ? i * R + r : 0] : load_weight(pb.q_val, x, pb.dtype);
        const int32_t b = min(int32_t(uint32_t(q[k]) >> bsh), int32_t(L.NB) - 1);
        b0[k] = bstart[b];
        hi[k] = bstart[b + 1];
        if (!ok) hi[k] = b0[k];
        lo[k] = b0[k];
    }
    // the last sorted position with (slot, token) <= (q, i), in each read's bucket
    for (;;) {
        bool act = false;
#pragma unroll
        for (int k = 0; k < KR; ++k) act |= lo[k] < hi[k];
        if (!__any(act)) break;
        int4 pk[KR];
#pragma unroll
        for (int k = 0; k < KR; ++k) pk[k] = spk[lo[k] < hi[k] ? (lo[k] + hi[k]) >> 1 : 0];
#pragma unroll
        for (int k = 0; k < KR; ++k) {
            if (lo[k] < hi[k]) {
                const int32_t mid = (lo[k] + hi[k]) >> 1;
                if (pk[k].x < q[k] || (pk[k].x == q[k] && pk[k].y <= i)) lo[k] = mid + 1;
                else hi[k] = mid;
            }
        }
    }
    int4 pk[KR], gh[KR];
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        const int32_t pos = lo[k] - 1;
        pk[k] = spk[pos >= b0[k] ? pos : 0];
        gh[k] = sgh[pos >= b0[k] ? pos : 0];   // group head, hot index, the head's L
    }
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        if (k >= nr) break;
        const int r = k * kWave + lane;
        const bool ok = r < R;
        float g = 0.0f, rv = 0.0f;
        int32_t h = -1;
        int4 cr = make_int4(0, 0, 0, 0);
        if (ok && live) {
            qid[int64_t(i) * R + r] = q[k];   // ids in entry order, for Phase 2
            const int32_t pos = lo[k] - 1;
            float l = 0.0f;
            if (pos >= b0[k] && pk[k].x == q[k]) {
                l = __int_as_float(pk[k].w);
                h = gh[k].y;
                if (h >= 0) rv = qv[k] * expf(l - __int_as_float(gh[k].z));
                else cr = make_int4(gh[k].x, pos + 1, __float_as_int(qv[k]), pk[k].w);
            }
            g = qv[k] * expf(l);
        }
        if (ok) {
            gr[int64_t(i) * R + r] = g;
            rcr[int64_t(i) * R + r] = cr;
        }
        // hot reads into the row, lanes ascending
        for (uint64_t m = __ballot(h >= 0); m; m &= m - 1) {
            const int src = __ffsll(static_cast<unsigned long long>(m)) - 1;
            if (lane == src) qr[h] += rv;
            __builtin_amdgcn_wave_barrier();
        }
    }
    __builtin_amdgcn_wave_barrier();
    for (int h = lane; h < HP; h += kWave) Qa[int64_t(i) * L.HCAP + h] = qr[h];
}

__device__ __forceinline__ void reads_token(const Problem &pb, const Slab &sl, int64_t n, int i, float *qr,
                                            const int4 *lspk = nullptr, const int4 *lsgh = nullptr,
                                            const int32_t *lbst = nullptr, const int32_t *lqid = nullptr,
                                            const float *lqv = nullptr) {
    static_assert(kMaxWidth <= 4 * kWave, "at most four reads per lane");
    if (pb.R <= kWave) reads_token_k<1>(pb, sl, n, i, qr, lspk, lsgh, lbst, lqid, lqv);
    else if (pb.R <= 2 * kWave) reads_token_k<2>(pb, sl, n, i, qr, lspk, lsgh, lbst, lqid, lqv);
    else reads_token_k<4>(pb, sl, n, i, qr, lspk, lsgh, lbst, lqid, lqv);
}

// The cold part of A (blockIdx.y = 0: write entries) or QK (blockIdx.y = 1: read
// entries), one wavefront per row i. Lane l holds columns 4l .. 4l + 3 of the row. The
// row's entries are taken 64 at a time (entry x = x0 + lane); each lane with earlier cold
// members writes its pair terms (column, value) into the wavefront's LDS list at its
// prefix-summed offset, and then every lane replays the list in order, adding the terms of
// its own columns. The sum of each element therefore runs in entry order, each entry's
// earlier group members in token order. Every row is written whole, zeros included, so A
// and QK are fully defined here (+0 outside their triangles) and the hot part is added
// afterwards.
constexpr int kColdBlock = 512;
constexpr int kTermCap = 512;   // terms per wavefront per round (>= 255 earlier members of one entry)

// Row i of the cold part of A (qk false) or QK (qk true) of chunk n by one wavefront;
// mcol, mval: kTermCap entries each of LDS.
// Row i from explicit arrays: spk the sorted member records, cr the transposed cold
// records of the row's region (width entries per token), Mout the C x C output.
__device__ __forceinline__ void cold_row_at(int C, int nl, const int4 *spk, const int4 *cr, float *Mout, int width,
                                            int i, int32_t *mcol, float *mval) {
    const int lane = threadIdx.x & 63;
    {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int x0 = 0; i < nl && x0 < width; x0 += kWave) {
            const int x = x0 + lane;
            // the row's own records are read once: streamed with the non-temporal hint, so
            // that the earlier members' records, which several rows read, stay cached
            int4 r = make_int4(0, 0, 0, 0);
            if (x < width) {
                typedef int32_t i4_t __attribute__((ext_vector_type(4)));
                const i4_t v = __builtin_nontemporal_load(reinterpret_cast<const i4_t *>(cr + int64_t(i) * width + x));
                r = make_int4(v[0], v[1], v[2], v[3]);
            }
            // earlier members of the entry's group; at most C - 1 <= 255 when the write slots
            // of a token are distinct, clamped so that a call breaking that contract still
            // advances through its rounds
            const int cnt = r.y > r.x ? min(r.y - r.x, kTermCap) : 0;
            if (__ballot(cnt > 0) == 0) continue;   // no entry here has earlier cold members
            // inclusive prefix of the counts over the lanes
            int incl = cnt;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int y = __shfl_up(incl, d, 64);
                if (lane >= d) incl += y;
            }
            const int excl = incl - cnt, total = __shfl(incl, 63, 64);
            const float kv = __int_as_float(r.z), Lv = __int_as_float(r.w);
            for (int base = 0; base < total;) {
                // this round: the lanes (in order) whose terms fit below base + kTermCap
                const bool in = cnt > 0 && excl >= base && incl <= base + kTermCap;
                // the in-round lanes are consecutive and their prefixes ascend: the round
                // ends at the last one's prefix
                const uint64_t inm = __ballot(in);
                const int end = inm ? __shfl(incl, 63 - __clzll(static_cast<long long>(inm)), 64) : base;
                if (in) {
                    for (int32_t j0 = 0; j0 < cnt; j0 += 4) {
                        int4 pk[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) pk[u] = j0 + u < cnt ? spk[r.x + j0 + u] : make_int4(0, 0, 0, 0);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            if (j0 + u >= cnt) break;
                            mcol[excl - base + j0 + u] = pk[u].y;
                            mval[excl - base + j0 + u] = (kv * __int_as_float(pk[u].z)) * expf(Lv - __int_as_float(pk[u].w));
                        }
                    }
                }
                __builtin_amdgcn_wave_barrier();
                // Replay, 64 terms at a time: the terms go to the lanes that own their columns
                // in rounds, round r carrying each owner's r-th term of the batch (its terms in
                // list order), through slots in the batch's own part of the list (its terms are
                // in registers by then). Every element still sums its terms in list order.
                const int nt = end - base;
                for (int j0 = 0; j0 < nt; j0 += kWave) {
                    const bool ok = j0 + lane < nt;
                    const int c = ok ? mcol[j0 + lane] : 0;
                    const float v = ok ? mval[j0 + lane] : 0.0f;
                    const int own = ok ? (c >> 2) : kWave;   // owner lane of column c (kWave: none)
                    uint64_t peers = ~uint64_t(0);
#pragma unroll
                    for (int b = 0; b < 7; ++b) {
                        const bool bit = (own >> b) & 1;
                        const uint64_t bb = __ballot(bit);
                        peers &= bit ? bb : ~bb;
                    }
                    const int rank = __popcll(peers & lanemask_lt(lane));
                    int32_t *scol = mcol + j0;
                    float *sval = mval + j0;
                    for (int rr = 0; __ballot(ok && rank == rr) != 0; ++rr) {
                        scol[lane] = -1;
                        __builtin_amdgcn_wave_barrier();
                        if (ok && rank == rr) {
                            scol[own] = c & 3;
                            sval[own] = v;
                        }
                        __builtin_amdgcn_wave_barrier();
                        const int q = scol[lane];
                        const float w = sval[lane];
                        if (q == 0) acc[0] += w;
                        else if (q == 1) acc[1] += w;
                        else if (q == 2) acc[2] += w;
                        else if (q == 3) acc[3] += w;
                        __builtin_amdgcn_wave_barrier();
                    }
                }
                __builtin_amdgcn_wave_barrier();
                base = end;
            }
        }
        const int c0 = 4 * lane;
        if (c0 + 3 < C && (C & 3) == 0) {
            *reinterpret_cast<float4 *>(Mout + int64_t(i) * C + c0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (c0 + q < C) Mout[int64_t(i) * C + c0 + q] = acc[q];
        }
    }
}

// Row i of the cold part of A (qk false) or QK (qk true) of chunk n, arrays in the workspace.
__device__ __forceinline__ void cold_row(const Problem &pb, const Slab &sl, int64_t n, bool qk, int i, int32_t *mcol,
                                         float *mval) {
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const ChunkLayout &L = sl.lay;
    uint32_t *cb = sl.chunk(n);
    cold_row_at(pb.C, n_live_tokens(pb, p, ti), reinterpret_cast<const int4 *>(cb + L.off_spk),
                reinterpret_cast<const int4 *>(cb + (qk ? L.off_rcr : L.off_ecr)),
                reinterpret_cast<float *>(cb + (qk ? L.off_QK : L.off_A)), qk ? pb.R : pb.W, i, mcol, mval);
}

// The hot part of A and QK on the matrix cores, from the dense operands of Phase 1
// ([C][HP] in the workspace, HP a multiple of 16): for hot write group h with reference
// log-decay L_ref (its first member's), token t writing it carries Ka[t][h] = k e^(L-L_ref)
// and Kb[t][h] = k e^(L_ref-L); a token reading it after a write carries Qa[t][h] =
// q e^(Lr-L_ref) (summed over its reads of the slot). Then A += tril(Ka Kb^T, -1) and
// QK += tril(Qa Kb^T): the factored exponents multiply back to the pair decays
// e^(L_t - L_t'). Each wavefront takes lower 16 x 16 tiles of A and QK in turn and
// accumulates them with v_mfma_f32_16x16x4_f32 over h in blocks of 16 ascending (a fixed
// order), operands read straight from memory, then adds them to the cold part.

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Hot tiles t0, t0 + tstep, ... (of the 2 T1 lower tiles of A and QK) of chunk n, one
// wavefront.
__device__ __forceinline__ void hot_tiles(const Problem &pb, const Slab &sl, int64_t n, int t0, int tstep) {
    const ChunkLayout &L = sl.lay;
    uint32_t *cb = sl.chunk(n);
    const int32_t *meta = reinterpret_cast<const int32_t *>(cb + L.off_meta);
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    const int nl = n_live_tokens(pb, p, ti);
    if (nl == 0) return;
    const int nhot = meta[3], HP = meta[5];
    if (nhot == 0) return;
    const int C = pb.C;
    const int nt = (C + 15) / 16, T1 = nt * (nt + 1) / 2;
    const float *Ka = reinterpret_cast<const float *>(cb + L.off_ka);
    const float *Kb = reinterpret_cast<const float *>(cb + L.off_kb);
    const float *Qa = reinterpret_cast<const float *>(cb + L.off_qa);
    float *A = reinterpret_cast<float *>(cb + L.off_A);
    float *QK = reinterpret_cast<float *>(cb + L.off_QK);
    const int lane = threadIdx.x & 63;
    const int ko = 4 * (lane >> 4);
    for (int t = t0; t < 2 * T1; t += tstep) {
        const bool isA = t < T1;
        const int tt = isA ? t : t - T1;
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= tt) ++I;
        const int J = tt - I * (I + 1) / 2;
        const float *Aop = isA ? Ka : Qa;
        const int ra = 16 * I + (lane & 15), rb = 16 * J + (lane & 15);
        f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int hb = 0; hb < HP; hb += 16) {
            float4 av = make_float4(0.0f, 0.0f, 0.0f, 0.0f), bv = av;
            if (ra < C) av = *reinterpret_cast<const float4 *>(Aop + int64_t(ra) * L.HCAP + hb + ko);
            if (rb < C) bv = *reinterpret_cast<const float4 *>(Kb + int64_t(rb) * L.HCAP + hb + ko);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, acc, 0, 0, 0);
        }
        // Add the hot part to the cold part, inside the triangles only (the four cold values
        // loaded before any sum is stored).
        float *M = isA ? A : QK;
        float cold[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * I + 4 * (lane >> 4) + v, c = 16 * J + (lane & 15);
            const bool in = r < C && c < C && (isA ? c < r : c <= r);
            cold[v] = M[in ? int64_t(r) * C + c : 0];
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * I + 4 * (lane >> 4) + v, c = 16 * J + (lane & 15);
            if (r < C && c < C && (isA ? c < r : c <= r)) M[int64_t(r) * C + c] = cold[v] + acc[v];
        }
    }
}

// ---------------------------------------------------------------------------------------
// Kernels: one stage per launch (large chunks), or every stage and the solve in one
// workgroup per chunk (small chunks), so that a small chunk pays one launch instead of six.
// ---------------------------------------------------------------------------------------
// Whether chunk n was handled by the partitioned kernel (phase1_part.hip), which ran first
// in this call and marked the chunks it left to the sorting kernels with meta[7] = 1.
__device__ __forceinline__ bool done_by_part(const Problem &pb, const Slab &sl, int64_t n) {
    return pb.part_on && reinterpret_cast<const int32_t *>(sl.chunk(n) + sl.lay.off_meta)[7] == 0;
}

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void p1_sort_kernel(Problem pb, Slab sl) {
    __shared__ __align__(16) char smem[sort_smem_bytes<BLOCK>()];
    if (done_by_part(pb, sl, blockIdx.x)) return;
    sort_chunk<BLOCK>(pb, sl, blockIdx.x, smem);
}

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void p1_groups_kernel(Problem pb, Slab sl) {
    __shared__ __align__(16) char smem[sizeof(GroupsSmem<BLOCK / kWave>)];
    if (done_by_part(pb, sl, blockIdx.x)) return;
    groups_chunk<BLOCK>(pb, sl, blockIdx.x, smem);
}

__global__ __launch_bounds__(kReadWaves * kWave) void p1_reads_kernel(Problem pb, Slab sl) {
    __shared__ float qrow[kReadWaves][kHotCap];
    if (done_by_part(pb, sl, blockIdx.y)) return;
    const int wave = threadIdx.x >> 6;
    reads_token(pb, sl, blockIdx.y, blockIdx.x * kReadWaves + wave, qrow[wave]);
}

__global__ __launch_bounds__(kColdBlock) void p1_gram_cold_kernel(Problem pb, Slab sl) {
    constexpr int NW = kColdBlock / kWave;
    __shared__ int32_t tcol[NW][kTermCap];
    __shared__ float tval[NW][kTermCap];
    const int wave = threadIdx.x >> 6;
    for (int i = wave; i < pb.C; i += NW) cold_row(pb, sl, blockIdx.x, blockIdx.y != 0, i, tcol[wave], tval[wave]);
}

// The hot pair terms of large chunks, one workgroup per (chunk, matrix): blockIdx.y = 0
// computes A's lower tiles from Ka and Kb, 1 QK's from Qa and Kb. The operands' columns are
// staged in LDS kHotKb at a time, each read once from memory (the next block's loads are in
// flight during this block's products), and each wavefront accumulates its tiles over every
// column block in registers with the MFMA chains of hot_tiles (16 columns at a time, lane
// group l / 16 taking columns 4 (l / 16) .. + 3, h ascending): the same bits. The chains of
// three tiles are interleaved step by step, so that the matrix unit always has an independent
// product to start while a dependent one is in flight.
// Chunks of fewer than kHotLdsMinC tokens have too few tiles for a workgroup per matrix:
// there each wavefront takes tiles straight from memory (hot_tiles), kHotBlock threads per
// workgroup, the tiles of a chunk split over up to eight workgroups. Both give the same bits.
constexpr int kHotBlock = 256;
constexpr int kHotLdsMinC = 128;

__global__ __launch_bounds__(kHotBlock) void p1_gram_hot_tiles_kernel(Problem pb, Slab sl) {
    constexpr int NWAVE = kHotBlock / kWave;
    hot_tiles(pb, sl, blockIdx.x, blockIdx.y * NWAVE + (threadIdx.x >> 6), gridDim.y * NWAVE);
}

constexpr int kHotLdsBlock = 1024;
constexpr int kHotKb = 32;                 // hot columns per staged block
constexpr int kHotPitch = kHotKb + 4;      // LDS row pitch (floats): 16-byte rows 4 banks apart
constexpr int kHotIl = 3;                  // tiles whose MFMA chains interleave
constexpr int kHotMaxT = ((kMaxChunk / 16) * (kMaxChunk / 16 + 1) / 2 + kHotLdsBlock / kWave - 1) / (kHotLdsBlock / kWave);
constexpr int kHotU = (2 * kMaxChunk * (kHotKb / 4) + kHotLdsBlock - 1) / kHotLdsBlock;   // 16-byte units per thread

// Component k (0..3, a constant after unrolling) of a float4.
__device__ __forceinline__ float f4_at(const float4 &v, int k) { return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w; }

size_t hot_lds_bytes(int C) { return size_t(2) * ((C + 15) & ~15) * kHotPitch * sizeof(float); }

__global__ __launch_bounds__(kHotLdsBlock) void p1_gram_hot_kernel(Problem pb, Slab sl) {
    extern __shared__ float hl[];   // [2][CP][kHotPitch]: Kb's staged columns, then Ka's or Qa's
    constexpr int NW = kHotLdsBlock / kWave;
    const int64_t n = blockIdx.x;
    const bool isA = blockIdx.y == 0;
    const ChunkLayout &L = sl.lay;
    uint32_t *cb = sl.chunk(n);
    const int32_t *meta = reinterpret_cast<const int32_t *>(cb + L.off_meta);
    const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
    if (n_live_tokens(pb, p, ti) == 0) return;
    const int nhot = meta[3], HP = meta[5];
    if (nhot == 0) return;
    const int C = pb.C, CP = (C + 15) & ~15, nt = CP / 16, T1 = nt * (nt + 1) / 2;
    const float *Kb = reinterpret_cast<const float *>(cb + L.off_kb);
    const float *Aop = reinterpret_cast<const float *>(cb + (isA ? L.off_ka : L.off_qa));
    float *bl = hl, *al = hl + CP * kHotPitch;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ko = 4 * (lane >> 4);
    const int nq = CP * (kHotKb / 4);   // 16-byte units of one staged operand block

    // unit i: operand i / nq (0 Kb, 1 Ka or Qa), row, column quad; rows past C and
    // columns past HP stage as 0 (loads unconditional, clamped in bounds)
    float4 st[kHotU];
    auto load = [&](int hb) {
        // the thread id re-read opaquely, so that the loads' 64-bit addresses are formed
        // here and not held across the block loop (they would spill)
        int tio = threadIdx.x;
        asm volatile("" : "+v"(tio));
#pragma unroll
        for (int u = 0; u < kHotU; ++u) {
            const int i = tio + u * kHotLdsBlock, w = i / nq, rem = i - w * nq;
            const int r = rem / (kHotKb / 4), col = hb + 4 * (rem % (kHotKb / 4));
            const bool ok = i < 2 * nq && r < C && col < HP;
            const float *src = (w == 0 ? Kb : Aop) + (ok ? int64_t(r) * L.HCAP + col : 0);
            const float4 x = *reinterpret_cast<const float4 *>(src);
            st[u] = ok ? x : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int u = 0; u < kHotU; ++u) {
            const int i = tid + u * kHotLdsBlock, w = i / nq, rem = i - w * nq;
            if (i < 2 * nq)
                *reinterpret_cast<float4 *>(hl + (w * CP + rem / (kHotKb / 4)) * kHotPitch + 4 * (rem % (kHotKb / 4))) =
                    st[u];
        }
    };
    f32x4 acc[kHotMaxT];
#pragma unroll
    for (int q = 0; q < kHotMaxT; ++q) acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // The wavefront's tiles t = wave + q NW: the LDS row offsets of their operands (wave-
    // uniform, held in scalar registers); tiles past the triangle repeat its last tile, whose
    // products are computed and never stored.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int aof[kHotMaxT], bof[kHotMaxT];
#pragma unroll
    for (int q = 0; q < kHotMaxT; ++q) {
        const int t = min(wv + q * NW, T1 - 1);
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= t) ++I;
        const int J = t - I * (I + 1) / 2;
        aof[q] = __builtin_amdgcn_readfirstlane(16 * I * kHotPitch);
        bof[q] = __builtin_amdgcn_readfirstlane(16 * J * kHotPitch);
    }
    const int lof = (lane & 15) * kHotPitch + ko;
    const int ntw = wv < T1 ? (T1 - wv + NW - 1) / NW : 0;
    load(0);
    for (int hb = 0; hb < HP; hb += kHotKb) {
        __syncthreads();   // the previous block's products are done with the LDS
        store();
        __syncthreads();
        if (hb + kHotKb < HP) load(hb + kHotKb);
        const int nsb = min(kHotKb, HP - hb) / 16;   // 16-column sub-blocks (HP is a multiple of 16)
        // kHotIl tiles at a time, their MFMA chains interleaved step by step: each tile's
        // chain is the same (sub-blocks ascending, four k-steps each), so are the bits
        for (int sb = 0; sb < nsb; ++sb) {
#pragma unroll
            for (int q0 = 0; q0 < kHotMaxT; q0 += kHotIl) {
                if (q0 >= ntw) break;
                float4 av[kHotIl], bv[kHotIl];
#pragma unroll
                for (int j = 0; j < kHotIl; ++j) {
                    const int q = q0 + j < kHotMaxT ? q0 + j : kHotMaxT - 1;
                    av[j] = *reinterpret_cast<const float4 *>(al + lof + aof[q] + 16 * sb);
                    bv[j] = *reinterpret_cast<const float4 *>(bl + lof + bof[q] + 16 * sb);
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int j = 0; j < kHotIl; ++j)
                        if (q0 + j < kHotMaxT)
                            acc[q0 + j] = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(av[j], kk), f4_at(bv[j], kk),
                                                                              acc[q0 + j], 0, 0, 0);
            }
        }
    }
    // Add the hot part to the cold part, inside the triangle only: every element's cold
    // value is loaded before any sum is stored (the compiler cannot tell that the elements
    // differ, and would otherwise wait for each load in turn)
    float *M = reinterpret_cast<float *>(cb + (isA ? L.off_A : L.off_QK));
    int32_t at_[kHotMaxT][4];
    float cold[kHotMaxT][4];
#pragma unroll
    for (int q = 0; q < kHotMaxT; ++q) {
        const int t = wave + q * NW;
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= t) ++I;
        const int J = t - I * (I + 1) / 2;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * I + 4 * (lane >> 4) + v, c = 16 * J + (lane & 15);
            const bool in = t < T1 && r < C && c < C && (isA ? c < r : c <= r);
            at_[q][v] = in ? r * C + c : -1;
            cold[q][v] = M[in ? r * C + c : 0];
        }
    }
#pragma unroll
    for (int q = 0; q < kHotMaxT; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            if (at_[q][v] >= 0) M[at_[q][v]] = cold[q][v] + acc[q][v];
}

constexpr int kFusedBlock = 1024;
constexpr int kFusedMaxEntries = 1024;   // write and read entries per chunk of the fused path
// the cold pass's term lists: two kTermCap arrays per wavefront
constexpr int kColdTermBytes = (kFusedBlock / kWave) * 2 * kTermCap * 4;
// the read pass's dense hot rows: kHotCap floats per wavefront
constexpr int kReadRowBytes = (kFusedBlock / kWave) * kHotCap * 4;

__global__ __launch_bounds__(kFusedBlock) void p1_fused_kernel(Problem pb, Slab sl, WyArgs wa) {
    extern __shared__ __align__(16) char fsm[];
    constexpr int NW = kFusedBlock / kWave;
    const int64_t n = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    sort_chunk<kFusedBlock>(pb, sl, n, fsm);
    __syncthreads();
    groups_chunk<kFusedBlock>(pb, sl, n, fsm);
    __syncthreads();
    {
        // The read lookups probe LDS copies of the sorted member records, the lookup records
        // and the bucket starts: one coalesced sweep instead of dependent memory round trips.
        const ChunkLayout &L = sl.lay;
        const uint32_t *cb = sl.chunk(n);
        int4 *lspk = reinterpret_cast<int4 *>(fsm + kReadRowBytes);
        int4 *lsgh = lspk + L.E;
        int32_t *lbst = reinterpret_cast<int32_t *>(lsgh + L.E);
        const int4 *gspk = reinterpret_cast<const int4 *>(cb + L.off_spk);
        const int4 *gsgh = reinterpret_cast<const int4 *>(cb + L.off_sgh);
        const int32_t *gbst = reinterpret_cast<const int32_t *>(cb + L.off_bstart);
        for (int e = threadIdx.x; e < L.E; e += kFusedBlock) {
            lspk[e] = gspk[e];
            lsgh[e] = gsgh[e];
        }
        for (int b = threadIdx.x; b <= L.NB; b += kFusedBlock) lbst[b] = gbst[b];
        int32_t *lqid = lbst + L.NB + 1;
        float *lqv = reinterpret_cast<float *>(lqid + L.F);
        {
            const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
            const int nlr = n_live_tokens(pb, p, ti) * pb.R;   // read entries of live tokens
            const int64_t q0 = (int64_t(p) * pb.T + int64_t(ti) * pb.C) * pb.R;
            for (int e = threadIdx.x; e < nlr; e += kFusedBlock) {
                lqid[e] = load_id(pb.q_idx, q0 + e, pb.q_id8);
                lqv[e] = load_weight(pb.q_val, q0 + e, pb.dtype);
            }
        }
        __syncthreads();
        float *qr = reinterpret_cast<float *>(fsm) + wave * kHotCap;
        for (int i = wave; i < pb.C; i += NW) reads_token(pb, sl, n, i, qr, lspk, lsgh, lbst, lqid, lqv);
    }
    __syncthreads();
    {
        // The cold pass reads its inputs (sorted member records, cold write and read records)
        // from LDS: one coalesced sweep instead of dependent memory round trips per row.
        const ChunkLayout &L = sl.lay;
        const uint32_t *cb = sl.chunk(n);
        int4 *lspk = reinterpret_cast<int4 *>(fsm + kColdTermBytes);
        int4 *lecr = lspk + L.E, *lrcr = lecr + L.E;
        const int4 *gspk = reinterpret_cast<const int4 *>(cb + L.off_spk);
        const int4 *gecr = reinterpret_cast<const int4 *>(cb + L.off_ecr);
        const int4 *grcr = reinterpret_cast<const int4 *>(cb + L.off_rcr);
        for (int e = threadIdx.x; e < L.E; e += kFusedBlock) {
            lspk[e] = gspk[e];
            lecr[e] = gecr[e];
        }
        for (int e = threadIdx.x; e < L.F; e += kFusedBlock) lrcr[e] = grcr[e];
        __syncthreads();
        const int p = int(n / sl.steps), ti = sl.ti0 + int(n % sl.steps);
        const int nl = n_live_tokens(pb, p, ti);
        float *A = reinterpret_cast<float *>(sl.chunk(n) + L.off_A);
        float *QK = reinterpret_cast<float *>(sl.chunk(n) + L.off_QK);
        int32_t *mcol = reinterpret_cast<int32_t *>(fsm) + wave * 2 * kTermCap;
        float *mval = reinterpret_cast<float *>(mcol + kTermCap);
        for (int k = wave; k < 2 * pb.C; k += NW) {
            const bool qk = k >= pb.C;
            cold_row_at(pb.C, nl, lspk, qk ? lrcr : lecr, qk ? QK : A, qk ? pb.R : pb.W, qk ? k - pb.C : k, mcol, mval);
        }
    }
    __syncthreads();
    hot_tiles(pb, sl, n, wave, NW);
    __syncthreads();
    wy_chunk<kFusedBlock>(wa, n, reinterpret_cast<float *>(fsm));
}

static size_t fused_smem_bytes(int C) {
    size_t b = sort_smem_bytes<kFusedBlock>();
    b = std::max(b, sizeof(GroupsSmem<kFusedBlock / kWave>));
    // read pass: hot rows, then the staged records (E <= kFusedMaxEntries, NB + 1 <= 1025)
    // and read ids and weights (F <= kFusedMaxEntries)
    b = std::max(b, size_t(kReadRowBytes) + 32 * size_t(kFusedMaxEntries) + 4 * size_t(kFusedMaxEntries + 1) +
                        8 * size_t(kFusedMaxEntries));
    b = std::max(b, size_t(kColdTermBytes) + 16 * size_t(2 * kFusedMaxEntries + kFusedMaxEntries));
    return std::max(b, wy_lds_bytes(C));
}

// Whether a chunk's Phase 1 and solve run fused: small chunks (E, F <= 1024) whose stages
// fit the device's LDS. SDM_P1_FUSED=0 turns it off, for sweeps and tests.
bool phase1_fused(const ChunkLayout &L, int C, int lds_limit) {
    // the fused cold pass stages at most kFusedMaxEntries write and read records in LDS
    if (fused_smem_bytes(C) > size_t(lds_limit) || L.E > kFusedMaxEntries || L.F > kFusedMaxEntries) return false;
    const char *env = getenv("SDM_P1_FUSED");
    return !(env && env[0] == '0');
}

// ---------------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------------
constexpr int kSortBlock = 1024;
constexpr int kGroupBlock = 1024;

size_t gram_lds_bytes(int) { return 0; }   // the cold Gram uses static LDS only


hipError_t phase1_prepare() {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&p1_fused_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(fused_smem_bytes(kMaxChunk)));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&p1_gram_hot_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(hot_lds_bytes(kMaxChunk)));
}

hipError_t launch_phase1_part(const Problem &pb, const Slab &sl, int lognp, hipStream_t st);

// ev: nullptr, or 5 events recorded before each of the five kernels (fused: the first
// before the fused kernel, the other four after it; partitioned: the first before the
// partitioned kernel, whose time counts with the sort's). fused: Phase 1 and the solve in
// one kernel (wa: the solve's arguments); otherwise the caller launches the solve.
// lognp >= 0 (with pb.part_on): the partitioned kernel runs first with 2^lognp partitions.
hipError_t launch_phase1(const Problem &pb, const Slab &sl, hipStream_t st, hipEvent_t *ev, bool fused,
                         const WyArgs &wa, int lognp) {
    const unsigned nch = unsigned(int64_t(pb.P) * sl.steps);
    hipError_t e;
    if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
    if (fused) {
        hipLaunchKernelGGL(p1_fused_kernel, dim3(nch), dim3(kFusedBlock), fused_smem_bytes(pb.C), st, pb, sl, wa);
        for (int k = 1; ev && k < 5; ++k)
            if ((e = hipEventRecord(ev[k], st)) != hipSuccess) return e;
        return hipGetLastError();
    }
    if (pb.part_on) {
        if ((e = launch_phase1_part(pb, sl, lognp, st)) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(p1_sort_kernel<kSortBlock>, dim3(nch), dim3(kSortBlock), 0, st, pb, sl);
    if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
    hipLaunchKernelGGL(p1_groups_kernel<kGroupBlock>, dim3(nch), dim3(kGroupBlock), 0, st, pb, sl);
    if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
    hipLaunchKernelGGL(p1_reads_kernel, dim3(unsigned((pb.C + kReadWaves - 1) / kReadWaves), nch),
                       dim3(kReadWaves * kWave), 0, st, pb, sl);
    if (ev && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
    hipLaunchKernelGGL(p1_gram_cold_kernel, dim3(nch, 2), dim3(kColdBlock), 0, st, pb, sl);
    if (ev && (e = hipEventRecord(ev[4], st)) != hipSuccess) return e;
    // SDM_P1_HOT_LDS=1 / 0 takes the staged / the per-tile kernel whatever the chunk (tests)
    const char *hot_env = getenv("SDM_P1_HOT_LDS");
    const bool hot_lds = hot_env ? hot_env[0] == '1' : pb.C >= kHotLdsMinC;
    if (hot_lds) {
        hipLaunchKernelGGL(p1_gram_hot_kernel, dim3(nch, 2), dim3(kHotLdsBlock), hot_lds_bytes(pb.C), st, pb, sl);
    } else {
        // tiles of A and QK split over enough workgroups per chunk to fill the device
        const int nt = (pb.C + 15) / 16, tiles = nt * (nt + 1);
        const unsigned gy = unsigned(min(8, max(1, tiles / (2 * (kHotBlock / kWave)))));
        hipLaunchKernelGGL(p1_gram_hot_tiles_kernel, dim3(nch, gy), dim3(kHotBlock), 0, st, pb, sl);
    }
    return hipGetLastError();
}

}  // namespace sdm

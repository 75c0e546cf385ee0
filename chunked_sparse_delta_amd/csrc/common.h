// Internal definitions shared by the SDM kernels and the C-ABI host code (gfx950).
#pragma once

#include <cstdlib>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {

constexpr int kWave = 64;          // CDNA4 wavefront
constexpr int kMaxChunk = 256;
constexpr int kMaxWidth = 256;
constexpr int kXcds = 8;           // MI355X: 8 XCDs of 32 CUs, workgroups dealt round-robin
constexpr int kHotMin = 16;        // write groups of at least this many members go to the dense Gram
constexpr float kHotSpan = 60.0f;  // ... if their log-decays stay within this of the first member's
constexpr int kHotCap = 512;       // at most this many hot groups per chunk (the rest stay cold)

// ---------------------------------------------------------------------------------------
// Element types. bf16 is carried as its 16-bit pattern.
// ---------------------------------------------------------------------------------------
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return __uint_as_float(uint32_t(x.bits) << 16); }

// Two floats -> two bf16 (low half first), round to nearest even, a NaN quieted (its top
// 16 bits with the quiet bit set): gfx950's packed conversion instruction, one per pair.
// Its result equals the integer rule (u + 0x7FFF + ((u >> 16) & 1)) >> 16 for every
// non-NaN input, denormals included, and (u >> 16) | 0x40 for every NaN.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// float -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
    bf16 r;
    r.bits = uint16_t(f32x2_to_bf16x2(f, 0.0f));
    return r;
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return f32_to_bf16(x); }

// A vector of V elements of T moved as one load/store (V * sizeof(T) is 16 B on the
// vector path, or one element on the scalar path for rows that are not 16 B multiples).
template <typename T, int V> struct Vec;

template <> struct Vec<float, 4> {
    using raw_t = float4;
    static __device__ __forceinline__ raw_t load_raw(const float *p) { return *reinterpret_cast<const float4 *>(p); }
    static __device__ __forceinline__ void unpack(const raw_t &x, float (&o)[4]) {
        o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    }
    static __device__ __forceinline__ void load(const float *p, float (&o)[4]) {
        float4 x = *reinterpret_cast<const float4 *>(p);
        o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    }
    static __device__ __forceinline__ void store(float *p, const float (&o)[4]) {
        *reinterpret_cast<float4 *>(p) = make_float4(o[0], o[1], o[2], o[3]);
    }
    // the same with the non-temporal hint (the line is not kept for reuse)
    static __device__ __forceinline__ raw_t load_raw_nt(const float *p) {
        typedef float f4_t __attribute__((ext_vector_type(4)));
        const f4_t x = __builtin_nontemporal_load(reinterpret_cast<const f4_t *>(p));
        return make_float4(x[0], x[1], x[2], x[3]);
    }
    static __device__ __forceinline__ void store_nt(float *p, const float (&o)[4]) {
        typedef float f4_t __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(f4_t{o[0], o[1], o[2], o[3]}, reinterpret_cast<f4_t *>(p));
    }
};
template <> struct Vec<bf16, 8> {
    using raw_t = uint4;
    static __device__ __forceinline__ raw_t load_raw(const bf16 *p) { return *reinterpret_cast<const uint4 *>(p); }
    static __device__ __forceinline__ void unpack(const raw_t &x, float (&o)[8]) {
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
    static __device__ __forceinline__ void load(const bf16 *p, float (&o)[8]) {
        uint4 x = *reinterpret_cast<const uint4 *>(p);
        uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
    static __device__ __forceinline__ void store(bf16 *p, const float (&o)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = f32x2_to_bf16x2(o[2 * i], o[2 * i + 1]);
        *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    // the same with the non-temporal hint (the line is not kept for reuse)
    static __device__ __forceinline__ raw_t load_raw_nt(const bf16 *p) {
        typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
        const u4_t x = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(p));
        return make_uint4(x[0], x[1], x[2], x[3]);
    }
    static __device__ __forceinline__ void store_nt(bf16 *p, const float (&o)[8]) {
        typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
        u4_t w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = f32x2_to_bf16x2(o[2 * i], o[2 * i + 1]);
        __builtin_nontemporal_store(w, reinterpret_cast<u4_t *>(p));
    }
};
// Four bfloat16 columns (8 bytes): the narrow slices of a resident bank (see plan_phase2).
template <> struct Vec<bf16, 4> {
    using raw_t = uint2;
    static __device__ __forceinline__ raw_t load_raw(const bf16 *p) { return *reinterpret_cast<const uint2 *>(p); }
    static __device__ __forceinline__ void unpack(const raw_t &x, float (&o)[4]) {
        o[0] = __uint_as_float(x.x << 16);
        o[1] = __uint_as_float(x.x & 0xFFFF0000u);
        o[2] = __uint_as_float(x.y << 16);
        o[3] = __uint_as_float(x.y & 0xFFFF0000u);
    }
    static __device__ __forceinline__ void load(const bf16 *p, float (&o)[4]) { unpack(load_raw(p), o); }
    static __device__ __forceinline__ void store(bf16 *p, const float (&o)[4]) {
        const uint32_t w0 = f32x2_to_bf16x2(o[0], o[1]);
        const uint32_t w1 = f32x2_to_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2 *>(p) = make_uint2(w0, w1);
    }
};
template <typename T> struct Vec<T, 1> {
    using raw_t = T;
    static __device__ __forceinline__ raw_t load_raw(const T *p) { return *p; }
    static __device__ __forceinline__ void unpack(const raw_t &x, float (&o)[1]) { o[0] = to_f32(x); }
    static __device__ __forceinline__ void load(const T *p, float (&o)[1]) { o[0] = to_f32(*p); }
    static __device__ __forceinline__ void store(T *p, const float (&o)[1]) { *p = from_f32<T>(o[0]); }
};

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (uint64_t(1) << lane) - 1; }

// Bit 30 of a slot id in a chunk's id copies (ids stay below 2^30: the host refuses a stream
// bank of 2 GiB or more): the partitioned Phase 1 sets it where no other entry of the chunk
// has the slot, and Phase 2 streams that row with the non-temporal hint on large workloads.
constexpr int32_t kIdOnce = 1 << 30;
constexpr int32_t kIdMask = kIdOnce - 1;

// The lanes of the wavefront whose digit (db low bits of d) equals this lane's, among the
// lanes with ok set: one ballot per digit bit.
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool ok, int db) {
    uint64_t peers = __ballot(ok);
    for (int b = 0; b < db; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t bb = __ballot(bit);
        peers &= bit ? bb : ~bb;
    }
    return peers;
}

// ---------------------------------------------------------------------------------------
// Problem description passed by value to every kernel.
// ---------------------------------------------------------------------------------------
struct Problem {
    int32_t P, T, C, Nt, W, R, G, hd;
    int64_t M;
    int32_t dtype;           // 0 f32, 1 bf16
    int32_t sort_passes;     // LSD radix passes over the slot id ...
    int32_t sort_digit;      // ... of this many bits each (the last one may use fewer)
    int32_t key_bits;        // bits of the largest slot id (M - 1)
    const void *k_idx;       // [P, T, W] int32, or int64 when k_id8
    const void *q_idx;       // [P, T, R] int32, or int64 when q_id8
    int32_t k_id8, q_id8;
    const void *k_val;       // [P, T, W] bank dtype
    const void *q_val;       // [P, T, R] bank dtype
    const float *beta;       // [P, T]
    const float *g;          // [P, T, G]
    const void *v;           // [P, T, hd]
    const int32_t *valid;    // [P] or nullptr
    void *bank;              // [P, M, hd], or one shared [M, hd]
    int64_t bank_stride;     // elements from one stream's bank to the next (0: shared bank)
    void *out;               // [P, T, hd]
    unsigned long long *repeats;   // optional device counter of repeated write slots
    int32_t part_on;         // Phase 1 of this call runs the partitioned kernel first: the sorting
                             // kernels then handle only the chunks it left to them (meta[7] = 1)
};

// Whether rows that one entry of a chunk alone reads are streamed with the non-temporal hint
// (the partitioned Phase 1 marks their ids with kIdOnce, the Phase-2 gather of a bank in
// memory loads them so): when a step's rows, P C (W + R) of head_dim columns, exceed the
// memory-side cache; beyond it their kept lines only displace rows the gather reuses, below
// it keeping every line measured faster. SDM_P2_NT = 0 / 1 turns it off / on whatever the
// shapes (tests: the bits are the same either way).
constexpr int64_t kMallBytes = int64_t(256) << 20;   // MI355X's memory-side (Infinity) cache
inline bool once_rows_streamed(const Problem &pb) {
    const char *e = getenv("SDM_P2_NT");
    if (e) return e[0] == '1';
    const double b = double(pb.P) * pb.C * (pb.W + pb.R) * pb.hd * (pb.dtype == 0 ? 4 : 2);
    return b > double(kMallBytes);
}

// Slot id i of an int32 or int64 id array (ids of valid calls lie in [0, M), M < 2^31): one
// 32-bit load either way (an int64 id's low word), with no branch on the width, so that
// loads of several ids issue back to back.
__device__ __forceinline__ int32_t load_id(const void *base, int64_t i, int32_t id8) {
    return *reinterpret_cast<const int32_t *>(static_cast<const char *>(base) + (id8 ? 8 * i : 4 * i));
}

__device__ __forceinline__ int32_t n_live_tokens(const Problem &pb, int p, int ti) {
    int32_t vt = pb.valid ? pb.valid[p] : pb.T;
    vt = vt < 0 ? 0 : (vt > pb.T ? pb.T : vt);
    int32_t n = vt - ti * pb.C;
    return n < 0 ? 0 : (n > pb.C ? pb.C : n);
}

// Element i of a float32 (dtype 0) or bfloat16 array as a float, from one aligned 32-bit load
// with no branch on the dtype (a bfloat16 is the half of its aligned word at its address;
// the word lies inside the element's 4-byte aligned page-internal span, so it is mapped).
__device__ __forceinline__ float load_weight(const void *base, int64_t i, int32_t dtype) {
    // the address stays derived from base (a global load, not a flat one)
    const char *b = static_cast<const char *>(base);
    const int64_t off = dtype ? 2 * i : 4 * i;
    const int mis = int((reinterpret_cast<uintptr_t>(b) + uintptr_t(off)) & 2);
    const uint32_t w = *reinterpret_cast<const uint32_t *>(b + (off - mis));
    return dtype ? __uint_as_float(mis ? (w & 0xFFFF0000u) : (w << 16)) : __uint_as_float(w);
}

// ---------------------------------------------------------------------------------------
// Workspace of one slab: `nchunks` chunks, chunk n = p * slab_steps + (ti - ti0).
// Every array is 256-byte aligned. E = C * W write entries, F = C * R read entries.
// "Sorted position" m indexes the chunk's write entries sorted by (slot, token); the
// entries of one slot form a contiguous write group, members in token order.
// Transposed per-entry arrays hold entry (token i, slot index x) at x * C + i, so that
// threads owning consecutive tokens read consecutive records.
// ---------------------------------------------------------------------------------------
struct ChunkLayout {
    int64_t E, F, C2, NB, HMAX, HCAP;
    // per-chunk strides (elements)
    int64_t off_key0, off_val0, off_key1, off_val1;   // radix-sort double buffer (u32)
    int64_t off_spk;      // [E] int4 per sorted position: {slot, token, bits k, bits L}
    int64_t off_shead;    // [E] i32: first sorted position of the group
    int64_t off_sgrp;     // [E] i32: group of sorted position
    int64_t off_gpos;     // [E+1] i32: group start positions
    int64_t off_grec;     // [E] int4: DW group record {slot, first position | (members - 1) << 16 |
                          //   first member's token << 24, bits of exp(L_last), bits of the first member's
                          //   k exp(L_last - L)}
    int64_t off_mrec;     // [E] int2: DW member record {token, bits of k exp(L_last - L)}
    int64_t off_gw;       // [E] f32: gather weight k exp(L), entry order
    int64_t off_kid;      // [E] i32: write slot ids of the chunk, entry order (copy of the input)
    int64_t off_ecr;      // [C][W] int4: cold write entry {a, m, bits k, bits L} (a == m: none)
    int64_t off_sgh;      // [E] int4 per sorted position: {group head, hot index or -1, bits of the head's L if hot, 0}
    int64_t off_ghot;     // [E] i32: hot index of group, or -1
    int64_t off_hgrp;     // [HMAX] i32: group of hot index
    int64_t off_brec;     // [HMAX] int4: DW group records of the groups with >= kHotMin members
    int64_t off_bstart;   // [NB+1] i32: first sorted position of each slot bucket
    int64_t off_gr;       // [F] f32: gather weight q exp(Lr), read-entry order
    int64_t off_qid;      // [F] i32: read slot ids of the chunk, entry order (copy of the input)
    int64_t off_rcr;      // [C][R] int4: cold read {a, end, bits q, bits Lr} (a == end: none)
    int64_t off_ka;       // [C][HCAP] f32: token t's write of hot group h (< HP = meta[5]), k exp(L - L_ref)
    int64_t off_kb;       // [C][HCAP] f32: the same write's k exp(L_ref - L)
    int64_t off_qa;       // [C][HCAP] f32: token t's reads of hot group h, sum of q exp(Lr - L_ref) in read order
    int64_t off_plist;    // [E + F] int4: the partitioned path's slot-partition lists {slot, code, bits of k
                          //   or q, bits of g}, then the entries' output records in the same slots
    int64_t off_oval;     // [E + F] u32: the partitioned path's gather weight of each list slot
    int64_t off_inv;      // [E + F] i32: list slot of each entry (token-major, a token's writes then reads);
                          //   these three share their words with the arrays only the sorting path uses
    int64_t off_meta;     // [64] i32: n_live, E_live, ngroups, hot groups, groups with >= kHotMin members,
                          //   HP (hot groups rounded up to 16), -, 1 if the chunk took the sorting path;
                          //   [8 + 2 slice], [9 + 2 slice]: the Phase-2 team words of each column slice
                          //   (gather pieces, then DW pieces: claim and done bits), zeroed by Phase 1
    int64_t off_xu;       // [S][2][C][CW] f32: Phase-2 teams' exchange, per column slice of CW columns:
                          //   u of every token, then inter; S * CW <= head_dim rounded up to 64
    int64_t off_beta;     // [C] f32: beta (0 for padding)
    int64_t off_A, off_QK, off_X, off_QX;   // [C, C] f32
    // [stage0, stage1): every array Phase 2 reads (records, weights, ids, meta, beta, X, QX),
    // contiguous, so that small chunks can be copied into LDS whole
    int64_t off_stage0, off_stage1;
    int64_t words;        // 4-byte words per chunk
};

inline int64_t align_words(int64_t w) { return (w + 63) & ~int64_t(63); }   // 256 B

// Number of slot buckets of the search index of a chunk of E write entries: about one
// bucket per entry, at most 2^14.
__host__ __device__ inline int bucket_bits(int64_t E) {
    int b = 1;
    while (b < 14 && (int64_t(1) << b) < E) ++b;
    return b;
}

constexpr int kTeamMaxSlices = 28;   // column slices with team words in a chunk's meta (8 + 2 x 28 = 64)

inline ChunkLayout make_layout(int C, int W, int R, int hd) {
    ChunkLayout L{};
    L.E = int64_t(C) * W;
    L.F = int64_t(C) * R;
    L.C2 = int64_t(C) * C;
    L.NB = int64_t(1) << bucket_bits(L.E);
    L.HMAX = L.E / kHotMin + 1;
    L.HCAP = ((L.HMAX + 15) / 16) * 16 < kHotCap ? ((L.HMAX + 15) / 16) * 16 : kHotCap;
    int64_t o = 0;
    auto take = [&](int64_t n) { int64_t r = o; o += align_words(n); return r; };
    // the arrays only the sorting path uses, then (in the same words) the partition lists
    // of the partitioned path: a chunk takes one path or the other
    L.off_key0 = take(L.E);
    L.off_val0 = take(L.E);
    L.off_key1 = take(L.E);
    L.off_val1 = take(L.E);
    L.off_shead = take(L.E);
    L.off_sgrp = take(L.E);
    L.off_gpos = take(L.E + 1);
    L.off_sgh = take(4 * L.E);
    L.off_ghot = take(L.E);
    L.off_hgrp = take(L.HMAX);
    L.off_bstart = take(L.NB + 1);
    L.off_plist = 0;
    L.off_oval = align_words(4 * (L.E + L.F));
    L.off_inv = L.off_oval + align_words(L.E + L.F);
    if (o < L.off_inv + align_words(L.E + L.F)) o = L.off_inv + align_words(L.E + L.F);
    L.off_spk = take(4 * L.E);
    L.off_ecr = take(4 * L.E);
    L.off_rcr = take(4 * L.F);
    L.off_ka = take(int64_t(C) * L.HCAP);
    L.off_kb = take(int64_t(C) * L.HCAP);
    L.off_qa = take(int64_t(C) * L.HCAP);
    L.off_A = take(L.C2);
    L.off_QK = take(L.C2);
    L.off_stage0 = o;
    L.off_grec = take(4 * L.E);
    L.off_mrec = take(2 * L.E);
    L.off_brec = take(4 * L.HMAX);
    L.off_gw = take(L.E);
    L.off_gr = take(L.F);
    L.off_kid = take(L.E);
    L.off_qid = take(L.F);
    L.off_meta = take(64);
    L.off_beta = take(C);
    L.off_X = take(L.C2);
    L.off_QX = take(L.C2);
    L.off_stage1 = o;
    L.off_xu = take(2 * int64_t(C) * ((hd + 63) / 64) * 64);
    L.words = o;
    return L;
}

// Phase-2 launch geometry: vectors per column slice, slices per row, and the mode: 0 all
// from memory, 1 the chunk's Phase-2 block staged in LDS, 2 staged and the bank slice
// resident in LDS; team: workgroups per (stream, slice) (1: one; 2 or 4 share its tokens,
// memory mode only).
struct P2Geom {
    int nv, S;
    int mode;
    int team;
};

struct Slab {
    int32_t ti0;        // first step of the slab
    int32_t steps;      // steps in the slab
    uint32_t *ws;       // workspace base
    ChunkLayout lay;
    // Chunk pointer helpers
    __host__ __device__ uint32_t *chunk(int64_t n) const { return ws + n * lay.words; }
};

}  // namespace sdm

// routing.h -- top-k ranking of one token by one wave, and bucketing of the
// (token, slot) pairs by expert inside one workgroup (the routing launch, or
// every gate/up workgroup of a batch of a few tokens).
//
// Ranking: experts ordered by (logit descending, index ascending); ids are the
// first k in that order; p = softmax over all experts; w_j = p_j / sum_j p_j.
// The pages print no routing formula; this is the plain reading of "softmax,
// top-k, renormalise" with exact ties going to the lower expert index.
#pragma once

#include "device.h"
#include "internal.h"

namespace moeffn {

struct RouteOut {
    int *ids;        // [k]
    float *w;        // [k]
    float *gate;     // [1] sigmoid(logit of the gate vector)
    int32_t *dbg_ids;
    float *dbg_w, *dbg_gate, *dbg_logits;
};

// Order-preserving 32-bit key of a logit: larger logit <=> larger key; -0 is
// read as +0 so that the two zeros tie like they compare.
__device__ __forceinline__ uint32_t logit_key(float v) {
    const uint32_t b = __float_as_uint(v == 0.f ? 0.f : v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Largest value over the wave, in every lane, in vector registers only (no round
// trip through scalar registers): a butterfly inside each row of 16 lanes (DPP),
// then the rows combined by swapping the two halves of the wave and then
// neighbouring rows (gfx950 permlane swaps), taking the max of each lane's value
// and the swapped one.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    // update_dpp with bound_ctrl lets the compiler fold each move into the max (v_max_u32_dpp)
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor1, 0xf, 0xf, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor2, 0xf, 0xf, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppHalfMirror, 0xf, 0xf, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppMirror, 0xf, 0xf, true));
    const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = max((uint32_t)a[0], (uint32_t)a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max((uint32_t)b[0], (uint32_t)b[1]);
}

// The logit of a key (the inverse of logit_key; a -0 logit comes back as +0, which
// gives the same weights).
__device__ __forceinline__ float key_logit(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Orders two (key, index) slots of a lane: larger key first, and among equal keys
// the lower expert index first.
__device__ __forceinline__ void slot_order(uint32_t &ka, uint32_t &ia, uint32_t &kb, uint32_t &ib) {
    const bool swap = kb > ka || (kb == ka && ib < ia);
    const uint32_t k0 = swap ? kb : ka, k1 = swap ? ka : kb;
    const uint32_t i0 = swap ? ib : ia, i1 = swap ? ia : ib;
    ka = k0; kb = k1; ia = i0; ib = i1;
}

// One wave ranks one token.  lg: the token's logits row (16-byte aligned, E router
// logits, the shared-gate logit at column E).  Expert e = lane * EPL + i starts in
// register slot i of its lane; each lane first sorts its EPL slots (key descending,
// index ascending), so its head is its best remaining expert.  The k picks are then
// taken one per round in rank order: the largest head over the wave, and among equal
// heads the lowest lane (lanes hold ascending index ranges, so that is the lowest
// expert index); the winning lane pops its head and lane r keeps pick r.  Keys of
// real logits are at least 1 (0 marks an empty slot), so the picks are k distinct
// experts whatever the logits hold.
// Weights: p_e = exp(l_e - max l) / sum_all exp(.) renormalised over the picks
// is w_j = exp(l_j - m) / sum_picks exp(l_i - m) for any m (the full sum
// cancels); m = the first pick, the largest logit.
// The ranking of one token by one wave in phases, so that a caller can act on the
// first picks before the last are known: begin (keys and the in-lane sort), rounds
// [r0, r1) (pick r in lane r), finish (weights, gate and outputs).
template <int EPL>
struct TokenRank {
    uint32_t key[EPL], idx[EPL];
    uint32_t my_id = 0, my_key = 0;
    float glog = 0.f;

    __device__ __forceinline__ void begin(const float *lg, int E, int lane) {
        if constexpr (EPL % 4 == 0) {
            // whole 16-byte groups: a group that starts below E lies inside the padded row
#pragma unroll
            for (int v = 0; v < EPL / 4; ++v) {
                const int e0 = lane * EPL + 4 * v;
                const float4 f = e0 < E ? *reinterpret_cast<const float4 *>(lg + e0) : make_float4(0.f, 0.f, 0.f, 0.f);
                const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) key[4 * v + q] = e0 + q < E ? max(logit_key(fv[q]), 1u) : 0u;
            }
        } else {
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane * EPL + i;
                key[i] = e < E ? max(logit_key(lg[e]), 1u) : 0u;
            }
        }
        glog = lg[E];
#pragma unroll
        for (int i = 0; i < EPL; ++i) idx[i] = (uint32_t)(lane * EPL + i);
        // in-lane sort: odd-even transposition, EPL rounds
#pragma unroll
        for (int r = 0; r < EPL; ++r)
#pragma unroll
            for (int i = r & 1; i + 1 < EPL; i += 2) slot_order(key[i], idx[i], key[i + 1], idx[i + 1]);
    }

    __device__ __forceinline__ void rounds(int r0, int r1, int lane) {
        for (int r = r0; r < r1; ++r) {
            const uint32_t M = wave_max_u32(key[0]);
            const unsigned long long hit = __ballot(key[0] == M);
            const int wl = (int)__builtin_ctzll(hit);
            const uint32_t win = (uint32_t)__builtin_amdgcn_readlane((int)idx[0], wl);
            if (lane == wl) {
#pragma unroll
                for (int i = 0; i + 1 < EPL; ++i) { key[i] = key[i + 1]; idx[i] = idx[i + 1]; }
                key[EPL - 1] = 0u;
            }
            if (lane == r) { my_id = win; my_key = M; }
        }
    }

    __device__ __forceinline__ void finish(const float *lg, int E, int k, int lane, const RouteOut &o) {
        const float my_v = key_logit(my_key);
        const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
        const float myp = lane < k ? expf(my_v - m) : 0.f;
        const float psum = seg_sum<64>(myp);
        if (lane < k) {
            const float w = myp / psum;
            o.ids[lane] = (int)my_id;
            o.w[lane] = w;
            if (o.dbg_ids) o.dbg_ids[lane] = (int)my_id;
            if (o.dbg_w) o.dbg_w[lane] = w;
        }
        if (lane == 0) {
            const float s = sigmoid_f(glog);
            o.gate[0] = s;
            if (o.dbg_gate) o.dbg_gate[0] = s;
        }
        if (o.dbg_logits)
            for (int e = lane; e < E; e += 64) o.dbg_logits[e] = lg[e];
    }
};

template <int EPL>
__device__ void route_token(const float *lg, int E, int k, int lane, const RouteOut &o) {
    TokenRank<EPL> st;
    st.begin(lg, E, lane);
    st.rounds(0, k, lane);
    st.finish(lg, E, k, lane, o);
}

__device__ __forceinline__ void route_token_any(const float *lg, int E, int k, int lane, const RouteOut &o) {
    const int epl = (E + 63) / 64;
    if (epl <= 1) route_token<1>(lg, E, k, lane, o);
    else if (epl <= 2) route_token<2>(lg, E, k, lane, o);
    else if (epl <= 4) route_token<4>(lg, E, k, lane, o);
    else route_token<8>(lg, E, k, lane, o);
}

// LDS ints the bucketing needs for E experts, T tokens and k picks a token: token
// bitmaps [E][ceil(T/32)], counts [E], positions [E], wave totals [32], first pairs [E],
// first-appearance bits [ceil(T*k/32)].
__host__ __device__ inline int bucket_scratch_ints(int E, int T, int k) {
    return E * ((T + 31) / 32) + 3 * E + 2 * 16 + (T * k + 31) / 32 + 16;
}

// The value of lane (lane ^ J) for J a power of two below 64, in vector registers
// only: DPP within rows of 16 lanes (xor 4 = half mirror then reversed quads, xor 8 =
// mirror then half mirror), the gfx950 permlane swaps across rows.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int lane) {
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor1, 0xf, 0xf, true);
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor2, 0xf, 0xf, true);
    } else if constexpr (J == 4) {
        const int m = __builtin_amdgcn_update_dpp(0, (int)v, kDppHalfMirror, 0xf, 0xf, true);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, m, kDppRevQuad, 0xf, 0xf, true);
    } else if constexpr (J == 8) {
        const int m = __builtin_amdgcn_update_dpp(0, (int)v, kDppMirror, 0xf, 0xf, true);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, m, kDppHalfMirror, 0xf, 0xf, true);
    } else if constexpr (J == 16) {
        const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? (uint32_t)a[0] : (uint32_t)a[1];
    } else {
        static_assert(J == 32, "lane distance");
        const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? (uint32_t)a[0] : (uint32_t)a[1];
    }
}

// One stage of a bitonic sort over the wave (ascending over lanes): blocks of KK lanes
// alternate direction, partners at distance J keep the smaller / larger key.
template <int KK, int J>
__device__ __forceinline__ uint32_t bitonic_stage(uint32_t key, int lane) {
    const uint32_t other = lane_xor<J>(key, lane);
    const bool up = (lane & KK) == 0, lower = (lane & J) == 0;
    return (lower == up) ? min(key, other) : max(key, other);
}

// Bucketing of up to 64 pairs by one wave (the same tables as bucket_pairs): lane q
// holds pair q as the key expert * 64 + q; a bitonic sort over the wave puts the keys
// in (expert, pair) order, so lane q then holds bucket position q; a bucket starts
// where the expert changes from the lane below.  Buckets are numbered in order of first
// appearance: a bucket's first pair is the first pair that picked its expert, and its
// slot is the number of buckets whose first pair comes earlier.  All 64 lanes of the
// wave must be active.
__device__ inline void bucket_pairs_wave(const int *ids, int NP, int E, int4 *slots, int *pairs,
                                         int *pos_expert, int *n_unique) {
    const int lane = threadIdx.x & 63;
    const int e0 = lane < NP ? ids[lane] : -1;
    uint32_t key = (e0 >= 0 && e0 < E) ? ((uint32_t)e0 << 6) | (uint32_t)lane : 0xffffffffu;
    key = bitonic_stage<2, 1>(key, lane);
    key = bitonic_stage<4, 2>(key, lane);
    key = bitonic_stage<4, 1>(key, lane);
    key = bitonic_stage<8, 4>(key, lane);
    key = bitonic_stage<8, 2>(key, lane);
    key = bitonic_stage<8, 1>(key, lane);
    key = bitonic_stage<16, 8>(key, lane);
    key = bitonic_stage<16, 4>(key, lane);
    key = bitonic_stage<16, 2>(key, lane);
    key = bitonic_stage<16, 1>(key, lane);
    key = bitonic_stage<32, 16>(key, lane);
    key = bitonic_stage<32, 8>(key, lane);
    key = bitonic_stage<32, 4>(key, lane);
    key = bitonic_stage<32, 2>(key, lane);
    key = bitonic_stage<32, 1>(key, lane);
    key = bitonic_stage<64, 32>(key, lane);
    key = bitonic_stage<64, 16>(key, lane);
    key = bitonic_stage<64, 8>(key, lane);
    key = bitonic_stage<64, 4>(key, lane);
    key = bitonic_stage<64, 2>(key, lane);
    key = bitonic_stage<64, 1>(key, lane);
    const bool ok = key != 0xffffffffu;
    const int e = (int)(key >> 6);
    const int below = __shfl_up(e, 1);
    const bool first = ok && (lane == 0 || below != e);
    const unsigned long long fm = __ballot(first);
    const int nvalid = __popcll(__ballot(ok));  // valid pairs: the last bucket ends there
    const int nb = __popcll(fm);
    const int q = (int)(key & 63u);
    if (ok) {
        pairs[lane] = q;
        pos_expert[lane] = e;
    }
    // each sorted lane tells the lane of its pair whether that pair opens a bucket (a
    // permutation of the wave: the lanes past the valid pairs keep their own), so that
    // bit q of `om` says whether pair q is the first of its expert
    const int opens = __builtin_amdgcn_ds_permute((ok ? q : lane) << 2, first ? 1 : 0);
    const unsigned long long om = __ballot(opens != 0 && lane < NP);
    if (first) {
        const int u = __popcll(om & ((1ull << q) - 1ull));
        const unsigned long long after = lane == 63 ? 0ull : fm & ~((2ull << lane) - 1ull);
        const int end = after ? (int)__builtin_ctzll(after) : nvalid;
        if (u < nb) slots[u] = make_int4(e, lane, end - lane, 0);
    }
    if (lane == 0) *n_unique = nb;
}

// Bucketing of all T*k pairs by one workgroup (any multiple of 64 threads up
// to 1024).  ids[], the scratch and the outputs are in LDS (the barriers
// inside order LDS accesses only).  Outputs:
// slots[u] = (expert, first position, count, 0) for used experts in order of first
// appearance (slot u is the expert of the u-th pair, in pair order, that is the first
// to pick its expert), pairs[pos] = t*k + j, pos_expert[pos], *n_unique.  Positions
// are expert-major (experts ascending), tokens ascending within an expert; a token's
// rank in its expert's bucket is the number of earlier tokens in the expert's token
// bitmap (a token picks an expert at most once).  Integer only: the result is unique.
__device__ void bucket_pairs(const int *ids, int T, int k, int E, uint32_t *scratch, int4 *slots,
                             int *pairs, int *pos_expert, int *n_unique) {
    const int nth = blockDim.x, nw = nth >> 6;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NP = T * k, W = (T + 31) / 32;
    const int NW = (NP + 31) / 32;
    uint32_t *mask = scratch;                     // [E][W] token bitmaps
    int *cnt = (int *)(mask + (size_t)E * W);     // [E]
    int *off = cnt + E;                           // [E] first position of expert e
    int *wtot = off + E;                          // [2 * 16] wave totals
    int *fq = wtot + 32;                          // [E] first pair of expert e
    uint32_t *fbits = (uint32_t *)(fq + E);       // [NW] bit q: pair q is the first of its expert
    for (int i = tid; i < E * W; i += nth) mask[i] = 0u;
    for (int i = tid; i < NW; i += nth) fbits[i] = 0u;
    lds_barrier();
    for (int q = tid; q < NP; q += nth) {
        const int t = q / k, e = ids[q];
        if (e >= 0 && e < E) atomicOr(&mask[e * W + (t >> 5)], 1u << (t & 31));
    }
    lds_barrier();
    for (int e = tid; e < E; e += nth) {
        int c = 0, t0 = -1;
        for (int w = 0; w < W; ++w) {
            const uint32_t m = mask[e * W + w];
            c += __popc(m);
            if (t0 < 0 && m) t0 = 32 * w + __builtin_ctz(m);
        }
        cnt[e] = c;
        int q0 = -1;  // the first token that picked e, at the slot where it did
        for (int jj = 0; t0 >= 0 && jj < k && q0 < 0; ++jj)
            if (ids[t0 * k + jj] == e) q0 = t0 * k + jj;
        fq[e] = q0;
        if (q0 >= 0) atomicOr(&fbits[q0 >> 5], 1u << (q0 & 31));
    }
    lds_barrier();
    // exclusive scans of cnt[] and (cnt[] > 0); thread owns EPT consecutive experts
    const int EPT = (E + nth - 1) / nth;
    int a = 0, b = 0;
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        if (e < E) { a += cnt[e]; b += cnt[e] > 0; }
    }
    const int ia = wave_incl_scan(a, lane), ib = wave_incl_scan(b, lane);
    if (lane == 63) { wtot[wave] = ia; wtot[16 + wave] = ib; }
    lds_barrier();
    int ba = ia - a;
    for (int w = 0; w < wave; ++w) ba += wtot[w];
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        if (e < E) {
            off[e] = ba;
            const int q0 = fq[e];
            if (cnt[e] > 0 && q0 >= 0 && q0 < NP) {
                // slot = first pairs of other experts that come before this one's
                int u = __popc(fbits[q0 >> 5] & ((1u << (q0 & 31)) - 1u));
                for (int w = 0; w < (q0 >> 5); ++w) u += __popc(fbits[w]);
                slots[u] = make_int4(e, ba, cnt[e], 0);
            }
            ba += cnt[e];
        }
    }
    if (tid == nth - 1) {
        int nu = 0;
        for (int w = 0; w < nw; ++w) nu += wtot[16 + w];
        *n_unique = nu;
    }
    lds_barrier();
    for (int q = tid; q < NP; q += nth) {
        const int t = q / k, e = ids[q];
        if (e < 0 || e >= E) continue;
        const uint32_t *me = mask + e * W;
        int rank = __popc(me[t >> 5] & ((1u << (t & 31)) - 1u));
        for (int w = 0; w < (t >> 5); ++w) rank += __popc(me[w]);
        const int pos = off[e] + rank;
        pairs[pos] = q;
        pos_expert[pos] = e;
    }
}

// ---- one workgroup routes a whole batch ------------------------------------------------

// LDS layout of the routing work area (byte offsets from its start).  With
// local tables the weights, gates and a copy of the batch's logits also live in LDS
// (a workgroup that routes for its own use, reading its jobs from the bucket slots);
// without, they only go to memory.  Job records only ever go to memory.
struct RouteLds {
    size_t ids, pairs, pose, nu, slots, scratch, w, g, lgt, bytes;
    bool local;
};

// A local routing workgroup (the gate/up launch) ranks from a copy of the batch's
// logits rows in LDS (its lgt region), loaded with one memory round trip ahead of
// every other load of the workgroup.

__host__ __device__ inline RouteLds route_lds_layout(int T, int k, int E, bool local) {
    const size_t np = (size_t)T * k, ns = (size_t)(E < T * k ? E : T * k);
    RouteLds L{};
    L.local = local;
    size_t o = 0;
    L.ids = o;     o += np * 4;
    L.pairs = o;   o += np * 4;
    L.pose = o;    o += np * 4;
    L.nu = o;      o += 16;
    o = (o + 15) & ~(size_t)15;
    L.slots = o;   o += ns * 16;
    L.scratch = o; o += (size_t)bucket_scratch_ints(E, T, k) * 4;
    o = (o + 15) & ~(size_t)15;
    L.w = o;       o += np * 4;
    L.g = o;       o += (size_t)T * 4;
    o = (o + 15) & ~(size_t)15;
    L.lgt = o;     o += local ? (size_t)T * logit_stride(E) * 4 : 0;
    L.bytes = (o + 15) & ~(size_t)15;
    return L;
}

// Where a routing result goes besides LDS (global tables; NULL = nowhere).
struct RouteGlobal {
    int *ids;
    float *wts;
    float *gate_s;
    int *records;
    int *n_unique;
    int *pairs;
    int *pos_expert;
    int32_t *dbg_ids;
    float *dbg_w, *dbg_logits, *dbg_gate;
};

// Ranks tokens [t_lo, t_hi) (waves take them in turn) into the LDS ids; weights and
// gates go to g when g.wts is set, else to LDS.  logits: row 0 of the [T][stride]
// table, in memory or in LDS.  No barrier inside.
__device__ inline void rank_tokens(const float *logits, int t_lo, int t_hi, int E, int k, uint8_t *area,
                                   const RouteLds &L, const RouteGlobal &g) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int *ids = reinterpret_cast<int *>(area + L.ids);
    float *lw = reinterpret_cast<float *>(area + L.w);
    float *lg = reinterpret_cast<float *>(area + L.g);
    for (int t = wave; t < t_hi; t += nw) {  // token t on wave t % nw, from t_lo on
        if (t < t_lo) continue;
        // every output goes to LDS (one known address space: a store through a pointer that
        // may be LDS or memory is a flat store, and waiting for one waits for every load in
        // flight); the publishing workgroup copies the tables to memory after the bucketing
        RouteOut o{ids + t * k, lw + t * k, lg + t,
                   g.dbg_ids ? g.dbg_ids + t * k : nullptr, g.dbg_w ? g.dbg_w + t * k : nullptr,
                   g.dbg_gate ? g.dbg_gate + t : nullptr,
                   g.dbg_logits ? g.dbg_logits + (size_t)t * E : nullptr};
        route_token_any(logits + (size_t)t * logit_stride(E), E, k, lane, o);
    }
}

// With every id in LDS: buckets the pairs into the LDS slots and pairs
// (expert-ascending buckets; a single token's buckets follow its rank order);
// builds the job records in g.records and copies the tables to g where its
// pointers are set.  Barriers inside: call from every thread of the workgroup.
// Returns the used-expert count.
// WAVE_ONLY: the caller guarantees T * k <= 64 (the workgroup bucketing is left out).
template <bool WAVE_ONLY = false>
__device__ inline int bucket_tokens(int T, int k, int E, uint8_t *area, const RouteLds &L,
                                    const RouteGlobal &g) {
    const int tid = threadIdx.x, NP = T * k;
    int *ids = reinterpret_cast<int *>(area + L.ids);
    int *pairs = reinterpret_cast<int *>(area + L.pairs);
    int *pose = reinterpret_cast<int *>(area + L.pose);
    int *nup = reinterpret_cast<int *>(area + L.nu);
    int4 *slots = reinterpret_cast<int4 *>(area + L.slots);
    lds_barrier();
    if (T == 1) {  // one token: its k picks are k distinct experts, one bucket each, in rank order
        if (threadIdx.x < 64) {
            const int j = threadIdx.x;
            if (j < k) {
                const int e = ids[j];
                slots[j] = make_int4(e, j, 1, 0);
                pairs[j] = j;
                pose[j] = e;
            }
            if (j == 0) *nup = k;
        }
    } else if (WAVE_ONLY || NP <= 64) {  // one wave sorts the pairs (no barrier inside)
        if (threadIdx.x < 64) bucket_pairs_wave(ids, NP, E, slots, pairs, pose, nup);
    } else {
        bucket_pairs(ids, T, k, E, reinterpret_cast<uint32_t *>(area + L.scratch), slots, pairs, pose, nup);
    }
    lds_barrier();
    const int nu = *nup;
    for (int i = tid; g.records && i < nu * kRecInts; i += blockDim.x) {
        const int u = i / kRecInts, f = i - u * kRecInts;
        const int4 sv = slots[u];
        int v;
        if (f == 0) v = sv.x;
        else if (f == 1) v = sv.y;
        else if (f == 2) v = sv.z;
        else if (f == 3) v = 0;
        else v = (f - 4 < sv.z) ? pairs[sv.y + f - 4] : -1;
        g.records[i] = v;
    }
    if (g.ids) {
        const float *lw = reinterpret_cast<const float *>(area + L.w);
        const float *lg = reinterpret_cast<const float *>(area + L.g);
        for (int i = tid; i < NP; i += blockDim.x) {
            g.ids[i] = ids[i];
            g.wts[i] = lw[i];
            g.pairs[i] = pairs[i];
            g.pos_expert[i] = pose[i];
        }
        for (int i = tid; i < T; i += blockDim.x) g.gate_s[i] = lg[i];
    }
    if (g.n_unique && tid == 0) *g.n_unique = nu;
    lds_barrier();
    return nu;
}

}  // namespace moeffn
